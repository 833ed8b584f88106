// fa_bwd.hip -- fused exact attention backward for gfx950.
//
// Gradient of L = sum(dO * O) for O = softmax(scale * Q K^T [+ causal]) V
// (chain rule of the attention the FlashAttention-4 pages compute; the
// backward is described in the gist.science technical summary,
// methodology item 3):
//   D_i = sum_k dO_ik O_ik                         (preprocess kernel)
//   P   = exp(scale * Q K^T - LSE)  recomputed tile by tile
//   dV  = P^T dO,  dP = dO V^T,  dS = P o (dP - D)
//   dQ  = scale * dS K   (global fp32 atomic adds),  dK = scale * dS^T Q
//
// Work decomposition of the main kernel
//   * one workgroup = 4 waves = 128 key/value rows (32 per wave) of one head;
//     it keeps its K and V rows resident (as MFMA B operands in registers,
//     and K once more in LDS for the dQ product) and its dK, dV
//     accumulators in registers, and streams query blocks of 64 rows;
//   * per query block: Q, dO, LSE, D copied straight from memory into a
//     double-buffered LDS stage (buffer_load ... lds); per wave
//     S = Q K^T and dP = dO V^T (keys on the lanes), P and dS in registers,
//     dV += P^T dO and dK += dS^T Q with P, dS straight from the
//     accumulators and dO, Q through transposing LDS reads; dS^T goes to
//     LDS, and each wave then forms a 64 x 32 slice of dS K and adds it to
//     dQ with fp32 atomics;
//   * scale is folded into dS once, so dK and dQ need no epilogue scaling;
//   * causal: a key block only meets query blocks at or below its diagonal;
//     workgroup ids are ordered so the longest key blocks (the first ones)
//     start first (LPT, technical summary, results).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBwdThreads = 256;
constexpr int kKvPerBlock = 128;  // key rows per workgroup
constexpr int kQPerIter = 64;     // query rows per iteration

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_pre_kernel(const uint16_t *__restrict__ O,
                                                              const uint16_t *__restrict__ dO,
                                                              float *__restrict__ Dvec,
                                                              float *__restrict__ dQ, int64_t rows) {
    constexpr int LPR = D / 8;  // lanes per row, 8 elements each
    constexpr int RPB = kBwdThreads / LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    float acc = 0.0f;
    if (row < rows) {
        const fa_u32x4 o = *(const fa_u32x4 *)(O + row * D + part * 8);
        const fa_u32x4 g = *(const fa_u32x4 *)(dO + row * D + part * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fmaf(bf16_lo(o[i]), bf16_lo(g[i]), acc);
            acc = fmaf(bf16_hi(o[i]), bf16_hi(g[i]), acc);
        }
        const fa_f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        fa_f32x4 *dq = (fa_f32x4 *)(dQ + row * D + part * 8);
        dq[0] = z;
        dq[1] = z;
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && part == 0) Dvec[row] = acc;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ LSE, const float *__restrict__ Dvec, const uint16_t *__restrict__ dO,
    float *__restrict__ dQ, uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int BH, int S,
    float scale, float c) {
    constexpr int ROWB = D * 2;
    constexpr int NCH = ROWB / 16;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int QTILE = kQPerIter * ROWB;
    constexpr int KTILE = kKvPerBlock * ROWB;
    constexpr int DSTILE = kKvPerBlock * kQPerIter * 2;  // dS^T: 128 key rows x 64 queries

    __shared__ __attribute__((aligned(1024))) char smem_raw[KTILE + 4 * QTILE + DSTILE + 4 * kQPerIter * 4];
    fa_lds_char *smem = (fa_lds_char *)smem_raw;
    fa_lds_char *sK = smem;
    fa_lds_char *sQ0 = smem + KTILE;             // [2] Q tiles
    fa_lds_char *sO0 = sQ0 + 2 * QTILE;          // [2] dO tiles
    fa_lds_char *sdS = sO0 + 2 * QTILE;          // dS^T tile
    fa_lds_char *sLD = sdS + DSTILE;             // [2][LSE 64 | D 64] floats

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int h = lane >> 5, n = lane & 31;

    const int bh = blockIdx.x % BH;
    const int kblk = blockIdx.x / BH;
    const int k0 = kblk * kKvPerBlock;
    const size_t head = (size_t)bh * (size_t)S * D;
    const int kv = k0 + 32 * w + n;  // this lane's key for S and dP

    // Per-head buffer resources (rows at or past S read as zero, are never written).
    const uint32_t head_bytes = (uint32_t)S * ROWB;
    const fa_rsrc rQ = make_rsrc(Q + head, head_bytes);
    const fa_rsrc rK = make_rsrc(K + head, head_bytes);
    const fa_rsrc rV = make_rsrc(V + head, head_bytes);
    const fa_rsrc rdO = make_rsrc(dO + head, head_bytes);
    const fa_rsrc rL = make_rsrc(LSE + (size_t)bh * S, (uint32_t)S * 4);
    const fa_rsrc rD = make_rsrc(Dvec + (size_t)bh * S, (uint32_t)S * 4);
    const fa_rsrc rdQ = make_rsrc(dQ + head, (uint32_t)S * D * 4);

    // Resident B operands: K[kv][16ks + 8h ..] and V[kv][..]; K tile in LDS
    // for the dQ product.
    fa_u32x4 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint32_t off = (uint32_t)kv * ROWB + (16 * ks + 8 * h) * 2;
        kf[ks] = buf_load16(rK, off);
        vf[ks] = buf_load16(rV, off);
    }
    tile_to_lds<NCH, kKvPerBlock>(rK, k0, sK, w, lane);

    fa_f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) {
        dkacc[i] = zero16();
        dvacc[i] = zero16();
    }

    const int nqb = (S + kQPerIter - 1) / kQPerIter;
    const int ib = CAUSAL ? k0 / kQPerIter : 0;

    // Query block i -> LDS buffer: Q and dO tiles (all waves), LSE (wave 0)
    // and D (wave 1).  Rows past S arrive as zeros; such rows then carry
    // dO = 0 and D = 0, so they add nothing to dV, dK or dS.
    auto issue = [&](int i, int buf) {
        tile_to_lds<NCH, kQPerIter>(rQ, i * kQPerIter, sQ0 + buf * QTILE, w, lane);
        tile_to_lds<NCH, kQPerIter>(rdO, i * kQPerIter, sO0 + buf * QTILE, w, lane);
        if (w < 2) {
            fa_lds_char *dst = sLD + (buf * 2 + w) * kQPerIter * 4;
            buf_load_lds<4>(w == 0 ? rL : rD, dst, (uint32_t)(i * kQPerIter + lane) * 4);
        }
    };

    if (ib < nqb) issue(ib, 0);
    wait_vmem();
    __syncthreads();

    for (int i = ib; i < nqb; ++i) {
        const int buf = (i - ib) & 1;
        if (i + 1 < nqb) issue(i + 1, buf ^ 1);
        const int q0 = i * kQPerIter;
        const fa_lds_char *sQ = sQ0 + buf * QTILE;
        const fa_lds_char *sO = sO0 + buf * QTILE;
        const fa_lds_char *sL = sLD + buf * 2 * kQPerIter * 4;
        const fa_lds_char *sD = sL + kQPerIter * 4;

        // S = Q K^T and dP = dO V^T: 64 queries x this wave's 32 keys.
        fa_f32x16 sacc[2] = {zero16(), zero16()};
        fa_f32x16 pacc[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int off = tile_off<NCH>(32 * qb + n, (2 * ks + h) * 16);
                sacc[qb] = mfma32(lds_read16(sQ, off), kf[ks], sacc[qb]);
                pacc[qb] = mfma32(lds_read16(sO, off), vf[ks], pacc[qb]);
            }
        }

        // P = 2^(s c - LSE log2 e) (masked -> 0), dS = scale P (dP - D).
        const bool need_mask = (CAUSAL && q0 < k0 + kKvPerBlock - 1) || (k0 + kKvPerBlock > S);
        fa_u32x4 pf[4], dsf[4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int qi = 32 * qb + 8 * g + 4 * h;
                const fa_f32x4 l4 = *(const __attribute__((address_space(3))) fa_f32x4 *)(sL + qi * 4);
                const fa_f32x4 d4 = *(const __attribute__((address_space(3))) fa_f32x4 *)(sD + qi * 4);
                float p[4], ds[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    float pv = __builtin_amdgcn_exp2f(fmaf(sacc[qb][r], c, -l4[e] * FA_LOG2E));
                    if (need_mask) {
                        const int q = q0 + qi + e;
                        const bool dead = (CAUSAL && kv > q) || kv >= S;
                        pv = dead ? 0.0f : pv;
                    }
                    p[e] = pv;
                    ds[e] = pv * (pacc[qb][r] - d4[e]) * scale;
                }
                const int t = 2 * qb + (g >> 1);
                const int wd = (g & 1) * 2;
                pf[t][wd] = pack_bf16(p[0], p[1]);
                pf[t][wd + 1] = pack_bf16(p[2], p[3]);
                dsf[t][wd] = pack_bf16(ds[0], ds[1]);
                dsf[t][wd + 1] = pack_bf16(ds[2], ds[3]);
                // dS^T row (this key), queries qi .. qi+3
                const fa_u32x2 v = {dsf[t][wd], dsf[t][wd + 1]};
                lds_write8(sdS, tile_off<8>(32 * w + n, qi * 2), v);
            }
        }

        // dV += P^T dO and dK += dS^T Q; query order of k-step t follows the
        // accumulator rows: 16t + 8(j/4) + 4h + j%4.
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int rbase = 16 * t + 4 * h;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                dvacc[db] = mfma32(pf[t], operand_tr<NCH>(sO, rbase, rbase + 8, 32 * db, lane), dvacc[db]);
                dkacc[db] = mfma32(dsf[t], operand_tr<NCH>(sQ, rbase, rbase + 8, 32 * db, lane), dkacc[db]);
            }
        }
        __syncthreads();  // dS^T of all four waves is in LDS

        // dQ slice of this wave: d = 128 -> (d block w, both query blocks);
        // d = 64 -> (query block w/2, d block w%2).  Keys in natural order.
        constexpr int NQB = (DB == 4) ? 2 : 1;
        fa_f32x16 dqacc[NQB];
#pragma unroll
        for (int u = 0; u < NQB; ++u) {
            const int qb = (DB == 4) ? u : (w >> 1);
            const int db = (DB == 4) ? w : (w & 1);
            dqacc[u] = zero16();
#pragma unroll
            for (int ks = 0; ks < kKvPerBlock / 16; ++ks) {
                const int r0 = 16 * ks + 8 * h;
                const fa_u32x4 a = operand_tr<8>(sdS, r0, r0 + 4, 32 * qb, lane);
                const fa_u32x4 b = operand_tr<NCH>(sK, r0, r0 + 4, 32 * db, lane);
                dqacc[u] = mfma32(a, b, dqacc[u]);
            }
        }
        wait_vmem();      // next query block landed (and older dQ atomics retired)
        __syncthreads();  // ... for every wave; dS^T and this block's tiles are free

        // dQ += partial, fp32 atomics; rows past S fall outside the resource.
#pragma unroll
        for (int u = 0; u < NQB; ++u) {
            const int qb = (DB == 4) ? u : (w >> 1);
            const int db = (DB == 4) ? w : (w & 1);
            const uint32_t base = ((uint32_t)(q0 + 32 * qb) * D + 32 * db + n) * 4;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qr = 8 * (r >> 2) + 4 * h + (r & 3);
                buf_atomic_add(rdQ, base + (uint32_t)qr * D * 4, dqacc[u][r]);
            }
        }
    }

    // Epilogue: dK, dV rows of this workgroup (lane = d column, registers = keys).
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kr = k0 + 32 * w + 8 * (r >> 2) + 4 * h + (r & 3);
            const uint32_t off = ((uint32_t)kr * D + 32 * db + n) * 2;
            buf_store2(make_rsrc(dK + head, head_bytes), off, (uint16_t)(pack_bf16(dkacc[db][r], 0.0f) & 0xFFFFu));
            buf_store2(make_rsrc(dV + head, head_bytes), off, (uint16_t)(pack_bf16(dvacc[db][r], 0.0f) & 0xFFFFu));
        }
    }
}

template <int D>
hipError_t launch_pre_d(const BwdArgs &a, hipStream_t st) {
    constexpr int RPB = kBwdThreads / (D / 8);
    const int64_t rows = (int64_t)a.BH * a.S;
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(kBwdThreads);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), grid, block, 0, st, (const uint16_t *)a.O,
                       (const uint16_t *)a.dO, a.Dvec, a.dQ, rows);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_main_t(const BwdArgs &a, hipStream_t st) {
    const int nkb = (a.S + kKvPerBlock - 1) / kKvPerBlock;
    const dim3 grid((unsigned)(a.BH * nkb)), block(kBwdThreads);
    hipLaunchKernelGGL((bwd_kernel<D, CAUSAL>), grid, block, 0, st, (const uint16_t *)a.Q,
                       (const uint16_t *)a.K, (const uint16_t *)a.V, a.LSE, (const float *)a.Dvec,
                       (const uint16_t *)a.dO, a.dQ, (uint16_t *)a.dK, (uint16_t *)a.dV, a.BH, a.S,
                       a.scale, a.scale * FA_LOG2E);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const BwdArgs &a, hipStream_t st) {
    return a.d == 128 ? launch_pre_d<128>(a, st) : launch_pre_d<64>(a, st);
}

hipError_t launch_bwd_main(const BwdArgs &a, hipStream_t st) {
    if (a.d == 128) return a.causal ? launch_main_t<128, true>(a, st) : launch_main_t<128, false>(a, st);
    return a.causal ? launch_main_t<64, true>(a, st) : launch_main_t<64, false>(a, st);
}

}  // namespace fa
