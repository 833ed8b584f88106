// fa_bwd.hip -- fused exact attention backward for gfx950.
//
// Gradient of L = sum(dO * O) for O = softmax(scale * Q K^T [+ causal]) V
// (chain rule of the attention the FlashAttention-4 pages compute; the
// backward is described in the gist.science technical summary,
// methodology item 3):
//   D_i = sum_k dO_ik O_ik                                  (preprocess)
//   P   = exp(scale * Q K^T - LSE)  recomputed tile by tile
//   dV  = P^T dO,  dP = dO V^T,  dS = P o (dP - D)
//   dK  = scale * dS^T Q                                    (dK/dV kernel)
//   dQ  = scale * dS K                                      (dQ kernel)
//
// Why two kernels and no atomics.  The pages accumulate dQ with global
// atomic adds (and halve their number on Blackwell by exchanging half tiles
// between a pair of CTAs).  On MI355X fp32 atomics are executed past the
// per-XCD L2 at about 1.36 TB/s: with 128-key blocks the dQ atomics of one
// S = 32768, 16-head backward are 68.7 GB, about 50 ms of atomic traffic,
// more than the whole compute.  So dQ gets its own pass, parallel over query
// blocks like the forward, which recomputes S and dP (7 MFMA contractions
// instead of 5) but writes dQ once with plain stores.  The backward is then
// free of atomics and bitwise deterministic.
//
// dK/dV kernel: one workgroup = 4 waves = 128 key rows (32 per wave); K and
// V rows stay resident as MFMA B operands in registers, dK and dV
// accumulate in registers; query blocks of 64 rows (Q, dO, LSE, D) stream
// through a double-buffered LDS stage filled by direct memory-to-LDS copies.
// Per wave and block: S = Q K^T and dP = dO V^T (keys on the lanes), P and
// dS in registers, dV += P^T dO and dK += dS^T Q with P and dS fed straight
// from the accumulators and dO, Q through transposing LDS reads.
//
// dQ kernel: one workgroup = 4 waves = 128 query rows (32 per wave), two
// workgroups per CU; Q and dO rows resident as B operands, keys/values
// streamed through LDS as in the forward.  Per wave and 64-key tile:
// S^T = K Q^T, dP^T = V dO^T (queries on the lanes, so LSE and D are per
// lane), dS^T in registers, dQ^T += K^T dS^T with K^T by transposing reads.
//
// scale is folded into dS once, so dK and dQ need no epilogue scaling.
// Causal: key blocks only meet query blocks at or below the diagonal; both
// kernels order workgroup ids so the longest blocks start first (LPT,
// technical summary, results).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kKvPerBlock = 128;  // dK/dV kernel: key rows per workgroup
constexpr int kQPerIter = 64;     // dK/dV kernel: query rows per iteration
constexpr int kQPerBlock = 128;   // dQ kernel: query rows per workgroup
constexpr int kKvPerTile = 64;    // dQ kernel: key rows per tile

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const uint16_t *__restrict__ O,
                                                           const uint16_t *__restrict__ dO,
                                                           float *__restrict__ Dvec, int64_t rows) {
    constexpr int LPR = D / 8;  // lanes per row, 8 elements each
    constexpr int RPB = kThreads / LPR;
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
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && part == 0) Dvec[row] = acc;
}

// ---------------------------------------------------------------- dK, dV
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ LSE, const float *__restrict__ Dvec, const uint16_t *__restrict__ dO,
    uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int BH, int S, float scale, float c) {
    constexpr int ROWB = D * 2;
    constexpr int NCH = ROWB / 16;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int QTILE = kQPerIter * ROWB;

    __shared__ __attribute__((aligned(1024))) char smem_raw[4 * QTILE + 4 * kQPerIter * 4];
    fa_lds_char *smem = (fa_lds_char *)smem_raw;
    fa_lds_char *sQ0 = smem;                     // [2] Q tiles
    fa_lds_char *sO0 = sQ0 + 2 * QTILE;          // [2] dO tiles
    fa_lds_char *sLD = sO0 + 2 * QTILE;          // [2][LSE 64 | D 64] floats

    const int lane = threadIdx.x & 63, w = wave_id();
    const int h = lane >> 5, n = lane & 31;

    const int bh = blockIdx.x % BH;
    const int kblk = blockIdx.x / BH;
    const int k0 = kblk * kKvPerBlock;
    const size_t head = (size_t)bh * (size_t)S * D;
    const int kv = k0 + 32 * w + n;  // this lane's key for S and dP

    const uint32_t head_bytes = (uint32_t)S * ROWB;
    const fa_rsrc rQ = make_rsrc(Q + head, head_bytes);
    const fa_rsrc rK = make_rsrc(K + head, head_bytes);
    const fa_rsrc rV = make_rsrc(V + head, head_bytes);
    const fa_rsrc rdO = make_rsrc(dO + head, head_bytes);
    const fa_rsrc rL = make_rsrc(LSE + (size_t)bh * S, (uint32_t)S * 4);
    const fa_rsrc rD = make_rsrc(Dvec + (size_t)bh * S, (uint32_t)S * 4);

    // Resident B operands: K[kv][16ks + 8h ..] and V[kv][..] (zero past S).
    fa_u32x4 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint32_t off = (uint32_t)kv * ROWB + (16 * ks + 8 * h) * 2;
        kf[ks] = buf_load16(rK, off);
        vf[ks] = buf_load16(rV, off);
    }

    fa_f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) {
        dkacc[i] = zero16();
        dvacc[i] = zero16();
    }

    const int nqb = (S + kQPerIter - 1) / kQPerIter;
    const int ib = CAUSAL ? k0 / kQPerIter : 0;

    // Query block i -> LDS stage: Q and dO tiles (all waves), LSE (wave 0)
    // and D (wave 1).  Rows past S arrive as zeros; such rows then carry
    // dO = 0 and D = 0, so they add nothing to dV or dK.
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
        wait_vmem();      // next query block has landed
        __syncthreads();  // ... for every wave, and this block's stage is free
    }

    // Epilogue: dK, dV rows of this workgroup (lane = d column, registers = keys).
    const fa_rsrc rdK = make_rsrc(dK + head, head_bytes);
    const fa_rsrc rdV = make_rsrc(dV + head, head_bytes);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kr = k0 + 32 * w + 8 * (r >> 2) + 4 * h + (r & 3);
            const uint32_t off = ((uint32_t)kr * D + 32 * db + n) * 2;
            buf_store2(rdK, off, (uint16_t)(pack_bf16(dkacc[db][r], 0.0f) & 0xFFFFu));
            buf_store2(rdV, off, (uint16_t)(pack_bf16(dvacc[db][r], 0.0f) & 0xFFFFu));
        }
    }
}

// ---------------------------------------------------------------- dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ LSE, const float *__restrict__ Dvec, const uint16_t *__restrict__ dO,
    float *__restrict__ dQ, int BH, int S, float scale, float c, int nqb) {
    constexpr int ROWB = D * 2;
    constexpr int NCH = ROWB / 16;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int TILE = kKvPerTile * ROWB;

    __shared__ __attribute__((aligned(1024))) char smem_raw[2 * 2 * TILE];
    fa_lds_char *smem = (fa_lds_char *)smem_raw;

    const int lane = threadIdx.x & 63, w = wave_id();
    const int h = lane >> 5, n = lane & 31;

    const int bh = blockIdx.x % BH;
    const int qi = blockIdx.x / BH;
    const int qblk = CAUSAL ? (nqb - 1 - qi) : qi;
    const int q0 = qblk * kQPerBlock;
    const size_t head = (size_t)bh * (size_t)S * D;
    const int kv_end = CAUSAL ? min(S, q0 + kQPerBlock) : S;
    const int nkv = (kv_end + kKvPerTile - 1) / kKvPerTile;
    const int qrow = q0 + 32 * w + n;
    const int wq_lo = q0 + 32 * w;

    const uint32_t head_bytes = (uint32_t)S * ROWB;
    const fa_rsrc rQ = make_rsrc(Q + head, head_bytes);
    const fa_rsrc rK = make_rsrc(K + head, head_bytes);
    const fa_rsrc rV = make_rsrc(V + head, head_bytes);
    const fa_rsrc rdO = make_rsrc(dO + head, head_bytes);

    // Q^T and dO^T as B operands (queries on the lanes); rows past S are
    // zero, and LSE = D = 0 there, so their dS is exactly 0.
    fa_u32x4 qf[KS], of[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint32_t off = (uint32_t)qrow * ROWB + (16 * ks + 8 * h) * 2;
        qf[ks] = buf_load16(rQ, off);
        of[ks] = buf_load16(rdO, off);
    }
    const float lse2 =
        buf_load4f(make_rsrc(LSE + (size_t)bh * S, (uint32_t)S * 4), (uint32_t)qrow * 4) * FA_LOG2E;
    const float dd = buf_load4f(make_rsrc(Dvec + (size_t)bh * S, (uint32_t)S * 4), (uint32_t)qrow * 4);

    fa_f32x16 dqacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) dqacc[i] = zero16();

    auto issue_tile = [&](int j, int buf) {
        fa_lds_char *sK = smem + buf * 2 * TILE;
        tile_to_lds<NCH, kKvPerTile>(rK, j * kKvPerTile, sK, w, lane);
        tile_to_lds<NCH, kKvPerTile>(rV, j * kKvPerTile, sK + TILE, w, lane);
    };

    if (nkv > 0) issue_tile(0, 0);
    wait_vmem();
    __syncthreads();

    for (int j = 0; j < nkv; ++j) {
        const int buf = j & 1;
        if (j + 1 < nkv) issue_tile(j + 1, buf ^ 1);
        const fa_lds_char *sK = smem + buf * 2 * TILE;
        const fa_lds_char *sV = sK + TILE;
        const int kv0 = j * kKvPerTile;
        const bool skip = CAUSAL && (kv0 > wq_lo + 31);

        if (!skip) {
            // S^T = K Q^T and dP^T = V dO^T: 64 keys x 32 queries each.
            fa_f32x16 sacc[2] = {zero16(), zero16()};
            fa_f32x16 pacc[2] = {zero16(), zero16()};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const int off = tile_off<NCH>(32 * mb + n, (2 * ks + h) * 16);
                    sacc[mb] = mfma32(lds_read16(sK, off), qf[ks], sacc[mb]);
                    pacc[mb] = mfma32(lds_read16(sV, off), of[ks], pacc[mb]);
                }
            }
            const bool need_mask = (CAUSAL && (kv0 + kKvPerTile - 1 > wq_lo)) || (kv0 + kKvPerTile > S);
            fa_u32x4 dsf[4];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float ds[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        float pv = __builtin_amdgcn_exp2f(fmaf(sacc[mb][r + e], c, -lse2));
                        if (need_mask) {
                            const int key = kv0 + 32 * mb + 8 * ((r + e) >> 2) + 4 * h + ((r + e) & 3);
                            const bool dead = (CAUSAL && key > qrow) || key >= S;
                            pv = dead ? 0.0f : pv;
                        }
                        ds[e] = pv * (pacc[mb][r + e] - dd) * scale;
                    }
                    dsf[2 * mb + (r >> 3)][(r & 7) >> 1] = pack_bf16(ds[0], ds[1]);
                }
            }
            // dQ^T += K^T dS^T, keys of k-step t in accumulator order.
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int rbase = 16 * t + 4 * h;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    dqacc[db] = mfma32(operand_tr<NCH>(sK, rbase, rbase + 8, 32 * db, lane), dsf[t], dqacc[db]);
            }
        }
        wait_vmem();
        __syncthreads();
    }

    // Epilogue: lane = query row, registers = 4 consecutive d per group.
    const fa_rsrc rdQ = make_rsrc(dQ + head, (uint32_t)S * D * 4);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            fa_u32x4 v = {__float_as_uint(dqacc[db][4 * g]), __float_as_uint(dqacc[db][4 * g + 1]),
                          __float_as_uint(dqacc[db][4 * g + 2]), __float_as_uint(dqacc[db][4 * g + 3])};
            buf_store16(rdQ, ((uint32_t)qrow * D + 32 * db + 8 * g + 4 * h) * 4, v);
        }
}

template <int D>
hipError_t launch_pre_d(const BwdArgs &a, hipStream_t st) {
    constexpr int RPB = kThreads / (D / 8);
    const int64_t rows = (int64_t)a.BH * a.S;
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(kThreads);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), grid, block, 0, st, (const uint16_t *)a.O,
                       (const uint16_t *)a.dO, a.Dvec, rows);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_t(const BwdArgs &a, hipStream_t st) {
    const int nkb = (a.S + kKvPerBlock - 1) / kKvPerBlock;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * nkb)), dim3(kThreads), 0, st,
                       (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V, a.LSE,
                       (const float *)a.Dvec, (const uint16_t *)a.dO, (uint16_t *)a.dK, (uint16_t *)a.dV,
                       a.BH, a.S, a.scale, a.scale * FA_LOG2E);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const BwdArgs &a, hipStream_t st) {
    const int nqb = (a.S + kQPerBlock - 1) / kQPerBlock;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * nqb)), dim3(kThreads), 0, st,
                       (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V, a.LSE,
                       (const float *)a.Dvec, (const uint16_t *)a.dO, a.dQ, a.BH, a.S, a.scale,
                       a.scale * FA_LOG2E, nqb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const BwdArgs &a, hipStream_t st) {
    return a.d == 128 ? launch_pre_d<128>(a, st) : launch_pre_d<64>(a, st);
}

hipError_t launch_bwd_dkdv(const BwdArgs &a, hipStream_t st) {
    if (a.d == 128) return a.causal ? launch_dkdv_t<128, true>(a, st) : launch_dkdv_t<128, false>(a, st);
    return a.causal ? launch_dkdv_t<64, true>(a, st) : launch_dkdv_t<64, false>(a, st);
}

hipError_t launch_bwd_dq(const BwdArgs &a, hipStream_t st) {
    if (a.d == 128) return a.causal ? launch_dq_t<128, true>(a, st) : launch_dq_t<128, false>(a, st);
    return a.causal ? launch_dq_t<64, true>(a, st) : launch_dq_t<64, false>(a, st);
}

}  // namespace fa
