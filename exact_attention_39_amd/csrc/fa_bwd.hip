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
// dK/dV kernel: one workgroup = 8 waves = 256 key rows; each wave owns 32
// keys and takes the two 32-row halves of every 64-row query block in turn,
// two waves per SIMD overlapping MFMA with softmax work.  Each wave's K and
// V rows sit in registers (loaded once: the B operands of S = Q K^T and
// dP = dO V^T), dK and dV accumulate in registers; query blocks (Q, dO,
// LSE, D) stream through a double-buffered LDS stage filled by direct
// memory-to-LDS copies, one barrier per 64 queries x 256 keys.  Per wave and half block: S = Q K^T
// and dP = dO V^T (keys on the lanes), P and dS in registers, dV += P^T dO
// and dK += dS^T Q with P and dS fed straight from the accumulators and dO,
// Q through transposing LDS reads.
//
// dQ kernel: 32 query rows per wave; 4 waves = 128 rows with 64-key tiles
// and two workgroups per CU, or (non-causal, S >= 8192) 8 waves = 256 rows
// with 128-key tiles and one per CU; Q and dO rows resident as B operands, keys/values
// streamed through LDS as in the forward.  Per wave and 64 keys:
// S^T = K Q^T, dP^T = V dO^T (queries on the lanes, so LSE and D are per
// lane), dS^T in registers, dQ^T += K^T dS^T with K^T by transposing reads.
//
// In both kernels the dP accumulators start at -D (the workspace keeps D
// negated), so they end as dP - D, and scale multiplies dK and dQ once in
// the epilogues rather than every dS element.
// Causal: key blocks only meet query blocks at or below the diagonal; both
// kernels order workgroup ids so the longest blocks start first (LPT,
// technical summary, results).
#include <algorithm>
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kQPerIter = 64;     // dK/dV kernel: query rows per iteration
// dQ kernel, two shapes: 4 waves / 128 queries with 64-key tiles (two
// workgroups per CU), or WIDE: 8 waves / 256 queries with 128-key tiles
// (one per CU, twice the work per barrier).
template <bool WIDE> constexpr int kDqWaves = WIDE ? 8 : 4;
template <bool WIDE> constexpr int kQPerBlock = 32 * kDqWaves<WIDE>;
template <bool WIDE> constexpr int kKvPerTile = WIDE ? 128 : 64;

// -D_i = -sum_k dO_ik O_ik and LSE_i * log2(e) (the base-2 exponent offset
// the two gradient kernels use), both into the workspace.  D is kept negated
// so that both gradient kernels can start their dP accumulators at -D and
// take dS = P (dP - D) straight from them.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const uint16_t *__restrict__ O,
                                                           const uint16_t *__restrict__ dO,
                                                           const float *__restrict__ LSE,
                                                           float *__restrict__ Dvec,
                                                           float *__restrict__ L2vec, int64_t rows,
                                                           int *__restrict__ sync, int64_t nsync) {
    // the sync words of the fused backward start at zero (a kernel, not a
    // memset, so that the sequence can be captured in a graph)
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid < nsync) sync[gid] = 0;
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
    if (row < rows && part == 0) {
        Dvec[row] = -acc;
        L2vec[row] = LSE[row] * FA_LOG2E;
    }
}

// ---------------------------------------------------------------- dK, dV
// 8 waves, 256 keys: wave w owns keys 32 w .. +31 of the block and takes the
// two 32-row halves of every 64-row query block in turn.  (Against 128 keys
// per workgroup with the query halves on the two waves of a SIMD: half the
// barriers and stage copies per MFMA, and no dK/dV exchange at the end.)
constexpr int kKB = 256;
template <int D, bool CAUSAL>
__global__ __launch_bounds__(2 * kThreads, 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ L2vec, const float *__restrict__ Dvec, const uint16_t *__restrict__ dO,
    uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int BH, int S, float scale, float c, int lpt) {
    constexpr int NW = 8;
    constexpr int ROWB = D * 2;
    constexpr int NCH = ROWB / 16;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int QTILE = kQPerIter * ROWB;
    constexpr int LDB = 4 * kQPerIter * 4;
    constexpr int SMEM = LDB + 4 * QTILE;

    // The query-side stages come first, so that each of their reads is one
    // register (lane offset with the stage folded in, flipped once per
    // iteration) plus an immediate below 64 KB, the reach of the LDS
    // instructions' offset field: no address arithmetic per read.
    __shared__ __attribute__((aligned(1024))) char smem_raw[SMEM];
    fa_lds_char *smem = (fa_lds_char *)smem_raw;
    fa_lds_char *sLD = smem;                     // [2][LSE 64 | D 64] floats
    fa_lds_char *sQ0 = sLD + LDB;                // [2] Q tiles
    fa_lds_char *sO0 = sQ0 + 2 * QTILE;          // [2] dO tiles

    const int lane = threadIdx.x & 63, w = wave_id();
    const int h = lane >> 5, n = lane & 31;

    const int bh = blockIdx.x % BH;
    const int nkb = (S + kKB - 1) / kKB;
    const int kblk = (CAUSAL && !lpt) ? (nkb - 1 - (int)(blockIdx.x / BH)) : (int)(blockIdx.x / BH);
    const int k0 = kblk * kKB;
    const size_t head = (size_t)bh * (size_t)S * D;
    const int kv = k0 + 32 * w + n;  // this lane's key for S and dP

    const uint32_t head_bytes = (uint32_t)S * ROWB;
    const fa_rsrc rQ = make_rsrc(Q + head, head_bytes);
    const fa_rsrc rdO = make_rsrc(dO + head, head_bytes);
    const fa_rsrc rL = make_rsrc(L2vec + (size_t)bh * S, (uint32_t)S * 4);
    const fa_rsrc rD = make_rsrc(Dvec + (size_t)bh * S, (uint32_t)S * 4);

    // this wave's K and V rows, the B operands of S = Q K^T and dP = dO V^T,
    // straight to registers (with them in registers the LDS holds only the
    // query-side stages, and each half block reads 8 KB less from it)
    fa_u32x4 kreg[KS], vreg[KS];
    {
        const fa_rsrc rK = make_rsrc(K + head, head_bytes);
        const fa_rsrc rV = make_rsrc(V + head, head_bytes);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kreg[ks] = buf_load16(rK, (uint32_t)kv * ROWB + (16 * ks + 8 * h) * 2);
            vreg[ks] = buf_load16(rV, (uint32_t)kv * ROWB + (16 * ks + 8 * h) * 2);
        }
    }

    fa_f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) {
        dkacc[i] = zero16();
        dvacc[i] = zero16();
    }

    const int nqb = (S + kQPerIter - 1) / kQPerIter;
    const int ib = CAUSAL ? k0 / kQPerIter : 0;

    auto issue = [&](int i, int buf) {
        tile_to_lds<NCH, kQPerIter, NW>(rQ, i * kQPerIter, sQ0 + buf * QTILE, w, lane);
        tile_to_lds<NCH, kQPerIter, NW>(rdO, i * kQPerIter, sO0 + buf * QTILE, w, lane);
        if (w < 2) {
            fa_lds_char *dst = sLD + (buf * 2 + w) * kQPerIter * 4;
            buf_load_lds<4>(w == 0 ? rL : rD, dst, (uint32_t)(i * kQPerIter + lane) * 4);
        }
    };

    if (ib < nqb) issue(ib, 0);
    wait_vmem();
    __syncthreads();

    // Lane-dependent LDS offsets within query half 0 (half 1 is 32 rows,
    // a multiple of the swizzle period, further on).  The swizzle XORs the
    // chunk index, so the Q/dO offset of k-step ks is that of k-step 0 with
    // 2 ks XORed into the chunk bits.  The query-side offsets (< QTILE / 2)
    // carry the stage as bit QTILE, flipped after every iteration; the LSE/D
    // offset carries it as bit 2 * kQPerIter * 4.
    int troff[DB][2];
    int qoff = tile_off<NCH>(n, h * 16);
    int ldoff = 16 * h;
    {
        const int L = lane & 15;
        const int col = ((lane >> 4) & 1) * 16 + (L & 3) * 4;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                troff[db][s2] = tile_off<NCH>(4 * h + 8 * s2 + (L >> 2), (32 * db + col) * 2);
    }

    auto compute_half = [&](int q0, auto QHC, auto MASKC) {
        constexpr int qh = decltype(QHC)::value;
        constexpr bool MASK = decltype(MASKC)::value;
        const fa_lds_char *sQ = sQ0 + qh * 32 * ROWB;
        const fa_lds_char *sO = sO0 + qh * 32 * ROWB;
        const fa_lds_char *sL = sLD + qh * 32 * 4 + ldoff;
        const fa_lds_char *sD = sL + kQPerIter * 4;

        // fresh copies per half, so that the eight offsets are formed at
        // their reads rather than hoisted out of the loop into registers
        int qb = qoff;
        asm volatile("" : "+v"(qb));
        // dP accumulates on top of -D of its query row, so it ends as dP - D
        fa_f32x16 sacc = zero16(), pacc;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const fa_f32x4 nd4 = *(const __attribute__((address_space(3))) fa_f32x4 *)(sD + 32 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) pacc[4 * g + e] = nd4[e];
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int qo = qb ^ (ks << 5);
            sacc = mfma32(lds_read16(sQ, qo), kreg[ks], sacc);
            pacc = mfma32(lds_read16(sO, qo), vreg[ks], pacc);
        }
        fa_u32x4 pf[2], dsf[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int qi = 8 * g + 4 * h;
            const fa_f32x4 l4 = *(const __attribute__((address_space(3))) fa_f32x4 *)(sL + 32 * g);
            float p[4], ds[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, -l4[e]));
                if constexpr (MASK) pv = kv > q0 + 32 * qh + qi + e ? 0.0f : pv;
                p[e] = pv;
                ds[e] = pv * pacc[r];
            }
            const int t = g >> 1;
            const int wd = (g & 1) * 2;
            pf[t][wd] = pack_bf16(p[0], p[1]);
            pf[t][wd + 1] = pack_bf16(p[2], p[3]);
            dsf[t][wd] = pack_bf16(ds[0], ds[1]);
            dsf[t][wd + 1] = pack_bf16(ds[2], ds[3]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const fa_u32x2 o0 = lds_read_tr(sO + 16 * t * ROWB, troff[db][0]);
                const fa_u32x2 o1 = lds_read_tr(sO + 16 * t * ROWB, troff[db][1]);
                const fa_u32x2 q0r = lds_read_tr(sQ + 16 * t * ROWB, troff[db][0]);
                const fa_u32x2 q1r = lds_read_tr(sQ + 16 * t * ROWB, troff[db][1]);
                const fa_u32x4 bo = {o0[0], o0[1], o1[0], o1[1]};
                const fa_u32x4 bq = {q0r[0], q0r[1], q1r[0], q1r[1]};
                dvacc[db] = mfma32(pf[t], bo, dvacc[db]);
                dkacc[db] = mfma32(dsf[t], bq, dkacc[db]);
            }
        }
    };

    auto step = [&](int i, auto MASKC) {
        const int buf = (i - ib) & 1;
        if (i + 1 < nqb) issue(i + 1, buf ^ 1);
        compute_half(i * kQPerIter, std::integral_constant<int, 0>{}, MASKC);
        __builtin_amdgcn_sched_barrier(0);
        compute_half(i * kQPerIter, std::integral_constant<int, 1>{}, MASKC);
        // the next iteration reads the other stage
        qoff ^= QTILE;
        ldoff ^= 2 * kQPerIter * 4;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            troff[db][0] ^= QTILE;
            troff[db][1] ^= QTILE;
        }
        wait_vmem();
        __syncthreads();
    };

    const int i_plain = CAUSAL ? min(nqb, (k0 + kKB - 1) / kQPerIter + 1) : ib;
    for (int i = ib; i < i_plain; ++i) step(i, std::true_type{});
    for (int i = i_plain; i < nqb; ++i) step(i, std::false_type{});

    const fa_rsrc rdK = make_rsrc(dK + head, head_bytes);
    const fa_rsrc rdV = make_rsrc(dV + head, head_bytes);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kr = k0 + 32 * w + 8 * (r >> 2) + 4 * h + (r & 3);
            const uint32_t off = ((uint32_t)kr * D + 32 * db + n) * 2;
            buf_store2(rdK, off, (uint16_t)(pack_bf16(dkacc[db][r] * scale, 0.0f) & 0xFFFFu));
            buf_store2(rdV, off, (uint16_t)(pack_bf16(dvacc[db][r], 0.0f) & 0xFFFFu));
        }
    }
}

// ---------------------------------------------------------------- dQ
template <int D, bool CAUSAL, bool WIDE>
__global__ __launch_bounds__(64 * kDqWaves<WIDE>, WIDE ? 1 : 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ L2vec, const float *__restrict__ Dvec, const uint16_t *__restrict__ dO,
    float *__restrict__ dQ, int BH, int S, float scale, float c, int nqb, int lpt) {
    constexpr int ROWB = D * 2;
    constexpr int NCH = ROWB / 16;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int QPB = kQPerBlock<WIDE>, KVT = kKvPerTile<WIDE>, NWV = kDqWaves<WIDE>;
    constexpr int TILE = KVT * ROWB;

    __shared__ __attribute__((aligned(1024))) char smem_raw[2 * 2 * TILE];
    fa_lds_char *smem = (fa_lds_char *)smem_raw;

    const int lane = threadIdx.x & 63, w = wave_id();
    const int h = lane >> 5, n = lane & 31;

    const int bh = blockIdx.x % BH;
    const int qi = blockIdx.x / BH;
    const int qblk = (CAUSAL && lpt) ? (nqb - 1 - qi) : qi;
    const int q0 = qblk * QPB;
    const size_t head = (size_t)bh * (size_t)S * D;
    const int kv_end = CAUSAL ? min(S, q0 + QPB) : S;
    const int nkv = (kv_end + KVT - 1) / KVT;
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
    const float lse2 = buf_load4f(make_rsrc(L2vec + (size_t)bh * S, (uint32_t)S * 4), (uint32_t)qrow * 4);
    const float ndd = buf_load4f(make_rsrc(Dvec + (size_t)bh * S, (uint32_t)S * 4), (uint32_t)qrow * 4);  // -D

    fa_f32x16 dqacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) dqacc[i] = zero16();
    // -D of this lane's query in every register: the dP^T accumulators
    // start from it (the MFMA's C operand), so they end as dP - D
    fa_f32x16 nd16;
#pragma unroll
    for (int r = 0; r < 16; ++r) nd16[r] = ndd;

    auto issue_tile = [&](int j, int buf) {
        fa_lds_char *sK = smem + buf * 2 * TILE;
        tile_to_lds<NCH, KVT, NWV>(rK, j * KVT, sK, w, lane);
        tile_to_lds<NCH, KVT, NWV>(rV, j * KVT, sK + TILE, w, lane);
    };

    // Lane-dependent LDS offsets, computed once (as in the forward kernel).
    int koff[KS], troff[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = tile_off<NCH>(n, (2 * ks + h) * 16);
    {
        const int L = lane & 15;
        const int col = ((lane >> 4) & 1) * 16 + (L & 3) * 4;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                troff[db][s2] = tile_off<NCH>(4 * h + 8 * s2 + (L >> 2), (32 * db + col) * 2);
    }

    // 64 keys (sub-tile sub of the tile in buffer buf).  MASK: they cross
    // this wave's diagonal or the end of the sequence.  The factor scale of
    // dS is applied to dQ at the end.
    auto compute_tile = [&](int buf, int kv0, int sub, auto MASKC) {
        constexpr bool MASK = decltype(MASKC)::value;
        const fa_lds_char *sK = smem + buf * 2 * TILE + sub * 64 * ROWB;
        const fa_lds_char *sV = sK + TILE;
        // S^T = K Q^T and dP^T = V dO^T: 64 keys x 32 queries each.
        fa_f32x16 sacc[2] = {zero16(), zero16()};
        fa_f32x16 pacc[2] = {nd16, nd16};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                sacc[mb] = mfma32(lds_read16(sK + 32 * mb * ROWB, koff[ks]), qf[ks], sacc[mb]);
                pacc[mb] = mfma32(lds_read16(sV + 32 * mb * ROWB, koff[ks]), of[ks], pacc[mb]);
            }
        }
        fa_u32x4 dsf[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float ds[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    float pv = __builtin_amdgcn_exp2f(fmaf(sacc[mb][r + e], c, -lse2));
                    if constexpr (MASK) {
                        const int key = kv0 + 32 * mb + 8 * ((r + e) >> 2) + 4 * h + ((r + e) & 3);
                        const bool dead = (CAUSAL && key > qrow) || key >= S;
                        pv = dead ? 0.0f : pv;
                    }
                    ds[e] = pv * pacc[mb][r + e];
                }
                dsf[2 * mb + (r >> 3)][(r & 7) >> 1] = pack_bf16(ds[0], ds[1]);
            }
        }
        // dQ^T += K^T dS^T, keys of k-step t in accumulator order.
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const fa_u32x2 lo = lds_read_tr(sK + 16 * t * ROWB, troff[db][0]);
                const fa_u32x2 hi = lds_read_tr(sK + 16 * t * ROWB, troff[db][1]);
                const fa_u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                dqacc[db] = mfma32(a, dsf[t], dqacc[db]);
            }
        }
    };

    auto step = [&](int j, auto MASKC) {
        const int buf = j & 1;
#pragma unroll
        for (int sub = 0; sub < KVT / 64; ++sub) {
            // the next tile's copies go out after the first 64-key sub-tile
            // of the wide shape (with one sub-tile: before it)
            if (sub == KVT / 128 && j + 1 < nkv) issue_tile(j + 1, buf ^ 1);
            const int kv0 = j * KVT + 64 * sub;
            if constexpr (decltype(MASKC)::value) {
                if (!(CAUSAL && kv0 > wq_lo + 31)) compute_tile(buf, kv0, sub, MASKC);
            } else {
                compute_tile(buf, kv0, sub, MASKC);
            }
            // one sub-tile's registers at a time
            if (sub + 1 < KVT / 64) __builtin_amdgcn_sched_barrier(0);
        }
        wait_vmem();
        __syncthreads();
    };

    if (nkv > 0) issue_tile(0, 0);
    wait_vmem();
    __syncthreads();

    const int n_plain = min(nkv, (CAUSAL ? min(q0, S) : S) / KVT);
    for (int j = 0; j < n_plain; ++j) step(j, std::false_type{});
    for (int j = n_plain; j < nkv; ++j) step(j, std::true_type{});

    // Epilogue: lane = query row, registers = 4 consecutive d per group.
    // The scaled rows go through LDS (the K/V stages are free: every wave
    // has passed the last barrier), 16-byte chunk index XORed with the row,
    // and leave as whole rows; stored straight from the accumulators, each
    // instruction would touch 32 rows with 32 bytes each.
    constexpr int RB4 = D * 4, NC4 = RB4 / 16;
    fa_lds_char *sQd = smem + w * (32 * RB4);
    auto off4 = [&](int row, int ch) { return row * RB4 + ((ch ^ (row & (NC4 - 1))) << 4); };
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            fa_u32x4 v = {__float_as_uint(dqacc[db][4 * g] * scale), __float_as_uint(dqacc[db][4 * g + 1] * scale),
                          __float_as_uint(dqacc[db][4 * g + 2] * scale), __float_as_uint(dqacc[db][4 * g + 3] * scale)};
            lds_write16(sQd, off4(n, 8 * db + 2 * g + h), v);
        }
    const fa_rsrc rdQ = make_rsrc(dQ + head, (uint32_t)S * D * 4);
    constexpr int RPI = 1024 / RB4;  // rows per 1 KB store instruction
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int row = i * RPI + lane / NC4, ch = lane % NC4;
        buf_store16(rdQ, (uint32_t)(wq_lo + row) * RB4 + ch * 16, lds_read16(sQd, off4(row, ch)));
    }
}

template <int D>
hipError_t launch_pre_d(const BwdArgs &a, hipStream_t st) {
    constexpr int RPB = kThreads / (D / 8);
    const int64_t rows = (int64_t)a.BH * a.S;
    const int64_t blocks = std::max((rows + RPB - 1) / RPB, ((int64_t)a.nsync + kThreads - 1) / kThreads);
    const dim3 grid((unsigned)blocks), block(kThreads);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), grid, block, 0, st, (const uint16_t *)a.O,
                       (const uint16_t *)a.dO, a.LSE, a.Dvec, a.Dvec + rows, rows, a.sync, (int64_t)a.nsync);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_t(const BwdArgs &a, hipStream_t st) {
    const int nkb = (a.S + kKB - 1) / kKB;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * nkb)), dim3(2 * kThreads), 0, st,
                       (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                       (const float *)a.Dvec + (size_t)a.BH * a.S, (const float *)a.Dvec,
                       (const uint16_t *)a.dO, (uint16_t *)a.dK, (uint16_t *)a.dV,
                       a.BH, a.S, a.scale, a.scale * FA_LOG2E, (int)a.lpt);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool WIDE>
hipError_t launch_dq_w(const BwdArgs &a, hipStream_t st) {
    const int nqb = (a.S + kQPerBlock<WIDE> - 1) / kQPerBlock<WIDE>;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, WIDE>), dim3((unsigned)(a.BH * nqb)), dim3(64 * kDqWaves<WIDE>), 0, st,
                       (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                       (const float *)a.Dvec + (size_t)a.BH * a.S, (const float *)a.Dvec,
                       (const uint16_t *)a.dO, a.dQ, a.BH, a.S, a.scale,
                       a.scale * FA_LOG2E, nqb, (int)a.lpt);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const BwdArgs &a, hipStream_t st) {
    // measured: the wide shape is 2 % faster non-causal from S = 8192 on,
    // even causal at S = 32768 and slower causal at S = 4096
    if constexpr (!CAUSAL) {
        if (a.S >= 8192) return launch_dq_w<D, CAUSAL, true>(a, st);
    }
    return launch_dq_w<D, CAUSAL, false>(a, st);
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
