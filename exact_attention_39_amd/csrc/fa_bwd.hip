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
//
// Stored dS (an option): the dK/dV kernel also writes its bf16 dS tiles to
// the workspace (2 bytes per query-key pair the mask keeps) and a third
// kernel computes dQ = scale * dS K from them: one contraction instead of
// three, bound by reading dS back from HBM.  MI355X's 288 GB hold the
// 32 GiB of one S = 32768, 16-head backward.
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

// ---------------------------------------------------------------- stored dS
// Optionally dS travels from the dK/dV kernel to the dQ kernel through HBM
// instead of being recomputed there (dQ = dS K then needs one product instead
// of three): one 32 KB bf16 tile per (head, 256-key block kb, 64-query
// iteration i), holding the dK/dV kernel's registers as they are (see the
// store).  Causal: only the tiles i >= 4 kb that a key block visits exist,
// packed block after block.
constexpr int kDsTileBytes = 256 * 64 * 2;
constexpr int kDsTileElems = kDsTileBytes / 2;
// cache policy of the dS stores and loads: non-temporal (each line is read
// once, by the next kernel, long after it has left L2)
constexpr int kNonTemporal = 2;

__host__ __device__ inline int64_t ds_tiles_per_head(int nkb, int nqi, bool causal) {
    return causal ? (int64_t)nkb * nqi - 2 * (int64_t)nkb * (nkb - 1) : (int64_t)nkb * nqi;
}

__host__ __device__ inline int64_t ds_tile(int64_t bh, int kb, int i, int nkb, int nqi, bool causal) {
    const int64_t head = bh * ds_tiles_per_head(nkb, nqi, causal);
    if (causal) return head + (int64_t)kb * nqi - 2 * (int64_t)kb * (kb - 1) + (i - 4 * kb);
    return head + (int64_t)kb * nqi + i;
}

// Copies issued from inline assembly (the stored-dS kernels).  After a copy
// through the compiler's intrinsic, the first transposing LDS read waits for
// every copy in flight, and so does the fence of __syncthreads: with copies
// two tiles ahead, or with dS stores in flight that only the next kernel
// reads, that wait would serialise them.  These kernels count their own
// memory operations instead (s_waitcnt vmcnt counts a wave's loads and
// stores in issue order) and their barriers carry no memory fence.
typedef uint32_t fa_srd __attribute__((ext_vector_type(4)));

__device__ __forceinline__ fa_srd make_srd(const void *base, uint32_t num_bytes) {
    const uint64_t p = (uint64_t)base;
    fa_srd r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane(num_bytes);
    r[3] = 0x00020000u;
    return r;
}

// buffer_load_dwordx4 / _dword ... lds: as buf_load_lds, invisible to the compiler.
__device__ __forceinline__ void copy16_async(fa_srd r, fa_lds_char *lds_wave_base, uint32_t off) {
    lds_poison(lds_wave_base, 16);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(off), "s"(r)
                 : "memory", "m0");
}

// The same with the non-temporal hint (data read once: the stored dS).
__device__ __forceinline__ void copy16_async_nt(fa_srd r, fa_lds_char *lds_wave_base, uint32_t off) {
    lds_poison(lds_wave_base, 16);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(m0), "v"(off), "s"(r)
                 : "memory", "m0");
}

__device__ __forceinline__ void copy4_async(fa_srd r, fa_lds_char *lds_wave_base, uint32_t off) {
    lds_poison(lds_wave_base, 4);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(off), "s"(r)
                 : "memory", "m0");
}

// tile_to_lds through copy16_async.
template <int NCH, int ROWS, int NW>
__device__ __forceinline__ void tile_to_lds_async(fa_srd r, int row0, fa_lds_char *tile, int w, int lane) {
    constexpr int ROWB = NCH * 16;
    constexpr int INSTS = ROWS * ROWB / 1024;
    static_assert(INSTS % NW == 0, "tile must split evenly over the waves");
#pragma unroll
    for (int k = 0; k < INSTS / NW; ++k) {
        const int inst = w + NW * k;
        const int row = inst * (1024 / ROWB) + lane / NCH;
        const int c = (lane % NCH) ^ swz<NCH>(row);
        copy16_async(r, tile + inst * 1024, (uint32_t)(row0 + row) * ROWB + c * 16);
    }
}

// ---------------------------------------------------------------- dK, dV
// 8 waves, 256 keys: wave w owns keys 32 w .. +31 of the block and takes the
// two 32-row halves of every 64-row query block in turn.  (Against 128 keys
// per workgroup with the query halves on the two waves of a SIMD: half the
// barriers and stage copies per MFMA, and no dK/dV exchange at the end.)
constexpr int kKB = 256;
template <int D, bool CAUSAL, bool DSOUT>
__global__ __launch_bounds__(2 * kThreads, 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ L2vec, const float *__restrict__ Dvec, const uint16_t *__restrict__ dO,
    uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, uint16_t *__restrict__ dS, int BH, int S,
    float scale, float c, int lpt) {
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

    [[maybe_unused]] const fa_srd aQ = make_srd(Q + head, head_bytes), adO = make_srd(dO + head, head_bytes);
    [[maybe_unused]] const fa_srd aLD = make_srd(w == 0 ? (const void *)(L2vec + (size_t)bh * S)
                                                         : (const void *)(Dvec + (size_t)bh * S),
                                                 (uint32_t)S * 4);
    auto issue = [&](int i, int buf) {
        if constexpr (DSOUT) {
            tile_to_lds_async<NCH, kQPerIter, NW>(aQ, i * kQPerIter, sQ0 + buf * QTILE, w, lane);
            tile_to_lds_async<NCH, kQPerIter, NW>(adO, i * kQPerIter, sO0 + buf * QTILE, w, lane);
            if (w < 2) copy4_async(aLD, sLD + (buf * 2 + w) * kQPerIter * 4, (uint32_t)(i * kQPerIter + lane) * 4);
        } else {
            tile_to_lds<NCH, kQPerIter, NW>(rQ, i * kQPerIter, sQ0 + buf * QTILE, w, lane);
            tile_to_lds<NCH, kQPerIter, NW>(rdO, i * kQPerIter, sO0 + buf * QTILE, w, lane);
            if (w < 2) {
                fa_lds_char *dst = sLD + (buf * 2 + w) * kQPerIter * 4;
                buf_load_lds<4>(w == 0 ? rL : rD, dst, (uint32_t)(i * kQPerIter + lane) * 4);
            }
        }
    };

    if (ib < nqb) issue(ib, 0);
    if constexpr (DSOUT) {
        // the compiler's own wait (vmcnt(0)): it then knows the K and V rows
        // have arrived and waits for nothing inside the loops
        __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
        wait_vmem();
    }
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

    auto compute_half = [&](int q0, fa_rsrc rds, auto QHC, auto MASKC) {
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
                if constexpr (MASK) {
                    // keys past S only reach the stored dS: zero them there
                    bool dead = DSOUT && kv >= S;
                    if constexpr (CAUSAL) dead = dead || kv > q0 + 32 * qh + qi + e;
                    pv = dead ? 0.0f : pv;
                }
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
        if constexpr (DSOUT) {
            // The stored tile holds each lane's registers as they are: 16
            // bytes (8 bf16 of key 32 w + n: queries 16 t + 4 h + 0..3, then
            // 16 t + 8 + 4 h + 0..3 of query half qh) at byte
            // ((2 qh + t) * 8 + w) * 1024 + lane * 16, so that every store
            // instruction writes 1 KB of whole lines.
#pragma unroll
            for (int t = 0; t < 2; ++t)
                __builtin_amdgcn_raw_buffer_store_b128(dsf[t], rds, (uint32_t)(((2 * qh + t) * 8 + w) * 1024 + lane * 16),
                                                       0, kNonTemporal);
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
        // (without a stored dS: an empty resource, never used)
        const fa_rsrc rds = DSOUT ? make_rsrc(dS + (size_t)ds_tile(bh, kblk, i, nkb, nqb, CAUSAL) * kDsTileElems,
                                              kDsTileBytes)
                                  : make_rsrc(dS, 0);
        compute_half(i * kQPerIter, rds, std::integral_constant<int, 0>{}, MASKC);
        __builtin_amdgcn_sched_barrier(0);
        compute_half(i * kQPerIter, rds, std::integral_constant<int, 1>{}, MASKC);
        // the next iteration reads the other stage
        qoff ^= QTILE;
        ldoff ^= 2 * kQPerIter * 4;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            troff[db][0] ^= QTILE;
            troff[db][1] ^= QTILE;
        }
        if constexpr (DSOUT) {
            // the copies for the next iteration are done once at most this
            // iteration's four dS stores are in flight; no fence (the
            // stores are read by another kernel)
            asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else {
            wait_vmem();
            __syncthreads();
        }
    };

    // masked iterations: the causal diagonal, and with a stored dS every
    // iteration of a block that reaches past S
    const int i_plain = (DSOUT && k0 + kKB > S) ? nqb : CAUSAL ? min(nqb, (k0 + kKB - 1) / kQPerIter + 1) : ib;
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

// ---------------------------------------------------------------- dQ from stored dS
// dQ = scale * dS K with dS read back from HBM (the dK/dV kernel stored it):
// a GEMM with the keys as its long inner dimension, bound by the dS reads.
// One workgroup = 8 waves = 256 queries (the four 64-query iterations
// 4 qb .. 4 qb + 3 of the stored layout); wave w takes 32 queries, iteration
// w / 2, half w % 2.  64-key tiles of K (swizzled rows) and of dS (four
// 64-row x 128-byte chunks, one per iteration) stream through three LDS
// stages, two tiles in flight.  Per wave and tile: dQ^T += K^T dS^T, both
// operands by transposing reads: K^T as in the other kernels, dS^T from the
// key rows of the stored tile (lane = query, 4 keys per read).
constexpr int kDqDsStages = 3;

// Copies of key tile kt into one stage: 2 (D = 128) or 1 (D = 64) for K and 4
// for dS per wave, the count the waits below rely on.
template <int D>
__device__ __forceinline__ void dq_ds_issue(fa_srd rK, const uint16_t *dS, int bh, int kt, int qb,
                                            int nkb, int nqi, bool causal, fa_lds_char *stage,
                                            int w, int lane) {
    constexpr int NCH = D / 8;
    // K rows kt*64 .. +63 (rows past S arrive as zeros)
    tile_to_lds_async<NCH, 64, 8>(rK, kt * 64, stage, w, lane);
    // dS: chunk k = iteration 4 qb + k, key rows (kt % 4) * 64 .. +63 of the
    // tile (kt / 4, 4 qb + k), into LDS rows of 128 bytes (one key, the 64
    // queries in the stored unit order); wave w copies rows 8 w .. 8 w + 7
    // of each chunk.  The 64-byte halves of a row swap on every other row
    // pair so that the transposing reads (4 rows x 64 bytes per half wave)
    // hit all 64 banks.  Unit u = 2 (2 qh + t) + h of key kk sits at byte
    // ((2 qh + t) * 8 + kk / 32) * 1024 + (32 h + kk % 32) * 16 of the tile.
    fa_lds_char *sds = stage + 64 * D * 2;
    const int r = 8 * w + lane / 8, pc = lane % 8;
    const int lc = pc ^ (((r >> 1) & 1) << 2);
    const int kk = (kt & 3) * 64 + r;
    const uint32_t goff = (uint32_t)((((lc >> 1) * 8 + (kk >> 5)) * 2 + (lc & 1)) * 512 + (kk & 31) * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = 4 * qb + k;
        // past the last iteration: an empty resource, the copy writes zeros
        const bool live = i < nqi;
        const int64_t tile = live ? ds_tile(bh, kt >> 2, i, nkb, nqi, causal) : 0;
        copy16_async_nt(make_srd(dS + tile * kDsTileElems, live ? (uint32_t)kDsTileBytes : 0u),
                        sds + k * 8192 + w * 1024, goff);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dq_ds_kernel(const uint16_t *__restrict__ K,
                                                           const uint16_t *__restrict__ dS,
                                                           float *__restrict__ dQ, int BH, int S,
                                                           float scale, int nqb, int lpt) {
    constexpr int ROWB = D * 2;
    constexpr int NCH = ROWB / 16;
    constexpr int DB = D / 32;
    constexpr int STAGE = 64 * ROWB + 4 * 8192;
    __shared__ __attribute__((aligned(1024))) char smem_raw[kDqDsStages * STAGE];
    fa_lds_char *smem = (fa_lds_char *)smem_raw;

    const int lane = threadIdx.x & 63, w = wave_id();
    const int h = lane >> 5, n = lane & 31;
    const int bh = blockIdx.x % BH;
    const int qi = blockIdx.x / BH;
    const int qb = (CAUSAL && lpt) ? (nqb - 1 - qi) : qi;
    const int q0 = qb * 256;
    const int wq_lo = q0 + 32 * w;
    const int nkb = (S + kKB - 1) / kKB, nqi = (S + kQPerIter - 1) / kQPerIter;
    const int kv_end = CAUSAL ? min(S, q0 + 256) : S;
    const int nkv = (kv_end + 63) / 64;
    const size_t head = (size_t)bh * (size_t)S * D;
    const fa_srd rK = make_srd(K + head, (uint32_t)S * ROWB);

    fa_f32x16 dqacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) dqacc[i] = zero16();

    // Lane offsets.  A (K^T, d rows): rows 16 ks + 8 h + 0..3 and + 4..7,
    // columns 32 db + the lane's 16-column group.  B (dS^T, queries): the
    // same key rows; in each 16-lane group (t = (lane >> 4) & 1), lane L
    // points at key row L / 4 of the four and at the 8-byte run L % 4 =
    // (hi, h_k) of unit (half, t, h_k): queries 16 t + 8 hi + 4 h_k + 0..3,
    // so lane i of the group receives query 16 t + i, the lane's own column.
    const int L = lane & 15, tq = (lane >> 4) & 1;
    int aoff[DB][2], boff[2];
    {
        const int col = tq * 16 + (L & 3) * 4;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) aoff[db][s2] = tile_off<NCH>(8 * h + 4 * s2 + (L >> 2), (32 * db + col) * 2);
        const int qh = w & 1, hk = L & 1, hi = (L >> 1) & 1;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int row = 8 * h + 4 * s2 + (L >> 2);  // + 16 ks, which keeps (row >> 1) & 1
            boff[s2] = 64 * ROWB + (w >> 1) * 8192 + row * 128 +
                       (((qh ^ ((row >> 1) & 1)) << 6) | (tq << 5) | (hk << 4) | (hi << 3));
        }
    }

    auto compute_tile = [&](const fa_lds_char *st) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const fa_u32x2 b0 = lds_read_tr(st + ks * 16 * 128, boff[0]);
            const fa_u32x2 b1 = lds_read_tr(st + ks * 16 * 128, boff[1]);
            const fa_u32x4 b = {b0[0], b0[1], b1[0], b1[1]};
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const fa_u32x2 a0 = lds_read_tr(st + ks * 16 * ROWB, aoff[db][0]);
                const fa_u32x2 a1 = lds_read_tr(st + ks * 16 * ROWB, aoff[db][1]);
                const fa_u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
                dqacc[db] = mfma32(a, b, dqacc[db]);
            }
        }
    };

    const int npre = min(nkv, kDqDsStages - 1);
    for (int j = 0; j < npre; ++j) dq_ds_issue<D>(rK, dS, bh, j, qb, nkb, nqi, CAUSAL, smem + j * STAGE, w, lane);
    // one tile; the stage is a constant (the loop below is unrolled by the
    // stage count), so every LDS read is a hoisted register plus an immediate
    auto step = [&](int j, auto STC) {
        constexpr int st = decltype(STC)::value;
        // tile j has landed (this wave's copies: the wait; everyone's: the
        // barrier), and every wave is done with the stage tile j + 2 goes to
        if (j + 1 < nkv) {
            if constexpr (D == 128) asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        if (j + 2 < nkv)
            dq_ds_issue<D>(rK, dS, bh, j + 2, qb, nkb, nqi, CAUSAL, smem + ((st + 2) % kDqDsStages) * STAGE, w, lane);
        // causal: a key tile wholly above this wave's queries has dS = 0
        if (!(CAUSAL && j * 64 > wq_lo + 31)) compute_tile(smem + st * STAGE);
    };
    static_assert(kDqDsStages == 3, "the loop is unrolled by the stage count");
    for (int j = 0; j < nkv; j += 3) {
        step(j, std::integral_constant<int, 0>{});
        if (j + 1 < nkv) step(j + 1, std::integral_constant<int, 1>{});
        if (j + 2 < nkv) step(j + 2, std::integral_constant<int, 2>{});
    }
    __syncthreads();

    // Epilogue as in the recomputing dQ kernel: scaled rows through LDS,
    // whole-row 16-byte stores.
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
    constexpr int RPI = 1024 / RB4;
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
                       (const uint16_t *)a.dO, a.LSE, a.Dvec, a.L2vec, rows, a.sync, (int64_t)a.nsync);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool DSOUT>
hipError_t launch_dkdv_s(const BwdArgs &a, hipStream_t st) {
    const int nkb = (a.S + kKB - 1) / kKB;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, DSOUT>), dim3((unsigned)(a.BH * nkb)), dim3(2 * kThreads), 0,
                       st, (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                       (const float *)a.L2vec, (const float *)a.Dvec,
                       (const uint16_t *)a.dO, (uint16_t *)a.dK, (uint16_t *)a.dV, (uint16_t *)a.dS,
                       a.BH, a.S, a.scale, a.scale * FA_LOG2E, (int)a.lpt);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_t(const BwdArgs &a, hipStream_t st) {
    return a.dS ? launch_dkdv_s<D, CAUSAL, true>(a, st) : launch_dkdv_s<D, CAUSAL, false>(a, st);
}

template <int D, bool CAUSAL>
hipError_t launch_dq_ds(const BwdArgs &a, hipStream_t st) {
    const int nqb = (a.S + 255) / 256;
    hipLaunchKernelGGL((bwd_dq_ds_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * nqb)), dim3(512), 0, st,
                       (const uint16_t *)a.K, (const uint16_t *)a.dS, a.dQ, a.BH, a.S, a.scale, nqb, (int)a.lpt);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool WIDE>
hipError_t launch_dq_w(const BwdArgs &a, hipStream_t st) {
    const int nqb = (a.S + kQPerBlock<WIDE> - 1) / kQPerBlock<WIDE>;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, WIDE>), dim3((unsigned)(a.BH * nqb)), dim3(64 * kDqWaves<WIDE>), 0, st,
                       (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                       (const float *)a.L2vec, (const float *)a.Dvec,
                       (const uint16_t *)a.dO, a.dQ, a.BH, a.S, a.scale,
                       a.scale * FA_LOG2E, nqb, (int)a.lpt);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const BwdArgs &a, hipStream_t st) {
    if (a.dS) return launch_dq_ds<D, CAUSAL>(a, st);
    // measured: the wide shape is 2 % faster non-causal from S = 8192 on,
    // even causal at S = 32768 and slower causal at S = 4096
    if constexpr (!CAUSAL) {
        if (a.S >= 8192) return launch_dq_w<D, CAUSAL, true>(a, st);
    }
    return launch_dq_w<D, CAUSAL, false>(a, st);
}

}  // namespace

int64_t bwd_ds_bytes(int BH, int S, bool causal) {
    const int nkb = (S + kKB - 1) / kKB, nqi = (S + kQPerIter - 1) / kQPerIter;
    return (int64_t)BH * ds_tiles_per_head(nkb, nqi, causal) * kDsTileBytes;
}

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
