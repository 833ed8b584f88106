// fa_bwd_fused.hip -- single-pass exact attention backward for gfx950:
// dK, dV and dQ from one recomputation of S and dP per tile.
//
// The pages' backward (gist.science technical summary, methodology item 3)
// keeps each key block's K, V resident, streams the query blocks past it,
// accumulates dK, dV in place and adds every key block's share of dQ into
// a global accumulator; their deterministic mode orders those additions
// with semaphores and schedules blocks so that the waits hide (technical
// summary, methodology item 3 and results).  On MI355X fp32 atomics run
// past the per-XCD L2 at a fraction of its bandwidth, so this kernel adds
// dQ with plain, ordered read-modify-writes that stay inside one XCD's L2:
//
//   * Persistent workgroups (one per CU) take (head, 256-key block) items
//     from one queue per XCD (the XCD comes from the XCC_ID register); the
//     heads of XCD x are those with head % nxcd == x.  So every workgroup
//     that adds into a head's dQ shares one L2, which is then the coherence
//     point: dQ and the turn flags are read with agent-scope loads (they
//     miss the CU's L1 and hit that L2) and written with plain stores.
//   * Queues are key-block major: key block 0 of every head of the XCD is
//     claimed first (under the causal mask the longest items first).
//   * An item walks its query blocks (32 queries each) from the last down
//     to 0 (causal: down to its diagonal).  Key block kb adds its dQ share
//     of query block i once the kb earlier shares are in: a turn flag per
//     (head, query block, wave slice) counts them; kb = 0 writes instead of
//     adding, so dQ needs no zeroing.  The order of the fp32 additions is
//     fixed (key blocks ascending): the result is bitwise repeatable.
//   * A workgroup only ever waits on an item claimed before its own from
//     the same queue, whose workgroup is running: no deadlock whatever the
//     dispatch order or residency.  Every wait is bounded; on expiry the
//     wave sets the error word of the workspace, stops waiting, and the
//     workgroups stop taking items, so the kernel always exits.
//
// Work of one item (8 waves, wave w owns keys 32w .. 32w+31 of the block):
//   prologue: the K block (256 rows) into LDS, this wave's V rows into
//   registers (the B operands of dP = dO V^T), dK, dV accumulators zeroed.
//   Step over query block i (32 rows; Q, dO, LSE*log2 e and -D double
//   buffered in LDS):
//     phase 2 of the previous block: dQ^T = K^T dS^T over all 256 keys;
//       wave w takes 16 query columns x D/4 head-dimension rows
//       (v_mfma_f32_16x16x32_bf16, K^T and dS^T by transposing LDS reads),
//       then adds scale * that into dQ in turn;
//     phase 1: S = Q K^T and dP = dO V^T (keys on the lanes), P and dS in
//       registers, dV += P^T dO, dK += dS^T Q, and dS^T into an LDS tile
//       (double buffered) for phase 2 of the next step.
//   One workgroup barrier per step.  Epilogue: dK * scale and dV stored.
//
// Workspace (fa_bwd_workspace_bytes): -D, LSE*log2 e, then the sync words:
// [0, 16) claim counters per XCD, [16] error word, [32, ...) turn flags
// [BH][ceil(S/32)][8].  The preprocess kernel zeroes the sync words.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kFThreads = 512;   // 8 waves
constexpr int kFKeys = 256;      // keys per item
constexpr int kFQ = 32;          // queries per step
constexpr int kSpinMax = 1 << 20;

__device__ __forceinline__ fa_f32x4 mfma16(fa_u32x4 a, fa_u32x4 b, fa_f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(fa_bf16x8, a),
                                                   __builtin_bit_cast(fa_bf16x8, b), c, 0, 0, 0);
}

// Agent-scope loads (cache policy sc1): they miss the CU's L1 and are
// served by the XCD's L2, where the other workgroups of the XCD stored.
// The turn flags are read as relaxed atomics, so that the compiler reloads
// them on every poll instead of hoisting one load out of the wait loop.
__device__ __forceinline__ int load_flag(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ fa_f32x4 load_dq4(fa_rsrc r, uint32_t off) {
    return __builtin_bit_cast(fa_f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}

__device__ __forceinline__ int xcc_id() {
    int x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return x & 15;
}

// dS^T tile in LDS: [256 keys][32 queries] bf16, 64-byte rows, the 16-byte
// chunk index XORed with (key / 4) % 4 so that both the row writes of the
// producers (8 bytes per lane, 32 consecutive keys) and the transposing
// reads of phase 2 (4 keys x 32 bytes per 16 lanes) are free of conflicts.
__device__ __forceinline__ int ds_off(int key, int byte) {
    return key * 64 + ((((byte >> 4) ^ (key >> 2)) & 3) << 4) + (byte & 15);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFThreads, 1) void bwd_fused_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ L2vec, const float *__restrict__ Dvec, const uint16_t *__restrict__ dO,
    float *__restrict__ dQ, uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int *__restrict__ sync,
    int BH, int S, float scale, float c, int nxcd) {
    constexpr int NW = 8;
    constexpr int ROWB = D * 2;
    constexpr int NCH = ROWB / 16;
    constexpr int KS = D / 16;          // k-steps of 16 over d (32x32x16 MFMAs)
    constexpr int DB = D / 32;          // 32-wide d blocks of dK, dV
    constexpr int NDB = D / 64;         // 16-wide d blocks of dQ^T per wave (phase 2)
    constexpr int QTILE = kFQ * ROWB;   // one Q or dO stage tile
    constexpr int STAGE = 2 * QTILE + 512;  // + LSE*log2 e [64] and -D [64] (32 used each)
    constexpr int KTILE = kFKeys * ROWB;
    constexpr int DSTILE = kFKeys * kFQ * 2;
    constexpr int SMEM = 2 * STAGE + KTILE + 2 * DSTILE;
    constexpr int SNW = QTILE / 1024 >= NW ? NW : QTILE / 1024;   // waves copying a stage tile
    static_assert(SMEM <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(1024))) char smem_raw[SMEM];
    __shared__ int s_item;
    fa_lds_char *smem = (fa_lds_char *)smem_raw;
    fa_lds_char *sStage = smem;            // [2] {Q tile, dO tile, LSE2[64], -D[64]}
    fa_lds_char *sK = smem + 2 * STAGE;    // the block's K rows (swizzled)
    fa_lds_char *sDS = sK + KTILE;         // [2] dS^T tiles

    const int lane = threadIdx.x & 63, w = wave_id();
    const int h = lane >> 5, n = lane & 31;
    const int x = xcc_id() % nxcd;
    const int hpx = x < BH ? (BH - x + nxcd - 1) / nxcd : 0;  // heads of this XCD
    const int nkb = (S + kFKeys - 1) / kFKeys;
    const int nqb = (S + kFQ - 1) / kFQ;
    const int n_items = hpx * nkb;
    const uint32_t head_bytes = (uint32_t)S * ROWB;
    const fa_rsrc rSync = make_rsrc(sync, 32 * 4);
    bool gave_up = false;

    // ---- lane offsets that do not depend on the item
    // Q / dO rows of k-step 0 (row n, chunk h); k-step ks XORs 2 ks into the chunk.
    const int qoff = tile_off<NCH>(n, h * 16);
    // K rows of this wave's keys, same pattern, 32 w rows further.
    const int koff = 32 * w * ROWB + tile_off<NCH>(n, h * 16);
    // transposing reads of dO^T / Q^T (rows 16 t + 4 h + 8 s2 + L/4)
    int troff[DB][2];
    {
        const int L = lane & 15;
        const int col = ((lane >> 4) & 1) * 16 + (L & 3) * 4;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                troff[db][s2] = tile_off<NCH>(4 * h + 8 * s2 + (L >> 2), (32 * db + col) * 2);
    }
    // Phase 2 of wave w: query columns 16 jq .. +15 of the block, d rows
    // d0 + 16 e .. +15 (e < NDB).  16x16x32 operands: lane l holds k
    // (keys) 8 (l / 16) .. +7 of column (B) / row (A) l % 16; the
    // accumulator holds rows 4 (l / 16) .. +3 of column l % 16.  Transposing
    // reads: lane L of a 16-lane group points at key row 8 g16 + L / 4 (+4
    // for the second read), columns c0 + 4 (L % 4), and receives column
    // c0 + L of those four rows.
    const int jq = w >> 2;
    const int d0 = (D / 4) * (w & 3);
    const int g16 = lane >> 4, i16 = lane & 15;
    const int tr_row = 8 * g16 + (i16 >> 2);
    const int tr_col = 4 * (i16 & 3);
    // (key rows 32 s + tr_row have the swizzle of tr_row: s is an immediate)
    const int dsr0 = ds_off(tr_row, (16 * jq + tr_col) * 2);
    const int dsr1 = ds_off(tr_row + 4, (16 * jq + tr_col) * 2);
    int ktr[NDB][2];
#pragma unroll
    for (int e = 0; e < NDB; ++e) {
        ktr[e][0] = tile_off<NCH>(tr_row, (d0 + 16 * e + tr_col) * 2);
        ktr[e][1] = tile_off<NCH>(tr_row + 4, (d0 + 16 * e + tr_col) * 2);
    }
    // dQ slice of wave w in a query block: row 16 jq + i16, d0 + 16 e + 4 g16 .. +3
    auto dq_off = [&](int blk, int e) __attribute__((always_inline)) {
        return ((uint32_t)(blk * kFQ + 16 * jq + i16) * D + d0 + 16 * e + 4 * g16) * 4;
    };

    for (;;) {
        // ---------------------------------------------------------- claim an item
        if (threadIdx.x == 0) {
            const int stop = load_flag(sync + 16);
            s_item = stop ? n_items : atomicAdd(&sync[x], 1);
        }
        __syncthreads();
        const int t_item = s_item;
        if (t_item >= n_items) break;
        const int kb = t_item / hpx;
        const int bh = x + nxcd * (t_item % hpx);
        const int k0 = kb * kFKeys;
        const size_t head = (size_t)bh * (size_t)S * D;
        const int i_lo = CAUSAL ? k0 / kFQ : 0;
        const int kv = k0 + 32 * w + n;   // this lane's key (S and dP columns)

        const fa_rsrc rQ = make_rsrc(Q + head, head_bytes);
        const fa_rsrc rdO = make_rsrc(dO + head, head_bytes);
        const fa_rsrc rL = make_rsrc(L2vec + (size_t)bh * S, (uint32_t)S * 4);
        const fa_rsrc rD = make_rsrc(Dvec + (size_t)bh * S, (uint32_t)S * 4);
        const fa_rsrc rdQ = make_rsrc(dQ + head, (uint32_t)S * D * 4);
        int *flags = sync + 32 + (size_t)bh * nqb * NW;   // turn flags of this head: [nqb][NW]
        const fa_rsrc rF = make_rsrc(flags, (uint32_t)nqb * NW * 4);

        // stage copies of query block i: Q and dO tiles, and 64 values of
        // LSE*log2 e and -D from row 32 i on (one 4-byte lane each; the
        // upper 32 are not used; rows past S read as zero)
        auto issue_stage = [&](int i, int buf) __attribute__((always_inline)) {
            fa_lds_char *st = sStage + buf * STAGE;
            if (w < SNW) {
                tile_to_lds<NCH, kFQ, SNW>(rQ, i * kFQ, st, w, lane);
                tile_to_lds<NCH, kFQ, SNW>(rdO, i * kFQ, st + QTILE, w, lane);
            }
            if (w == 0) buf_load_lds<4>(rL, st + 2 * QTILE, (uint32_t)(i * kFQ + lane) * 4);
            if (w == 1) buf_load_lds<4>(rD, st + 2 * QTILE + 256, (uint32_t)(i * kFQ + lane) * 4);
        };

        // ---------------------------------------------------------- prologue
        tile_to_lds<NCH, kFKeys, NW>(make_rsrc(K + head, head_bytes), k0, sK, w, lane);
        issue_stage(S > 0 ? nqb - 1 : 0, 0);
        fa_u32x4 vreg[KS];
        {
            const fa_rsrc rV = make_rsrc(V + head, head_bytes);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) vreg[ks] = buf_load16(rV, (uint32_t)kv * ROWB + (16 * ks + 8 * h) * 2);
        }
        fa_f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
        for (int i = 0; i < DB; ++i) {
            dkacc[i] = zero16();
            dvacc[i] = zero16();
        }
        wait_vmem();
        __syncthreads();

        // phase 2 (dQ^T of one block from the dS^T tile in buffer pbuf)
        auto phase2 = [&](int pbuf, fa_f32x4 *acc) __attribute__((always_inline)) {
            const fa_lds_char *sd = sDS + pbuf * DSTILE;
#pragma unroll
            for (int e = 0; e < NDB; ++e) acc[e] = fa_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < kFKeys / 32; ++s) {
                const fa_u32x2 b0 = lds_read_tr(sd + 32 * s * 64, dsr0);
                const fa_u32x2 b1 = lds_read_tr(sd + 32 * s * 64, dsr1);
                const fa_u32x4 b = {b0[0], b0[1], b1[0], b1[1]};
#pragma unroll
                for (int e = 0; e < NDB; ++e) {
                    const fa_u32x2 a0 = lds_read_tr(sK + 32 * s * ROWB, ktr[e][0]);
                    const fa_u32x2 a1 = lds_read_tr(sK + 32 * s * ROWB, ktr[e][1]);
                    const fa_u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
                    acc[e] = mfma16(a, b, acc[e]);
                }
            }
        };
        // wait until kb earlier key blocks have added into block blk (bounded)
        auto wait_turn = [&](int blk, int seen) __attribute__((always_inline)) {
            if (kb == 0 || gave_up) return;
            int spin = 0;
            while (seen < kb) {
                if (++spin > kSpinMax) {
                    gave_up = true;
                    if (lane == 0) buf_store4(rSync, 16 * 4, 1u);
                    return;
                }
                __builtin_amdgcn_s_sleep(2);
                seen = load_flag(flags + blk * NW + w);
            }
            // the dQ loads that follow stay after the wait
            asm volatile("" ::: "memory");
        };

        // Step over query block i (stage buffer / dS^T buffer `buf`); `it`
        // counts the steps of the item.  MASK: the block crosses the causal
        // diagonal of this key block.  `seen` carries the turn flag of the
        // block whose dQ share this step adds (polled one step ahead).
        int seen = 0;
        auto step = [&](int i, int it, auto MASKC) __attribute__((always_inline)) {
            constexpr bool MASK = decltype(MASKC)::value;
            const int buf = it & 1;
            const bool has2 = it > 0;     // phase 2 of block i + 1 (dS^T in buffer buf ^ 1)
            const int blk2 = i + 1;
            // Memory operations in issue order: dQ loads, next turn flag, dQ
            // stores, stage copies.  They complete in that order, so waiting
            // for the dQ loads never waits for the copies, and the wait at the
            // end of the step (for the copies) covers the dQ stores, after
            // which this step's turn is published.
            fa_f32x4 old[NDB];
#pragma unroll
            for (int e = 0; e < NDB; ++e) old[e] = fa_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (has2 && kb > 0) {
                wait_turn(blk2, seen);
#pragma unroll
                for (int e = 0; e < NDB; ++e) old[e] = load_dq4(rdQ, dq_off(blk2, e));
            }
            if (kb > 0) seen = load_flag(flags + i * NW + w);   // for the next step
            if (has2) {
                fa_f32x4 q2[NDB];
                phase2(buf ^ 1, q2);
#pragma unroll
                for (int e = 0; e < NDB; ++e) {
                    const fa_f32x4 v = old[e] + q2[e] * scale;
                    buf_store16(rdQ, dq_off(blk2, e), __builtin_bit_cast(fa_u32x4, v));
                }
            }
            asm volatile("" ::: "memory");
            if (i - 1 >= i_lo) issue_stage(i - 1, buf ^ 1);
            asm volatile("" ::: "memory");

            // ---- phase 1 on block i
            const fa_lds_char *st = sStage + buf * STAGE;
            const fa_lds_char *sQ = st;
            const fa_lds_char *sO = st + QTILE;
            const fa_lds_char *sL = st + 2 * QTILE + 16 * h;
            const fa_lds_char *sD = st + 2 * QTILE + 256 + 16 * h;
            fa_f32x16 sacc = zero16(), pacc;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const fa_f32x4 nd4 = *(const __attribute__((address_space(3))) fa_f32x4 *)(sD + 32 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) pacc[4 * g + e] = nd4[e];
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                sacc = mfma32(lds_read16(sQ, qoff ^ (ks << 5)), lds_read16(sK, koff ^ (ks << 5)), sacc);
                pacc = mfma32(lds_read16(sO, qoff ^ (ks << 5)), vreg[ks], pacc);
            }
            fa_u32x4 pf[2], dsf[2];
            const int q0 = i * kFQ;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int qi = 8 * g + 4 * h;
                const fa_f32x4 l4 = *(const __attribute__((address_space(3))) fa_f32x4 *)(sL + 32 * g);
                float p[4], ds[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, -l4[e]));
                    if constexpr (MASK) pv = kv > q0 + qi + e ? 0.0f : pv;
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
            // dS^T of this wave's 32 keys into the tile for the next step's phase 2
            fa_lds_char *sdw = sDS + buf * DSTILE;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const fa_u32x2 v = {dsf[t][2 * hf], dsf[t][2 * hf + 1]};
                    lds_write8(sdw, ds_off(32 * w + n, 32 * t + 16 * hf + 8 * h), v);
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
            wait_vmem();
            // this step's dQ stores are complete: publish the turn
            if (has2 && lane == 0) buf_store4(rF, (uint32_t)(blk2 * NW + w) * 4, (uint32_t)(kb + 1));
            __syncthreads();
        };

        int it = 0;
        const int i_plain = CAUSAL ? min(nqb, i_lo + kFKeys / kFQ) : 0;   // blocks below need the mask
        for (int i = nqb - 1; i >= i_plain; --i, ++it) step(i, it, std::false_type{});
        for (int i = min(nqb - 1, i_plain - 1); i >= i_lo; --i, ++it) step(i, it, std::true_type{});

        // ---------------------------------------------------------- drain: phase 2 of block i_lo
        {
            fa_f32x4 old[NDB], q2[NDB];
#pragma unroll
            for (int e = 0; e < NDB; ++e) old[e] = fa_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (kb > 0) {
                wait_turn(i_lo, seen);
#pragma unroll
                for (int e = 0; e < NDB; ++e) old[e] = load_dq4(rdQ, dq_off(i_lo, e));
            }
            phase2((it - 1) & 1, q2);
#pragma unroll
            for (int e = 0; e < NDB; ++e) {
                const fa_f32x4 v = old[e] + q2[e] * scale;
                buf_store16(rdQ, dq_off(i_lo, e), __builtin_bit_cast(fa_u32x4, v));
            }
            wait_vmem();
            if (lane == 0) buf_store4(rF, (uint32_t)(i_lo * NW + w) * 4, (uint32_t)(kb + 1));
        }

        // ---------------------------------------------------------- dK, dV of the block
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
        // every wave is done with the K, dS^T and stage tiles before the next
        // item's copies overwrite them
        __syncthreads();
    }
    // the turn flags of the last item, and its dK / dV stores, complete
    // before the workgroup ends (kernel end makes them visible)
}

template <int D, bool CAUSAL>
hipError_t launch_fused_t(const BwdArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((bwd_fused_kernel<D, CAUSAL>), dim3((unsigned)a.n_cu), dim3(kFThreads), 0, st,
                       (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                       (const float *)a.L2vec, (const float *)a.Dvec,
                       (const uint16_t *)a.dO, a.dQ, (uint16_t *)a.dK, (uint16_t *)a.dV, a.sync, a.BH, a.S,
                       a.scale, a.scale * FA_LOG2E, a.nxcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_fused(const BwdArgs &a, hipStream_t st) {
    if (a.d == 128) return a.causal ? launch_fused_t<128, true>(a, st) : launch_fused_t<128, false>(a, st);
    return a.causal ? launch_fused_t<64, true>(a, st) : launch_fused_t<64, false>(a, st);
}

}  // namespace fa
