// fa_fwd.hip -- fused exact attention forward for gfx950.
//
// Computes, per (batch, head), O = softmax(scale * Q K^T [+ causal mask]) V
// and LSE = ln of each row's softmax denominator, in one pass over key/value
// tiles without forming the S x S matrix (the FlashAttention-4 pages: exact
// attention, hyper.ai story; tiled pipeline, gist.science technical
// summary, methodology item 1).
//
// Work decomposition
//   * one workgroup = 4 waves = 128 query rows (32 per wave) of one head;
//     two workgroups share a CU (256 VGPRs per wave, 64 KB LDS each), so
//     each SIMD interleaves the MFMA phase of one wave with the softmax of
//     the other -- the MFMA/softmax overlap the pages call ping-pong,
//     obtained here from the SIMD's wave arbitration;
//   * key/value tiles of 64 rows stream through LDS, double buffered: the
//     direct memory-to-LDS copies of tile j+1 (buffer_load ... lds) are
//     issued before tile j is computed and land in the other buffer;
//   * per wave and tile: S^T = K Q^T (16 MFMA 32x32x16), online softmax in
//     registers, O^T += V^T P^T (16 MFMA).  Keeping the transposed products
//     puts the query index on the lanes, so row max, row sum and the
//     rescale factor are per lane; only one v_permlane32_swap per tile
//     joins the two half-waves that hold the two halves of a row.
//
// Softmax (the pages' ideas, adapted):
//   * log2 domain: t = s * scale * log2(e), P = 2^(t - m_ref);
//   * conditional rescale: the reference max m_ref only moves when a tile's
//     row max exceeds it by more than tau; otherwise O and l are left alone
//     and P may reach 2^tau (gist.science German explainer, section 3: skip
//     the rescale when the numbers do not grow too large).  The decision is
//     per row, the multiply is skipped for the whole wave when no row needs
//     it.  The result does not depend on tau beyond rounding;
//   * hybrid exp2: POLY eighths of the exponentials (a static subset of the
//     registers) use the FMA polynomial of exp2_poly.h, the rest v_exp_f32
//     (technical summary, methodology item 2);
//   * causal tiles are processed longest first: workgroup ids map to the
//     last query blocks first (LPT, technical summary, results).
#include <type_traits>

#include "fa_common.h"
#include "exp2_poly.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kFwdThreads = 256;
constexpr int kBr = 128;  // query rows per workgroup
constexpr int kBc = 64;   // key/value rows per tile

template <int POLY, int DEG>
__device__ __forceinline__ float exp2_sel(float x, int r) {
    if constexpr (POLY > 0) {
        if ((r & 7) < POLY) return fa_exp2::exp2_poly<DEG>(x);
    }
    return __builtin_amdgcn_exp2f(x);
}

// VARLEN: packed variable-length batch.  Workgroup (unit u, block qi) with
// u = blockIdx % BH takes sequence u / H, head u % H; its rows are tokens
// cu[s] .. cu[s+1]-1 of a [total][H][D] tensor (row pitch H * D elements),
// LSE is [H][total].  cu entries are clamped to [0, total] and made
// non-decreasing, so no access leaves the tensors whatever they hold.
// Otherwise unit u is head u of a [BH][S][D] tensor, LSE [BH][S].
template <int D, bool CAUSAL, int POLY, int DEG, bool VARLEN>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    uint16_t *__restrict__ O, float *__restrict__ LSE, int BH, int S_arg, float c, float tau, int nqb,
    int lpt, const int *__restrict__ cu, int H, int total) {
    constexpr int ROWB = D * 2;        // bytes per row
    constexpr int NCH = ROWB / 16;     // 16-byte chunks per row
    constexpr int KS = D / 16;         // k-steps over d
    constexpr int DB = D / 32;         // 32-wide d blocks of O^T
    constexpr int TILE = kBc * ROWB;   // bytes of one K or V tile

    __shared__ __attribute__((aligned(1024))) char smem_raw[2 * 2 * TILE];
    fa_lds_char *smem = (fa_lds_char *)smem_raw;

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int h = lane >> 5, n = lane & 31;

    const int bh = blockIdx.x % BH;
    const int qi = blockIdx.x / BH;
    const int qblk = (CAUSAL && lpt) ? (nqb - 1 - qi) : qi;
    const int q0 = qblk * kBr;
    int S;                // rows of this unit
    size_t head;          // element offset of its row 0
    size_t lse0;          // index of its row 0 in LSE
    uint32_t pitch;       // bytes between consecutive rows
    if constexpr (VARLEN) {
        const int seq = bh / H, hh = bh - seq * H;
        const int start = min(max(cu[seq], 0), total);
        const int end = min(max(cu[seq + 1], start), total);
        S = end - start;
        if (q0 >= S) return;  // whole workgroup, before any barrier
        head = ((size_t)start * H + hh) * D;
        lse0 = (size_t)hh * total + start;
        pitch = (uint32_t)H * ROWB;
    } else {
        S = S_arg;
        head = (size_t)bh * (size_t)S * D;
        lse0 = (size_t)bh * S;
        pitch = ROWB;
    }
    const int kv_end = CAUSAL ? min(S, q0 + kBr) : S;
    const int nkv = (kv_end + kBc - 1) / kBc;

    const int qrow = q0 + 32 * w + n;   // this lane's query row
    const int wq_lo = q0 + 32 * w;      // first query row of the wave

    // Per-unit buffer resources end with row S - 1: rows at or past S read
    // as zero and are never written.
    const uint32_t head_bytes = (uint32_t)(S - 1) * pitch + ROWB;
    const fa_rsrc rQ = make_rsrc(Q + head, head_bytes);
    const fa_rsrc rK = make_rsrc(K + head, head_bytes);
    const fa_rsrc rV = make_rsrc(V + head, head_bytes);

    // Q^T as the B operand of S^T = K Q^T: lane holds Q[qrow][16ks + 8h .. +7].
    fa_u32x4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = buf_load16(rQ, (uint32_t)qrow * pitch + (16 * ks + 8 * h) * 2);

    fa_f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = zero16();
    float m_ref = -1.0e30f;  // finite sentinel: no inf - inf when a row's tile is fully masked
    float l_sum = 0.0f;

    auto issue_tile = [&](int j, int buf) {
        fa_lds_char *sK = smem + buf * 2 * TILE;
        tile_to_lds_pitched<NCH, kBc>(rK, j * kBc, pitch, sK, w, lane);
        tile_to_lds_pitched<NCH, kBc>(rV, j * kBc, pitch, sK + TILE, w, lane);
    };

    // Lane-dependent LDS offsets, computed once.  Row reads of key row
    // 32 mb + n at chunk 2 ks + h: the swizzle only sees the low 4 bits of
    // the row, so mb is an immediate (32 rows) and one offset per ks remains.
    // Transposing reads of V rows 16 t + 4 h + 8 s + L/4: the swizzle is the
    // same for every t, so t is an immediate and one offset per (db, s)
    // remains.
    int koff[KS], voff[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = tile_off<NCH>(n, (2 * ks + h) * 16);
    {
        const int L = lane & 15;
        const int col = ((lane >> 4) & 1) * 16 + (L & 3) * 4;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) voff[db][s2] = tile_off<NCH>(4 * h + 8 * s2 + (L >> 2), (32 * db + col) * 2);
    }

    // One key/value tile from LDS buffer BUF (a compile-time constant, so
    // every LDS address is a loop-invariant register plus an immediate).
    // MASK: the tile crosses this wave's diagonal or the end of the sequence.
    auto compute_tile = [&](int buf, auto MASKC, int kv0) {
        constexpr bool MASK = decltype(MASKC)::value;
        const fa_lds_char *sK = smem + buf * 2 * TILE;
        const fa_lds_char *sV = sK + TILE;
        // S^T = K Q^T for 64 keys x 32 queries: two 32x32 blocks.
        fa_f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const fa_u32x4 a = lds_read16(sK + 32 * mb * ROWB, koff[ks]);
                sacc[mb] = mfma32(a, qf[ks], sacc[mb]);
            }
        }
        if constexpr (MASK) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kv = kv0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
                    const bool dead = (CAUSAL && kv > qrow) || kv >= S;
                    sacc[mb][r] = dead ? -INFINITY : sacc[mb][r];
                }
        }
        // row max over this lane's 32 keys, then across the two half-waves
        float mx = sacc[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
        mx = max_halves(mx);
        const float m_new = mx * c;
        const bool need = m_new > m_ref + tau;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
            m_ref = need ? m_new : m_ref;
            l_sum *= alpha;
#pragma unroll
            for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
        }
        const float nm = -m_ref;
        // P = 2^(s c - m_ref), packed to bf16 in MFMA k order.  The row sum
        // adds the fp32 values (two partial sums): summing the bf16-rounded
        // ones would put up to 2^-9 relative error into the LSE of rows with
        // few keys.
        fa_u32x4 pf[4];
        float la = 0.0f, lb = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = exp2_sel<POLY, DEG>(fmaf(sacc[mb][r], c, nm), r);
                const float p1 = exp2_sel<POLY, DEG>(fmaf(sacc[mb][r + 1], c, nm), r + 1);
                la += p0;
                lb += p1;
                pf[2 * mb + (r >> 3)][(r & 7) >> 1] = pack_bf16(p0, p1);
            }
        }
        l_sum += la + lb;
        // O^T += V^T P^T, k-step t covers keys 16t .. 16t+15 of the tile in
        // accumulator order; V^T operand by transposing reads of V rows.
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const fa_u32x2 lo = lds_read_tr(sV + 16 * t * ROWB, voff[db][0]);
                const fa_u32x2 hi = lds_read_tr(sV + 16 * t * ROWB, voff[db][1]);
                const fa_u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                oacc[db] = mfma32(a, pf[t], oacc[db]);
            }
        }
    };

    // One loop step: prefetch tile j+1 into the other buffer, compute tile j,
    // then wait for the prefetch and synchronise.  Interior tiles (no key
    // past the diagonal of any row of the workgroup, none past S) run
    // without masking in a first loop; the at most two boundary tiles run
    // masked in a second loop, where a wave whose rows all lie above the
    // tile skips the compute.
    auto step = [&](int j, auto MASKC) {
        const int buf = j & 1;
        if (j + 1 < nkv) issue_tile(j + 1, buf ^ 1);
        const int kv0 = j * kBc;
        if constexpr (decltype(MASKC)::value) {
            if (!(CAUSAL && kv0 > wq_lo + 31)) compute_tile(buf, MASKC, kv0);
        } else {
            compute_tile(buf, MASKC, kv0);
        }
        wait_vmem();      // tile j+1 has landed in the other buffer
        __syncthreads();  // ... for every wave, and nobody still reads this one
    };

    if (nkv > 0) issue_tile(0, 0);
    wait_vmem();
    __syncthreads();

    const int n_plain = min(nkv, (CAUSAL ? min(q0, S) : S) / kBc);
    for (int j = 0; j < n_plain; ++j) step(j, std::false_type{});
    for (int j = n_plain; j < nkv; ++j) step(j, std::true_type{});

    // Epilogue: join the half-row sums, normalise, store O (bf16) and LSE.
    const float l_tot = sum_halves(l_sum);
    const float inv = 1.0f / l_tot;
    const fa_rsrc rO = make_rsrc(O + head, head_bytes);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            fa_u32x2 v = {pack_bf16(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                          pack_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
            buf_store8(rO, (uint32_t)qrow * pitch + (32 * db + 8 * g + 4 * h) * 2, v);
        }
    if (h == 0) {
        const fa_rsrc rL = make_rsrc(LSE + lse0, (uint32_t)S * 4);
        buf_store4(rL, (uint32_t)qrow * 4, __float_as_uint((m_ref + __log2f(l_tot)) * FA_LN2));
    }
}

template <int D, bool CAUSAL, int POLY, int DEG>
hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t st) {
    const int nqb = (a.S + kBr - 1) / kBr;
    const dim3 grid((unsigned)(a.BH * nqb)), block(kFwdThreads);
    if (a.cu_seqlens)
        hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, POLY, DEG, true>), grid, block, 0, st,
                           (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           (uint16_t *)a.O, a.LSE, a.BH, a.S, a.scale * FA_LOG2E, a.tau, nqb, (int)a.lpt,
                           a.cu_seqlens, a.H, a.total);
    else
        hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, POLY, DEG, false>), grid, block, 0, st,
                           (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           (uint16_t *)a.O, a.LSE, a.BH, a.S, a.scale * FA_LOG2E, a.tau, nqb, (int)a.lpt,
                           (const int *)nullptr, 0, 0);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_d(const FwdArgs &a, hipStream_t st) {
    if (a.poly_eighths == 0) return launch_fwd_t<D, CAUSAL, 0, 3>(a, st);
    if (a.poly_eighths == 1) return a.poly_degree == 5 ? launch_fwd_t<D, CAUSAL, 1, 5>(a, st)
                                                       : launch_fwd_t<D, CAUSAL, 1, 3>(a, st);
    return a.poly_degree == 5 ? launch_fwd_t<D, CAUSAL, 2, 5>(a, st)
                              : launch_fwd_t<D, CAUSAL, 2, 3>(a, st);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, hipStream_t st) {
    if (a.d == 128) return a.causal ? launch_fwd_d<128, true>(a, st) : launch_fwd_d<128, false>(a, st);
    return a.causal ? launch_fwd_d<64, true>(a, st) : launch_fwd_d<64, false>(a, st);
}

}  // namespace fa
