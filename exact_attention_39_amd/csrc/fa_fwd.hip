// fa_fwd.hip -- fused exact attention forward for gfx950.
//
// Computes, per (batch, head), O = softmax(scale * Q K^T [+ causal mask]) V
// and LSE = ln of each row's softmax denominator, in one pass over key/value
// tiles without forming the S x S matrix (the FlashAttention-4 pages: exact
// attention, hyper.ai story; tiled pipeline, gist.science technical
// summary, methodology item 1).
//
// Work decomposition (warp specialisation, the MFMA/softmax overlap of the
// gist.science technical summary, methodology item 1, mapped to CDNA4):
//   * one workgroup = 8 waves = 256 query rows of one head, one workgroup
//     per CU.  Waves 0-3 are score waves, waves 4-7 PV waves; wave w and
//     wave w + 4 (one of each per SIMD) form a pair that owns 64 query rows
//     as two halves of 32;
//   * the score wave forms S^T = K Q^T for its 64 rows (16 MFMA 32x32x16
//     per half; every K operand read from LDS feeds the MFMAs of both
//     halves), runs the online softmax and hands P, already packed as the
//     PV MFMA operand, plus the per-row rescale factors to its partner
//     through LDS;
//   * the PV wave holds O^T of the 64 rows and adds V^T P^T one tile later
//     (every V^T operand feeds both halves).  On each SIMD the PV wave's
//     MFMAs run while the score wave computes exponentials;
//   * key/value tiles of 64 rows stream through LDS, K and V double
//     buffered and filled by direct memory-to-LDS copies (buffer_load ...
//     lds) one iteration ahead; one workgroup barrier per tile;
//   * the transposed products put the query index on the lanes, so row max,
//     row sum and the rescale factor are per lane; one v_permlane32_swap
//     joins the two half-waves that hold the two halves of a row.
//
// Softmax (the pages' ideas, adapted):
//   * log2 domain: t = s * scale * log2(e), P = 2^(t - m_ref);
//   * conditional rescale: the reference max m_ref only moves when a tile's
//     row max exceeds it by more than tau; otherwise O and l are left alone
//     and P may reach 2^tau (gist.science German explainer, section 3: skip
//     the rescale when the numbers do not grow too large).  The decision is
//     per row, the multiply is skipped for the whole wave when no row needs
//     it.  The result does not depend on tau beyond rounding.  With tau > 0
//     P is formed against the reference first and the row maxima are only
//     taken when some lane's partial row sum exceeds 2^tau (then some P may
//     have), which leaves the common tile with no max reduction at all;
//     tau <= 0 takes the maxima first (the classic order);
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

constexpr int kFwdThreads = 512;  // waves 0-3 score waves, 4-7 PV waves (one of each per SIMD)
constexpr int kBr = 256;  // query rows per workgroup: 64 per wave pair
constexpr int kBc = 64;   // key/value rows per tile

template <int POLY, int DEG>
__device__ __forceinline__ float exp2_sel(float x, int r) {
    if constexpr (POLY > 0) {
        if ((r & 7) < POLY) return fa_exp2::exp2_poly<DEG>(x);
    }
    return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return __builtin_amdgcn_readfirstlane(v);
}

// Work item (sequence, query block) g of a packed batch, in longest-first
// order, or !valid past the last item.  The cost of an item is its number of
// key tiles: qblk + 1 blocks' worth when causal, the whole sequence when
// not.  Items are grouped into levels, highest first, so no early-exit
// workgroups sit between the working ones whatever the order of the
// sequences in the batch:
//   * causal: the level of a sequence is floor(log2(its block count)); the
//     sequences of a level follow in index order, each with all its blocks,
//     highest first.  So the workgroups running together are mostly blocks
//     of one sequence (and, heads innermost, of one head on one XCD), which
//     read the same key/value tiles: one tile in L2 serves many of them.
//     The longest blocks of the longest sequences start first and the last
//     items are blocks of the shortest sequences, which keeps the tail
//     short (the longest-first idea at the granularity of sequences);
//   * non-causal: level = blocks of the sequence - 1 (all blocks of a
//     sequence cost the same), all blocks of each such sequence in turn.
// Every wave computes this on its own from cu (no LDS, no barrier); the
// level is found by bisection over F(c) = number of items at levels >= c.
// Blocks of a sequence past nqb (a sequence longer than max_seqlen) are not
// counted.
struct VarlenItem {
    int seq, qblk;
    bool valid;
};

template <bool CAUSAL>
__device__ VarlenItem varlen_item(const int *__restrict__ cu, int nseq, int total, int nqb, int g, int lpt,
                                  int lane) {
    auto nb_at = [&](int s) -> int {
        if (s >= nseq) return 0;
        const int a = min(max(cu[s], 0), total);
        const int b = min(max(cu[s + 1], a), total);
        return min((b - a + kBr - 1) / kBr, nqb);
    };
    const int nb0 = nb_at(lane);  // the first 64 sequences, kept
    auto nb_chunk = [&](int s0) { return s0 == 0 ? nb0 : nb_at(s0 + lane); };
    // items of one sequence at level c, and at levels >= c
    auto level_of = [](int nb) { return 31 - __builtin_clz((unsigned)nb); };   // nb >= 1
    auto at_level = [&](int nb, int c) -> int {
        if constexpr (CAUSAL) return (nb > 0 && level_of(nb) == c) ? nb : 0;
        return nb == c + 1 ? nb : 0;
    };
    auto from_level = [&](int nb, int c) -> int {
        if constexpr (CAUSAL) return (nb > 0 && level_of(nb) >= c) ? nb : 0;
        return nb > c ? nb : 0;
    };
    auto F = [&](int c) -> int {
        int acc = 0;
        for (int s0 = 0; s0 < nseq; s0 += 64) acc += wave_sum(from_level(nb_chunk(s0), c));
        return acc;
    };
    VarlenItem it{0, 0, false};
    const int items = F(0);
    if (g >= items) return it;
    if (!lpt) g = items - 1 - g;
    const int nlev = CAUSAL ? 32 - __builtin_clz((unsigned)max(nqb, 1)) : nqb;
    int lo = 0, hi = nlev, f_hi = 0;  // F(lo) > g >= F(hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        const int f = F(mid);
        if (f > g) {
            lo = mid;
        } else {
            hi = mid;
            f_hi = f;
        }
    }
    // item r of level lo: the sequence holding it by a running count over
    // the sequences in index order, then the block within that sequence
    int r = g - f_hi;
    for (int s0 = 0; s0 < nseq; s0 += 64) {
        const int cnt = at_level(nb_chunk(s0), lo);
        int incl = cnt;   // inclusive prefix over the lanes of this chunk
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        const uint64_t m = __builtin_amdgcn_ballot_w64(incl > r);
        if (m != 0) {
            const int ln = __builtin_ctzll(m);
            const int c_ln = __shfl(cnt, ln), incl_ln = __shfl(incl, ln);
            const int k = r - (incl_ln - c_ln);          // position within the sequence's items
            it.seq = s0 + ln;
            it.qblk = CAUSAL ? c_ln - 1 - k : k;
            it.valid = true;
            return it;
        }
        r -= __shfl(incl, 63);
    }
    return it;  // not reached: F counted the item
}

// VARLEN: packed variable-length batch; the workgroup's sequence, head and
// query block come from varlen_item.  Its rows are tokens cu[s] .. cu[s+1]-1
// of a [total][H][D] tensor (row pitch H * D elements), LSE is [H][total].
// cu entries are clamped to [0, total] and made non-decreasing, so no access
// leaves the tensors whatever they hold.  Otherwise unit u = blockIdx % BH
// is head u of a [BH][S][D] tensor, LSE [BH][S].
template <int D, bool CAUSAL, int POLY, int DEG, bool VARLEN>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    uint16_t *__restrict__ O, float *__restrict__ LSE, int BH, int S_arg, float c, float tau, int nqb,
    int lpt, const int *__restrict__ cu, int H, int total) {
    constexpr int ROWB = D * 2;        // bytes per row
    constexpr int NCH = ROWB / 16;     // 16-byte chunks per row
    constexpr int KS = D / 16;         // k-steps over d
    constexpr int DB = D / 32;         // 32-wide d blocks of O^T
    constexpr int TILE = kBc * ROWB;   // bytes of one K or V tile

    // LDS: K slots [2], V slots [2] (tile t in slot t & 1); P hand-off
    // buffers [2] (P of tile t in buffer t & 1), per wave pair, query half
    // sb and k-step u one 16-byte operand per lane; rescale factors [2]
    // (the same indexing, one float per lane).
    constexpr int PBUF = 4 * 2 * 4 * 64 * 16;
    constexpr int ABUF = 4 * 2 * 64 * 4;
    __shared__ __attribute__((aligned(1024))) char smem_raw[4 * TILE + 2 * PBUF + 2 * ABUF];
    fa_lds_char *smem = (fa_lds_char *)smem_raw;
    fa_lds_char *sPb = smem + 4 * TILE;
    fa_lds_char *sAb = sPb + 2 * PBUF;

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int h = lane >> 5, n = lane & 31;

    int qblk;             // query block of this workgroup
    int S;                // rows of this unit
    size_t head;          // element offset of its row 0
    size_t lse0;          // index of its row 0 in LSE
    uint32_t pitch;       // bytes between consecutive rows
    if constexpr (VARLEN) {
        // Heads innermost: workgroup b takes head b % H of work item b / H
        // (a sequence and one of its query blocks) in longest-first order.
        const int hh = blockIdx.x % H;
        const VarlenItem it = varlen_item<CAUSAL>(cu, BH / H, total, nqb, blockIdx.x / H, lpt, lane);
        if (!it.valid) return;  // whole workgroup, before any barrier
        qblk = it.qblk;
        const int start = min(max(cu[it.seq], 0), total);
        const int end = min(max(cu[it.seq + 1], start), total);
        S = end - start;
        head = ((size_t)start * H + hh) * D;
        lse0 = (size_t)hh * total + start;
        pitch = (uint32_t)H * ROWB;
    } else {
        const int bh = blockIdx.x % BH;
        const int qi = blockIdx.x / BH;
        qblk = (CAUSAL && lpt) ? (nqb - 1 - qi) : qi;
        S = S_arg;
        head = (size_t)bh * (size_t)S * D;
        lse0 = (size_t)bh * S;
        pitch = ROWB;
    }
    const int q0 = qblk * kBr;
    const int kv_end = CAUSAL ? min(S, q0 + kBr) : S;
    const int nkv = (kv_end + kBc - 1) / kBc;

    const int pair = w & 3;             // the 64 query rows q0 + 64 pair ..
    const bool score_wave = w < 4;      // S^T and softmax; the partner does O^T += V^T P^T
    const int prow0 = q0 + 64 * pair;   // first query row of the pair

    // Per-unit buffer resources end with row S - 1: rows at or past S read
    // as zero and are never written.
    const uint32_t head_bytes = (uint32_t)(S - 1) * pitch + ROWB;
    const fa_rsrc rQ = make_rsrc(Q + head, head_bytes);
    const fa_rsrc rK = make_rsrc(K + head, head_bytes);
    const fa_rsrc rV = make_rsrc(V + head, head_bytes);

    auto issue_k = [&](int t) __attribute__((always_inline)) {
        tile_to_lds_pitched<NCH, kBc, 8>(rK, t * kBc, pitch, smem + (t & 1) * TILE, w, lane);
    };
    auto issue_v = [&](int t) __attribute__((always_inline)) {
        tile_to_lds_pitched<NCH, kBc, 8>(rV, t * kBc, pitch, smem + (2 + (t & 1)) * TILE, w, lane);
    };
    // this lane's 16-byte P operand of half sb, k-step u in buffer b, and
    // its rescale factor of half sb
    auto p_slot = [&](int b, int sb, int u) __attribute__((always_inline)) {
        return sPb + b * PBUF + (((pair * 2 + sb) * 4 + u) * 64 + lane) * 16;
    };
    auto a_slot = [&](int b, int sb) __attribute__((always_inline)) {
        return sAb + b * ABUF + ((pair * 2 + sb) * 64 + lane) * 4;
    };

    // Iteration j (0 <= j <= nkv): the copies of K_{j+1} and V_j start; the
    // score wave turns tile j into P(j); the PV wave adds tile j - 1 to O.
    // K_{j+1} and V_j go to the slots last read in iteration j - 1 (K_{j-1}
    // by the score wave, V_{j-2} by the PV wave); P(j) to the buffer the PV
    // wave read in iteration j - 1.  One barrier per iteration.
    const int n_plain = min(nkv, (CAUSAL ? min(q0, S) : S) / kBc);
    issue_k(0);
    wait_vmem();
    __syncthreads();

    if (score_wave) {
        // ------------------------------------------------ score wave
        // Q^T of both halves as B operands: lane holds Q[row][16ks + 8h .. +7].
        fa_u32x4 qf[2][KS];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[sb][ks] = buf_load16(rQ, (uint32_t)(prow0 + 32 * sb + n) * pitch + (16 * ks + 8 * h) * 2);
        float m_ref[2] = {-1.0e30f, -1.0e30f};  // finite sentinel: no inf - inf for fully masked rows
        float l_sum[2] = {0.0f, 0.0f};
        // Row reads of key row 32 mb + n at chunk 2 ks + h: the swizzle only
        // sees the low 4 bits of the row, so mb is an immediate.
        int koff[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) koff[ks] = tile_off<NCH>(n, (2 * ks + h) * 16);

        // S^T = K_t Q^T, 64 keys x 2 halves of 32 queries; each K operand
        // feeds the MFMAs of both halves.
        fa_f32x16 sacc[2][2];
        auto s_product = [&](int t) __attribute__((always_inline)) {
            const fa_lds_char *sK = smem + (t & 1) * TILE;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) sacc[sb][0] = sacc[sb][1] = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const fa_u32x4 a = lds_read16(sK + 32 * mb * ROWB, koff[ks]);
#pragma unroll
                    for (int sb = 0; sb < 2; ++sb) sacc[sb][mb] = mfma32(a, qf[sb][ks], sacc[sb][mb]);
                }
            }
        };

        // Online softmax of S^T(t) into P(t) and the rescale factors, both
        // handed to the PV wave through buffer t & 1.  tau_pow sits just
        // below 2^tau, so that a P of 2^tau times (1 - 1 ulp) from a row max
        // exactly tau past its reference still takes the row-max path.
        // With tau <= 0 every new row max moves the reference, so P is formed
        // after the row maxima (MAXFIRST), the classic order.
        const float tau_pow = __builtin_amdgcn_exp2f(tau) * 0.999f;
        auto softmax = [&](int t, auto MASKC, auto MAXFIRSTC) __attribute__((always_inline)) {
            constexpr bool MAXFIRST = decltype(MAXFIRSTC)::value;
            const int kv0 = t * kBc;
            if constexpr (decltype(MASKC)::value) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int kv = kv0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
                            const bool dead = (CAUSAL && kv > prow0 + 32 * sb + n) || kv >= S;
                            sacc[sb][mb][r] = dead ? -INFINITY : sacc[sb][mb][r];
                        }
            }
            // P = 2^(s c - m_ref) of half sb, packed to bf16 in MFMA k order
            // and handed over; returns the lane's partial row sum.  The row
            // sum adds the fp32 values (two partial sums): summing the
            // bf16-rounded ones would put up to 2^-9 relative error into the
            // LSE of rows with few keys.
            auto form_p = [&](int sb, float nm) __attribute__((always_inline)) {
                float la = 0.0f, lb = 0.0f;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                    for (int r8 = 0; r8 < 16; r8 += 8) {
                        fa_u32x4 pk;
#pragma unroll
                        for (int r = r8; r < r8 + 8; r += 2) {
                            const float p0 = exp2_sel<POLY, DEG>(fmaf(sacc[sb][mb][r], c, nm), r);
                            const float p1 = exp2_sel<POLY, DEG>(fmaf(sacc[sb][mb][r + 1], c, nm), r + 1);
                            la += p0;
                            lb += p1;
                            pk[(r & 7) >> 1] = pack_bf16(p0, p1);
                        }
                        lds_write16(p_slot(t & 1, sb, 2 * mb + (r8 >> 3)), 0, pk);
                    }
                }
                return la + lb;
            };
            // P is first formed against the current reference max.  If no
            // lane's partial row sum exceeds 2^tau, no P exceeds 2^tau, so no
            // row max has moved more than tau past its reference: that is the
            // result, and no row max is taken.  Otherwise (a larger or
            // non-finite sum; always on a row's first tile, whose reference
            // is the finite sentinel) take the row maxima, move the reference
            // of the rows whose max exceeds it by more than tau, and form P
            // again for a half in which any row moved.
            float part[2], alpha[2] = {1.0f, 1.0f};
            // row max over this lane's 32 keys, then across the half-waves;
            // moves the reference of the rows whose max exceeds it by more
            // than tau
            auto move_reference = [&](int sb) __attribute__((always_inline)) {
                float mx = sacc[sb][0][0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[sb][0][r]);
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][1][r]);
                mx = max_halves(mx);
                const float m_new = mx * c;
                const bool need = m_new > m_ref[sb] + tau;
                alpha[sb] = need ? __builtin_amdgcn_exp2f(m_ref[sb] - m_new) : 1.0f;
                m_ref[sb] = need ? m_new : m_ref[sb];
                return need;
            };
            if constexpr (MAXFIRST) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    move_reference(sb);
                    part[sb] = form_p(sb, -m_ref[sb]);
                }
            } else {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) part[sb] = form_p(sb, -m_ref[sb]);
                if (__builtin_amdgcn_ballot_w64(!(part[0] <= tau_pow) || !(part[1] <= tau_pow))) {
#pragma unroll
                    for (int sb = 0; sb < 2; ++sb)
                        if (__builtin_amdgcn_ballot_w64(move_reference(sb))) part[sb] = form_p(sb, -m_ref[sb]);
                }
            }
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                l_sum[sb] = fmaf(l_sum[sb], alpha[sb], part[sb]);
                *(__attribute__((address_space(3))) float *)a_slot(t & 1, sb) = alpha[sb];
            }
        };

        // Iteration j: S^T(j), then its softmax.
        // The score waves issue their share of the copies after the S^T
        // MFMAs, off the head of the critical path, and without a branch
        // between S^T and the softmax (which would keep the compiler from
        // interleaving them).  The copies past the last tile read rows at or
        // past S (zeros) or rows no iteration uses, into slots no later
        // iteration reads.
        auto iteration = [&](int j, auto MASKC, auto MAXFIRSTC) __attribute__((always_inline)) {
            if (j < nkv) {
                s_product(j);
                issue_k(j + 1);
                issue_v(j);
                softmax(j, MASKC, MAXFIRSTC);
            } else {
                issue_k(j + 1);
                issue_v(j);
            }
            wait_vmem();
            __syncthreads();
        };
        auto tiles = [&](auto MAXFIRSTC) __attribute__((always_inline)) {
            int j = 0;
            for (; j < n_plain; ++j) iteration(j, std::false_type{}, MAXFIRSTC);
            for (; j <= nkv; ++j) iteration(j, std::true_type{}, MAXFIRSTC);
        };
        if (tau > 0.0f)
            tiles(std::false_type{});
        else
            tiles(std::true_type{});

        // hand the row sums and reference maxima to the PV wave; store LSE
        const fa_rsrc rL = make_rsrc(LSE + lse0, (uint32_t)S * 4);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const float l_tot = sum_halves(l_sum[sb]);
            *(__attribute__((address_space(3))) float *)a_slot(0, sb) = l_tot;
            if (h == 0)
                buf_store4(rL, (uint32_t)(prow0 + 32 * sb + n) * 4,
                           __float_as_uint((m_ref[sb] + __log2f(l_tot)) * FA_LN2));
        }
        __syncthreads();
    } else {
        // ------------------------------------------------ PV wave
        fa_f32x16 oacc[2][DB];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[sb][db] = zero16();
        // Transposing reads of V rows 16 u + 4 h + 8 s + L/4: the swizzle is
        // the same for every u, so u is an immediate and one offset per
        // (db, s) remains.
        int voff[DB][2];
        {
            const int L = lane & 15;
            const int col = ((lane >> 4) & 1) * 16 + (L & 3) * 4;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    voff[db][s2] = tile_off<NCH>(4 * h + 8 * s2 + (L >> 2), (32 * db + col) * 2);
        }

        // O^T = alpha O^T + V^T P^T for tile t (P(t) in buffer t & 1, V_t in
        // V slot t & 1); each V^T operand feeds the MFMAs of both halves.
        auto pv_tile = [&](int t) __attribute__((always_inline)) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                const float alpha = *(const __attribute__((address_space(3))) float *)a_slot(t & 1, sb);
                if (__builtin_amdgcn_ballot_w64(alpha < 1.0f)) {
#pragma unroll
                    for (int db = 0; db < DB; ++db) oacc[sb][db] *= alpha;
                }
            }
            const fa_lds_char *sV = smem + (2 + (t & 1)) * TILE;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const fa_u32x4 p0 = lds_read16(p_slot(t & 1, 0, u), 0);
                const fa_u32x4 p1 = lds_read16(p_slot(t & 1, 1, u), 0);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const fa_u32x2 lo = lds_read_tr(sV + 16 * u * ROWB, voff[db][0]);
                    const fa_u32x2 hi = lds_read_tr(sV + 16 * u * ROWB, voff[db][1]);
                    const fa_u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[0][db] = mfma32(a, p0, oacc[0][db]);
                    oacc[1][db] = mfma32(a, p1, oacc[1][db]);
                }
            }
        };

        for (int j = 0; j <= nkv; ++j) {
            if (j + 1 < nkv) issue_k(j + 1);
            if (j < nkv) issue_v(j);
            if (j >= 1) pv_tile(j - 1);
            wait_vmem();
            __syncthreads();
        }
        __syncthreads();  // the score wave's row sums are in the buffer

        // Epilogue: normalise O (bf16) into this wave's 64 rows of a
        // swizzled LDS tile (the K/V slots are free now), then store whole
        // rows: each lane holds 4 consecutive d of a column of O^T, so
        // stores straight from the accumulators would touch 32 rows per
        // instruction with 8 bytes each.
        fa_lds_char *sO = smem + (w - 4) * (64 * ROWB);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const float inv = 1.0f / *(const __attribute__((address_space(3))) float *)a_slot(0, sb);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    fa_u32x2 v = {pack_bf16(oacc[sb][db][4 * g] * inv, oacc[sb][db][4 * g + 1] * inv),
                                  pack_bf16(oacc[sb][db][4 * g + 2] * inv, oacc[sb][db][4 * g + 3] * inv)};
                    lds_write8(sO, tile_off<NCH>(32 * sb + n, (32 * db + 8 * g + 4 * h) * 2), v);
                }
        }
        const fa_rsrc rO = make_rsrc(O + head, head_bytes);
        constexpr int RPI = 1024 / ROWB;  // rows per 1 KB store instruction
#pragma unroll
        for (int i = 0; i < 64 / RPI; ++i) {
            const int row = i * RPI + lane / NCH, ch = lane % NCH;
            buf_store16(rO, (uint32_t)(prow0 + row) * pitch + ch * 16, lds_read16(sO, tile_off<NCH>(row, ch * 16)));
        }
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
