/*
 * fa.h -- C ABI of the MI355X (gfx950) fused exact-attention library.
 *
 * What the operations compute.  FlashAttention-4 (hyper.ai news story, one
 * paragraph; gist.science explainer "FlashAttention-4: Algorithm and Kernel
 * Pipelining Co-Design for Asymmetric Hardware Scaling", technical summary)
 * is an exact, faster implementation of the standard attention of a
 * Transformer.  Per (batch b, head h), with queries, keys and values
 * Q, K, V in R^{S x d}:
 *
 *   forward   S = scale * Q K^T, optional causal mask (key j visible to
 *             query i iff j <= i), P = row-softmax(S), O = P V,
 *             LSE_i = ln sum_j exp(S_ij) over the visible j.
 *   backward  for the loss gradient dO:  D_i = sum_k dO_ik O_ik,
 *             P recomputed from LSE, dV = P^T dO, dP = dO V^T,
 *             dS = P o (dP - D), dQ = scale * dS K, dK = scale * dS^T Q.
 *
 * The forward never forms S x S: it streams key/value tiles with an online
 * softmax (running row max and sum, output rescaled only when the running
 * max grows past a threshold, the "skip the rescale when it is not needed"
 * idea of the gist.science explainer, section 3 of the German page), and
 * schedules causal tiles longest-first (the LPT causal scheduler of the
 * technical summary, "Belangrijkste Resultaten").  The backward recomputes P
 * tile by tile from the saved LSE (technical summary, methodology item 3).
 * Unlike the pages, which add dQ with global atomics, the default backward
 * computes dQ in its own pass over query blocks (fp32 atomics are slow on
 * this GPU); a single-pass variant that adds every key block's share of dQ
 * in a fixed order -- the pages' deterministic mode -- with plain
 * read-modify-writes kept inside one XCD's L2 is available (fa_bwd_fused),
 * and so is a dQ pass that reads the dS the dK/dV pass stored in the
 * workspace instead of recomputing it (fa_options.stored_ds: O(S^2) bytes of
 * workspace per head, traded for two of the dQ pass's three products).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing and keeps no mutable state: everything a call uses
 *     arrives in its arguments (the tuning options as a per-call struct,
 *     copied on entry), so one call cannot see another's settings.
 *   - Q, K, V, O, dO, dK, dV: bf16 (raw 16-bit patterns), contiguous
 *     row-major [B][H][S][d].  LSE: fp32 [B][H][S].  dQ: fp32 [B][H][S][d].
 *     The backward workspace holds -D (fp32 [B][H][S], D_i = sum_k dO_ik
 *     O_ik, kept negated), LSE * log2(e) (fp32 [B][H][S]) and, from byte
 *     round_up(8*B*H*S, 256) on, the int32 sync words of the single-pass
 *     backward: 16 work-queue counters, an error word (index 16: nonzero
 *     after a call means a bounded wait expired and the gradients of that
 *     call are invalid; it cannot happen unless the hardware stops making
 *     progress), padding to 32, then one turn flag per (b*H + h, block of
 *     32 queries, wave slice of 8).  With fa_options.stored_ds the bf16 dS
 *     tiles follow, from byte fa_bwd_workspace_bytes(B, H, S, d) on, in a
 *     layout private to the library.
 *   - Every pointer must be 16-byte aligned.
 *   - d must be 64 or 128.  S may be any value >= 0 (ragged tails are
 *     masked).  B, H >= 0.  B*H*S == 0 is a valid empty call that launches
 *     nothing.  S <= 2^22 (per-head offsets are 32-bit) and B*H <= 2^31-1.
 *   - scale must be finite and > 0 (1/sqrt(d) is the usual value).
 *   - causal must be 0 or 1.
 *   - opts (where taken) may be NULL for the defaults of fa_default_options;
 *     out-of-range fields give FA_ERR_INVALID.
 *   - stream is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work and never synchronize; results are ready when the stream
 *     reaches them.  Argument errors are reported synchronously, before
 *     anything is enqueued.  A failed launch is reported as FA_ERR_HIP.
 *     Faults inside a kernel surface at the caller's next synchronization.
 *   - Calls on different streams are independent; the library is safe to
 *     call from several threads at once.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID = 1,     /* null/misaligned pointer, bad size, scale or flag */
    FA_ERR_UNSUPPORTED = 2, /* head dimension other than 64 or 128; fa_bwd_fused: B*H vs XCDs */
    FA_ERR_HIP = 3,         /* the HIP runtime refused a launch or a device symbol lookup */
    FA_ERR_TOO_LARGE = 4    /* fa_bwd_noalloc: the workspace would not fit its static array */
} fa_status;

/*
 * Tuning options of one call.  None of them changes the mathematical result
 * (only rounding, and for the block order not even that).
 *   rescale_tau: the running row max (in log2 units) is moved, and O and
 *     the row sum rescaled, only when a new tile's max exceeds it by more
 *     than tau -- the rescale that is skipped while the numbers do not grow
 *     too much (gist.science explainer, German page, section 3).  Finite,
 *     0 <= tau <= 64; 0 rescales on every increase (classic online
 *     softmax).  Unnormalised probabilities stay below 2^tau.  Default 8.
 *   poly_eighths: how many eighths (0, 1 or 2) of the forward's
 *     exponentials use the FMA polynomial exp2 instead of the hardware
 *     v_exp_f32 (the hybrid split of the technical summary, methodology
 *     item 2).  Default 0: on gfx950 the hardware exponential costs about two
 *     FMA slots, the polynomial about seven.
 *   poly_degree: 3 or 5 (default 3).
 *   longest_first: causal block order.  1 (default): longest blocks first,
 *     the LPT order of the technical summary's results (forward and dQ
 *     kernel: last query blocks first; dK/dV kernel and single-pass
 *     backward: first key blocks first).  0: shortest first, kept for
 *     measuring what the order is worth; it selects the split backward.
 *     The result does not depend on it beyond the rounding of dQ sums.
 *   fused_backward: 0 (default): fa_bwd / fa_bwd_opt run the split
 *     backward (fa_bwd_dkdv + fa_bwd_dq), the faster one on MI355X; 1: the
 *     single-pass backward (fa_bwd_fused) when B*H is a multiple of the
 *     GPU's XCD count (8 on MI355X), else the split one.  Both are bitwise
 *     repeatable; they differ in the rounding of dQ, dK and dV.
 *   stored_ds: split backward only.  0 (default): the dQ kernel recomputes
 *     S, dP and dS for itself (three matrix products per tile; workspace
 *     O(B*H*S)).  1: the dK/dV kernel also writes its bf16 dS to the
 *     workspace and the dQ kernel reads it back (one product per tile),
 *     trading HBM capacity and traffic for two products: the workspace grows
 *     by 2 bytes per (query, key) pair the mask keeps, about 2*B*H*S*S
 *     (half that causal; fa_bwd_workspace_bytes_opt), or with a smaller
 *     workspace fa_bwd_opt takes the heads in groups (see
 *     fa_bwd_workspace_bytes_min).  dK and dV are bitwise the same either
 *     way, dQ differs in rounding.  Measured on MI355X: faster at d = 128
 *     (backward -7 to -10 % at S = 4096 to 32768), slower at d = 64.  Cannot be
 *     combined with fused_backward (FA_ERR_INVALID).
 * The forward reads the first four fields, the backward the last three.
 */
typedef struct fa_options {
    float rescale_tau;
    int poly_eighths;
    int poly_degree;
    int longest_first;
    int fused_backward;
    int stored_ds;
} fa_options;

/* The defaults: {8.0f, 0, 3, 1, 0, 0}. */
fa_options fa_default_options(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *fa_status_string(fa_status s);

/*
 * Forward pass.  Writes O (bf16 [B][H][S][d]) and LSE (fp32 [B][H][S],
 * natural log of the softmax denominator of each query row).  Q, K, V are
 * read only.  O and LSE must not overlap the inputs.
 */
fa_status fa_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE,
                 int B, int H, int S, int d, float scale, int causal, void *stream);

/* fa_fwd with explicit tuning options (NULL = defaults). */
fa_status fa_fwd_opt(const void *Q, const void *K, const void *V, void *O, float *LSE,
                     int B, int H, int S, int d, float scale, int causal,
                     const fa_options *opts, void *stream);

/*
 * Forward pass over a packed batch of variable-length sequences (the
 * forward-only prefill case; the pages' kernel serves prefill in inference
 * engines, hyper.ai story).  Sequence s (0 <= s < nseq) is tokens
 * cu_seqlens[s] .. cu_seqlens[s+1]-1; attention never crosses sequences,
 * and under causal = 1 token i of a sequence sees its tokens 0 .. i.
 *   Q, K, V, O: bf16 [total][H][d] (token-major, heads interleaved), device.
 *   LSE: fp32 [H][total], device.
 *   cu_seqlens: device int32 array of nseq + 1 offsets, 4-byte aligned,
 *     expected non-decreasing from 0 to total.  The kernel clamps every
 *     entry to [0, total] and to at least the previous one, so bad offsets
 *     cannot make it touch memory outside the tensors; tokens covered by no
 *     sequence are not written.
 *   max_seqlen: an upper bound of the sequence lengths (the launch covers
 *     this many rows per sequence; rows of a longer sequence past it are
 *     not written).
 * Row offsets inside one (sequence, head) are 32-bit: with R = max(max_seqlen
 * rounded up to 256, total + 192) rows (the furthest the kernel's query and
 * key/value tiles reach), R * H * d * 2 must not exceed 2^32, else
 * FA_ERR_INVALID.  max_seqlen <= 2^22.  nseq, H, total or max_seqlen equal
 * to 0 is a valid empty call.  Other rules as fa_fwd_opt.
 */
fa_status fa_fwd_varlen(const void *Q, const void *K, const void *V, void *O, float *LSE,
                        const int *cu_seqlens, int nseq, int H, int total, int max_seqlen, int d,
                        float scale, int causal, const fa_options *opts, void *stream);

/* Bytes of workspace fa_bwd needs: round_up(8*B*H*S, 256) for -D and LSE*log2 e,
 * plus round_up(4*(32 + 8*B*H*ceil(S/32)), 256) for the sync words. */
size_t fa_bwd_workspace_bytes(int B, int H, int S, int d);

/* Workspace bytes of fa_bwd_opt (and of its steps) with these options (NULL
 * = defaults) and this causal flag; 0 for invalid options or an empty
 * problem.  Equal to fa_bwd_workspace_bytes(B, H, S, d) unless stored_ds. */
size_t fa_bwd_workspace_bytes_opt(int B, int H, int S, int d, int causal, const fa_options *opts);

/* The least workspace fa_bwd_opt accepts with these options: the same as
 * fa_bwd_workspace_bytes_opt, except with stored_ds, where it is the
 * default workspace plus the dS of one head.  Between this and
 * fa_bwd_workspace_bytes_opt, fa_bwd_opt runs the heads in equal groups, as
 * few as the workspace allows (dK/dV, then dQ, per group; bitwise the same
 * result, more launches).  0 for invalid options or an empty problem. */
size_t fa_bwd_workspace_bytes_min(int B, int H, int S, int d, int causal, const fa_options *opts);

/*
 * Backward pass for the O and LSE that fa_fwd produced from the same Q, K,
 * V, scale and causal flag.  Writes dQ (fp32 [B][H][S][d]), dK and dV
 * (bf16 [B][H][S][d]) without atomics: dK, dV are written once, dQ is
 * either written once (split backward) or summed over key blocks in a
 * fixed order (single-pass backward), so the result is bitwise
 * reproducible.  workspace must hold at least fa_bwd_workspace_bytes(B, H,
 * S, d) bytes of device memory (fa_bwd_opt: fa_bwd_workspace_bytes_min with
 * the same options and causal flag); its contents on entry are ignored.  Outputs
 * must not overlap inputs.  Steps: fa_bwd_preprocess, then the single-pass
 * kernel, or fa_bwd_dkdv and fa_bwd_dq (see fa_options.fused_backward), with
 * default options.  Calls that share a workspace must be ordered (one
 * stream).
 */
fa_status fa_bwd(const void *Q, const void *K, const void *V, const void *O, const float *LSE,
                 const void *dO, float *dQ, void *dK, void *dV,
                 int B, int H, int S, int d, float scale, int causal,
                 void *workspace, size_t workspace_bytes, void *stream);

/* fa_bwd with explicit options (NULL = defaults). */
fa_status fa_bwd_opt(const void *Q, const void *K, const void *V, const void *O, const float *LSE,
                     const void *dO, float *dQ, void *dK, void *dV,
                     int B, int H, int S, int d, float scale, int causal, const fa_options *opts,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Step 1 of fa_bwd: -D_i = -sum_k dO_ik O_ik and LSE_i * log2(e), fp32, into
 * workspace, and the sync words zeroed.  Same argument rules as fa_bwd.
 */
fa_status fa_bwd_preprocess(const void *O, const void *dO, const float *LSE,
                            int B, int H, int S, int d,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Step 2 of fa_bwd: recompute P from LSE tile by tile and write dK and dV
 * (one workgroup per block of 256 keys).  Reads the -D and LSE*log2(e) that
 * fa_bwd_preprocess left in workspace on the same stream; with stored_ds it
 * also writes dS into workspace.
 */
fa_status fa_bwd_dkdv(const void *Q, const void *K, const void *V,
                      const void *dO, void *dK, void *dV,
                      int B, int H, int S, int d, float scale, int causal, const fa_options *opts,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Step 3 of fa_bwd: recompute P and dP per block of 128 queries (256 for
 * non-causal S >= 8192) and write dQ = scale * dS K in fp32.  Reads the
 * workspace like fa_bwd_dkdv.  With stored_ds (the same options as step 2,
 * on the same stream after it) it reads the dS that step 2 wrote instead,
 * per block of 256 queries.
 */
fa_status fa_bwd_dq(const void *Q, const void *K, const void *V,
                    const void *dO, float *dQ,
                    int B, int H, int S, int d, float scale, int causal, const fa_options *opts,
                    const void *workspace, size_t workspace_bytes, void *stream);

/*
 * Step 2 of fa_bwd's single-pass variant (methodology item 3 of the
 * technical summary: one pass over key blocks, dQ added in a fixed order):
 * recompute P from LSE tile by tile and write dK, dV and dQ.  Reads the -D
 * and LSE*log2 e that fa_bwd_preprocess left in workspace on the same
 * stream, and uses (and leaves nonzero) its sync words, which that step
 * zeroes: run fa_bwd_preprocess before every call.  FA_ERR_UNSUPPORTED if
 * B*H is not a multiple of the GPU's XCD count or the device cannot be
 * queried.  Longest-first order always.
 */
fa_status fa_bwd_fused(const void *Q, const void *K, const void *V, const void *dO,
                       float *dQ, void *dK, void *dV,
                       int B, int H, int S, int d, float scale, int causal,
                       const void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): fa_bwd
 * with its workspace taken from a static device array of the library,
 * FA_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held by each GPU the library
 * runs on until the process ends.  Same arguments and results as fa_bwd
 * (default options), minus the workspace; it allocates nothing.
 *   - Limit: fa_bwd_workspace_bytes(B, H, S, d) (about 9 bytes per query
 *     row: B*H*S up to about 1.86 million rows) must not exceed
 *     FA_NOALLOC_SCRATCH_BYTES, else FA_ERR_TOO_LARGE, reported before any
 *     HIP call.
 *   - The array's device address is looked up (hipGetSymbolAddress) on the
 *     first call on each device, with that device current; a failed lookup
 *     gives FA_ERR_HIP.
 *   - All calls on one GPU share its array, which keeps the last call's
 *     contents (-D, LSE*log2 e, sync words).  Calls that overlap on one GPU (on
 *     different streams, or from several threads without ordering) race on
 *     it and give wrong gradients; order them on one stream.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
fa_status fa_bwd_noalloc(const void *Q, const void *K, const void *V, const void *O, const float *LSE,
                         const void *dO, float *dQ, void *dK, void *dV,
                         int B, int H, int S, int d, float scale, int causal, void *stream);

/*
 * Diagnostic: y[i] = exp2 of x[i] through the device polynomial of the given
 * degree (3 or 5), as the forward kernel evaluates it.  x, y: device fp32
 * arrays of n elements.  For x < -126 the result is 0; the polynomial is
 * meant for x <= 2^7.
 */
fa_status fa_exp2_poly(const float *x, float *y, int64_t n, int degree, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
