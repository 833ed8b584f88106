// fa_api.hip -- the C ABI declared in include/fa.h: argument validation and
// template dispatch.  No allocation, no synchronisation, no mutable state:
// the tuning options arrive with each call and are copied once on entry;
// every launch goes on the caller's stream.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "exp2_poly.h"
#include "fa.h"
#include "fa_common.h"
#include "fa_launch.h"

namespace {

constexpr fa_options kDefaultOptions = {8.0f, 0, 3, 1, 0, 0};

// Copies the caller's options (NULL = defaults) into *out once, so the
// launches of one call all see the same values; false if a field is out of
// range.
bool read_options(const fa_options *opts, fa_options *out) {
    const fa_options o = opts ? *opts : kDefaultOptions;
    if (!isfinite(o.rescale_tau) || o.rescale_tau < 0.0f || o.rescale_tau > 64.0f) return false;
    if (o.poly_eighths < 0 || o.poly_eighths > 2) return false;
    if (o.poly_degree != 3 && o.poly_degree != 5) return false;
    if (o.longest_first != 0 && o.longest_first != 1) return false;
    if (o.fused_backward != 0 && o.fused_backward != 1) return false;
    if (o.stored_ds != 0 && o.stored_ds != 1) return false;
    if (o.fused_backward && o.stored_ds) return false;  // two different backward algorithms
    *out = o;
    return true;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Shared shape/flag checks.  Returns FA_OK when the call is well formed;
// *empty is set when there is nothing to compute.
fa_status check_shape(int B, int H, int S, int d, bool *empty) {
    if (B < 0 || H < 0 || S < 0) return FA_ERR_INVALID;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (S > (1 << 22)) return FA_ERR_INVALID;  // per-head byte offsets stay 32-bit
    const int64_t bh = (int64_t)B * (int64_t)H;
    if (bh > INT32_MAX) return FA_ERR_INVALID;
    // grid sizes: BH * ceil(S / 64) must fit a 32-bit grid dimension
    if (bh * (((int64_t)S + 63) / 64) > INT32_MAX) return FA_ERR_INVALID;
    *empty = (bh == 0 || S == 0);
    return FA_OK;
}

bool good_scale(float s) { return isfinite(s) && s > 0.0f; }

// Workspace layout of the backward: -D and LSE*log2 e (fp32 [BH][S] each),
// then, 256-byte aligned, the sync words of the single-pass backward: 16
// claim counters, an error word, padding to 32, and one turn flag per
// (head, block of 32 queries, wave slice of 8).
size_t sync_offset(int64_t bh, int64_t S) { return ((size_t)(8 * bh * S) + 255) / 256 * 256; }
int64_t sync_words(int64_t bh, int64_t S) { return 32 + bh * ((S + 31) / 32) * 8; }

// Compute units and XCDs of the current device, looked up once per device.
constexpr int kMaxDev = 64;
std::atomic<int> g_ncu[kMaxDev], g_nxcd[kMaxDev];

void device_counts(int *ncu, int *nxcd) {
    *ncu = *nxcd = 0;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return;
    int c = g_ncu[dev].load(std::memory_order_relaxed), x = g_nxcd[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 0;
        if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess) x = 0;
        g_nxcd[dev].store(x, std::memory_order_relaxed);
        g_ncu[dev].store(c, std::memory_order_relaxed);
    }
    *ncu = c;
    *nxcd = x;
}

fa_status hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

__global__ void exp2_poly_kernel(const float *__restrict__ x, float *__restrict__ y, int64_t n,
                                 int degree) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = degree == 5 ? fa_exp2::exp2_poly<5>(x[i]) : fa_exp2::exp2_poly<3>(x[i]);
}

}  // namespace

namespace fa {
hipError_t launch_exp2_poly(const float *x, float *y, int64_t n, int degree, hipStream_t st) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(exp2_poly_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, y, n, degree);
    return hipGetLastError();
}
}  // namespace fa

extern "C" {

const char *fa_status_string(fa_status s) {
    switch (s) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID: return "FA_ERR_INVALID: invalid argument";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension must be 64 or 128";
        case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch or device symbol lookup failed";
        case FA_ERR_TOO_LARGE:
            return "FA_ERR_TOO_LARGE: the workspace (fa_bwd_workspace_bytes) exceeds the static scratch "
                   "array of fa_bwd_noalloc (FA_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown fa_status";
}

fa_options fa_default_options(void) { return kDefaultOptions; }

fa_status fa_fwd_opt(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H,
                     int S, int d, float scale, int causal, const fa_options *opts, void *stream) {
    fa_options o;
    if (!read_options(opts, &o)) return FA_ERR_INVALID;
    bool empty = false;
    fa_status st = check_shape(B, H, S, d, &empty);
    if (st != FA_OK) return st;
    if (!good_scale(scale) || (causal != 0 && causal != 1)) return FA_ERR_INVALID;
    if (empty) return FA_OK;
    if (!Q || !K || !V || !O || !LSE) return FA_ERR_INVALID;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
        return FA_ERR_INVALID;
    fa::FwdArgs a{Q, K, V, O, LSE, B * H, S, d, scale, causal == 1,
                  o.rescale_tau, o.poly_eighths, o.poly_degree, o.longest_first != 0};
    return hip_status(fa::launch_fwd(a, (hipStream_t)stream));
}

fa_status fa_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H,
                 int S, int d, float scale, int causal, void *stream) {
    return fa_fwd_opt(Q, K, V, O, LSE, B, H, S, d, scale, causal, nullptr, stream);
}

fa_status fa_fwd_varlen(const void *Q, const void *K, const void *V, void *O, float *LSE,
                        const int *cu_seqlens, int nseq, int H, int total, int max_seqlen, int d,
                        float scale, int causal, const fa_options *opts, void *stream) {
    fa_options o;
    if (!read_options(opts, &o)) return FA_ERR_INVALID;
    if (nseq < 0 || H < 0 || total < 0 || max_seqlen < 0) return FA_ERR_INVALID;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (!good_scale(scale) || (causal != 0 && causal != 1)) return FA_ERR_INVALID;
    if (max_seqlen > (1 << 22)) return FA_ERR_INVALID;
    // Byte offsets inside one (sequence, head) are 32-bit.  The kernel
    // addresses query/output rows up to max_seqlen rounded up to its 256-row
    // blocks, and key/value rows up to 191 past the end of a sequence (tile
    // copies of the next iteration), at a pitch of H * d * 2 bytes: every such
    // offset must stay below 2^32, or it would wrap onto valid rows.
    const int64_t reach = std::max(((int64_t)max_seqlen + 255) / 256 * 256, (int64_t)total + 192);
    if (reach * H * d * 2 > ((int64_t)1 << 32)) return FA_ERR_INVALID;
    const int64_t units = (int64_t)nseq * H;
    if (units > INT32_MAX || units * (((int64_t)max_seqlen + 63) / 64) > INT32_MAX) return FA_ERR_INVALID;
    if (units == 0 || total == 0 || max_seqlen == 0) return FA_OK;
    if (!Q || !K || !V || !O || !LSE || !cu_seqlens) return FA_ERR_INVALID;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE) ||
        ((uintptr_t)cu_seqlens & 3u) != 0)
        return FA_ERR_INVALID;
    fa::FwdArgs a{Q, K, V, O, LSE, (int)units, max_seqlen, d, scale, causal == 1,
                  o.rescale_tau, o.poly_eighths, o.poly_degree, o.longest_first != 0};
    a.cu_seqlens = cu_seqlens;
    a.H = H;
    a.total = total;
    return hip_status(fa::launch_fwd(a, (hipStream_t)stream));
}

size_t fa_bwd_workspace_bytes(int B, int H, int S, int d) {
    (void)d;
    if (B <= 0 || H <= 0 || S <= 0) return 0;
    const int64_t bh = (int64_t)B * H;
    return sync_offset(bh, S) + ((size_t)sync_words(bh, S) * 4 + 255) / 256 * 256;
}

size_t fa_bwd_workspace_bytes_opt(int B, int H, int S, int d, int causal, const fa_options *opts) {
    fa_options o;
    if (!read_options(opts, &o)) return 0;
    const size_t base = fa_bwd_workspace_bytes(B, H, S, d);
    if (!o.stored_ds || base == 0) return base;
    return base + (size_t)fa::bwd_ds_bytes(B * H, S, causal != 0);
}

size_t fa_bwd_workspace_bytes_min(int B, int H, int S, int d, int causal, const fa_options *opts) {
    fa_options o;
    if (!read_options(opts, &o)) return 0;
    const size_t base = fa_bwd_workspace_bytes(B, H, S, d);
    if (!o.stored_ds || base == 0) return base;
    return base + (size_t)fa::bwd_ds_bytes(1, S, causal != 0);
}

static fa_status check_bwd_common(int B, int H, int S, int d, int causal, const fa_options &o,
                                  const void *workspace, size_t workspace_bytes, bool *empty) {
    fa_status st = check_shape(B, H, S, d, empty);
    if (st != FA_OK) return st;
    if (*empty) return FA_OK;
    if (!workspace || !aligned16(workspace)) return FA_ERR_INVALID;
    if (workspace_bytes < fa_bwd_workspace_bytes_opt(B, H, S, d, causal, &o)) return FA_ERR_INVALID;
    return FA_OK;
}

fa_status fa_bwd_preprocess(const void *O, const void *dO, const float *LSE, int B, int H, int S,
                            int d, void *workspace, size_t workspace_bytes, void *stream) {
    bool empty = false;
    fa_status st = check_bwd_common(B, H, S, d, 0, kDefaultOptions, workspace, workspace_bytes, &empty);
    if (st != FA_OK || empty) return st;
    if (!O || !dO || !LSE || !aligned16(O) || !aligned16(dO) || !aligned16(LSE)) return FA_ERR_INVALID;
    fa::BwdArgs a{};
    a.O = O;
    a.dO = dO;
    a.LSE = LSE;
    a.Dvec = (float *)workspace;
    a.L2vec = a.Dvec + (size_t)B * H * S;
    a.BH = B * H;
    a.S = S;
    a.d = d;
    a.sync = (int *)((char *)workspace + sync_offset(a.BH, S));
    a.nsync = (int)sync_words(a.BH, S);
    return hip_status(fa::launch_bwd_preprocess(a, (hipStream_t)stream));
}

// Common checks of the two gradient kernels; fills the launch arguments.
static fa_status bwd_grad_args(const void *Q, const void *K, const void *V,
                               const void *dO, int B, int H, int S, int d, float scale, int causal,
                               const fa_options *opts, const void *workspace, size_t workspace_bytes,
                               fa::BwdArgs *a, bool *empty) {
    fa_options o;
    if (!read_options(opts, &o)) return FA_ERR_INVALID;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID;
    fa_status st = check_bwd_common(B, H, S, d, causal, o, workspace, workspace_bytes, empty);
    if (st != FA_OK) return st;
    if (!good_scale(scale)) return FA_ERR_INVALID;
    if (*empty) return FA_OK;
    const void *ptrs[] = {Q, K, V, dO};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return FA_ERR_INVALID;
    *a = fa::BwdArgs{};
    a->Q = Q;
    a->K = K;
    a->V = V;
    a->dO = dO;
    a->Dvec = (float *)workspace;
    a->L2vec = a->Dvec + (size_t)B * H * S;
    a->BH = B * H;
    a->S = S;
    a->d = d;
    a->scale = scale;
    a->causal = causal == 1;
    a->lpt = o.longest_first != 0;
    a->sync = (int *)((char *)workspace + sync_offset(a->BH, S));
    a->nsync = (int)sync_words(a->BH, S);
    // the stored dS follows the base workspace (whose size is a multiple of 256)
    if (o.stored_ds) a->dS = (char *)workspace + fa_bwd_workspace_bytes(B, H, S, d);
    return FA_OK;
}

fa_status fa_bwd_dkdv(const void *Q, const void *K, const void *V, const void *dO,
                      void *dK, void *dV, int B, int H, int S, int d, float scale, int causal,
                      const fa_options *opts, void *workspace, size_t workspace_bytes,
                      void *stream) {
    fa::BwdArgs a;
    bool empty = false;
    fa_status st = bwd_grad_args(Q, K, V, dO, B, H, S, d, scale, causal, opts, workspace,
                                 workspace_bytes, &a, &empty);
    if (st != FA_OK || empty) return st;
    if (!dK || !dV || !aligned16(dK) || !aligned16(dV)) return FA_ERR_INVALID;
    a.dK = dK;
    a.dV = dV;
    return hip_status(fa::launch_bwd_dkdv(a, (hipStream_t)stream));
}

fa_status fa_bwd_dq(const void *Q, const void *K, const void *V, const void *dO,
                    float *dQ, int B, int H, int S, int d, float scale, int causal,
                    const fa_options *opts, const void *workspace, size_t workspace_bytes,
                    void *stream) {
    fa::BwdArgs a;
    bool empty = false;
    fa_status st = bwd_grad_args(Q, K, V, dO, B, H, S, d, scale, causal, opts, workspace,
                                 workspace_bytes, &a, &empty);
    if (st != FA_OK || empty) return st;
    if (!dQ || !aligned16(dQ)) return FA_ERR_INVALID;
    a.dQ = dQ;
    return hip_status(fa::launch_bwd_dq(a, (hipStream_t)stream));
}

// Whether the single-pass backward can run on the current device for B*H
// heads: one work queue per XCD holding whole heads.  Fills the launch counts.
static bool fused_supported(fa::BwdArgs *a) {
    int ncu = 0, nxcd = 0;
    device_counts(&ncu, &nxcd);
    if (ncu <= 0 || nxcd <= 0 || nxcd > 16 || a->BH % nxcd != 0) return false;
    a->n_cu = ncu;
    a->nxcd = nxcd;
    return true;
}

fa_status fa_bwd_fused(const void *Q, const void *K, const void *V, const void *dO, float *dQ, void *dK,
                       void *dV, int B, int H, int S, int d, float scale, int causal, const void *workspace,
                       size_t workspace_bytes, void *stream) {
    fa::BwdArgs a;
    bool empty = false;
    fa_status st = bwd_grad_args(Q, K, V, dO, B, H, S, d, scale, causal, nullptr, workspace,
                                 workspace_bytes, &a, &empty);
    if (st != FA_OK || empty) return st;
    const void *outs[] = {dQ, dK, dV};
    for (const void *p : outs)
        if (!p || !aligned16(p)) return FA_ERR_INVALID;
    if (!fused_supported(&a)) return FA_ERR_UNSUPPORTED;
    a.dQ = dQ;
    a.dK = dK;
    a.dV = dV;
    return hip_status(fa::launch_bwd_fused(a, (hipStream_t)stream));
}

// The stored-dS backward in groups of heads that a smaller workspace holds:
// each group runs the dK/dV kernel (writing its dS) and then the dQ kernel
// on its own heads, reusing the same dS area.  Every head's arithmetic is
// that of the single launch, so the result is bitwise the same.  Groups are
// made of whole units of 8 heads (or of the largest power of two that fits,
// below 8), so that a head's workgroups stay on the XCDs they use in the
// single launch (head = workgroup id mod the group's head count), and the
// units are spread evenly over as few groups as the workspace allows (a
// small last group would leave most of the GPU idle, worst under the causal
// mask, where one key block then sets the time).
static fa_status bwd_stored_ds_groups(fa::BwdArgs a, int max_heads_per_group, hipStream_t stream) {
    const int BH = a.BH;
    int unit = 1;
    while (unit * 2 <= std::min(max_heads_per_group, 8)) unit *= 2;
    const int units_per_group = max_heads_per_group / unit;
    const int nunits = (BH + unit - 1) / unit;
    const int ngroups = (nunits + units_per_group - 1) / units_per_group;
    const size_t rows = (size_t)a.S, elems = rows * a.d;
    for (int gi = 0, h0 = 0; gi < ngroups; ++gi) {
        fa::BwdArgs g = a;
        const int units = nunits / ngroups + (gi < nunits % ngroups ? 1 : 0);
        g.BH = std::min(units * unit, BH - h0);
        g.Q = (const char *)a.Q + h0 * elems * 2;
        g.K = (const char *)a.K + h0 * elems * 2;
        g.V = (const char *)a.V + h0 * elems * 2;
        g.dO = (const char *)a.dO + h0 * elems * 2;
        g.dK = (char *)a.dK + h0 * elems * 2;
        g.dV = (char *)a.dV + h0 * elems * 2;
        g.dQ = a.dQ + h0 * elems;
        g.Dvec = a.Dvec + h0 * rows;
        g.L2vec = a.L2vec + h0 * rows;
        fa_status st = hip_status(fa::launch_bwd_dkdv(g, stream));
        if (st != FA_OK) return st;
        st = hip_status(fa::launch_bwd_dq(g, stream));
        if (st != FA_OK) return st;
        h0 += g.BH;
    }
    return FA_OK;
}

fa_status fa_bwd_opt(const void *Q, const void *K, const void *V, const void *O, const float *LSE,
                     const void *dO, float *dQ, void *dK, void *dV, int B, int H, int S, int d,
                     float scale, int causal, const fa_options *opts, void *workspace,
                     size_t workspace_bytes, void *stream) {
    fa_options o;
    if (!read_options(opts, &o)) return FA_ERR_INVALID;
    // Stored dS with a workspace too small for every head's dS at once, but
    // large enough for at least one head's: run the heads in groups.
    int group = 0;
    if (o.stored_ds && causal >= 0 && causal <= 1) {
        const size_t full = fa_bwd_workspace_bytes_opt(B, H, S, d, causal, &o);
        const size_t base = fa_bwd_workspace_bytes(B, H, S, d);
        const size_t per_head = base ? (size_t)fa::bwd_ds_bytes(1, S, causal != 0) : 0;
        if (full && workspace_bytes < full && per_head && workspace_bytes >= base + per_head) {
            group = (int)std::min<size_t>((workspace_bytes - base) / per_head, (size_t)B * H);
            o.stored_ds = 0;  // so that the checks below ask only for the base workspace
        }
    }
    fa::BwdArgs a;
    bool empty = false;
    fa_status st = bwd_grad_args(Q, K, V, dO, B, H, S, d, scale, causal, &o, workspace,
                                 workspace_bytes, &a, &empty);
    if (st != FA_OK || empty) return st;
    const void *outs[] = {O, LSE, dQ, dK, dV};
    for (const void *p : outs)
        if (!p || !aligned16(p)) return FA_ERR_INVALID;
    st = fa_bwd_preprocess(O, dO, LSE, B, H, S, d, workspace, workspace_bytes, stream);
    if (st != FA_OK) return st;
    if (group > 0) {
        a.dQ = dQ;
        a.dK = dK;
        a.dV = dV;
        a.dS = (char *)workspace + fa_bwd_workspace_bytes(B, H, S, d);
        return bwd_stored_ds_groups(a, group, (hipStream_t)stream);
    }
    // The single-pass backward needs one work queue per XCD holding whole
    // heads (B*H a multiple of the XCD count) and runs its own longest-first
    // order; otherwise, or when asked, the split dK/dV and dQ kernels run.
    if (o.fused_backward && o.longest_first && fused_supported(&a)) {
        a.dQ = dQ;
        a.dK = dK;
        a.dV = dV;
        return hip_status(fa::launch_bwd_fused(a, (hipStream_t)stream));
    }
    st = fa_bwd_dkdv(Q, K, V, dO, dK, dV, B, H, S, d, scale, causal, &o, workspace, workspace_bytes,
                     stream);
    if (st != FA_OK) return st;
    return fa_bwd_dq(Q, K, V, dO, dQ, B, H, S, d, scale, causal, &o, workspace, workspace_bytes, stream);
}

fa_status fa_bwd(const void *Q, const void *K, const void *V, const void *O, const float *LSE,
                 const void *dO, float *dQ, void *dK, void *dV, int B, int H, int S, int d,
                 float scale, int causal, void *workspace, size_t workspace_bytes, void *stream) {
    return fa_bwd_opt(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, S, d, scale, causal, nullptr, workspace,
                      workspace_bytes, stream);
}

// ------------------------------------------------------------ no-allocation backward
// The workspace of fa_bwd_noalloc: one array per GPU the library runs on,
// held until the process ends.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, once per
// device, with that device current, and only that address is passed on.
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up on the first
// call there; nullptr (and *err set) if the lookup fails.
void *scratch_address(hipError_t *err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !p) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}
}  // namespace

fa_status fa_bwd_noalloc(const void *Q, const void *K, const void *V, const void *O, const float *LSE,
                         const void *dO, float *dQ, void *dK, void *dV, int B, int H, int S, int d,
                         float scale, int causal, void *stream) {
    // Host checks first (no HIP call for a malformed or oversized call).
    bool empty = false;
    fa_status st = check_shape(B, H, S, d, &empty);
    if (st != FA_OK) return st;
    if (!good_scale(scale) || (causal != 0 && causal != 1)) return FA_ERR_INVALID;
    if (empty) return FA_OK;
    const size_t need = fa_bwd_workspace_bytes(B, H, S, d);
    if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
    const void *ptrs[] = {Q, K, V, O, LSE, dO, dQ, dK, dV};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return FA_ERR_INVALID;
    hipError_t err = hipSuccess;
    void *ws = scratch_address(&err);
    if (!ws) return FA_ERR_HIP;
    // Every element of the workspace that the gradient kernels read is
    // written by the preprocess step of this call first: nothing to clear.
    return fa_bwd_opt(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, S, d, scale, causal, nullptr, ws, need,
                      stream);
}

fa_status fa_exp2_poly(const float *x, float *y, int64_t n, int degree, void *stream) {
    if (n < 0 || (degree != 3 && degree != 5)) return FA_ERR_INVALID;
    if (n == 0) return FA_OK;
    if (!x || !y) return FA_ERR_INVALID;
    if ((n + 255) / 256 > INT32_MAX) return FA_ERR_INVALID;
    return hip_status(fa::launch_exp2_poly(x, y, n, degree, (hipStream_t)stream));
}

}  // extern "C"
