// fa_launch.h -- internal launcher interface between the C ABI (fa_api.hip)
// and the kernel files.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
    const void *Q, *K, *V;
    void *O;
    float *LSE;
    int BH, S, d;
    float scale;
    bool causal;
    float tau;         // rescale threshold, log2 units
    int poly_eighths;  // 0, 1 or 2
    int poly_degree;   // 3 or 5
    bool lpt;          // causal: longest query blocks first
    // Packed variable-length batch (cu_seqlens != nullptr): nseq sequences,
    // sequence s = tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 of Q, K, V, O
    // laid out [total][H][d]; LSE [H][total].  BH = nseq * H and S =
    // max_seqlen then.
    const int *cu_seqlens = nullptr;
    int H = 0;
    int total = 0;
};

struct BwdArgs {
    const void *Q, *K, *V, *O, *dO;
    const float *LSE;
    float *dQ;
    void *dK, *dV;
    float *Dvec;           // workspace: -D (BH*S floats) ...
    float *L2vec = nullptr;  // ... then LSE*log2(e) (BH*S floats)
    int *sync = nullptr;  // workspace: sync words of the fused backward (zeroed by the preprocess)
    int nsync = 0;        // their count
    int BH, S, d;
    float scale;
    bool causal;
    bool lpt;     // causal: longest blocks first
    int n_cu = 0;   // fused backward: compute units (one persistent workgroup each)
    int nxcd = 0;   // fused backward: XCDs (one work queue each)
    void *dS = nullptr;  // stored dS (bwd_ds_bytes): the dK/dV kernel writes it, the dQ kernel reads it
};

// Bytes of the stored dS of a backward over BH heads of length S.
int64_t bwd_ds_bytes(int BH, int S, bool causal);

hipError_t launch_fwd(const FwdArgs &a, hipStream_t st);
hipError_t launch_bwd_preprocess(const BwdArgs &a, hipStream_t st);
hipError_t launch_bwd_dkdv(const BwdArgs &a, hipStream_t st);
hipError_t launch_bwd_dq(const BwdArgs &a, hipStream_t st);
hipError_t launch_bwd_fused(const BwdArgs &a, hipStream_t st);
hipError_t launch_exp2_poly(const float *x, float *y, int64_t n, int degree, hipStream_t st);

}  // namespace fa
