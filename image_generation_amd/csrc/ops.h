// Launchers of the bandwidth-bound kernels (internal to libdit).
#pragma once
#include <hip/hip_runtime.h>
#include "common.h"

namespace dit {

// Result of the First-Block-Cache test, written by the device, read by the host.
struct FbcResult {
  double rel;      // relative L1 change (+inf without an anchor)
  int skip;        // 1: skip the remaining blocks
  int nonfinite;   // 1: a NaN / Inf reached the reduction
};

constexpr int FBC_PARTS = 1024;   // blocks of the first reduction pass

// WT, TT, OT: bf16_t or float
template <class WT>
hipError_t embed_latents(const float* lat, const WT* W, const float* bias, float* x,
                         float* before, int B, int Lt, int Li, int D, int Cin, hipStream_t st);
template <class TT>
hipError_t text_to_stream(const TT* txt, float* x, int B, int Lt, int L, int D, hipStream_t st);
constexpr int SIG_CHUNK = 64;
struct SigChunk { double s[SIG_CHUNK]; };
// Timestep embedding of host sigmas (passed through kernel arguments).
template <class OT>
hipError_t sinusoid_host(const double* sig_host, OT* e, int M, int half, hipStream_t st);
hipError_t rope_table(float* tab, int grid_w, int Lt, int L, int d, double theta, hipStream_t st);
hipError_t fbc_reduce(const float* x, const float* before, const float* anchor, float* staging,
                      double* part, int nparts, FbcResult* res, int B, int Lt, int Li, int D,
                      int has_anchor, double threshold, hipStream_t st);
hipError_t fbc_commit(const float* x, const float* before, const float* staging, float* cached,
                      float* anchor, int B, int Lt, int Li, int D, hipStream_t st);
hipError_t fbc_apply(float* x, const float* cached, int B, int Lt, int Li, int D, hipStream_t st);
// x (n elements, n % 4 == 0) between bf16 and fp32
hipError_t widen_bf16(const bf16_t* a, float* b, size_t n, hipStream_t st);
hipError_t narrow_f32(const float* a, bf16_t* b, size_t n, hipStream_t st);
hipError_t euler_update(float* lat, const float* v, int n, int cfg, float g, float dt,
                        hipStream_t st);

}  // namespace dit
