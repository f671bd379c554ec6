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

// Device state of a graph-replayed denoise loop: everything a replayed step reads
// that changes from step to step (step index, sigma step, First-Block-Cache
// decision and policy counters).  One per loop, in caller memory.
struct LoopState {
  int next;           // step index the next replay runs
  int cur;            // step index being run
  int n_steps;
  int skip;           // this step's decision, 1: blocks 1.. skipped (the launch gate)
  int has_anchor, steps_done, skip_run;
  int warmup_steps, max_skips;
  int cache_on;
  float threshold;
  float dt;           // sigma[cur + 1] - sigma[cur]
  int overrun;        // a replay found next >= n_steps and left the latents alone
};
// Per-step record of a graph-replayed loop.
struct LoopLog {
  double rel;
  int skip;
  int nonfinite;
};

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
// skip, run_if: when skip is set, the kernel runs only while (*skip != 0) == run_if;
// has_anchor_out (optional) is set to 1 by the commit.
hipError_t fbc_commit(const float* x, const float* before, const float* staging, float* cached,
                      float* anchor, int B, int Lt, int Li, int D, hipStream_t st,
                      const int* skip = nullptr, int run_if = 0, int* has_anchor_out = nullptr);
hipError_t fbc_apply(float* x, const float* cached, int B, int Lt, int Li, int D, hipStream_t st,
                     const int* skip = nullptr, int run_if = 1);
// Loop form of the test: the anchor flag, threshold and skip policy come from the
// loop state, which receives the decision; the step's record goes to log[cur].
hipError_t fbc_reduce_loop(const float* x, const float* before, const float* anchor,
                           float* staging, double* part, int nparts, LoopState* s, LoopLog* log,
                           int B, int Lt, int Li, int D, hipStream_t st);
// Start of a replayed step: i = s->next; mod_cur <- mod_all[i] (n_mod floats),
// s->cur = i, s->dt = sig[i + 1] - sig[i], s->skip = 0, log[i] = (+inf, 0, 0).
hipError_t loop_begin(LoopState* s, const float* mod_all, size_t n_mod, const double* sig,
                      float* mod_cur, LoopLog* log, hipStream_t st);
// Euler update with dt from the loop state, then s->next += 1.
hipError_t euler_update_loop(float* lat, const float* v, int n, int cfg, float g, LoopState* s,
                             hipStream_t st);
// x (n elements, n % 4 == 0) between bf16 and fp32
hipError_t widen_bf16(const bf16_t* a, float* b, size_t n, hipStream_t st);
hipError_t narrow_f32(const float* a, bf16_t* b, size_t n, hipStream_t st);
hipError_t euler_update(float* lat, const float* v, int n, int cfg, float g, float dt,
                        hipStream_t st);

}  // namespace dit
