// Host-side launch interface of the HIP kernels (internal to libdit).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "common.h"

namespace dit {

// Launch sites, numbered as the DIT_SITE_* constants of the public header.
enum KSite {
  KS_ATTENTION = 0, KS_GEMM_QKV, KS_GEMM_RESID, KS_GEMM_GELU, KS_GEMM_LIN1, KS_GEMM_F32,
  KS_GEMM_SILU, KS_LN, KS_FBC, KS_OTHER
};
// Bracket a launch with the calling thread's installed event timer (no-op if none).
void ktimer_start(int site, hipStream_t st);
void ktimer_stop(int site, hipStream_t st);
struct KTimerScope {
  int site; hipStream_t st;
  KTimerScope(int s, hipStream_t t) : site(s), st(t) { ktimer_start(site, st); }
  ~KTimerScope() { ktimer_stop(site, st); }
};

// One GEMM problem: C[M, N] = A[M, K] W[N, K]^T + bias.  bf16 operands, K % 64 == 0,
// lda / ldw multiples of 8 elements, 16-byte aligned base pointers.
struct GemmProblem {
  const bf16_t* A; int lda;
  const bf16_t* W; int ldw;
  const float* bias;
  int M, N, K;
};

// Destinations of the fused QKV epilogue.
struct QKVOut {
  bf16_t* q;          // [B, H, L, d]
  bf16_t* k;          // [B, H, L, d]
  uint16_t* vt;       // [B, H, d, L] fp16
  const float* rope;  // [L, d/2, 2] (cos, sin)
  int D, H, d;
};

hipError_t gemm_store_f32(const GemmProblem& g, float* out, int ldo, hipStream_t st);
hipError_t gemm_store_bf16(const GemmProblem& g, bf16_t* out, int ldo, hipStream_t st);
hipError_t gemm_silu_bf16(const GemmProblem& g, bf16_t* out, int ldo, hipStream_t st);
hipError_t gemm_gelu_bf16(const GemmProblem* g, int ng, bf16_t* const* out, const int* ldo,
                          hipStream_t st);
template <class XT>
hipError_t gemm_gated_residual(const GemmProblem* g, int ng, XT* x, int D,
                               const float* const* gate, int gate_bstride, const RowMap* map,
                               hipStream_t st);
hipError_t gemm_qkv(const GemmProblem* g, int ng, const QKVOut& o, const RowMap* map,
                    hipStream_t st);
hipError_t gemm_linear1(const GemmProblem& g, const QKVOut& o, const RowMap& map,
                        bf16_t* cat, int ldcat, hipStream_t st);

// Flash attention: q, k bf16 [B, H, L, d], vt fp16 [B, H, d, L]; output (bf16) of
// token (b, t), head h goes to o[map.stream_row(b, t) * ldo + h * d + c].
hipError_t attention_bf16(const bf16_t* q, const bf16_t* k, const uint16_t* vt, bf16_t* o,
                          int ldo, const RowMap& map, int B, int H, int L, int d,
                          float softmax_scale, hipStream_t st);

// LayerNorm (eps 1e-6, no affine) + modulate: out[r] = LN(x[map(r)]) * (1 + scale) + shift.
// Rows r < n_img take the image vectors, the rest the text vectors; per batch b
// the vectors sit at mod + b * mod_bstride.
template <class XT>
hipError_t ln_modulate(const XT* x, bf16_t* out, int rows, int D, const RowMap& map,
                       int n_img_rows, const float* shift_img, const float* scale_img,
                       const float* shift_txt, const float* scale_txt, int mod_bstride,
                       hipStream_t st);

}  // namespace dit
