// Host-side launch interface of the HIP kernels (internal to libdit).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "common.h"

namespace dit {

// Launch sites, numbered as the DIT_SITE_* constants of the public header.
enum KSite {
  KS_ATTENTION = 0, KS_GEMM_QKV, KS_GEMM_RESID, KS_GEMM_GELU, KS_GEMM_LIN1, KS_GEMM_F32,
  KS_GEMM_SILU, KS_LN, KS_FBC, KS_OTHER, KS_QUANT
};
// Bracket a launch with the calling thread's installed event timer (no-op if none).
void ktimer_start(int site, hipStream_t st);
void ktimer_stop(int site, hipStream_t st);
struct KTimerScope {
  int site; hipStream_t st;
  KTimerScope(int s, hipStream_t t) : site(s), st(t) { ktimer_start(site, st); }
  ~KTimerScope() { ktimer_stop(site, st); }
};

// Gate of the launches made while a GateScope is alive on the calling thread: a
// device int that each gated kernel reads on entry, returning at once unless it
// holds 0 (a graph-replayed loop keeps the First-Block-Cache decision there).
// nullptr, the default: kernels run unconditionally.
const int* launch_gate();
struct GateScope {
  const int* prev;
  explicit GateScope(const int* g);
  ~GateScope();
};

// One GEMM problem: C[M, N] = A[M, K] W[N, K]^T + bias.
//   bf16: A, W; K % 64 == 0.
//   fp8 (e4m3): A8, W8 with per-row scales sa[M] and per-output-channel scales
//   sw[N], C = (A8 W8^T) * sa[m] * sw[n] + bias; K % 128 == 0.
// lda / ldw in elements, rows 16-byte aligned.
struct GemmProblem {
  const bf16_t* A; int lda;
  const bf16_t* W; int ldw;
  const float* bias;
  int M, N, K;
  const fp8_t* A8 = nullptr;
  const fp8_t* W8 = nullptr;
  const float* sa = nullptr;
  const float* sw = nullptr;
  // fp32 (reference-precision blocks): A32 [M, K], W32 [N, K]; K % 4 == 0
  const float* A32 = nullptr;
  const float* W32 = nullptr;
  // MXFP4 (W4A4): E2M1 codes A4 [M, lda / 2 bytes], W4 [N, ldw / 2 bytes] (lda, ldw in
  // elements) and E8M0 block scales xa [K / 256][pad_m][8], xw [K / 256][pad_n][8]
  // (pad_m, pad_n multiples of 256; a row's 8 scales of a 256-wide K slab are
  // stored as blocks 0, 2, 4, 6, 1, 3, 5, 7); K % 256 == 0
  const uint8_t* A4 = nullptr;
  const uint8_t* W4 = nullptr;
  const uint8_t* xa = nullptr;
  const uint8_t* xw = nullptr;
  int pad_m = 0, pad_n = 0;
};

// Destinations of the fused QKV epilogue.
struct QKVOut {
  bf16_t* q;          // [B, H, L, d] (rotated)
  bf16_t* k;          // [B, H, L, d] (rotated)
  bf16_t* v;          // [B, H, L, d]
  const float* rope;  // [L, d/2, 2] (cos, sin)
  int D, H, d;
  // optional [3, B, H]: largest stored |q|, |k|, |v| per (b, h) as fp32 bits,
  // accumulated with atomic max (zero it before the GEMM); direct-to-LDS kernel only
  unsigned int* amax = nullptr;
};

hipError_t gemm_store_f32(const GemmProblem& g, float* out, int ldo, hipStream_t st);
hipError_t gemm_store_bf16(const GemmProblem& g, bf16_t* out, int ldo, hipStream_t st);
// MXFP4 (W4A4) GEMM, out = A W^T + bias, A4 / W4 / xa / xw set in g.
hipError_t gemm_mx4_store_f32(const GemmProblem& g, float* out, int ldo, hipStream_t st);
hipError_t gemm_mx4_store_bf16(const GemmProblem& g, bf16_t* out, int ldo, hipStream_t st);
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

// fp32 GEMMs (VALU, 64 x 64 tiles) with the same fused epilogues writing fp32:
// Q, K, V [B, H, L, d], GELU hidden, gated residual, plain stores.
struct QKVOut32 {
  float* q; float* k; float* v; const float* rope; int D, H, d;
};
hipError_t gemm32_store(const GemmProblem& g, float* out, int ldo, hipStream_t st);
hipError_t gemm32_silu(const GemmProblem& g, float* out, int ldo, hipStream_t st);
hipError_t gemm32_gelu(const GemmProblem* g, int ng, float* const* out, const int* ldo,
                       hipStream_t st);
hipError_t gemm32_gated_residual(const GemmProblem* g, int ng, float* x, int D,
                                 const float* const* gate, int gate_bstride, const RowMap* map,
                                 hipStream_t st);
hipError_t gemm32_qkv(const GemmProblem* g, int ng, const QKVOut32& o, const RowMap* map,
                      hipStream_t st);
hipError_t gemm32_linear1(const GemmProblem& g, const QKVOut32& o, const RowMap& map, float* cat,
                          int ldcat, hipStream_t st);

// fp32 attention, head dim 32 or 64: q, k, v [B, H, L, d], o fp32.
hipError_t attention_f32(const float* q, const float* k, const float* v, float* o, int ldo,
                         const RowMap& map, int B, int H, int L, int d, float softmax_scale,
                         hipStream_t st);

// Flash attention: q, k, v bf16 [B, H, L, d], d 64 or 128, any L >= 1; output
// (bf16) of token (b, t), head h goes to o[map.stream_row(b, t) * ldo + h * d + c].
hipError_t attention_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* v, bf16_t* o,
                          int ldo, const RowMap& map, int B, int H, int L, int d,
                          float softmax_scale, hipStream_t st);

// LayerNorm (eps 1e-6, no affine) + modulate: out[r] = LN(x[map(r)]) * (1 + scale) + shift
// (OT = bf16_t or float).
// Rows r < n_img take the image vectors, the rest the text vectors; per batch b
// the vectors sit at mod + b * mod_bstride.
template <class XT, class OT>
hipError_t ln_modulate(const XT* x, OT* out, int rows, int D, const RowMap& map,
                       int n_img_rows, const float* shift_img, const float* scale_img,
                       const float* shift_txt, const float* scale_txt, int mod_bstride,
                       hipStream_t st);

// LayerNorm + modulate emitting e4m3 with a per-row scale (out8 [rows, D], scale [rows]).
hipError_t ln_modulate_fp8(const float* x, fp8_t* out8, float* scale, int rows, int D,
                           const RowMap& map, int n_img_rows, const float* shift_img,
                           const float* scale_img, const float* shift_txt, const float* scale_txt,
                           int mod_bstride, hipStream_t st);
// LN + modulate straight to MXFP4 (codes [rows, D/2], scales [D/256][pad_rows][8])
// of the bf16-rounded output: the same codes and scales as ln_modulate to bf16
// followed by quant_mxfp4.
hipError_t ln_modulate_mx4(const float* x, uint8_t* codes, uint8_t* scales, int pad_rows, int rows,
                           int D, const RowMap& map, int n_img_rows, const float* shift_img,
                           const float* scale_img, const float* shift_txt, const float* scale_txt,
                           int mod_bstride, hipStream_t st);

// Per-row dynamic quantisation: dst[r, :width] = e4m3(src[r, :width] * 448 / amax_r),
// scale[r] = amax_r / 448.  T = bf16_t or f16_t.
template <class T>
hipError_t quant_rows(const T* src, int lds, fp8_t* dst, int ldd, float* scale, int rows, int width,
                      hipStream_t st);
// One scale per contiguous slice of n elements (nslices slices), from each slice's
// largest magnitude given as fp32 bits in amax[nslices] (the QKV epilogues gather it).
template <class T>
hipError_t quant_slices(const T* src, size_t n, int nslices, const unsigned int* amax,
                        fp8_t* dst, float* scale, hipStream_t st);
hipError_t zero_u32(unsigned int* p, int n, hipStream_t st);
// MXFP4 quantisation of rows (see GemmProblem for the code and scale layouts);
// width % 256 == 0, pad_rows = rows rounded up to 256 (pad rows get scale 2^0).
template <class T>
hipError_t quant_mxfp4(const T* src, int lds, int rows, int width, uint8_t* codes, uint8_t* scales,
                       int pad_rows, hipStream_t st);

// fp8 attention: q8, k8, v8 e4m3 [B, H, L, d], one fp32 scale per (b, h) for each
// of q, k, v; output bf16 as attention_bf16.
hipError_t attention_fp8(const fp8_t* q8, const fp8_t* k8, const fp8_t* v8, const float* sq,
                         const float* sk, const float* sv, bf16_t* o, int ldo, const RowMap& map,
                         int B, int H, int L, int d, float softmax_scale, hipStream_t st);

}  // namespace dit
