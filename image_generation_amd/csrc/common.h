// Device-side helpers shared by the HIP kernels of the DiT denoise step (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef uint16_t bf16_t;   // bfloat16 storage
typedef uint8_t fp8_t;     // OCP e4m3 storage
typedef _Float16 f16_t;    // fp16 storage

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;   // 16-byte load/store unit

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
__device__ __forceinline__ float bf2f(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (the gfx950 convert instruction).
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}

template <class OT> __device__ __forceinline__ OT from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f2bf(v); }

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// Round-to-nearest-even fp32 -> fp16 bits.
__device__ __forceinline__ uint16_t f2h(float f) {
  f16_t h = (f16_t)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
}

// Two floats -> two packed bf16 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// x * sigmoid(x)
__device__ __forceinline__ float silu_f(float x) {
  return x * fast_rcp(1.0f + fast_exp2(-x * 1.4426950408889634f));
}

// tanh-approximated GELU written as x * sigmoid(2u), u = sqrt(2/pi)(x + 0.044715 x^3):
// 0.5 x (1 + tanh u) = x / (1 + e^{-2u}).
__device__ __forceinline__ float gelu_tanh_f(float x) {
  const float k0 = 0.7978845608028654f;   // sqrt(2/pi)
  const float k1 = 0.044715f;
  float u = k0 * (x + k1 * x * x * x);
  return x * fast_rcp(1.0f + fast_exp2(-2.0f * 1.4426950408889634f * u));
}

// A set launch gate holding a non-zero value: the kernel returns before any work.
// Every thread reads the same word, so the exit is uniform.
__device__ __forceinline__ bool gate_closed(const int* gate) {
  return gate != nullptr && *gate != 0;
}

// ---- MXFP4 (OCP E2M1 elements, E8M0 scale per 32 consecutive K values)
// E2M1 code of x / 2^e (exact in fp32), rounded to nearest by counting the
// midpoints it passes, ties to the even mantissa (0.25 -> 0, 0.75 -> 1,
// 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4), beyond 6 saturating.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | (__float_as_uint(v) >> 31 << 3);
}
// Block exponent: floor(log2 amax) - 2, clamped to the E8M0 range; 0 for amax 0.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int k;
  frexpf(amax, &k);                    // amax = m 2^k, m in [0.5, 1)
  return min(max(k - 3, -127), 127);
}
// Byte of block j (0..7 within a 256-wide slab) in a row's 8 stored scales: the
// GEMM reads them in the order 0, 2, 4, 6, 1, 3, 5, 7.
__device__ __forceinline__ int mx_scale_pos(int j) { return (j & 1) ? 4 + (j >> 1) : j >> 1; }

template <typename T> struct XIO;
template <> struct XIO<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct XIO<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
};

// Row map of the "stream-major" row space used inside a double-stream block:
// rows [0, B*Li) are image tokens (batch-major), rows [B*Li, B*(Li+Lt)) are text
// tokens; a single-stream block uses the joint order directly (stream_major = 0).
struct RowMap {
  int B, Lt, Li, L;
  int stream_major;  // 1: image rows first then text rows; 0: joint [b][t] order
  int base;          // added to a row index before mapping (row offset of a GEMM group)
  __device__ __forceinline__ void token(int r, int& b, int& t) const {
    r += base;
    if (!stream_major) { b = r / L; t = r - b * L; return; }
    const int ni = B * Li;
    if (r < ni) { b = r / Li; t = Lt + (r - b * Li); }
    else { const int q = r - ni; b = q / Lt; t = q - b * Lt; }
  }
  // Joint-buffer row (b * L + t) of row r.
  __device__ __forceinline__ int joint_row(int r) const {
    int b, t; token(r, b, t); return b * L + t;
  }
  // Inverse (ignores base): row of token (b, t) in this map's row space.
  __device__ __forceinline__ int stream_row(int b, int t) const {
    if (!stream_major) return b * L + t;
    if (t >= Lt) return b * Li + (t - Lt);
    return B * Li + b * Lt + t;
  }
};

}  // namespace dit
