// Dynamic fp8 (OCP e4m3) quantisation kernels for the W8A8 path (gfx950).
//
// Rows: per-row scale = amax / 448 (amax 0 -> 1); codes = RNE-saturating e4m3 of
// x * (448 / amax), both factors one correctly rounded fp32 division.  The
// gfx950 convert (v_cvt_pk_fp8_f32) rounds to nearest even and saturates.
// Heads: one scale per contiguous slice (a (batch, head) of Q, K or V^T).
#include "common.h"
#include "kernels.h"
#include "ops.h"

namespace dit {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// 8 consecutive source elements -> f32
template <class T> struct Load8;
template <> struct Load8<bf16_t> {
  static __device__ __forceinline__ void get(const bf16_t* p, float* v) {
    const uint4 u = *(const uint4*)p;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Load8<float> {
  static __device__ __forceinline__ void get(const float* p, float* v) {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
};
template <> struct Load8<f16_t> {
  static __device__ __forceinline__ void get(const f16_t* p, float* v) {
    const f16x8 h = *(const f16x8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
  }
};

// 16 raw bytes (8 elements) -> f32
template <class T>
__device__ __forceinline__ void decode8(const i32x4 u, float* v);
template <>
__device__ __forceinline__ void decode8<bf16_t>(const i32x4 u, float* v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float((uint32_t)u[i] << 16);
    v[2 * i + 1] = __uint_as_float((uint32_t)u[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void decode8<f16_t>(const i32x4 u, float* v) {
  const f16x8 h = __builtin_bit_cast(f16x8, u);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
}

__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ void store_fp8x8(fp8_t* p, const float* v, float inv) {
  uint2 u;
  u.x = pack_fp8x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  u.y = pack_fp8x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  *(uint2*)p = u;
}

__device__ __forceinline__ void scale_of(float amax, float& scale, float& inv) {
  if (amax > 0.f) {
    scale = amax / 448.0f;
    inv = 448.0f / amax;
  } else {
    scale = 1.f;
    inv = 1.f;
  }
}

// One wave per row; the row is read twice (amax, then quantise).
template <class T>
__global__ __launch_bounds__(256) void quant_rows_kernel(const T* __restrict__ src, int lds,
                                                         fp8_t* __restrict__ dst, int ldd,
                                                         float* __restrict__ scale, int rows,
                                                         int width, const int* __restrict__ gate) {
  if (gate_closed(gate)) return;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const T* s = src + (size_t)r * lds;
  float amax = 0.f;
  for (int c = lane * 8; c < width; c += 512) {
    float v[8];
    Load8<T>::get(s + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  float sc, inv;
  scale_of(amax, sc, inv);
  fp8_t* d = dst + (size_t)r * ldd;
  for (int c = lane * 8; c < width; c += 512) {
    float v[8];
    Load8<T>::get(s + c, v);
    store_fp8x8(d + c, v, inv);
  }
  if (lane == 0) scale[r] = sc;
}

// One wave per row with the row held in registers (NCH x 512 elements at most):
// one read of the source instead of two.
template <class T, int NCH>
__global__ __launch_bounds__(256) void quant_rows_reg_kernel(const T* __restrict__ src, int lds,
                                                             fp8_t* __restrict__ dst, int ldd,
                                                             float* __restrict__ scale, int rows,
                                                             int width,
                                                             const int* __restrict__ gate) {
  if (gate_closed(gate)) return;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const T* s = src + (size_t)r * lds;
  i32x4 raw[NCH];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = i * 512 + lane * 8;
    if (c < width) {
      raw[i] = *(const i32x4*)(s + c);
      float v[8];
      decode8<T>(raw[i], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
  }
  amax = wave_max(amax);
  float sc, inv;
  scale_of(amax, sc, inv);
  fp8_t* d = dst + (size_t)r * ldd;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = i * 512 + lane * 8;
    if (c < width) {
      float v[8];
      decode8<T>(raw[i], v);
      store_fp8x8(d + c, v, inv);
    }
  }
  if (lane == 0) scale[r] = sc;
}

// One workgroup (4 waves) per row, the row split over the waves and held in
// registers (4 x NCH x 512 elements at most; NCH chunks of 512 per wave): the
// row's amax combines the waves' maxima through LDS, then each wave quantises its
// part.  Splitting a row keeps the registers per wave low, so more rows are in
// flight than with one wave per row.
template <class T, int NCH>
__global__ __launch_bounds__(256) void quant_rows_split_kernel(const T* __restrict__ src, int lds,
                                                               fp8_t* __restrict__ dst, int ldd,
                                                               float* __restrict__ scale,
                                                               int rows, int width,
                                                               const int* __restrict__ gate) {
  if (gate_closed(gate)) return;
  __shared__ float wmax[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = blockIdx.x;
  const T* s = src + (size_t)r * lds;
  i32x4 raw[NCH];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (wave * NCH + i) * 512 + lane * 8;
    if (c < width) {
      raw[i] = *(const i32x4*)(s + c);
      float v[8];
      decode8<T>(raw[i], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
  }
  amax = wave_max(amax);
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  float sc, inv;
  scale_of(amax, sc, inv);
  fp8_t* d = dst + (size_t)r * ldd;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (wave * NCH + i) * 512 + lane * 8;
    if (c < width) {
      float v[8];
      decode8<T>(raw[i], v);
      store_fp8x8(d + c, v, inv);
    }
  }
  if (threadIdx.x == 0) scale[r] = sc;
}

// e4m3 codes of one contiguous slice per blockIdx.y, scaled by that slice's given
// amax (fp32 bits; a non-negative float's bits order like its value).
template <class T>
__global__ __launch_bounds__(256) void quant_slices_kernel(const T* __restrict__ src, size_t n,
                                                           const unsigned int* __restrict__ amax,
                                                           fp8_t* __restrict__ dst,
                                                           float* __restrict__ scale,
                                                           const int* __restrict__ gate) {
  if (gate_closed(gate)) return;
  float sc, inv;
  scale_of(__uint_as_float(amax[blockIdx.y]), sc, inv);
  const T* s = src + (size_t)blockIdx.y * n;
  fp8_t* d = dst + (size_t)blockIdx.y * n;
  for (size_t c = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8; c < n; c += (size_t)gridDim.x * 2048) {
    float v[8];
    Load8<T>::get(s + c, v);
    store_fp8x8(d + c, v, inv);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[blockIdx.y] = sc;
}

__global__ void zero_u32_kernel(unsigned int* p, int n, const int* __restrict__ gate) {
  if (gate_closed(gate)) return;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <class T>
hipError_t quant_rows(const T* src, int lds, fp8_t* dst, int ldd, float* scale, int rows, int width,
                      hipStream_t st) {
  if (width % 8 || lds % 8 || ldd % 8) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  KTimerScope timer(KS_QUANT, st);
  const dim3 grid((rows + 3) / 4);
  if (width <= 8 * 512)
    hipLaunchKernelGGL((quant_rows_reg_kernel<T, 8>), grid, dim3(256), 0, st, src, lds, dst, ldd,
                       scale, rows, width, launch_gate());
  else if (width <= 4 * 8 * 512)
    hipLaunchKernelGGL((quant_rows_split_kernel<T, 8>), dim3(rows), dim3(256), 0, st, src, lds,
                       dst, ldd, scale, rows, width, launch_gate());
  else
    hipLaunchKernelGGL(quant_rows_kernel<T>, grid, dim3(256), 0, st, src, lds, dst, ldd, scale,
                       rows, width, launch_gate());
  return hipGetLastError();
}
template hipError_t quant_rows<bf16_t>(const bf16_t*, int, fp8_t*, int, float*, int, int, hipStream_t);
template hipError_t quant_rows<f16_t>(const f16_t*, int, fp8_t*, int, float*, int, int, hipStream_t);

template <class T>
hipError_t quant_slices(const T* src, size_t n, int nslices, const unsigned int* amax,
                        fp8_t* dst, float* scale, hipStream_t st) {
  if (n % 8) return hipErrorInvalidValue;
  if (nslices == 0 || n == 0) return hipSuccess;
  KTimerScope timer(KS_QUANT, st);
  size_t blocks = (n / 8 + 255) / 256;
  const int bx = (int)(blocks < 64 ? blocks : 64);
  hipLaunchKernelGGL(quant_slices_kernel<T>, dim3(bx, nslices), dim3(256), 0, st, src, n, amax,
                     dst, scale, launch_gate());
  return hipGetLastError();
}
template hipError_t quant_slices<bf16_t>(const bf16_t*, size_t, int, const unsigned int*, fp8_t*,
                                         float*, hipStream_t);
template hipError_t quant_slices<f16_t>(const f16_t*, size_t, int, const unsigned int*, fp8_t*,
                                        float*, hipStream_t);

// ---------------------------------------------------------------- MXFP4
// One lane per block of 32 consecutive elements of a row: e = floor(log2 amax) - 2
// (clamped to the E8M0 range; 0 for an all-zero block), each element x / 2^e
// (exact in fp32) rounded to E2M1 by counting the midpoints it passes, ties going
// to the even mantissa (0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2,
// 3.5 -> 4, 5 -> 4) and values beyond 6 saturating.  16 code bytes per block,
// element 2j in the low nibble of byte j; the scale byte goes to the GEMM order
// [slab][pad_rows][8] with a row's 8 slab blocks stored as 0, 2, 4, 6, 1, 3, 5, 7.
// (e2m1_code, mx_exponent and mx_scale_pos live in common.h: the fused LN pass
// uses them too.)

template <class T>
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const T* __restrict__ src, int lds,
                                                          int rows, int width, int pad_rows,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          const int* __restrict__ gate) {
  if (gate_closed(gate)) return;
  const int nb = width >> 5;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)pad_rows * nb) return;
  const int r = (int)(idx / nb), b = (int)(idx - (long long)r * nb);
  uint8_t* sp = scales + (((size_t)(b >> 3) * pad_rows + r) << 3) + mx_scale_pos(b & 7);
  if (r >= rows) {   // padding rows of the scale array
    *sp = 127;
    return;
  }
  float v[32];
  const T* p = src + (size_t)r * lds + (b << 5);
#pragma unroll
  for (int q = 0; q < 4; ++q) Load8<T>::get(p + q * 8, v + q * 8);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_exponent(amax);
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t u = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) u |= e2m1_code(ldexpf(v[q * 8 + i], -e)) << (4 * i);
    w[q] = u;
  }
  *(uint4*)(codes + (size_t)r * (width >> 1) + (b << 4)) = make_uint4(w[0], w[1], w[2], w[3]);
  *sp = (uint8_t)(e + 127);
}

template <class T>
hipError_t quant_mxfp4(const T* src, int lds, int rows, int width, uint8_t* codes, uint8_t* scales,
                       int pad_rows, hipStream_t st) {
  if (width % 256 || lds % 8 || pad_rows < rows || pad_rows % 256) return hipErrorInvalidValue;
  if (pad_rows == 0) return hipSuccess;
  KTimerScope timer(KS_QUANT, st);
  const long long n = (long long)pad_rows * (width >> 5);
  hipLaunchKernelGGL(quant_mxfp4_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     src, lds, rows, width, pad_rows, codes, scales, launch_gate());
  return hipGetLastError();
}
template hipError_t quant_mxfp4<bf16_t>(const bf16_t*, int, int, int, uint8_t*, uint8_t*, int,
                                        hipStream_t);
template hipError_t quant_mxfp4<float>(const float*, int, int, int, uint8_t*, uint8_t*, int,
                                       hipStream_t);

hipError_t zero_u32(unsigned int* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, launch_gate());
  return hipGetLastError();
}

}  // namespace dit
