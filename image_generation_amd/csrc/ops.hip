// Bandwidth-bound kernels of the DiT denoise step (gfx950): adaLN LayerNorm-modulate,
// embeddings, the First-Block-Cache relative-L1 reduction, cache commit/apply and
// the Euler / CFG update.
#include "common.h"
#include "kernels.h"
#include "ops.h"

namespace dit {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------- LN + modulate
// One wave per output row; the row (D <= 64 * 4 * LN_MAXCH) stays in registers
// between the mean pass, the variance pass and the output pass.
constexpr int LN_MAXCH = 12;

template <class XT>
__device__ __forceinline__ f32x4 load4(const XT* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) { return *(const f32x4*)p; }
template <>
__device__ __forceinline__ f32x4 load4<bf16_t>(const bf16_t* p) {
  uint2 u = *(const uint2*)p;
  f32x4 v;
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xffff0000u);
  return v;
}

// OUT: 0 = bf16, 1 = e4m3 + per-row scale, 2 = fp32, 3 = MXFP4 codes [rows, D/2] +
// E8M0 block scales mxs [D/256][pad_rows][8] of the bf16-rounded output (the
// values the separate quantiser would see; rows in [rows, pad_rows) get scale 2^0)
template <class XT, int OUT>
__global__ __launch_bounds__(256) void ln_modulate_kernel(
    const XT* __restrict__ x, void* __restrict__ out_, float* __restrict__ oscale, int rows, int D,
    RowMap map, int n_img,
    const float* __restrict__ sh_i, const float* __restrict__ sc_i,
    const float* __restrict__ sh_t, const float* __restrict__ sc_t, int bstride,
    const int* __restrict__ gate, uint8_t* __restrict__ mxs, int pad_rows) {
  if (gate_closed(gate)) return;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) {
    if constexpr (OUT == 3) {
      if (r < pad_rows && lane < 8)
        for (int c = 0; c < (D >> 8); ++c) mxs[((size_t)c * pad_rows + r) * 8 + lane] = 127;
    }
    return;
  }
  int b, t;
  map.token(r, b, t);
  const XT* xr = x + ((size_t)b * map.L + t) * D;
  const int nch = D >> 8;
  f32x4 v[LN_MAXCH];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < LN_MAXCH; ++c) {
    if (c < nch) {
      v[c] = load4<XT>(xr + c * 256 + lane * 4);
      s += (v[c][0] + v[c][1]) + (v[c][2] + v[c][3]);
    }
  }
  const float inv_d = 1.0f / (float)D;
  const float mean = wave_sum(s) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < LN_MAXCH; ++c) {
    if (c < nch) {
      v[c] -= mean;
      q += (v[c][0] * v[c][0] + v[c][1] * v[c][1]) + (v[c][2] * v[c][2] + v[c][3] * v[c][3]);
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) * inv_d + 1e-6f);
  const bool img = r < n_img;
  const float* sh = (img ? sh_i : sh_t) + (size_t)b * bstride;
  const float* sc = (img ? sc_i : sc_t) + (size_t)b * bstride;
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < LN_MAXCH; ++c) {
    if (c < nch) {
      const int col = c * 256 + lane * 4;
      const f32x4 a = *(const f32x4*)(sc + col);
      const f32x4 z = *(const f32x4*)(sh + col);
      v[c] = v[c] * rstd * (1.0f + a) + z;
      if constexpr (OUT == 1)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[c][0]), fabsf(v[c][1])),
                                 fmaxf(fabsf(v[c][2]), fabsf(v[c][3]))));
    }
  }
  if constexpr (OUT == 3) {
    uint8_t* crow = (uint8_t*)out_ + (size_t)r * (D >> 1);
#pragma unroll
    for (int c = 0; c < LN_MAXCH; ++c) {
      if (c < nch) {
        // a 32-value block is 8 consecutive lanes' 4 values
        f32x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = bf2f(f2bf(v[c][i]));
        float m = fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3])));
        m = fmaxf(m, __shfl_xor(m, 1));
        m = fmaxf(m, __shfl_xor(m, 2));
        m = fmaxf(m, __shfl_xor(m, 4));
        const int e = mx_exponent(m);
        uint32_t u = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) u |= e2m1_code(ldexpf(h[i], -e)) << (4 * i);
        *(uint16_t*)(crow + c * 128 + lane * 2) = (uint16_t)u;
        if ((lane & 7) == 0)
          mxs[((size_t)c * pad_rows + r) * 8 + mx_scale_pos(lane >> 3)] = (uint8_t)(e + 127);
      }
    }
  } else if constexpr (OUT == 2) {
    float* orow = (float*)out_ + (size_t)r * D;
#pragma unroll
    for (int c = 0; c < LN_MAXCH; ++c)
      if (c < nch) *(f32x4*)(orow + c * 256 + lane * 4) = v[c];
  } else if constexpr (OUT == 0) {
    bf16_t* orow = (bf16_t*)out_ + (size_t)r * D;
#pragma unroll
    for (int c = 0; c < LN_MAXCH; ++c) {
      if (c < nch) {
        uint2 u;
        u.x = pack_bf16x2(v[c][0], v[c][1]);
        u.y = pack_bf16x2(v[c][2], v[c][3]);
        *(uint2*)(orow + c * 256 + lane * 4) = u;
      }
    }
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    float scl = 1.f, inv = 1.f;
    if (amax > 0.f) {
      scl = amax / 448.0f;
      inv = 448.0f / amax;
    }
    fp8_t* orow = (fp8_t*)out_ + (size_t)r * D;
#pragma unroll
    for (int c = 0; c < LN_MAXCH; ++c) {
      if (c < nch) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[c][0] * inv, v[c][1] * inv, 0, false);
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[c][2] * inv, v[c][3] * inv, lo, true);
        *(int*)(orow + c * 256 + lane * 4) = w;
      }
    }
    if (lane == 0) oscale[r] = scl;
  }
}

template <class XT, class OT>
hipError_t ln_modulate(const XT* x, OT* out, int rows, int D, const RowMap& map,
                       int n_img_rows, const float* shift_img, const float* scale_img,
                       const float* shift_txt, const float* scale_txt, int mod_bstride,
                       hipStream_t st) {
  if (D % 256 != 0 || D > 256 * LN_MAXCH) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  KTimerScope timer(KS_LN, st);
  constexpr int mode = sizeof(OT) == 4 ? 2 : 0;
  hipLaunchKernelGGL((ln_modulate_kernel<XT, mode>), dim3((rows + 3) / 4), dim3(256), 0, st, x,
                     (void*)out, nullptr, rows, D, map, n_img_rows, shift_img, scale_img,
                     shift_txt, scale_txt, mod_bstride, launch_gate(), (uint8_t*)nullptr, 0);
  return hipGetLastError();
}
template hipError_t ln_modulate<float, bf16_t>(const float*, bf16_t*, int, int, const RowMap&, int,
                                               const float*, const float*, const float*,
                                               const float*, int, hipStream_t);
template hipError_t ln_modulate<float, float>(const float*, float*, int, int, const RowMap&, int,
                                              const float*, const float*, const float*,
                                              const float*, int, hipStream_t);

hipError_t ln_modulate_fp8(const float* x, fp8_t* out8, float* scale, int rows, int D,
                           const RowMap& map, int n_img_rows, const float* shift_img,
                           const float* scale_img, const float* shift_txt, const float* scale_txt,
                           int mod_bstride, hipStream_t st) {
  if (D % 256 != 0 || D > 256 * LN_MAXCH) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  KTimerScope timer(KS_LN, st);
  hipLaunchKernelGGL((ln_modulate_kernel<float, 1>), dim3((rows + 3) / 4), dim3(256), 0, st, x,
                     (void*)out8, scale, rows, D, map, n_img_rows, shift_img, scale_img,
                     shift_txt, scale_txt, mod_bstride, launch_gate(), (uint8_t*)nullptr, 0);
  return hipGetLastError();
}

hipError_t ln_modulate_mx4(const float* x, uint8_t* codes, uint8_t* scales, int pad_rows, int rows,
                           int D, const RowMap& map, int n_img_rows, const float* shift_img,
                           const float* scale_img, const float* shift_txt, const float* scale_txt,
                           int mod_bstride, hipStream_t st) {
  if (D % 256 != 0 || D > 256 * LN_MAXCH || pad_rows < rows || pad_rows % 256)
    return hipErrorInvalidValue;
  if (pad_rows == 0) return hipSuccess;
  KTimerScope timer(KS_LN, st);
  hipLaunchKernelGGL((ln_modulate_kernel<float, 3>), dim3((pad_rows + 3) / 4), dim3(256), 0, st, x,
                     (void*)codes, nullptr, rows, D, map, n_img_rows, shift_img, scale_img,
                     shift_txt, scale_txt, mod_bstride, launch_gate(), scales, pad_rows);
  return hipGetLastError();
}

// ---------------------------------------------------------------- embeddings

// Image tokens: x[b, Lt + i, :] = before[b, i, :] = lat[i] W_in^T + b_in for every
// batch row b (a CFG pair shares its latents).  16 tokens x 256 columns per block.
template <class WT>
__global__ __launch_bounds__(256) void embed_latents_kernel(
    const float* __restrict__ lat, const WT* __restrict__ W, const float* __restrict__ bias,
    float* __restrict__ x, float* __restrict__ before, int B, int Lt, int Li, int L, int D,
    int Cin) {
  __shared__ float sl[16][64];
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * 16;
  const int n = blockIdx.y * 256 + tid;
  for (int e = tid; e < 16 * Cin; e += 256) {
    const int i = e / Cin, k = e - i * Cin;
    sl[i][k] = (i0 + i < Li) ? lat[(size_t)(i0 + i) * Cin + k] : 0.f;
  }
  __syncthreads();
  if (n >= D) return;
  float w[64];
#pragma unroll
  for (int k = 0; k < 64; ++k) w[k] = k < Cin ? to_f32(W[(size_t)n * Cin + k]) : 0.f;
  const float bn = bias[n];
  for (int i = 0; i < 16 && i0 + i < Li; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 64; ++k) acc = fmaf(sl[i][k], w[k], acc);
    acc += bn;
    for (int b = 0; b < B; ++b) {
      x[((size_t)b * L + Lt + i0 + i) * D + n] = acc;
      before[((size_t)b * Li + i0 + i) * D + n] = acc;
    }
  }
}

// Text tokens: x[b, t, :] = txt[b, t, :] (bf16 or fp32 -> fp32 residual stream).
template <class TT>
__global__ __launch_bounds__(256) void text_to_stream_kernel(
    const TT* __restrict__ txt, float* __restrict__ x, int B, int Lt, int L, int D) {
  const size_t n4 = (size_t)B * Lt * D / 4;
  for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n4; j += (size_t)gridDim.x * 256) {
    const size_t e = j * 4;
    const size_t row = e / D;
    const int c = (int)(e - row * D);
    const int b = (int)(row / Lt), t = (int)(row - (size_t)b * Lt);
    *(f32x4*)(x + ((size_t)b * L + t) * D + c) = load4<TT>(txt + e);
  }
}

// Sinusoidal timestep embedding of t = sigma_m, in fp64: [cos(1000 t w_k), sin(1000 t w_k)],
// w_k = 10000^(-k/half); out [M, 2*half] (bf16 or fp32).  Sigmas travel in the
// kernel arguments, up to SIG_CHUNK per launch.
template <class OT>
__global__ void sinusoid_kernel(SigChunk sig, OT* __restrict__ e, int half) {
  const int m = blockIdx.x;
  for (int k = threadIdx.x; k < half; k += blockDim.x) {
    const double w = exp(-log(10000.0) * (double)k / (double)half);
    const double a = 1000.0 * sig.s[m] * w;
    e[(size_t)m * 2 * half + k] = from_f32<OT>((float)cos(a));
    e[(size_t)m * 2 * half + half + k] = from_f32<OT>((float)sin(a));
  }
}

// 2-D RoPE table [L, d/2, 2] (cos, sin), fp64 angles: pair p < d/4 turns with the
// patch row, p >= d/4 with the patch column, at 10000^(-j/(d/4)) per position.
__global__ void rope_table_kernel(float* __restrict__ tab, int grid_w, int Lt, int L, int d,
                                  double theta) {
  const int t = blockIdx.x;
  if (t >= L) return;
  const int q = d / 4;
  double row = 0.0, col = 0.0;
  if (t >= Lt) {
    row = (double)((t - Lt) / grid_w);
    col = (double)((t - Lt) % grid_w);
  }
  for (int p = threadIdx.x; p < d / 2; p += blockDim.x) {
    const int j = p % q;
    const double f = exp(-log(theta) * (double)j / (double)q);
    const double a = (p < q ? row : col) * f;
    tab[((size_t)t * (d / 2) + p) * 2 + 0] = (float)cos(a);
    tab[((size_t)t * (d / 2) + p) * 2 + 1] = (float)sin(a);
  }
}

// ---------------------------------------------------------------- First-Block-Cache

// Pass 1: r = x_img(after block 0) - x_img(before); staging = r; per-block sums of
// |r - anchor| and |anchor| in fp64 (fixed assignment of elements to blocks).
__global__ __launch_bounds__(256) void fbc_partial_kernel(
    const float* __restrict__ x, const float* __restrict__ before,
    const float* __restrict__ anchor, float* __restrict__ staging, double* __restrict__ part,
    int B, int Lt, int Li, int L, int D, int has_anchor) {
  const size_t n4 = (size_t)B * Li * D / 4;
  float num = 0.f, den = 0.f;
  double dnum = 0.0, dden = 0.0;
  int cnt = 0;
  for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n4; j += (size_t)gridDim.x * 256) {
    const size_t e = j * 4;
    const size_t row = e / D;
    const int c = (int)(e - row * D);
    const int b = (int)(row / Li), i = (int)(row - (size_t)b * Li);
    const f32x4 xa = *(const f32x4*)(x + ((size_t)b * L + Lt + i) * D + c);
    const f32x4 r = xa - *(const f32x4*)(before + e);
    *(f32x4*)(staging + e) = r;
    if (has_anchor) {
      const f32x4 a = *(const f32x4*)(anchor + e);
      num += (fabsf(r[0] - a[0]) + fabsf(r[1] - a[1])) + (fabsf(r[2] - a[2]) + fabsf(r[3] - a[3]));
      den += (fabsf(a[0]) + fabsf(a[1])) + (fabsf(a[2]) + fabsf(a[3]));
      if (++cnt == 16) {   // flush fp32 partials into fp64 every 64 elements
        dnum += num; dden += den; num = 0.f; den = 0.f; cnt = 0;
      }
    }
  }
  dnum += num;
  dden += den;
  __shared__ double sn[256], sd[256];
  sn[threadIdx.x] = dnum;
  sd[threadIdx.x] = dden;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      sn[threadIdx.x] += sn[threadIdx.x + o];
      sd[threadIdx.x] += sd[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = sn[0];
    part[2 * blockIdx.x + 1] = sd[0];
  }
}

// Pass 2 (one block): fixed-order fp64 sum of the partials; the result is valid
// in thread 0.  rel = num / den (+inf without an anchor or with a zero
// denominator, NaN for 0/0 of NaN sums); nonfinite flags a NaN / Inf in the sums.
__device__ void fbc_final_sums(const double* __restrict__ part, int nparts, int has_anchor,
                               double* rel_out, int* nonfinite_out) {
  __shared__ double sn[256], sd[256];
  double a = 0.0, c = 0.0;
  for (int i = threadIdx.x; i < nparts; i += 256) {
    a += part[2 * i];
    c += part[2 * i + 1];
  }
  sn[threadIdx.x] = a;
  sd[threadIdx.x] = c;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      sn[threadIdx.x] += sn[threadIdx.x + o];
      sd[threadIdx.x] += sd[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double num = sn[0], den = sd[0];
    double rel;
    int nonfinite = 0;
    if (!has_anchor) {
      rel = INFINITY;
    } else {
      nonfinite = !(isfinite(num) && isfinite(den));
      rel = den > 0.0 ? num / den : (num == num ? INFINITY : NAN);
    }
    *rel_out = rel;
    *nonfinite_out = nonfinite;
  }
}

// The decision skip = has_anchor && rel < threshold (strict; NaN and a zero
// denominator never skip).
__global__ __launch_bounds__(256) void fbc_final_kernel(const double* __restrict__ part, int nparts,
                                                        int has_anchor, double threshold,
                                                        FbcResult* __restrict__ res) {
  double rel;
  int nonfinite;
  fbc_final_sums(part, nparts, has_anchor, &rel, &nonfinite);
  if (threadIdx.x == 0) {
    res->rel = rel;
    res->skip = (has_anchor && !nonfinite && rel < threshold) ? 1 : 0;
    res->nonfinite = nonfinite;
  }
}

// Loop form: the same test with the anchor flag and threshold of the loop state,
// then the skip policy (no skip during the warm-up steps nor past max_skips
// consecutive skips) and its counters, all on the device.  A NaN / Inf in the sums
// never skips and is recorded in the step's log entry.
__global__ __launch_bounds__(256) void fbc_final_loop_kernel(const double* __restrict__ part,
                                                             int nparts, LoopState* __restrict__ s,
                                                             LoopLog* __restrict__ log) {
  const int has_anchor = s->has_anchor;
  double rel;
  int nonfinite;
  fbc_final_sums(part, nparts, has_anchor, &rel, &nonfinite);
  if (threadIdx.x == 0) {
    const int test = (has_anchor && !nonfinite && rel < (double)s->threshold) ? 1 : 0;
    const int skip = test && s->steps_done >= s->warmup_steps &&
                     (s->max_skips == 0 || s->skip_run < s->max_skips);
    s->steps_done += 1;
    s->skip_run = skip ? s->skip_run + 1 : 0;
    s->skip = skip;
    if (s->cur < s->n_steps) {
      log[s->cur].rel = rel;
      log[s->cur].skip = skip;
      log[s->cur].nonfinite = nonfinite;
    }
  }
}

// After a fully computed step: cached = (x_final - before) - r, anchor = r.
__global__ __launch_bounds__(256) void fbc_commit_kernel(
    const float* __restrict__ x, const float* __restrict__ before,
    const float* __restrict__ staging, float* __restrict__ cached, float* __restrict__ anchor,
    int B, int Lt, int Li, int L, int D, const int* __restrict__ skip, int run_if,
    int* __restrict__ has_anchor_out) {
  if (skip != nullptr && (*skip != 0) != run_if) return;
  if (has_anchor_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *has_anchor_out = 1;
  const size_t n4 = (size_t)B * Li * D / 4;
  for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n4; j += (size_t)gridDim.x * 256) {
    const size_t e = j * 4;
    const size_t row = e / D;
    const int c = (int)(e - row * D);
    const int b = (int)(row / Li), i = (int)(row - (size_t)b * Li);
    const f32x4 xf = *(const f32x4*)(x + ((size_t)b * L + Lt + i) * D + c);
    const f32x4 r = *(const f32x4*)(staging + e);
    *(f32x4*)(cached + e) = (xf - *(const f32x4*)(before + e)) - r;
    *(f32x4*)(anchor + e) = r;
  }
}

// Skipped step: x_img += cached.
__global__ __launch_bounds__(256) void fbc_apply_kernel(float* __restrict__ x,
                                                        const float* __restrict__ cached, int B,
                                                        int Lt, int Li, int L, int D,
                                                        const int* __restrict__ skip, int run_if) {
  if (skip != nullptr && (*skip != 0) != run_if) return;
  const size_t n4 = (size_t)B * Li * D / 4;
  for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n4; j += (size_t)gridDim.x * 256) {
    const size_t e = j * 4;
    const size_t row = e / D;
    const int c = (int)(e - row * D);
    const int b = (int)(row / Li), i = (int)(row - (size_t)b * Li);
    f32x4* p = (f32x4*)(x + ((size_t)b * L + Lt + i) * D + c);
    *p = *p + *(const f32x4*)(cached + e);
  }
}

// ---------------------------------------------------------------- Euler + CFG
// lat += dt * v, with v = v_neg + g (v_pos - v_neg) for a CFG pair (pos = batch row 0).
// With a loop state s, dt comes from it and the step counter advances.
__global__ __launch_bounds__(256) void euler_kernel(float* __restrict__ lat,
                                                    const float* __restrict__ v, int n, int cfg,
                                                    float g, float dt, LoopState* __restrict__ s) {
  if (s != nullptr) {
    dt = s->dt;
    if (blockIdx.x == 0 && threadIdx.x == 0) s->next = s->next + 1;
  }
  for (int j = blockIdx.x * 256 + threadIdx.x; j < n; j += gridDim.x * 256) {
    float vv = v[j];
    if (cfg) {
      const float vn = v[n + j];
      vv = vn + g * (vv - vn);
    }
    lat[j] += dt * vv;
  }
}

// Start of a replayed step (see loop_begin).  A replay past the last step copies
// nothing and sets dt = 0, so it leaves the latents as they are.
__global__ __launch_bounds__(256) void loop_begin_kernel(LoopState* __restrict__ s,
                                                         const float* __restrict__ mod_all,
                                                         size_t n_mod, const double* __restrict__ sig,
                                                         float* __restrict__ mod_cur,
                                                         LoopLog* __restrict__ log) {
  const int i = s->next;
  const int n = s->n_steps;
  if (i < n) {
    const f32x4* src = (const f32x4*)(mod_all + (size_t)i * n_mod);
    f32x4* dst = (f32x4*)mod_cur;
    for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n_mod / 4;
         j += (size_t)gridDim.x * 256)
      dst[j] = src[j];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    s->cur = i;
    s->skip = 0;
    if (i < n) {
      s->dt = (float)(sig[i + 1] - sig[i]);
      log[i].rel = INFINITY;
      log[i].skip = 0;
      log[i].nonfinite = 0;
    } else {
      s->dt = 0.0f;
      s->overrun = 1;
    }
  }
}

// ---------------------------------------------------------------- dtype moves
__global__ __launch_bounds__(256) void bf16_to_f32_kernel(const bf16_t* __restrict__ a,
                                                          float* __restrict__ b, size_t n4) {
  for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n4; j += (size_t)gridDim.x * 256)
    *(f32x4*)(b + 4 * j) = load4<bf16_t>(a + 4 * j);
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ a,
                                                          bf16_t* __restrict__ b, size_t n4) {
  for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n4; j += (size_t)gridDim.x * 256) {
    const f32x4 v = *(const f32x4*)(a + 4 * j);
    uint2 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    *(uint2*)(b + 4 * j) = u;
  }
}

// ---------------------------------------------------------------- launchers

static int grid_for(size_t n4) {
  size_t g = (n4 + 255) / 256;
  return (int)(g < 2048 ? (g == 0 ? 1 : g) : 2048);
}

hipError_t widen_bf16(const bf16_t* a, float* b, size_t n, hipStream_t st) {
  KTimerScope timer(KS_OTHER, st);
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3(grid_for(n / 4)), dim3(256), 0, st, a, b, n / 4);
  return hipGetLastError();
}

hipError_t narrow_f32(const float* a, bf16_t* b, size_t n, hipStream_t st) {
  KTimerScope timer(KS_OTHER, st);
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(grid_for(n / 4)), dim3(256), 0, st, a, b, n / 4);
  return hipGetLastError();
}

template <class WT>
hipError_t embed_latents(const float* lat, const WT* W, const float* bias, float* x,
                         float* before, int B, int Lt, int Li, int D, int Cin, hipStream_t st) {
  KTimerScope timer(KS_OTHER, st);
  if (Cin > 64) return hipErrorInvalidValue;
  dim3 grid((Li + 15) / 16, (D + 255) / 256);
  hipLaunchKernelGGL(embed_latents_kernel<WT>, grid, dim3(256), 0, st, lat, W, bias, x, before, B,
                     Lt, Li, Lt + Li, D, Cin);
  return hipGetLastError();
}
template hipError_t embed_latents<bf16_t>(const float*, const bf16_t*, const float*, float*,
                                          float*, int, int, int, int, int, hipStream_t);
template hipError_t embed_latents<float>(const float*, const float*, const float*, float*, float*,
                                         int, int, int, int, int, hipStream_t);

template <class TT>
hipError_t text_to_stream(const TT* txt, float* x, int B, int Lt, int L, int D, hipStream_t st) {
  KTimerScope timer(KS_OTHER, st);
  hipLaunchKernelGGL(text_to_stream_kernel<TT>, dim3(grid_for((size_t)B * Lt * D / 4)), dim3(256),
                     0, st, txt, x, B, Lt, L, D);
  return hipGetLastError();
}
template hipError_t text_to_stream<bf16_t>(const bf16_t*, float*, int, int, int, int, hipStream_t);
template hipError_t text_to_stream<float>(const float*, float*, int, int, int, int, hipStream_t);

template <class OT>
hipError_t sinusoid_host(const double* sig_host, OT* e, int M, int half, hipStream_t st) {
  for (int m0 = 0; m0 < M; m0 += SIG_CHUNK) {
    SigChunk c;
    const int n = M - m0 < SIG_CHUNK ? M - m0 : SIG_CHUNK;
    for (int i = 0; i < SIG_CHUNK; ++i) c.s[i] = i < n ? sig_host[m0 + i] : 0.0;
    hipLaunchKernelGGL(sinusoid_kernel<OT>, dim3(n), dim3(128), 0, st, c,
                       e + (size_t)m0 * 2 * half, half);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}
template hipError_t sinusoid_host<bf16_t>(const double*, bf16_t*, int, int, hipStream_t);
template hipError_t sinusoid_host<float>(const double*, float*, int, int, hipStream_t);

hipError_t rope_table(float* tab, int grid_w, int Lt, int L, int d, double theta, hipStream_t st) {
  KTimerScope timer(KS_OTHER, st);
  hipLaunchKernelGGL(rope_table_kernel, dim3(L), dim3(64), 0, st, tab, grid_w, Lt, L, d, theta);
  return hipGetLastError();
}

hipError_t fbc_reduce(const float* x, const float* before, const float* anchor, float* staging,
                      double* part, int nparts, FbcResult* res, int B, int Lt, int Li, int D,
                      int has_anchor, double threshold, hipStream_t st) {
  KTimerScope timer(KS_FBC, st);
  hipLaunchKernelGGL(fbc_partial_kernel, dim3(nparts), dim3(256), 0, st, x, before, anchor, staging,
                     part, B, Lt, Li, Lt + Li, D, has_anchor);
  hipLaunchKernelGGL(fbc_final_kernel, dim3(1), dim3(256), 0, st, part, nparts, has_anchor,
                     threshold, res);
  return hipGetLastError();
}

hipError_t fbc_commit(const float* x, const float* before, const float* staging, float* cached,
                      float* anchor, int B, int Lt, int Li, int D, hipStream_t st,
                      const int* skip, int run_if, int* has_anchor_out) {
  KTimerScope timer(KS_OTHER, st);
  hipLaunchKernelGGL(fbc_commit_kernel, dim3(grid_for((size_t)B * Li * D / 4)), dim3(256), 0, st,
                     x, before, staging, cached, anchor, B, Lt, Li, Lt + Li, D, skip, run_if,
                     has_anchor_out);
  return hipGetLastError();
}

hipError_t fbc_apply(float* x, const float* cached, int B, int Lt, int Li, int D, hipStream_t st,
                     const int* skip, int run_if) {
  KTimerScope timer(KS_OTHER, st);
  hipLaunchKernelGGL(fbc_apply_kernel, dim3(grid_for((size_t)B * Li * D / 4)), dim3(256), 0, st,
                     x, cached, B, Lt, Li, Lt + Li, D, skip, run_if);
  return hipGetLastError();
}

hipError_t fbc_reduce_loop(const float* x, const float* before, const float* anchor,
                           float* staging, double* part, int nparts, LoopState* s, LoopLog* log,
                           int B, int Lt, int Li, int D, hipStream_t st) {
  KTimerScope timer(KS_FBC, st);
  // the sums are always taken; without an anchor the final pass ignores them
  hipLaunchKernelGGL(fbc_partial_kernel, dim3(nparts), dim3(256), 0, st, x, before, anchor, staging,
                     part, B, Lt, Li, Lt + Li, D, 1);
  hipLaunchKernelGGL(fbc_final_loop_kernel, dim3(1), dim3(256), 0, st, part, nparts, s, log);
  return hipGetLastError();
}

hipError_t loop_begin(LoopState* s, const float* mod_all, size_t n_mod, const double* sig,
                      float* mod_cur, LoopLog* log, hipStream_t st) {
  if (n_mod % 4) return hipErrorInvalidValue;
  KTimerScope timer(KS_OTHER, st);
  hipLaunchKernelGGL(loop_begin_kernel, dim3(grid_for(n_mod / 4 + 1)), dim3(256), 0, st, s,
                     mod_all, n_mod, sig, mod_cur, log);
  return hipGetLastError();
}

hipError_t euler_update(float* lat, const float* v, int n, int cfg, float g, float dt,
                        hipStream_t st) {
  KTimerScope timer(KS_OTHER, st);
  hipLaunchKernelGGL(euler_kernel, dim3(grid_for((size_t)n / 4 + 1)), dim3(256), 0, st, lat, v, n,
                     cfg, g, dt, (LoopState*)nullptr);
  return hipGetLastError();
}

hipError_t euler_update_loop(float* lat, const float* v, int n, int cfg, float g, LoopState* s,
                             hipStream_t st) {
  KTimerScope timer(KS_OTHER, st);
  hipLaunchKernelGGL(euler_kernel, dim3(grid_for((size_t)n / 4 + 1)), dim3(256), 0, st, lat, v, n,
                     cfg, g, 0.0f, s);
  return hipGetLastError();
}

}  // namespace dit
