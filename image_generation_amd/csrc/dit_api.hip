// C ABI of libdit: argument validation, workspace layout and the host-side
// sequencing of the HIP kernels for a block, a denoise step, the modulation
// precompute and the First-Block-Cache test.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>
#include <new>

#include "../../include/dit.h"
#include "common.h"
#include "kernels.h"
#include "ops.h"

using namespace dit;

namespace {

thread_local std::string g_last_error;
thread_local dit_kernel_timer* g_timer = nullptr;
thread_local const int* g_gate = nullptr;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

#define DIT_CHECK_HIP(expr)                                                              \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(DIT_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));           \
  } while (0)

// Arch check, cached per device (the answer never changes for a device).
int check_device() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(DIT_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(DIT_ERR_UNSUPPORTED, "device index %d", dev);
  int v = cache[dev].load();
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(DIT_ERR_HIP, "hipGetDeviceProperties failed");
    v = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    cache[dev].store(v);
  }
  if (v != 1) return fail(DIT_ERR_UNSUPPORTED, "libdit runs on gfx950 only");
  return DIT_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

struct Dims {
  int B, Lt, Li, L, D, H, d, F, gw;
};

int make_dims(const dit_dims* in, Dims* o) {
  if (!in) return fail(DIT_ERR_INVALID_ARG, "dims is NULL");
  if (in->B < 1 || in->Lt < 0 || in->grid_h < 1 || in->grid_w < 1 || in->D < 1 || in->H < 1 ||
      in->F < 1)
    return fail(DIT_ERR_INVALID_ARG, "non-positive dimension");
  o->B = in->B;
  o->Lt = in->Lt;
  o->Li = in->grid_h * in->grid_w;
  o->L = o->Lt + o->Li;
  o->D = in->D;
  o->H = in->H;
  o->F = in->F;
  o->gw = in->grid_w;
  if (o->D % o->H) return fail(DIT_ERR_INVALID_ARG, "D %% H != 0");
  o->d = o->D / o->H;
  if ((long long)o->B * o->L * (o->D + o->F) > (1LL << 31) - 1)
    return fail(DIT_ERR_UNSUPPORTED, "problem too large for 32-bit row indexing");
  return DIT_OK;
}

int check_block_dims(const Dims& dm, int dtype) {
  if (dtype != DIT_BF16 && dtype != DIT_FP8 && dtype != DIT_F32 && dtype != DIT_MXFP4 &&
      dtype != DIT_MXFP4_FP8ATTN)
    return fail(DIT_ERR_UNSUPPORTED, "block dtype %d", dtype);
  if (dm.D % 256 || dm.D > 3072)
    return fail(DIT_ERR_UNSUPPORTED, "hidden size %d (needs a multiple of 256, <= 3072)", dm.D);
  if (dtype == DIT_F32) {
    if (dm.d != 32 && dm.d != 64)
      return fail(DIT_ERR_UNSUPPORTED, "fp32 blocks: head dim %d (32 or 64)", dm.d);
    if (dm.F % 4) return fail(DIT_ERR_UNSUPPORTED, "fp32 blocks: MLP size %d (multiple of 4)", dm.F);
    return DIT_OK;
  }
  if (dm.d != 64 && dm.d != 128)
    return fail(DIT_ERR_UNSUPPORTED, "head dim %d (bf16/fp8 run 64 or 128)", dm.d);
  if (dm.F % 64) return fail(DIT_ERR_UNSUPPORTED, "MLP size %d (needs a multiple of 64)", dm.F);
  // e4m3 K slabs are 128 deep
  if (dtype == DIT_FP8 && dm.F % 128)
    return fail(DIT_ERR_UNSUPPORTED, "fp8: MLP size %d (multiple of 128)", dm.F);
  if ((dtype == DIT_MXFP4 || dtype == DIT_MXFP4_FP8ATTN) && dm.F % 256)   // 256-deep MX slabs
    return fail(DIT_ERR_UNSUPPORTED, "mxfp4: MLP size %d (multiple of 256)", dm.F);
  return DIT_OK;
}

// ---- workspace layout (256-byte aligned carving)
struct Carver {
  char* base;
  size_t off;
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~(size_t)255;
    T* r = (T*)(base + off);
    off += n * sizeof(T);
    return r;
  }
};

struct BlockWS {
  float* xf;    // fp32 residual stream for a bf16-stored x [B, L, D]
  bf16_t* u;    // LN-modulate output [B*L, D] (row order of the block)
  bf16_t* q;    // [B, H, L, d] (rotated)
  bf16_t* k;    // [B, H, L, d] (rotated)
  bf16_t* v;    // [B, H, L, d]
  bf16_t* cat;  // [B*L, D + F]: attention output | MLP hidden
  // e4m3 operands of the fp8 blocks and their scales
  fp8_t* u8;    // [B*L, D], scale su [B*L]
  fp8_t* q8;    // [B, H, L, d]
  fp8_t* k8;    // [B, H, L, d]
  fp8_t* v8;    // [B, H, L, d]
  fp8_t* cat8;  // [B*L, D + F], scales s_att (attention part or whole row), s_hid
  float *su, *s_att, *s_hid;
  float* s_qkv;          // [3, B*H]: q, k, v scales per (b, h)
  unsigned int* amax;    // [3, B*H]: largest stored |q|, |k|, |v| per (b, h) (fp32 bits)
  // MXFP4 blocks: one linear input at a time as E2M1 codes [B*L, K/2] (over cat8)
  // and E8M0 scales [K/256][mx_pad][8]
  uint8_t* a4;
  uint8_t* a4s;
  int mx_pad;            // scale rows: B*L rounded up to 256, plus 256 so a GEMM group
                         // starting inside the array reads whole 256-row tiles
  // fp32 blocks (overlaying the buffers above): LN out, Q, K, V, attention | MLP
  float *u32, *q32, *k32, *v32, *cat32;
};

BlockWS carve_block(Carver& c, const Dims& dm, bool with_xf) {
  const size_t n = (size_t)dm.B * dm.L * dm.D;
  const size_t rows = (size_t)dm.B * dm.L;
  const size_t bh = (size_t)dm.B * dm.H;
  BlockWS w;
  w.xf = with_xf ? c.take<float>(n) : nullptr;
  Carver c32 = c;   // the fp32 layout reuses the space of the bf16 / fp8 one
  w.u = c.take<bf16_t>(n);
  w.q = c.take<bf16_t>(n);
  w.k = c.take<bf16_t>(n);
  w.v = c.take<bf16_t>(n);
  w.cat = c.take<bf16_t>(rows * (dm.D + dm.F));
  w.u8 = c.take<fp8_t>(n);
  w.q8 = c.take<fp8_t>(n);
  w.k8 = c.take<fp8_t>(n);
  w.v8 = c.take<fp8_t>(n);
  w.cat8 = c.take<fp8_t>(rows * (dm.D + dm.F));
  w.su = c.take<float>(rows);
  w.s_att = c.take<float>(rows);
  w.s_hid = c.take<float>(rows);
  w.s_qkv = c.take<float>(3 * bh);
  w.amax = c.take<unsigned int>(3 * bh);
  w.a4 = (uint8_t*)w.cat8;
  w.mx_pad = (int)((rows + 255) / 256 * 256 + 256);
  w.a4s = c.take<uint8_t>(((size_t)(dm.D + dm.F) / 256 + 1) * w.mx_pad * 8);
  w.u32 = c32.take<float>(n);
  w.q32 = c32.take<float>(n);
  w.k32 = c32.take<float>(n);
  w.v32 = c32.take<float>(n);
  w.cat32 = c32.take<float>(rows * (dm.D + dm.F));
  if (c32.off > c.off) c.off = c32.off;
  return w;
}

struct StepWS {
  BlockWS blk;
  float* x;         // joint residual stream [B, L, D]
  float* before;    // image hidden before block 0 [B, Li, D]
  float* staging;   // first block's residual [B, Li, D]
  float* v;         // velocity [B * Li, 64]
  float* rope;      // [L, d/2, 2]
  double* part;     // [2 * FBC_PARTS]
  FbcResult* res;
};

StepWS carve_step(Carver& c, const Dims& dm) {
  StepWS w;
  w.blk = carve_block(c, dm, false);
  w.x = c.take<float>((size_t)dm.B * dm.L * dm.D);
  w.before = c.take<float>((size_t)dm.B * dm.Li * dm.D);
  w.staging = c.take<float>((size_t)dm.B * dm.Li * dm.D);
  w.v = c.take<float>((size_t)dm.B * dm.Li * 64);
  w.rope = c.take<float>((size_t)dm.L * dm.d);
  w.part = c.take<double>(2 * FBC_PARTS);
  w.res = c.take<FbcResult>(1);
  return w;
}

struct ModWS {
  void* emb;  // [n, 256]  (bf16, or fp32 for an fp32 model)
  void* h;    // [n, D]
  void* cs;   // [n, D]
};

ModWS carve_mod(Carver& c, const Dims& dm, int n) {
  ModWS w;   // sized for fp32 elements, so either element type fits
  w.emb = c.take<float>((size_t)n * 256);
  w.h = c.take<float>((size_t)n * dm.D);
  w.cs = c.take<float>((size_t)n * dm.D);
  return w;
}

// Caller memory of a graph-replayed loop (dit_loop_state_bytes).
struct LoopBufs {
  LoopState* state;
  double* sig;       // [n + 1]
  LoopLog* log;      // [n]
  float* mod_cur;    // [N_mod]: the running step's modulation vectors
};

size_t n_mod_of(const dit_model* m) {
  return (12 * (size_t)m->n_double + 3 * (size_t)m->n_single + 2) * (size_t)m->dims.D;
}

LoopBufs carve_loop(Carver& c, size_t n_mod, int n) {
  LoopBufs b;
  b.state = c.take<LoopState>(1);
  b.sig = c.take<double>((size_t)n + 1);
  b.log = c.take<LoopLog>((size_t)n);
  b.mod_cur = c.take<float>(n_mod);
  return b;
}

size_t ws_size(const Dims& dm, int purpose, int n) {
  Carver c{nullptr, 0};
  switch (purpose) {
    case DIT_WS_ATTENTION: return 0;
    case DIT_WS_BLOCK: carve_block(c, dm, true); break;
    case DIT_WS_STEP: carve_step(c, dm); break;
    case DIT_WS_MODULATION: carve_mod(c, dm, n); break;
    case DIT_WS_FBCACHE:
      c.take<double>(2 * FBC_PARTS);
      c.take<FbcResult>(1);
      break;
    default: return 0;
  }
  return (c.off + 255) & ~(size_t)255;
}

// fp8: the layer must carry its per-channel weight scales; MXFP4 its block scales
int check_linear(const dit_linear& l, const char* name, int dtype = DIT_BF16) {
  if (!l.w || !l.b) return fail(DIT_ERR_INVALID_ARG, "%s: NULL weight or bias", name);
  if (!aligned16(l.w) || !aligned16(l.b))
    return fail(DIT_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", name);
  if (dtype == DIT_FP8 && (!l.w_scale || !aligned16(l.w_scale)))
    return fail(DIT_ERR_INVALID_ARG, "%s: fp8 layer needs a 16-byte aligned w_scale", name);
  if ((dtype == DIT_MXFP4 || dtype == DIT_MXFP4_FP8ATTN) && (!l.w_mx || !aligned16(l.w_mx)))
    return fail(DIT_ERR_INVALID_ARG, "%s: mxfp4 layer needs 16-byte aligned w_mx scales", name);
  return DIT_OK;
}

int check_block(const dit_block* blk, int dtype) {
  if (!blk) return fail(DIT_ERR_INVALID_ARG, "block is NULL");
  int rc;
  if (blk->kind == DIT_BLOCK_DOUBLE) {
    for (int s = 0; s < 2; ++s) {
      if ((rc = check_linear(blk->qkv[s], "qkv", dtype)) ||
          (rc = check_linear(blk->proj[s], "proj", dtype)) ||
          (rc = check_linear(blk->mlp1[s], "mlp1", dtype)) ||
          (rc = check_linear(blk->mlp2[s], "mlp2", dtype)))
        return rc;
    }
  } else if (blk->kind == DIT_BLOCK_SINGLE) {
    if ((rc = check_linear(blk->lin1, "lin1", dtype)) ||
        (rc = check_linear(blk->lin2, "lin2", dtype)))
      return rc;
  } else {
    return fail(DIT_ERR_INVALID_ARG, "unknown block kind %d", blk->kind);
  }
  return DIT_OK;
}

GemmProblem gp(const bf16_t* A, int lda, const dit_linear& l, int K, int M, int N) {
  GemmProblem g;
  g.A = A;
  g.lda = lda;
  g.W = (const bf16_t*)l.w;
  g.ldw = K;
  g.bias = l.b;
  g.M = M;
  g.N = N;
  g.K = K;
  return g;
}

// e4m3 problem: A8 [M, K] with row scales sa, weight codes with l.w_scale
GemmProblem gp8(const fp8_t* A8, int lda, const float* sa, const dit_linear& l, int K, int M, int N) {
  GemmProblem g = gp(nullptr, lda, l, K, M, N);
  g.W = nullptr;
  g.A8 = A8;
  g.W8 = (const fp8_t*)l.w;
  g.sa = sa;
  g.sw = l.w_scale;
  return g;
}

// fp32 problem: A32 [M, K] (row stride lda), fp32 weight [N, K]
GemmProblem gp32(const float* A, int lda, const dit_linear& l, int K, int M, int N) {
  GemmProblem g = gp(nullptr, lda, l, K, M, N);
  g.W = nullptr;
  g.A32 = A;
  g.W32 = (const float*)l.w;
  return g;
}

// fp32 block (reference precision): the same sequence as block_impl on fp32 buffers
hipError_t block_f32(const Dims& dm, const dit_block& blk, float* x, const float* mod, int bs,
                     const float* rope, const BlockWS& w, hipStream_t st) {
  const int B = dm.B, Lt = dm.Lt, Li = dm.Li, L = dm.L, D = dm.D, F = dm.F;
  const int DF = D + F;
  const QKVOut32 qo{w.q32, w.k32, w.v32, rope, D, dm.H, dm.d};
  const float scale = 1.0f / sqrtf((float)dm.d);
  hipError_t e;
  if (blk.kind == DIT_BLOCK_DOUBLE) {
    const RowMap sm{B, Lt, Li, L, 1, 0};
    RowMap st_txt = sm;
    st_txt.base = B * Li;
    const RowMap maps[2] = {sm, st_txt};
    const int ng = (B * Lt > 0) ? 2 : 1;
    const float* mi = mod;
    const float* mt = mod + 6 * (size_t)D;
    const size_t ti = (size_t)B * Li;
    float* u = w.u32;
    float* cat = w.cat32;
    if ((e = ln_modulate<float>(x, u, B * L, D, sm, B * Li, mi, mi + D, mt, mt + D, bs, st))) return e;
    GemmProblem g[2] = {gp32(u, D, blk.qkv[0], D, B * Li, 3 * D),
                        gp32(u + ti * D, D, blk.qkv[1], D, B * Lt, 3 * D)};
    if ((e = gemm32_qkv(g, ng, qo, maps, st))) return e;
    if ((e = attention_f32(w.q32, w.k32, w.v32, cat, DF, sm, B, dm.H, L, dm.d, scale, st)))
      return e;
    g[0] = gp32(cat, DF, blk.proj[0], D, B * Li, D);
    g[1] = gp32(cat + ti * DF, DF, blk.proj[1], D, B * Lt, D);
    const float* gate1[2] = {mi + 2 * D, mt + 2 * D};
    if ((e = gemm32_gated_residual(g, ng, x, D, gate1, bs, maps, st))) return e;
    if ((e = ln_modulate<float>(x, u, B * L, D, sm, B * Li, mi + 3 * D, mi + 4 * D, mt + 3 * D,
                                mt + 4 * D, bs, st)))
      return e;
    g[0] = gp32(u, D, blk.mlp1[0], D, B * Li, F);
    g[1] = gp32(u + ti * D, D, blk.mlp1[1], D, B * Lt, F);
    float* hid[2] = {cat + D, cat + ti * DF + D};
    const int ldh[2] = {DF, DF};
    if ((e = gemm32_gelu(g, ng, hid, ldh, st))) return e;
    g[0] = gp32(cat + D, DF, blk.mlp2[0], F, B * Li, D);
    g[1] = gp32(cat + ti * DF + D, DF, blk.mlp2[1], F, B * Lt, D);
    const float* gate2[2] = {mi + 5 * D, mt + 5 * D};
    return gemm32_gated_residual(g, ng, x, D, gate2, bs, maps, st);
  }
  const RowMap jm{B, Lt, Li, L, 0, 0};
  if ((e = ln_modulate<float>(x, w.u32, B * L, D, jm, B * L, mod, mod + D, mod, mod + D, bs, st)))
    return e;
  const GemmProblem g1 = gp32(w.u32, D, blk.lin1, D, B * L, 3 * D + F);
  if ((e = gemm32_linear1(g1, qo, jm, w.cat32, DF, st))) return e;
  if ((e = attention_f32(w.q32, w.k32, w.v32, w.cat32, DF, jm, B, dm.H, L, dm.d, scale, st)))
    return e;
  const GemmProblem g2 = gp32(w.cat32, DF, blk.lin2, DF, B * L, D);
  const float* gate[1] = {mod + 2 * D};
  return gemm32_gated_residual(&g2, 1, x, D, gate, bs, &jm, st);
}

// per-(b, h) e4m3 copies of the QKV epilogue's Q, K and V (bf16); their per-head
// amax was gathered by that epilogue into w.amax
hipError_t quant_qkv(const Dims& dm, const BlockWS& w, hipStream_t st) {
  const size_t n = (size_t)dm.L * dm.d;
  const int bh = dm.B * dm.H;
  hipError_t e;
  if ((e = quant_slices<bf16_t>(w.q, n, bh, w.amax, w.q8, w.s_qkv, st))) return e;
  if ((e = quant_slices<bf16_t>(w.k, n, bh, w.amax + bh, w.k8, w.s_qkv + bh, st))) return e;
  return quant_slices<bf16_t>(w.v, n, bh, w.amax + 2 * bh, w.v8, w.s_qkv + 2 * bh, st);
}

// fp8 block (x fp32): e4m3 GEMM operands with per-token activation scales, e4m3
// attention with per-(b, h) scales; the same row spaces and epilogues as bf16.
hipError_t block_fp8(const Dims& dm, const dit_block& blk, float* x, const float* mod, int bs,
                     const float* rope, const BlockWS& w, hipStream_t st) {
  const int B = dm.B, Lt = dm.Lt, Li = dm.Li, L = dm.L, D = dm.D, F = dm.F, H = dm.H;
  const int DF = D + F, BH = B * H;
  QKVOut qo{w.q, w.k, w.v, rope, D, H, dm.d};
  qo.amax = w.amax;
  const float scale = 1.0f / sqrtf((float)dm.d);
  const float *sq = w.s_qkv, *sk = w.s_qkv + BH, *sv = w.s_qkv + 2 * BH;
  hipError_t e;
  if (blk.kind == DIT_BLOCK_DOUBLE) {
    const RowMap sm{B, Lt, Li, L, 1, 0};
    RowMap st_txt = sm;
    st_txt.base = B * Li;
    const RowMap maps[2] = {sm, st_txt};
    const int ng = (B * Lt > 0) ? 2 : 1;
    const float* mi = mod;
    const float* mt = mod + 6 * (size_t)D;
    const size_t ti = (size_t)B * Li;

    if ((e = ln_modulate_fp8(x, w.u8, w.su, B * L, D, sm, B * Li, mi, mi + D, mt, mt + D, bs, st)))
      return e;
    GemmProblem g[2] = {gp8(w.u8, D, w.su, blk.qkv[0], D, B * Li, 3 * D),
                        gp8(w.u8 + ti * D, D, w.su + ti, blk.qkv[1], D, B * Lt, 3 * D)};
    if ((e = zero_u32(w.amax, 3 * BH, st))) return e;
    if ((e = gemm_qkv(g, ng, qo, maps, st))) return e;
    if ((e = quant_qkv(dm, w, st))) return e;
    if ((e = attention_fp8(w.q8, w.k8, w.v8, sq, sk, sv, w.cat, DF, sm, B, H, L, dm.d, scale, st)))
      return e;
    if ((e = quant_rows<bf16_t>(w.cat, DF, w.cat8, DF, w.s_att, B * L, D, st))) return e;
    g[0] = gp8(w.cat8, DF, w.s_att, blk.proj[0], D, B * Li, D);
    g[1] = gp8(w.cat8 + ti * DF, DF, w.s_att + ti, blk.proj[1], D, B * Lt, D);
    const float* gate1[2] = {mi + 2 * D, mt + 2 * D};
    if ((e = gemm_gated_residual<float>(g, ng, x, D, gate1, bs, maps, st))) return e;
    if ((e = ln_modulate_fp8(x, w.u8, w.su, B * L, D, sm, B * Li, mi + 3 * D, mi + 4 * D,
                             mt + 3 * D, mt + 4 * D, bs, st)))
      return e;
    g[0] = gp8(w.u8, D, w.su, blk.mlp1[0], D, B * Li, F);
    g[1] = gp8(w.u8 + ti * D, D, w.su + ti, blk.mlp1[1], D, B * Lt, F);
    bf16_t* hid[2] = {w.cat + D, w.cat + ti * DF + D};
    const int ldh[2] = {DF, DF};
    if ((e = gemm_gelu_bf16(g, ng, hid, ldh, st))) return e;
    if ((e = quant_rows<bf16_t>(w.cat + D, DF, w.cat8 + D, DF, w.s_hid, B * L, F, st))) return e;
    g[0] = gp8(w.cat8 + D, DF, w.s_hid, blk.mlp2[0], F, B * Li, D);
    g[1] = gp8(w.cat8 + ti * DF + D, DF, w.s_hid + ti, blk.mlp2[1], F, B * Lt, D);
    const float* gate2[2] = {mi + 5 * D, mt + 5 * D};
    return gemm_gated_residual<float>(g, ng, x, D, gate2, bs, maps, st);
  }
  const RowMap jm{B, Lt, Li, L, 0, 0};
  if ((e = ln_modulate_fp8(x, w.u8, w.su, B * L, D, jm, B * L, mod, mod + D, mod, mod + D, bs, st)))
    return e;
  const GemmProblem g1 = gp8(w.u8, D, w.su, blk.lin1, D, B * L, 3 * D + F);
  if ((e = zero_u32(w.amax, 3 * BH, st))) return e;
  if ((e = gemm_linear1(g1, qo, jm, w.cat, DF, st))) return e;
  if ((e = quant_qkv(dm, w, st))) return e;
  if ((e = attention_fp8(w.q8, w.k8, w.v8, sq, sk, sv, w.cat, DF, jm, B, H, L, dm.d, scale, st)))
    return e;
  // linear2 takes [attention | GELU] as one row, so one scale per joint row
  if ((e = quant_rows<bf16_t>(w.cat, DF, w.cat8, DF, w.s_att, B * L, DF, st))) return e;
  const GemmProblem g2 = gp8(w.cat8, DF, w.s_att, blk.lin2, DF, B * L, D);
  const float* gate[1] = {mod + 2 * D};
  return gemm_gated_residual<float>(&g2, 1, x, D, gate, bs, &jm, st);
}

hipError_t run_block(const Dims& dm, int dtype, const dit_block& blk, float* x, const float* mod,
                     int bs, const float* rope, const BlockWS& w, hipStream_t st);

// MXFP4 problem: activation codes [M, K/2] and their E8M0 scales, both starting at
// row r0 of the quantised activation (scale slab stride: pad rows); weight codes
// l.w [N, K/2] with block scales l.w_mx
GemmProblem gp4(const uint8_t* a4, const uint8_t* a4s, int r0, int pad, const dit_linear& l, int K,
                int M, int N) {
  GemmProblem g = gp(nullptr, K, l, K, M, N);
  g.W = nullptr;
  g.A4 = a4 + (size_t)r0 * (K / 2);
  g.W4 = (const uint8_t*)l.w;
  g.xa = a4s + (size_t)r0 * 8;
  g.xw = l.w_mx;
  g.pad_m = pad;
  g.pad_n = (N + 255) / 256 * 256;
  return g;
}

// MXFP4 (W4A4) block: the bf16 block's sequence with every linear's bf16 input
// quantised to MXFP4 just before its GEMM (32-value blocks along K, E8M0 scales;
// the LN outputs straight from the LN pass); attention stays bf16
// A8: attention in e4m3 as in the fp8 block (per-(b, h) scales from the QKV
// epilogue's amax), the linears still MXFP4
template <bool A8>
hipError_t block_mx4(const Dims& dm, const dit_block& blk, float* x, const float* mod, int bs,
                     const float* rope, const BlockWS& w, hipStream_t st) {
  const int B = dm.B, Lt = dm.Lt, Li = dm.Li, L = dm.L, D = dm.D, F = dm.F, H = dm.H;
  const int DF = D + F, BH = B * H;
  const int P = w.mx_pad;
  QKVOut qo{w.q, w.k, w.v, rope, D, dm.H, dm.d};
  if (A8) qo.amax = w.amax;
  const float scale = 1.0f / sqrtf((float)dm.d);
  const float *sq = w.s_qkv, *sk = w.s_qkv + BH, *sv = w.s_qkv + 2 * BH;
  // joint attention into the first D columns of cat, in the given row map
  auto attend = [&](const RowMap& map) -> hipError_t {
    if (!A8) return attention_bf16(w.q, w.k, w.v, w.cat, DF, map, B, H, L, dm.d, scale, st);
    hipError_t e2;
    if ((e2 = quant_qkv(dm, w, st))) return e2;
    return attention_fp8(w.q8, w.k8, w.v8, sq, sk, sv, w.cat, DF, map, B, H, L, dm.d, scale, st);
  };
  hipError_t e;
  if (blk.kind == DIT_BLOCK_DOUBLE) {
    const RowMap sm{B, Lt, Li, L, 1, 0};
    RowMap st_txt = sm;
    st_txt.base = B * Li;
    const RowMap maps[2] = {sm, st_txt};
    const int ng = (B * Lt > 0) ? 2 : 1;
    const float* mi = mod;
    const float* mt = mod + 6 * (size_t)D;
    const int ti = B * Li;   // first text row of the stream-major row space

    if ((e = ln_modulate_mx4(x, w.a4, w.a4s, P, B * L, D, sm, B * Li, mi, mi + D, mt, mt + D, bs,
                             st)))
      return e;
    GemmProblem g[2] = {gp4(w.a4, w.a4s, 0, P, blk.qkv[0], D, B * Li, 3 * D),
                        gp4(w.a4, w.a4s, ti, P, blk.qkv[1], D, B * Lt, 3 * D)};
    if (A8 && (e = zero_u32(w.amax, 3 * BH, st))) return e;
    if ((e = gemm_qkv(g, ng, qo, maps, st))) return e;
    if ((e = attend(sm))) return e;
    if ((e = quant_mxfp4<bf16_t>(w.cat, DF, B * L, D, w.a4, w.a4s, P, st))) return e;
    g[0] = gp4(w.a4, w.a4s, 0, P, blk.proj[0], D, B * Li, D);
    g[1] = gp4(w.a4, w.a4s, ti, P, blk.proj[1], D, B * Lt, D);
    const float* gate1[2] = {mi + 2 * D, mt + 2 * D};
    if ((e = gemm_gated_residual<float>(g, ng, x, D, gate1, bs, maps, st))) return e;
    if ((e = ln_modulate_mx4(x, w.a4, w.a4s, P, B * L, D, sm, B * Li, mi + 3 * D, mi + 4 * D,
                             mt + 3 * D, mt + 4 * D, bs, st)))
      return e;
    g[0] = gp4(w.a4, w.a4s, 0, P, blk.mlp1[0], D, B * Li, F);
    g[1] = gp4(w.a4, w.a4s, ti, P, blk.mlp1[1], D, B * Lt, F);
    bf16_t* hid[2] = {w.cat + D, w.cat + (size_t)ti * DF + D};
    const int ldh[2] = {DF, DF};
    if ((e = gemm_gelu_bf16(g, ng, hid, ldh, st))) return e;
    if ((e = quant_mxfp4<bf16_t>(w.cat + D, DF, B * L, F, w.a4, w.a4s, P, st))) return e;
    g[0] = gp4(w.a4, w.a4s, 0, P, blk.mlp2[0], F, B * Li, D);
    g[1] = gp4(w.a4, w.a4s, ti, P, blk.mlp2[1], F, B * Lt, D);
    const float* gate2[2] = {mi + 5 * D, mt + 5 * D};
    return gemm_gated_residual<float>(g, ng, x, D, gate2, bs, maps, st);
  }
  // single-stream block, joint row order
  const RowMap jm{B, Lt, Li, L, 0, 0};
  if ((e = ln_modulate_mx4(x, w.a4, w.a4s, P, B * L, D, jm, B * L, mod, mod + D, mod, mod + D, bs,
                           st)))
    return e;
  const GemmProblem g1 = gp4(w.a4, w.a4s, 0, P, blk.lin1, D, B * L, 3 * D + F);
  if (A8 && (e = zero_u32(w.amax, 3 * BH, st))) return e;
  if ((e = gemm_linear1(g1, qo, jm, w.cat, DF, st))) return e;
  if ((e = attend(jm))) return e;
  // linear2 takes [attention | GELU] as one row
  if ((e = quant_mxfp4<bf16_t>(w.cat, DF, B * L, DF, w.a4, w.a4s, P, st))) return e;
  const GemmProblem g2 = gp4(w.a4, w.a4s, 0, P, blk.lin2, DF, B * L, D);
  const float* gate[1] = {mod + 2 * D};
  return gemm_gated_residual<float>(&g2, 1, x, D, gate, bs, &jm, st);
}


// ---- one block, already validated
template <class XT>
hipError_t block_impl(const Dims& dm, const dit_block& blk, XT* x, const float* mod, int bs,
                      const float* rope, const BlockWS& w, hipStream_t st) {
  const int B = dm.B, Lt = dm.Lt, Li = dm.Li, L = dm.L, D = dm.D, F = dm.F;
  const int DF = D + F;
  const QKVOut qo{w.q, w.k, w.v, rope, D, dm.H, dm.d};
  const float scale = 1.0f / sqrtf((float)dm.d);
  hipError_t e;
  if (blk.kind == DIT_BLOCK_DOUBLE) {
    const RowMap sm{B, Lt, Li, L, 1, 0};
    RowMap st_txt = sm;
    st_txt.base = B * Li;
    const RowMap maps[2] = {sm, st_txt};
    const int ng = (B * Lt > 0) ? 2 : 1;
    const float* mi = mod;
    const float* mt = mod + 6 * (size_t)D;
    const size_t ti = (size_t)B * Li;   // first text row of the stream-major row space

    if ((e = ln_modulate<XT>(x, w.u, B * L, D, sm, B * Li, mi, mi + D, mt, mt + D, bs, st))) return e;
    GemmProblem g[2] = {gp(w.u, D, blk.qkv[0], D, B * Li, 3 * D),
                        gp(w.u + ti * D, D, blk.qkv[1], D, B * Lt, 3 * D)};
    if ((e = gemm_qkv(g, ng, qo, maps, st))) return e;
    if ((e = attention_bf16(w.q, w.k, w.v, w.cat, DF, sm, B, dm.H, L, dm.d, scale, st))) return e;
    g[0] = gp(w.cat, DF, blk.proj[0], D, B * Li, D);
    g[1] = gp(w.cat + ti * DF, DF, blk.proj[1], D, B * Lt, D);
    const float* gate1[2] = {mi + 2 * D, mt + 2 * D};
    if ((e = gemm_gated_residual<XT>(g, ng, x, D, gate1, bs, maps, st))) return e;
    if ((e = ln_modulate<XT>(x, w.u, B * L, D, sm, B * Li, mi + 3 * D, mi + 4 * D, mt + 3 * D,
                             mt + 4 * D, bs, st)))
      return e;
    g[0] = gp(w.u, D, blk.mlp1[0], D, B * Li, F);
    g[1] = gp(w.u + ti * D, D, blk.mlp1[1], D, B * Lt, F);
    bf16_t* hid[2] = {w.cat + D, w.cat + ti * DF + D};
    const int ldh[2] = {DF, DF};
    if ((e = gemm_gelu_bf16(g, ng, hid, ldh, st))) return e;
    g[0] = gp(w.cat + D, DF, blk.mlp2[0], F, B * Li, D);
    g[1] = gp(w.cat + ti * DF + D, DF, blk.mlp2[1], F, B * Lt, D);
    const float* gate2[2] = {mi + 5 * D, mt + 5 * D};
    return gemm_gated_residual<XT>(g, ng, x, D, gate2, bs, maps, st);
  }
  // single-stream block, joint row order
  const RowMap jm{B, Lt, Li, L, 0, 0};
  if ((e = ln_modulate<XT>(x, w.u, B * L, D, jm, B * L, mod, mod + D, mod, mod + D, bs, st))) return e;
  const GemmProblem g1 = gp(w.u, D, blk.lin1, D, B * L, 3 * D + F);
  if ((e = gemm_linear1(g1, qo, jm, w.cat, DF, st))) return e;
  if ((e = attention_bf16(w.q, w.k, w.v, w.cat, DF, jm, B, dm.H, L, dm.d, scale, st))) return e;
  const GemmProblem g2 = gp(w.cat, DF, blk.lin2, DF, B * L, D);
  const float* gate[1] = {mod + 2 * D};
  return gemm_gated_residual<XT>(&g2, 1, x, D, gate, bs, &jm, st);
}

hipError_t run_block(const Dims& dm, int dtype, const dit_block& blk, float* x, const float* mod,
                     int bs, const float* rope, const BlockWS& w, hipStream_t st) {
  if (dtype == DIT_FP8) return block_fp8(dm, blk, x, mod, bs, rope, w, st);
  if (dtype == DIT_MXFP4) return block_mx4<false>(dm, blk, x, mod, bs, rope, w, st);
  if (dtype == DIT_MXFP4_FP8ATTN) return block_mx4<true>(dm, blk, x, mod, bs, rope, w, st);
  if (dtype == DIT_F32) return block_f32(dm, blk, x, mod, bs, rope, w, st);
  return block_impl<float>(dm, blk, x, mod, bs, rope, w, st);
}

// ---- the pieces of one denoise step, shared by the eager and the replayed loop

// Model checks common to the step entry points.
int check_model(const dit_model* m, Dims* dm, const char* fn) {
  int rc;
  if ((rc = make_dims(&m->dims, dm))) return rc;
  if ((rc = check_block_dims(*dm, m->dtype))) return rc;
  if (m->n_double < 1 || m->n_single < 0 || !m->blocks)
    return fail(DIT_ERR_INVALID_ARG, "%s: needs >= 1 double block", fn);
  for (int j = 0; j < m->n_double + m->n_single; ++j) {
    if ((rc = check_block(&m->blocks[j], m->dtype))) return rc;
    const int want = j < m->n_double ? DIT_BLOCK_DOUBLE : DIT_BLOCK_SINGLE;
    if (m->blocks[j].kind != want)
      return fail(DIT_ERR_INVALID_ARG, "%s: block %d has the wrong kind", fn, j);
  }
  if ((rc = check_linear(m->img_in, "img_in")) || (rc = check_linear(m->final_out, "final_out")))
    return rc;
  if (m->C_in < 4 || m->C_in > 64 || m->C_in % 4)
    return fail(DIT_ERR_UNSUPPORTED, "%s: C_in %d (4..64, multiple of 4)", fn, m->C_in);
  if (dm->B > 2) return fail(DIT_ERR_UNSUPPORTED, "%s: B must be 1 or 2", fn);
  if (dm->B == 2 && !std::isfinite(m->guidance))
    return fail(DIT_ERR_INVALID_ARG, "%s: non-finite guidance", fn);
  return DIT_OK;
}

int check_cache(const dit_fbcache* cache, const char* fn) {
  if (!cache || !cache->enabled) return DIT_OK;
  if (!cache->anchor || !cache->cached || !aligned16(cache->anchor) || !aligned16(cache->cached))
    return fail(DIT_ERR_INVALID_ARG, "%s: cache buffers NULL or misaligned", fn);
  if (std::isnan(cache->threshold)) return fail(DIT_ERR_INVALID_ARG, "%s: NaN threshold", fn);
  if (cache->warmup_steps < 0 || cache->max_skips < 0 || cache->steps_done < 0 ||
      cache->skip_run < 0)
    return fail(DIT_ERR_INVALID_ARG, "%s: negative cache policy field", fn);
  return DIT_OK;
}

// RoPE table, text tokens and embedded latents into the joint stream; the image
// hidden before block 0 into w.before.
hipError_t step_embed(const dit_model* m, const Dims& dm, const void* txt, const float* latents,
                      const StepWS& w, hipStream_t st) {
  const int B = dm.B, Lt = dm.Lt, Li = dm.Li, D = dm.D;
  hipError_t e;
  if ((e = rope_table(w.rope, dm.gw, Lt, dm.L, dm.d, 10000.0, st))) return e;
  if (m->dtype == DIT_F32) {
    if (Lt > 0 && (e = text_to_stream((const float*)txt, w.x, B, Lt, dm.L, D, st))) return e;
    return embed_latents(latents, (const float*)m->img_in.w, m->img_in.b, w.x, w.before, B, Lt, Li,
                         D, m->C_in, st);
  }
  if (Lt > 0 && (e = text_to_stream((const bf16_t*)txt, w.x, B, Lt, dm.L, D, st))) return e;
  return embed_latents(latents, (const bf16_t*)m->img_in.w, m->img_in.b, w.x, w.before, B, Lt, Li,
                       D, m->C_in, st);
}

// Blocks 1.. (all but the first).
hipError_t step_rest(const dit_model* m, const Dims& dm, const float* mod_step, const StepWS& w,
                     hipStream_t st) {
  const size_t D12 = 12 * (size_t)dm.D, D3 = 3 * (size_t)dm.D;
  hipError_t e;
  for (int j = 1; j < m->n_double; ++j)
    if ((e = run_block(dm, m->dtype, m->blocks[j], w.x, mod_step + j * D12, 0, w.rope, w.blk, st)))
      return e;
  const float* ms = mod_step + m->n_double * D12;
  for (int j = 0; j < m->n_single; ++j)
    if ((e = run_block(dm, m->dtype, m->blocks[m->n_double + j], w.x, ms + j * D3, 0, w.rope, w.blk,
                       st)))
      return e;
  return hipSuccess;
}

// Velocity head on the image rows into w.v [B * Li, C_in].
hipError_t step_velocity(const dit_model* m, const Dims& dm, const float* mod_step,
                         const StepWS& w, hipStream_t st) {
  const int B = dm.B, Li = dm.Li, D = dm.D;
  const float* mf = mod_step + m->n_double * 12 * (size_t)D + m->n_single * 3 * (size_t)D;
  const RowMap sm{B, dm.Lt, Li, dm.L, 1, 0};
  hipError_t e;
  if (m->dtype == DIT_F32) {
    if ((e = ln_modulate<float>(w.x, w.blk.u32, B * Li, D, sm, B * Li, mf, mf + D, mf, mf + D, 0,
                                st)))
      return e;
    return gemm32_store(gp32(w.blk.u32, D, m->final_out, D, B * Li, m->C_in), w.v, m->C_in, st);
  }
  if ((e = ln_modulate<float>(w.x, w.blk.u, B * Li, D, sm, B * Li, mf, mf + D, mf, mf + D, 0, st)))
    return e;
  return gemm_store_f32(gp(w.blk.u, D, m->final_out, D, B * Li, m->C_in), w.v, m->C_in, st);
}

// One step of a replayed loop, every per-step value read from the loop state.
hipError_t enqueue_loop_step(const dit_model* m, const Dims& dm, const float* mod_all,
                             const void* txt, float* latents, float* anchor, float* cached,
                             bool cache_on, const StepWS& w, const LoopBufs& lb, hipStream_t st) {
  const int B = dm.B, Lt = dm.Lt, Li = dm.Li, D = dm.D;
  hipError_t e;
  if ((e = loop_begin(lb.state, mod_all, n_mod_of(m), lb.sig, lb.mod_cur, lb.log, st))) return e;
  if ((e = step_embed(m, dm, txt, latents, w, st))) return e;
  if ((e = run_block(dm, m->dtype, m->blocks[0], w.x, lb.mod_cur, 0, w.rope, w.blk, st))) return e;
  if (cache_on) {
    int* skip = &lb.state->skip;
    if ((e = fbc_reduce_loop(w.x, w.before, anchor, w.staging, w.part, FBC_PARTS, lb.state, lb.log,
                             B, Lt, Li, D, st)))
      return e;
    {
      GateScope gate(skip);
      if ((e = step_rest(m, dm, lb.mod_cur, w, st))) return e;
    }
    if ((e = fbc_apply(w.x, cached, B, Lt, Li, D, st, skip, 1))) return e;
    if ((e = fbc_commit(w.x, w.before, w.staging, cached, anchor, B, Lt, Li, D, st, skip, 0,
                        &lb.state->has_anchor)))
      return e;
  } else if ((e = step_rest(m, dm, lb.mod_cur, w, st))) {
    return e;
  }
  if ((e = step_velocity(m, dm, lb.mod_cur, w, st))) return e;
  return euler_update_loop(latents, w.v, Li * m->C_in, B == 2 ? 1 : 0, m->guidance, lb.state, st);
}

}  // namespace

// Host handle of a captured step graph.
struct dit_loop_graph {
  hipGraphExec_t exec;
  int device;
  int n_steps;
  int launched;        // replays enqueued since create / reset
  int cache_on;
  float* anchor;       // the cache buffers baked into the graph
  float* cached;
  LoopState* state;
  LoopLog* log;
};

namespace dit {
void ktimer_start(int site, hipStream_t st) {
  dit_kernel_timer* t = g_timer;
  if (!t || !((t->site_mask >> site) & 1u) || t->count >= t->capacity) return;
  t->sites[t->count] = site;
  (void)hipEventRecord((hipEvent_t)t->start[t->count], st);
}
const int* launch_gate() { return g_gate; }
GateScope::GateScope(const int* g) : prev(g_gate) { g_gate = g; }
GateScope::~GateScope() { g_gate = prev; }
void ktimer_stop(int site, hipStream_t st) {
  dit_kernel_timer* t = g_timer;
  if (!t || !((t->site_mask >> site) & 1u) || t->count >= t->capacity) return;
  (void)hipEventRecord((hipEvent_t)t->stop[t->count], st);
  ++t->count;
}
}  // namespace dit

// ====================================================================== C ABI

extern "C" {

const char* dit_status_string(int status) {
  switch (status) {
    case DIT_OK: return "ok";
    case DIT_ERR_INVALID_ARG: return "invalid argument";
    case DIT_ERR_UNSUPPORTED: return "unsupported";
    case DIT_ERR_WORKSPACE: return "workspace too small";
    case DIT_ERR_HIP: return "HIP runtime error";
    case DIT_ERR_NONFINITE: return "non-finite value in the cache test";
    default: return "unknown status";
  }
}

const char* dit_last_error(void) { return g_last_error.c_str(); }

int dit_set_kernel_timer(dit_kernel_timer* timer) {
  if (timer && (timer->capacity < 0 || timer->count < 0 ||
                (timer->capacity > 0 && (!timer->sites || !timer->start || !timer->stop))))
    return fail(DIT_ERR_INVALID_ARG, "dit_set_kernel_timer: bad timer");
  g_timer = timer;
  return DIT_OK;
}

size_t dit_workspace_bytes(const dit_dims* dims, int purpose, int n_steps) {
  Dims dm;
  if (make_dims(dims, &dm) != DIT_OK) return 0;
  if (purpose == DIT_WS_MODULATION && n_steps < 1) return 0;
  return ws_size(dm, purpose, n_steps);
}

int dit_sigmas(int n_steps, double shift, double* out_host) {
  if (n_steps < 1 || !out_host || !(shift > 0.0) || !std::isfinite(shift))
    return fail(DIT_ERR_INVALID_ARG, "dit_sigmas: n_steps >= 1, shift > 0, out non-NULL");
  for (int i = 0; i <= n_steps; ++i) {
    const double tau = 1.0 - (double)i / (double)n_steps;
    out_host[i] = shift * tau / (1.0 + (shift - 1.0) * tau);
  }
  return DIT_OK;
}

int dit_rope_table(int grid_h, int grid_w, int Lt, int head_dim, double theta, float* table,
                   void* stream) {
  if (grid_h < 1 || grid_w < 1 || Lt < 0 || head_dim < 4 || head_dim % 4 || !table ||
      !(theta > 0.0))
    return fail(DIT_ERR_INVALID_ARG, "dit_rope_table: bad argument");
  int rc = check_device();
  if (rc) return rc;
  DIT_CHECK_HIP(rope_table(table, grid_w, Lt, Lt + grid_h * grid_w, head_dim, theta,
                           (hipStream_t)stream));
  return DIT_OK;
}

int dit_linear_forward(const void* x, int M, int K, const dit_linear* lin, int N, void* y, int y_dtype,
               void* stream) {
  if (!x || !lin || !y) return fail(DIT_ERR_INVALID_ARG, "dit_linear_forward: NULL pointer");
  int rc;
  if ((rc = check_linear(*lin, "dit_linear_forward"))) return rc;
  if (!aligned16(x) || !aligned16(y))
    return fail(DIT_ERR_INVALID_ARG, "dit_linear_forward: pointers must be 16-byte aligned");
  if (M < 1 || K < 64 || K % 64 || N < 4 || N % 4)
    return fail(DIT_ERR_INVALID_ARG, "dit_linear_forward: M >= 1, K a multiple of 64, N a multiple of 4");
  if ((long long)M * N > (1LL << 40) || (long long)M * K > (1LL << 40))
    return fail(DIT_ERR_UNSUPPORTED, "dit_linear_forward: problem too large");
  if (y_dtype != DIT_F32 && y_dtype != DIT_BF16)
    return fail(DIT_ERR_INVALID_ARG, "dit_linear_forward: y_dtype %d", y_dtype);
  if ((rc = check_device())) return rc;
  const GemmProblem g = gp((const bf16_t*)x, K, *lin, K, M, N);
  if (y_dtype == DIT_F32)
    DIT_CHECK_HIP(gemm_store_f32(g, (float*)y, N, (hipStream_t)stream));
  else
    DIT_CHECK_HIP(gemm_store_bf16(g, (bf16_t*)y, N, (hipStream_t)stream));
  return DIT_OK;
}

int dit_block_views_of(const dit_dims* dims, void* workspace, size_t ws_bytes,
                       dit_block_views* out) {
  if (!workspace || !out) return fail(DIT_ERR_INVALID_ARG, "dit_block_views_of: NULL pointer");
  Dims dm;
  int rc;
  if ((rc = make_dims(dims, &dm))) return rc;
  const size_t need = ws_size(dm, DIT_WS_BLOCK, 0);
  if (ws_bytes < need)
    return fail(DIT_ERR_WORKSPACE, "dit_block_views_of: workspace %zu < %zu bytes", ws_bytes, need);
  Carver c{(char*)workspace, 0};
  const BlockWS w = carve_block(c, dm, true);
  out->ln = w.u;
  out->ln8 = w.u8;
  out->ln_scale = w.su;
  out->q = w.q;
  out->k = w.k;
  out->v = w.v;
  out->q8 = w.q8;
  out->k8 = w.k8;
  out->v8 = w.v8;
  out->qkv_scale = w.s_qkv;
  out->cat = w.cat;
  out->cat8 = w.cat8;
  out->att_scale = w.s_att;
  out->hid_scale = w.s_hid;
  return DIT_OK;
}

int dit_attention(const void* q, const void* k, const void* v, void* o, const float* q_scale,
                  const float* k_scale, const float* v_scale, int B, int H, int L, int head_dim,
                  int dtype, float softmax_scale, void* stream) {
  if (!q || !k || !v || !o) return fail(DIT_ERR_INVALID_ARG, "dit_attention: NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(DIT_ERR_INVALID_ARG, "dit_attention: pointers must be 16-byte aligned");
  if (dtype != DIT_BF16 && dtype != DIT_FP8 && dtype != DIT_F32)
    return fail(DIT_ERR_UNSUPPORTED, "dit_attention: dtype %d", dtype);
  if (B < 1 || H < 1 || L < 1)
    return fail(DIT_ERR_INVALID_ARG, "dit_attention: B, H and L must be >= 1");
  if (dtype == DIT_FP8 && (!q_scale || !k_scale || !v_scale))
    return fail(DIT_ERR_INVALID_ARG, "dit_attention: fp8 needs q, k and v scales");
  if (dtype == DIT_F32 ? (head_dim != 32 && head_dim != 64) : (head_dim != 64 && head_dim != 128))
    return fail(DIT_ERR_UNSUPPORTED, "dit_attention: head_dim %d for dtype %d", head_dim, dtype);
  if (!std::isfinite(softmax_scale))
    return fail(DIT_ERR_INVALID_ARG, "dit_attention: softmax_scale must be finite");
  if ((long long)B * H * L * head_dim > (1LL << 40) || (long long)B * L > (1LL << 31) - 1 ||
      (long long)L * head_dim > (1LL << 31) - 1)
    return fail(DIT_ERR_UNSUPPORTED, "dit_attention: problem too large");
  int rc = check_device();
  if (rc) return rc;
  const RowMap jm{B, 0, L, L, 0, 0};
  if (dtype == DIT_F32)
    DIT_CHECK_HIP(attention_f32((const float*)q, (const float*)k, (const float*)v, (float*)o,
                                H * head_dim, jm, B, H, L, head_dim, softmax_scale,
                                (hipStream_t)stream));
  else if (dtype == DIT_FP8)
    DIT_CHECK_HIP(attention_fp8((const fp8_t*)q, (const fp8_t*)k, (const fp8_t*)v, q_scale,
                                k_scale, v_scale, (bf16_t*)o, H * head_dim, jm, B, H, L, head_dim,
                                softmax_scale, (hipStream_t)stream));
  else
    DIT_CHECK_HIP(attention_bf16((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)o,
                                 H * head_dim, jm, B, H, L, head_dim, softmax_scale,
                                 (hipStream_t)stream));
  return DIT_OK;
}

int dit_quantize_rows(const void* src, int src_dtype, int src_ld, int rows, int width, void* dst,
                      int dst_ld, float* scale, void* stream) {
  if (!src || !dst || !scale) return fail(DIT_ERR_INVALID_ARG, "dit_quantize_rows: NULL pointer");
  if (!aligned16(src) || !aligned16(dst) || !aligned16(scale))
    return fail(DIT_ERR_INVALID_ARG, "dit_quantize_rows: pointers must be 16-byte aligned");
  if (src_dtype != DIT_BF16)
    return fail(DIT_ERR_UNSUPPORTED, "dit_quantize_rows: src_dtype %d (DIT_BF16)", src_dtype);
  if (rows < 0 || width < 8 || width % 8 || src_ld < width || src_ld % 8 || dst_ld < width ||
      dst_ld % 8)
    return fail(DIT_ERR_INVALID_ARG,
                "dit_quantize_rows: width, src_ld, dst_ld multiples of 8, strides >= width");
  if ((long long)rows * src_ld > (1LL << 40) || (long long)rows * dst_ld > (1LL << 40))
    return fail(DIT_ERR_UNSUPPORTED, "dit_quantize_rows: problem too large");
  int rc = check_device();
  if (rc) return rc;
  DIT_CHECK_HIP(quant_rows<bf16_t>((const bf16_t*)src, src_ld, (fp8_t*)dst, dst_ld, scale, rows,
                                   width, (hipStream_t)stream));
  return DIT_OK;
}

int dit_mx_rows(int rows) { return rows <= 0 ? 0 : (rows + 255) / 256 * 256; }

int dit_quantize_mxfp4(const void* src, int src_dtype, int src_ld, int rows, int width,
                       void* codes, unsigned char* scales, void* stream) {
  if (!src || !codes || !scales)
    return fail(DIT_ERR_INVALID_ARG, "dit_quantize_mxfp4: NULL pointer");
  if (!aligned16(src) || !aligned16(codes) || !aligned16(scales))
    return fail(DIT_ERR_INVALID_ARG, "dit_quantize_mxfp4: pointers must be 16-byte aligned");
  if (src_dtype != DIT_BF16 && src_dtype != DIT_F32)
    return fail(DIT_ERR_UNSUPPORTED, "dit_quantize_mxfp4: src_dtype %d (DIT_BF16, DIT_F32)",
                src_dtype);
  if (rows < 0 || width < 256 || width % 256 || src_ld < width || src_ld % 8)
    return fail(DIT_ERR_INVALID_ARG,
                "dit_quantize_mxfp4: width a multiple of 256, src_ld >= width, src_ld % 8 == 0");
  if ((long long)rows * src_ld > (1LL << 40))
    return fail(DIT_ERR_UNSUPPORTED, "dit_quantize_mxfp4: problem too large");
  int rc = check_device();
  if (rc) return rc;
  const int pad = dit_mx_rows(rows);
  if (src_dtype == DIT_BF16)
    DIT_CHECK_HIP(quant_mxfp4<bf16_t>((const bf16_t*)src, src_ld, rows, width, (uint8_t*)codes,
                                      scales, pad, (hipStream_t)stream));
  else
    DIT_CHECK_HIP(quant_mxfp4<float>((const float*)src, src_ld, rows, width, (uint8_t*)codes,
                                     scales, pad, (hipStream_t)stream));
  return DIT_OK;
}

int dit_linear_mxfp4(const void* x_codes, const unsigned char* x_scales, int M, int K,
                     const void* w_codes, const unsigned char* w_scales, const float* b, int N,
                     void* y, int y_dtype, void* stream) {
  if (!x_codes || !x_scales || !w_codes || !w_scales || !y)
    return fail(DIT_ERR_INVALID_ARG, "dit_linear_mxfp4: NULL pointer");
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(y) || (b && !aligned16(b)))
    return fail(DIT_ERR_INVALID_ARG, "dit_linear_mxfp4: pointers must be 16-byte aligned");
  if (M < 1 || K < 256 || K % 256 || N < 4 || N % 4)
    return fail(DIT_ERR_INVALID_ARG,
                "dit_linear_mxfp4: M >= 1, K a multiple of 256, N a multiple of 4");
  if ((long long)M * (K / 2) >= (1LL << 31) || (long long)N * (K / 2) >= (1LL << 31) ||
      (long long)M * N > (1LL << 40))
    return fail(DIT_ERR_UNSUPPORTED, "dit_linear_mxfp4: problem too large");
  if (y_dtype != DIT_F32 && y_dtype != DIT_BF16)
    return fail(DIT_ERR_INVALID_ARG, "dit_linear_mxfp4: y_dtype %d", y_dtype);
  int rc = check_device();
  if (rc) return rc;
  GemmProblem g{};
  g.lda = K;
  g.ldw = K;
  g.bias = b;
  g.M = M;
  g.N = N;
  g.K = K;
  g.A4 = (const uint8_t*)x_codes;
  g.W4 = (const uint8_t*)w_codes;
  g.xa = x_scales;
  g.xw = w_scales;
  g.pad_m = dit_mx_rows(M);
  g.pad_n = dit_mx_rows(N);
  if (y_dtype == DIT_F32)
    DIT_CHECK_HIP(gemm_mx4_store_f32(g, (float*)y, N, (hipStream_t)stream));
  else
    DIT_CHECK_HIP(gemm_mx4_store_bf16(g, (bf16_t*)y, N, (hipStream_t)stream));
  return DIT_OK;
}

int dit_block_forward(const dit_dims* dims, const dit_block* blk, int dtype, void* x, int x_dtype,
                      const float* mod, long mod_bstride, const float* rope, void* workspace,
                      size_t ws_bytes, void* stream) {
  Dims dm;
  int rc;
  if ((rc = make_dims(dims, &dm))) return rc;
  if ((rc = check_block_dims(dm, dtype))) return rc;
  if ((rc = check_block(blk, dtype))) return rc;
  if (!x || !mod || !rope || !workspace)
    return fail(DIT_ERR_INVALID_ARG, "dit_block_forward: NULL pointer");
  if (!aligned16(x) || !aligned16(mod) || !aligned16(rope) || !aligned16(workspace))
    return fail(DIT_ERR_INVALID_ARG, "dit_block_forward: pointers must be 16-byte aligned");
  if (mod_bstride < 0 || mod_bstride % 4 || mod_bstride > (1L << 30))
    return fail(DIT_ERR_INVALID_ARG, "dit_block_forward: mod_bstride must be >= 0, a multiple of 4");
  if (x_dtype != DIT_F32 && x_dtype != DIT_BF16)
    return fail(DIT_ERR_INVALID_ARG, "dit_block_forward: x_dtype %d", x_dtype);
  const size_t need = ws_size(dm, DIT_WS_BLOCK, 0);
  if (ws_bytes < need)
    return fail(DIT_ERR_WORKSPACE, "dit_block_forward: workspace %zu < %zu bytes", ws_bytes, need);
  if ((rc = check_device())) return rc;
  Carver c{(char*)workspace, 0};
  const BlockWS w = carve_block(c, dm, true);
  hipStream_t st = (hipStream_t)stream;
  if (x_dtype == DIT_F32) {
    DIT_CHECK_HIP(run_block(dm, dtype, *blk, (float*)x, mod, (int)mod_bstride, rope, w, st));
  } else {
    // a bf16 residual stream is carried in fp32 through the block and rounded once
    const size_t n = (size_t)dm.B * dm.L * dm.D;
    DIT_CHECK_HIP(widen_bf16((const bf16_t*)x, w.xf, n, st));
    DIT_CHECK_HIP(run_block(dm, dtype, *blk, w.xf, mod, (int)mod_bstride, rope, w, st));
    DIT_CHECK_HIP(narrow_f32(w.xf, (bf16_t*)x, n, st));
  }
  return DIT_OK;
}

}  // extern "C"

namespace {

// Argument checks of the modulation entry points; *need receives the scratch bytes.
int check_modulation(const dit_model* m, const double* sigmas_host, int n, const float* out,
                     Dims* dm, long long* nmod, size_t* need, const char* fn) {
  if (!m || !sigmas_host || !out || n < 1)
    return fail(DIT_ERR_INVALID_ARG, "%s: NULL pointer or n < 1", fn);
  int rc;
  if ((rc = make_dims(&m->dims, dm))) return rc;
  if ((rc = check_linear(m->time1, "time1")) || (rc = check_linear(m->time2, "time2")) ||
      (rc = check_linear(m->mod, "mod")))
    return rc;
  if (!aligned16(out)) return fail(DIT_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
  if (m->n_double < 0 || m->n_single < 0)
    return fail(DIT_ERR_INVALID_ARG, "%s: negative block count", fn);
  if (dm->D % 64) return fail(DIT_ERR_UNSUPPORTED, "%s: D %% 64 != 0", fn);
  for (int i = 0; i < n; ++i)
    if (!std::isfinite(sigmas_host[i])) return fail(DIT_ERR_INVALID_ARG, "%s: non-finite sigma", fn);
  *nmod = (12LL * m->n_double + 3LL * m->n_single + 2) * dm->D;
  if (*nmod > (1LL << 31) - 1) return fail(DIT_ERR_UNSUPPORTED, "%s: too many vectors", fn);
  if (m->dtype != DIT_BF16 && m->dtype != DIT_FP8 && m->dtype != DIT_F32 &&
      m->dtype != DIT_MXFP4 && m->dtype != DIT_MXFP4_FP8ATTN)
    return fail(DIT_ERR_INVALID_ARG, "%s: model dtype %d", fn, m->dtype);
  *need = ws_size(*dm, DIT_WS_MODULATION, n);
  return DIT_OK;
}

// The modulation kernels with their intermediates (timestep sinusoid, hidden
// activation, SiLU(c)) carved from scratch; every intermediate is written in
// full before it is read, so the scratch needs no clearing.
int modulation_run(const dit_model* m, const Dims& dm, long long nmod, const double* sigmas_host,
                   int n, float* out, void* scratch_base, hipStream_t st) {
  Carver c{(char*)scratch_base, 0};
  const ModWS w = carve_mod(c, dm, n);
  if (m->dtype == DIT_F32) {
    float *emb = (float*)w.emb, *h = (float*)w.h, *cs = (float*)w.cs;
    DIT_CHECK_HIP(sinusoid_host(sigmas_host, emb, n, 128, st));
    DIT_CHECK_HIP(gemm32_silu(gp32(emb, 256, m->time1, 256, n, dm.D), h, dm.D, st));
    DIT_CHECK_HIP(gemm32_silu(gp32(h, dm.D, m->time2, dm.D, n, dm.D), cs, dm.D, st));
    DIT_CHECK_HIP(gemm32_store(gp32(cs, dm.D, m->mod, dm.D, n, (int)nmod), out, (int)nmod, st));
    return DIT_OK;
  }
  bf16_t *emb = (bf16_t*)w.emb, *h = (bf16_t*)w.h, *cs = (bf16_t*)w.cs;
  DIT_CHECK_HIP(sinusoid_host(sigmas_host, emb, n, 128, st));
  DIT_CHECK_HIP(gemm_silu_bf16(gp(emb, 256, m->time1, 256, n, dm.D), h, dm.D, st));
  DIT_CHECK_HIP(gemm_silu_bf16(gp(h, dm.D, m->time2, dm.D, n, dm.D), cs, dm.D, st));
  DIT_CHECK_HIP(gemm_store_f32(gp(cs, dm.D, m->mod, dm.D, n, (int)nmod), out, (int)nmod, st));
  return DIT_OK;
}

// Static scratch of dit_modulation_static: one copy per GPU, kept until the
// process ends.  Host code never passes `scratch` itself (its host-side name is
// a stand-in, not a device address): the device address of each GPU's copy is
// looked up once per device with that device current and kept in
// g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[DIT_MOD_STATIC_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};

int static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(DIT_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(DIT_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DIT_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return DIT_OK;
}

}  // namespace

extern "C" {

int dit_modulation(const dit_model* m, const double* sigmas_host, int n, float* out,
                   void* workspace, size_t ws_bytes, void* stream) {
  Dims dm;
  long long nmod = 0;
  size_t need = 0;
  int rc;
  if ((rc = check_modulation(m, sigmas_host, n, out, &dm, &nmod, &need, "dit_modulation")))
    return rc;
  if (!workspace) return fail(DIT_ERR_INVALID_ARG, "dit_modulation: NULL workspace");
  if (!aligned16(workspace))
    return fail(DIT_ERR_INVALID_ARG, "dit_modulation: pointers must be 16-byte aligned");
  if (ws_bytes < need)
    return fail(DIT_ERR_WORKSPACE, "dit_modulation: workspace %zu < %zu bytes", ws_bytes, need);
  if ((rc = check_device())) return rc;
  return modulation_run(m, dm, nmod, sigmas_host, n, out, workspace, (hipStream_t)stream);
}

int dit_modulation_static(const dit_model* m, const double* sigmas_host, int n, float* out,
                          void* stream) {
  Dims dm;
  long long nmod = 0;
  size_t need = 0;
  int rc;
  if ((rc = check_modulation(m, sigmas_host, n, out, &dm, &nmod, &need, "dit_modulation_static")))
    return rc;
  if (need > (size_t)DIT_MOD_STATIC_BYTES)
    return fail(DIT_ERR_WORKSPACE,
                "dit_modulation_static: %d steps at D %d need %zu bytes of scratch, more than "
                "the library's static %u bytes (call dit_modulation with a workspace, or fewer "
                "steps per call)",
                n, dm.D, need, (unsigned)DIT_MOD_STATIC_BYTES);
  if ((rc = check_device())) return rc;
  void* base = nullptr;
  if ((rc = static_scratch(&base))) return rc;
  return modulation_run(m, dm, nmod, sigmas_host, n, out, base, (hipStream_t)stream);
}

int fbcache_should_skip(const float* x_after, const float* x_before, const float* anchor,
                        float* staging, int B, int Lt, int Li, int D, float threshold,
                        int has_anchor, void* workspace, size_t ws_bytes, void* stream,
                        double* rel_out, int* skip_out) {
  if (!x_after || !x_before || !staging || !workspace || !rel_out || !skip_out ||
      (has_anchor && !anchor))
    return fail(DIT_ERR_INVALID_ARG, "fbcache_should_skip: NULL pointer");
  if (!aligned16(x_after) || !aligned16(x_before) || !aligned16(staging) ||
      !aligned16(workspace) || (anchor && !aligned16(anchor)))
    return fail(DIT_ERR_INVALID_ARG, "fbcache_should_skip: pointers must be 16-byte aligned");
  if (B < 1 || Lt < 0 || Li < 1 || D < 4 || D % 4)
    return fail(DIT_ERR_INVALID_ARG, "fbcache_should_skip: bad shape");
  if (std::isnan(threshold)) return fail(DIT_ERR_INVALID_ARG, "fbcache_should_skip: NaN threshold");
  dit_dims dd{B, Lt, 1, Li, D, 1, 1};
  Dims dm;
  int rc;
  if ((rc = make_dims(&dd, &dm))) return rc;
  const size_t need = ws_size(dm, DIT_WS_FBCACHE, 0);
  if (ws_bytes < need)
    return fail(DIT_ERR_WORKSPACE, "fbcache_should_skip: workspace %zu < %zu bytes", ws_bytes, need);
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  Carver c{(char*)workspace, 0};
  double* part = c.take<double>(2 * FBC_PARTS);
  FbcResult* res = c.take<FbcResult>(1);
  DIT_CHECK_HIP(fbc_reduce(x_after, x_before, anchor, staging, part, FBC_PARTS, res, B, Lt, Li, D,
                           has_anchor ? 1 : 0, (double)threshold, st));
  FbcResult h;
  DIT_CHECK_HIP(hipMemcpyAsync(&h, res, sizeof(h), hipMemcpyDeviceToHost, st));
  DIT_CHECK_HIP(hipStreamSynchronize(st));
  *rel_out = h.rel;
  *skip_out = h.skip;
  if (h.nonfinite) return fail(DIT_ERR_NONFINITE, "fbcache_should_skip: non-finite residual");
  return DIT_OK;
}

int dit_denoise_step(const dit_model* m, const float* mod_step, const void* txt, float* latents,
                     double sigma, double sigma_next, dit_fbcache* cache, void* workspace,
                     size_t ws_bytes, void* stream, dit_step_info* info_out) {
  if (!m || !mod_step || !latents || !workspace || (m->dims.Lt > 0 && !txt))
    return fail(DIT_ERR_INVALID_ARG, "dit_denoise_step: NULL pointer");
  Dims dm;
  int rc;
  if ((rc = check_model(m, &dm, "dit_denoise_step"))) return rc;
  if (!std::isfinite(sigma) || !std::isfinite(sigma_next))
    return fail(DIT_ERR_INVALID_ARG, "dit_denoise_step: non-finite sigma");
  if (!aligned16(mod_step) || !aligned16(latents) || !aligned16(workspace) ||
      (txt && !aligned16(txt)))
    return fail(DIT_ERR_INVALID_ARG, "dit_denoise_step: pointers must be 16-byte aligned");
  const bool use_cache = cache && cache->enabled;
  if ((rc = check_cache(cache, "dit_denoise_step"))) return rc;
  const size_t need = ws_size(dm, DIT_WS_STEP, 0);
  if (ws_bytes < need)
    return fail(DIT_ERR_WORKSPACE, "dit_denoise_step: workspace %zu < %zu bytes", ws_bytes, need);
  if ((rc = check_device())) return rc;

  hipStream_t st = (hipStream_t)stream;
  Carver c{(char*)workspace, 0};
  const StepWS w = carve_step(c, dm);
  const int B = dm.B, Lt = dm.Lt, Li = dm.Li, D = dm.D;

  DIT_CHECK_HIP(step_embed(m, dm, txt, latents, w, st));
  DIT_CHECK_HIP(run_block(dm, m->dtype, m->blocks[0], w.x, mod_step, 0, w.rope, w.blk, st));

  double rel = INFINITY;
  int skip = 0;
  if (use_cache) {
    DIT_CHECK_HIP(fbc_reduce(w.x, w.before, cache->anchor, w.staging, w.part, FBC_PARTS, w.res, B,
                             Lt, Li, D, cache->has_anchor ? 1 : 0, (double)cache->threshold, st));
    FbcResult h;
    DIT_CHECK_HIP(hipMemcpyAsync(&h, w.res, sizeof(h), hipMemcpyDeviceToHost, st));
    DIT_CHECK_HIP(hipStreamSynchronize(st));
    if (h.nonfinite) return fail(DIT_ERR_NONFINITE, "dit_denoise_step: non-finite residual");
    rel = h.rel;
    // the rel test, then the policy: no skip during warm-up nor past max_skips in a row
    skip = h.skip && cache->steps_done >= cache->warmup_steps &&
           (cache->max_skips == 0 || cache->skip_run < cache->max_skips);
    cache->steps_done += 1;
    cache->skip_run = skip ? cache->skip_run + 1 : 0;
  }
  if (skip) {
    DIT_CHECK_HIP(fbc_apply(w.x, cache->cached, B, Lt, Li, D, st));
  } else {
    DIT_CHECK_HIP(step_rest(m, dm, mod_step, w, st));
    if (use_cache) {
      DIT_CHECK_HIP(fbc_commit(w.x, w.before, w.staging, cache->cached, cache->anchor, B, Lt, Li, D,
                               st));
      cache->has_anchor = 1;
    }
  }
  // velocity head on the image rows, then the Euler (+CFG) update
  DIT_CHECK_HIP(step_velocity(m, dm, mod_step, w, st));
  DIT_CHECK_HIP(euler_update(latents, w.v, Li * m->C_in, B == 2 ? 1 : 0, m->guidance,
                             (float)(sigma_next - sigma), st));
  if (info_out) {
    info_out->rel = rel;
    info_out->skipped = skip;
  }
  return DIT_OK;
}

// Workspace of dit_denoise_step_at: the step's own workspace, then the step's
// modulation row, then the modulation scratch for one row.
struct StepAtLayout {
  size_t step, row_off, mod_off, total;
};

static bool step_at_layout(const dit_model* m, StepAtLayout* o) {
  Dims dm;
  if (!m || m->n_double < 0 || m->n_single < 0) return false;
  if (make_dims(&m->dims, &dm) != DIT_OK) return false;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  o->step = ws_size(dm, DIT_WS_STEP, 0);
  o->row_off = up(o->step);
  o->mod_off = o->row_off + up(n_mod_of(m) * sizeof(float));
  o->total = o->mod_off + ws_size(dm, DIT_WS_MODULATION, 1);
  return true;
}

size_t dit_step_at_workspace_bytes(const dit_model* m) {
  StepAtLayout lay;
  return step_at_layout(m, &lay) ? lay.total : 0;
}

int dit_denoise_step_at(const dit_model* m, float* latents, const void* txt, int step,
                        int num_steps, const double* sigmas_host, dit_fbcache* cache,
                        void* workspace, size_t ws_bytes, void* stream,
                        dit_step_info* info_out) {
  const char* fn = "dit_denoise_step_at";
  if (!m || !sigmas_host || !workspace) return fail(DIT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (num_steps < 1 || step < 0 || step >= num_steps)
    return fail(DIT_ERR_INVALID_ARG, "%s: step %d of %d", fn, step, num_steps);
  if (!aligned16(workspace))
    return fail(DIT_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
  Dims dm;
  int rc;
  if ((rc = check_model(m, &dm, fn))) return rc;
  StepAtLayout lay;
  if (!step_at_layout(m, &lay)) return fail(DIT_ERR_INVALID_ARG, "%s: bad model dimensions", fn);
  if (ws_bytes < lay.total)
    return fail(DIT_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, lay.total);
  float* row = (float*)((char*)workspace + lay.row_off);
  long long nmod = 0;
  size_t mod_need = 0;
  if ((rc = check_modulation(m, sigmas_host + step, 1, row, &dm, &nmod, &mod_need, fn))) return rc;
  if (!std::isfinite(sigmas_host[step + 1]))
    return fail(DIT_ERR_INVALID_ARG, "%s: non-finite sigma", fn);
  // the step's own checks run before anything is enqueued; the row is written next
  if (!latents || (m->dims.Lt > 0 && !txt)) return fail(DIT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(latents) || (txt && !aligned16(txt)))
    return fail(DIT_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
  if ((rc = check_cache(cache, fn))) return rc;
  if ((rc = check_device())) return rc;
  if ((rc = modulation_run(m, dm, nmod, sigmas_host + step, 1, row,
                           (char*)workspace + lay.mod_off, (hipStream_t)stream)))
    return rc;
  return dit_denoise_step(m, row, txt, latents, sigmas_host[step], sigmas_host[step + 1], cache,
                          workspace, lay.step, stream, info_out);
}

size_t dit_loop_state_bytes(const dit_model* m, int n_steps) {
  if (!m || n_steps < 1 || m->n_double < 0 || m->n_single < 0 || m->dims.D <= 0) return 0;
  Carver c{nullptr, 0};
  carve_loop(c, n_mod_of(m), n_steps);
  return (c.off + 255) & ~(size_t)255;
}

// Initial device state of a replayed loop from the caller's cache state.
static int write_loop_state(LoopState* dst, int n_steps, int first_step, const dit_fbcache* cache,
                            hipStream_t st) {
  LoopState h{};
  h.next = first_step;
  h.cur = first_step;
  h.n_steps = n_steps;
  if (cache && cache->enabled) {
    h.cache_on = 1;
    h.has_anchor = cache->has_anchor ? 1 : 0;
    h.steps_done = cache->steps_done;
    h.skip_run = cache->skip_run;
    h.warmup_steps = cache->warmup_steps;
    h.max_skips = cache->max_skips;
    h.threshold = cache->threshold;
  }
  DIT_CHECK_HIP(hipMemcpyAsync(dst, &h, sizeof(h), hipMemcpyHostToDevice, st));
  DIT_CHECK_HIP(hipStreamSynchronize(st));
  return DIT_OK;
}

int dit_loop_graph_create(const dit_model* m, const float* mod_all, const void* txt,
                          float* latents, const double* sigmas_host, int n_steps,
                          const dit_fbcache* cache, void* workspace, size_t ws_bytes,
                          void* loop_state, size_t state_bytes, void* stream,
                          dit_loop_graph** out) {
  const char* fn = "dit_loop_graph_create";
  if (!out) return fail(DIT_ERR_INVALID_ARG, "%s: NULL out", fn);
  *out = nullptr;
  if (!m || !mod_all || !latents || !sigmas_host || !workspace || !loop_state ||
      (m->dims.Lt > 0 && !txt))
    return fail(DIT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (n_steps < 1) return fail(DIT_ERR_INVALID_ARG, "%s: n_steps %d < 1", fn, n_steps);
  Dims dm;
  int rc;
  if ((rc = check_model(m, &dm, fn))) return rc;
  for (int i = 0; i <= n_steps; ++i)
    if (!std::isfinite(sigmas_host[i])) return fail(DIT_ERR_INVALID_ARG, "%s: non-finite sigma", fn);
  if (!aligned16(mod_all) || !aligned16(latents) || !aligned16(workspace) ||
      !aligned16(loop_state) || (txt && !aligned16(txt)))
    return fail(DIT_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
  if ((rc = check_cache(cache, fn))) return rc;
  const size_t need = ws_size(dm, DIT_WS_STEP, 0);
  if (ws_bytes < need) return fail(DIT_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  const size_t need_state = dit_loop_state_bytes(m, n_steps);
  if (state_bytes < need_state)
    return fail(DIT_ERR_WORKSPACE, "%s: loop state %zu < %zu bytes", fn, state_bytes, need_state);
  if ((rc = check_device())) return rc;
  int dev = 0;
  DIT_CHECK_HIP(hipGetDevice(&dev));

  hipStream_t st = (hipStream_t)stream;
  Carver c{(char*)workspace, 0};
  const StepWS w = carve_step(c, dm);
  Carver cl{(char*)loop_state, 0};
  const LoopBufs lb = carve_loop(cl, n_mod_of(m), n_steps);
  const bool cache_on = cache && cache->enabled;
  DIT_CHECK_HIP(hipMemcpyAsync(lb.sig, sigmas_host, sizeof(double) * (n_steps + 1),
                               hipMemcpyHostToDevice, st));
  if ((rc = write_loop_state(lb.state, n_steps, 0, cache, st))) return rc;

  // capture one step on a private stream; nothing runs until the graph is launched
  hipStream_t cs = nullptr;
  DIT_CHECK_HIP(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  if (e == hipSuccess) {
    dit_kernel_timer* timer = g_timer;   // event records stay out of the graph
    g_timer = nullptr;
    e = enqueue_loop_step(m, dm, mod_all, txt, latents, cache_on ? cache->anchor : nullptr,
                          cache_on ? cache->cached : nullptr, cache_on, w, lb, cs);
    g_timer = timer;
    const hipError_t e2 = hipStreamEndCapture(cs, &graph);
    if (e == hipSuccess) e = e2;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (graph) (void)hipGraphDestroy(graph);
  (void)hipStreamDestroy(cs);
  if (e != hipSuccess)
    return fail(DIT_ERR_HIP, "%s: step capture failed: %s", fn, hipGetErrorString(e));
  dit_loop_graph* g = new (std::nothrow) dit_loop_graph;
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    return fail(DIT_ERR_INVALID_ARG, "%s: out of host memory", fn);
  }
  g->exec = exec;
  g->device = dev;
  g->n_steps = n_steps;
  g->launched = 0;
  g->cache_on = cache_on ? 1 : 0;
  g->anchor = cache_on ? cache->anchor : nullptr;
  g->cached = cache_on ? cache->cached : nullptr;
  g->state = lb.state;
  g->log = lb.log;
  *out = g;
  return DIT_OK;
}

int dit_loop_graph_run(dit_loop_graph* g, int n, void* stream) {
  if (!g || n < 0) return fail(DIT_ERR_INVALID_ARG, "dit_loop_graph_run: NULL graph or n < 0");
  if (g->launched + n > g->n_steps)
    return fail(DIT_ERR_INVALID_ARG, "dit_loop_graph_run: %d + %d replays exceed the %d steps",
                g->launched, n, g->n_steps);
  int dev = 0;
  DIT_CHECK_HIP(hipGetDevice(&dev));
  if (dev != g->device)
    return fail(DIT_ERR_INVALID_ARG, "dit_loop_graph_run: graph of device %d, current %d",
                g->device, dev);
  for (int i = 0; i < n; ++i) {
    DIT_CHECK_HIP(hipGraphLaunch(g->exec, (hipStream_t)stream));
    g->launched += 1;
  }
  return DIT_OK;
}

int dit_loop_graph_sync(dit_loop_graph* g, dit_fbcache* cache, dit_step_info* info, int n_info,
                        void* stream, int* steps_run) {
  if (!g || n_info < 0 || (n_info > 0 && !info))
    return fail(DIT_ERR_INVALID_ARG, "dit_loop_graph_sync: NULL graph or info");
  if (cache && (cache->enabled ? 1 : 0) != g->cache_on)
    return fail(DIT_ERR_INVALID_ARG, "dit_loop_graph_sync: cache enabled flag differs from create");
  hipStream_t st = (hipStream_t)stream;
  LoopState h;
  std::vector<LoopLog> log((size_t)g->n_steps);
  DIT_CHECK_HIP(hipMemcpyAsync(&h, g->state, sizeof(h), hipMemcpyDeviceToHost, st));
  DIT_CHECK_HIP(hipMemcpyAsync(log.data(), g->log, sizeof(LoopLog) * log.size(),
                               hipMemcpyDeviceToHost, st));
  DIT_CHECK_HIP(hipStreamSynchronize(st));
  const int done = h.next < g->n_steps ? h.next : g->n_steps;
  int nonfinite = 0;
  for (int i = 0; i < g->n_steps; ++i) {
    if (i < n_info) {
      info[i].rel = log[i].rel;
      info[i].skipped = log[i].skip;
    }
    if (i < done && log[i].nonfinite) nonfinite = 1;
  }
  if (steps_run) *steps_run = done;
  if (cache && g->cache_on) {
    cache->has_anchor = h.has_anchor;
    cache->steps_done = h.steps_done;
    cache->skip_run = h.skip_run;
  }
  if (nonfinite)
    return fail(DIT_ERR_NONFINITE, "dit_loop_graph_sync: a step met a non-finite residual");
  return DIT_OK;
}

int dit_loop_graph_reset(dit_loop_graph* g, const dit_fbcache* cache, int first_step,
                         void* stream) {
  const char* fn = "dit_loop_graph_reset";
  if (!g) return fail(DIT_ERR_INVALID_ARG, "%s: NULL graph", fn);
  if (first_step < 0 || first_step > g->n_steps)
    return fail(DIT_ERR_INVALID_ARG, "%s: first_step %d outside [0, %d]", fn, first_step,
                g->n_steps);
  const int on = cache && cache->enabled ? 1 : 0;
  if (on != g->cache_on || (on && (cache->anchor != g->anchor || cache->cached != g->cached)))
    return fail(DIT_ERR_INVALID_ARG, "%s: the cache must be the one the graph was created with", fn);
  int rc;
  if ((rc = check_cache(cache, fn))) return rc;
  if ((rc = write_loop_state(g->state, g->n_steps, first_step, cache, (hipStream_t)stream)))
    return rc;
  g->launched = first_step;
  return DIT_OK;
}

int dit_loop_graph_destroy(dit_loop_graph* g) {
  if (!g) return DIT_OK;
  const hipError_t e = hipGraphExecDestroy(g->exec);
  delete g;
  if (e != hipSuccess)
    return fail(DIT_ERR_HIP, "dit_loop_graph_destroy: %s", hipGetErrorString(e));
  return DIT_OK;
}

}  // extern "C"
