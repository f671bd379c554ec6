// bf16 MFMA GEMM with fused epilogues for the DiT block linears (gfx950).
//
//   C[m, n] = sum_k A[m, k] * W[n, k] + bias[n]      (A: activations, W: [out, in])
//
// One workgroup = 4 or 8 wave64s computing a BM x BN tile with
// v_mfma_f32_32x32x16_bf16.  K is staged through LDS 64 at a time,
// double-buffered, with the next slab's global loads in flight during the
// current slab's MFMAs.  Up to two problems (the image and text streams of a
// double block, each with its own weights) share one launch.
//
// Epilogue: each wave parks one 32-column slice of its accumulators in LDS at a
// time and reads it back row-wise (4 consecutive columns of one row per lane:
// coalesced stores, RoPE pairs in-register), then calls the fused
// epilogue functor; a pass wholly in bounds hands the functor all of a lane's rows
// at once, so the loads they need (RoPE entries, residual rows, gates) are in
// flight together.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dit {

constexpr int GEMM_BK = 64;
constexpr int GEMM_LDS = GEMM_BK + 8;   // padded LDS row (bf16 elements): 144 B
constexpr int EPI_LDS = 36;             // padded fp32 row of a parked 32-column slice

// ---------------------------------------------------------------- epilogues
// row4(r, c, v): v = C[r, c..c+3] (bias added), c % 4 == 0
// rows<NR>(r0, rs, c, v) (optional): v[i] = C[r0 + i rs, c..c+3] for i < NR, every
//   row in bounds and the calling wave's columns inside one tensor and head, so
//   branches on c agree across the wave; the functor issues all its loads before
//   its first store.  Returns the largest |stored value| (amax-tracking functors).

struct EpiStoreF32 {
  float* out; int ldo;
  __device__ __forceinline__ void row4(int r, int c, f32x4 v) const {
    *(f32x4*)(out + (size_t)r * ldo + c) = v;
  }
};

__device__ __forceinline__ void store_bf16x4(bf16_t* p, float a, float b, float c, float d) {
  uint2 u;
  u.x = pack_bf16x2(a, b);
  u.y = pack_bf16x2(c, d);
  *(uint2*)p = u;
}

struct EpiStoreBf16 {
  bf16_t* out; int ldo;
  __device__ __forceinline__ void row4(int r, int c, f32x4 v) const {
    store_bf16x4(out + (size_t)r * ldo + c, v[0], v[1], v[2], v[3]);
  }
};

struct EpiSiluBf16 {
  bf16_t* out; int ldo;
  __device__ __forceinline__ void row4(int r, int c, f32x4 v) const {
    store_bf16x4(out + (size_t)r * ldo + c, silu_f(v[0]), silu_f(v[1]), silu_f(v[2]), silu_f(v[3]));
  }
};

struct EpiGeluBf16 {
  bf16_t* out; int ldo; int col_off;
  __device__ __forceinline__ void row4(int r, int c, f32x4 v) const {
    store_bf16x4(out + (size_t)r * ldo + col_off + c, gelu_tanh_f(v[0]), gelu_tanh_f(v[1]),
                 gelu_tanh_f(v[2]), gelu_tanh_f(v[3]));
  }
};

// x[token] += gate[b] * v, x being the joint residual stream [B, L, D].
template <class XT>
struct EpiGatedResidual {
  XT* x; int D; const float* gate; int gate_bstride; RowMap map;
  __device__ __forceinline__ void row4(int r, int c, f32x4 v) const {
    int b, t; map.token(r, b, t);
    XT* p = x + ((size_t)b * map.L + t) * D + c;
    const f32x4 g = *(const f32x4*)(gate + (size_t)b * gate_bstride + c);
    if constexpr (sizeof(XT) == 4) {
      f32x4 o = *(f32x4*)p;
      *(f32x4*)p = o + g * v;
    } else {
      uint2 u = *(uint2*)p;
      float o0 = __uint_as_float(u.x << 16), o1 = __uint_as_float(u.x & 0xffff0000u);
      float o2 = __uint_as_float(u.y << 16), o3 = __uint_as_float(u.y & 0xffff0000u);
      store_bf16x4((bf16_t*)p, o0 + g[0] * v[0], o1 + g[1] * v[1], o2 + g[2] * v[2],
                   o3 + g[3] * v[3]);
    }
  }
  template <int NR>
  __device__ __forceinline__ float rows(int r0, int rs, int c, const f32x4 (&v)[NR]) const {
    XT* p[NR];
    f32x4 g[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      int b, t; map.token(r0 + i * rs, b, t);
      p[i] = x + ((size_t)b * map.L + t) * D + c;
      g[i] = *(const f32x4*)(gate + (size_t)b * gate_bstride + c);
    }
    if constexpr (sizeof(XT) == 4) {
      f32x4 o[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) o[i] = *(const f32x4*)p[i];
#pragma unroll
      for (int i = 0; i < NR; ++i) *(f32x4*)p[i] = o[i] + g[i] * v[i];
    } else {
      uint2 u[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) u[i] = *(const uint2*)p[i];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const float o0 = __uint_as_float(u[i].x << 16), o1 = __uint_as_float(u[i].x & 0xffff0000u);
        const float o2 = __uint_as_float(u[i].y << 16), o3 = __uint_as_float(u[i].y & 0xffff0000u);
        store_bf16x4((bf16_t*)p[i], o0 + g[i][0] * v[i][0], o1 + g[i][1] * v[i][1],
                     o2 + g[i][2] * v[i][2], o3 + g[i][3] * v[i][3]);
      }
    }
    return 0.f;
  }
};

// Epilogues that also report the largest magnitude they stored, per slot
// (kTrackAmax): row4 returns the largest |value| before the store's rounding,
// slot(r, c) names the slot of an output (-1: not tracked) and stored(slot, m)
// applies that slot's rounding (round-to-nearest is monotonic, so rounding the
// largest magnitude gives the largest stored magnitude).  The kernel folds these
// into amax[slot] with an atomic max of the fp32 bit patterns (non-negative values
// order like their bits).
template <class E, class = void> struct TracksAmax : std::false_type {};
template <class E>
struct TracksAmax<E, std::void_t<decltype(E::kTrackAmax)>> : std::bool_constant<E::kTrackAmax> {};

template <class E>
__device__ __forceinline__ unsigned int* amax_of(const E& e) {
  if constexpr (TracksAmax<E>::value) return e.amax_ptr();
  else return nullptr;
}

// One output's magnitude m straight into amax[sl] (tiles whose wave spans slots).
template <class Epi>
__device__ __forceinline__ void track_amax(const Epi& epi, int sl, float m, unsigned int* amax) {
  if (sl >= 0 && amax) atomicMax(amax + sl, __float_as_uint(epi.stored(sl, m)));
}

__device__ __forceinline__ float amax4(float a, float b, float c, float d) {
  return fmaxf(fmaxf(fabsf(a), fabsf(b)), fmaxf(fabsf(c), fabsf(d)));
}

template <class E, class = void> struct HasRows : std::false_type {};
template <class E>
struct HasRows<E, std::void_t<decltype(&E::template rows<1>)>> : std::true_type {};

// NR in-bounds rows r0 + i rs through the functor's rows() if it has one, else row4
// one row at a time; the largest |stored value| when the functor tracks it.
template <int NR, class Epi>
__device__ __forceinline__ float epi_rows(const Epi& e, int r0, int rs, int c, const f32x4 (&v)[NR]) {
  if constexpr (HasRows<Epi>::value) {
    return e.template rows<NR>(r0, rs, c, v);
  } else {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if constexpr (TracksAmax<Epi>::value) m = fmaxf(m, e.row4(r0 + i * rs, c, v[i]));
      else e.row4(r0 + i * rs, c, v[i]);
    }
    return m;
  }
}

// Split the fused projection into head-major Q, K (rotated) and V, all bf16
// [B, H, L, d].  AMAX: the largest stored magnitude of every (tensor, b, h) is
// gathered too into amax [3, B, H] (q, k, v: the per-head e4m3 scales of the
// fp8 path).
template <bool AMAX>
struct EpiQKVT {
  static constexpr bool kTrackAmax = AMAX;
  bf16_t* q; bf16_t* k; bf16_t* v; const float* rope;  // rope: [L, d/2, 2] (cos, sin)
  int D, H, d; RowMap map;
  unsigned int* amax;
  __device__ __forceinline__ unsigned int* amax_ptr() const { return amax; }
  __device__ __forceinline__ int slot(int r, int c) const {
    const int which = c / D;
    const int h = (c - which * D) / d;
    int b, t; map.token(r, b, t);
    return (which * map.B + b) * H + h;
  }
  // The slot shared by rows [r0, r1] at column c, or -2 when they span several.
  // Within the image rows and within the text rows the batch index never
  // decreases, so equal end slots on one side of that split cover the range.
  __device__ __forceinline__ int slot_span(int r0, int r1, int c) const {
    const int s0 = slot(r0, c);
    if (s0 != slot(r1, c)) return -2;
    if (map.stream_major) {
      const int ni = map.B * map.Li;
      if ((r0 + map.base < ni) != (r1 + map.base < ni)) return -2;
    }
    return s0;
  }
  __device__ __forceinline__ float row4(int r, int c, f32x4 x) const {
    const int which = c / D;
    const int cc = c - which * D;
    const int h = cc / d;
    const int dd = cc - h * d;
    int b, t; map.token(r, b, t);
    const size_t bh = (size_t)b * H + h;
    bf16_t* dst = (which == 0 ? q : which == 1 ? k : v) + (bh * map.L + t) * d + dd;
    if (which == 2) {
      store_bf16x4(dst, x[0], x[1], x[2], x[3]);
      return amax4(x[0], x[1], x[2], x[3]);
    }
    // pairs (dd, dd+1) and (dd+2, dd+3): table entries p = dd/2 and dd/2 + 1
    const f32x4 cs = *(const f32x4*)(rope + ((size_t)t * (d >> 1) + (dd >> 1)) * 2);
    const float o0 = x[0] * cs[0] - x[1] * cs[1];
    const float o1 = x[0] * cs[1] + x[1] * cs[0];
    const float o2 = x[2] * cs[2] - x[3] * cs[3];
    const float o3 = x[2] * cs[3] + x[3] * cs[2];
    store_bf16x4(dst, o0, o1, o2, o3);
    return amax4(o0, o1, o2, o3);
  }
  // the rows' tokens (and RoPE entries for Q, K) first, then the stores
  template <int NR>
  __device__ __forceinline__ float rows(int r0, int rs, int c, const f32x4 (&x)[NR]) const {
    const int which = c / D;
    const int cc = c - which * D;
    const int h = cc / d;
    const int dd = cc - h * d;
    bf16_t* const base = which == 0 ? q : which == 1 ? k : v;
    bf16_t* dst[NR];
    int tok[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      int b, t; map.token(r0 + i * rs, b, t);
      dst[i] = base + (((size_t)b * H + h) * map.L + t) * d + dd;
      tok[i] = t;
    }
    float m = 0.f;
    if (which == 2) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        store_bf16x4(dst[i], x[i][0], x[i][1], x[i][2], x[i][3]);
        m = fmaxf(m, amax4(x[i][0], x[i][1], x[i][2], x[i][3]));
      }
      return m;
    }
    f32x4 cs[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i)
      cs[i] = *(const f32x4*)(rope + ((size_t)tok[i] * (d >> 1) + (dd >> 1)) * 2);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float o0 = x[i][0] * cs[i][0] - x[i][1] * cs[i][1];
      const float o1 = x[i][0] * cs[i][1] + x[i][1] * cs[i][0];
      const float o2 = x[i][2] * cs[i][2] - x[i][3] * cs[i][3];
      const float o3 = x[i][2] * cs[i][3] + x[i][3] * cs[i][2];
      store_bf16x4(dst[i], o0, o1, o2, o3);
      m = fmaxf(m, amax4(o0, o1, o2, o3));
    }
    return m;
  }
  // every slot stores bf16
  __device__ __forceinline__ float stored(int, float m) const { return bf2f(f2bf(m)); }
};

using EpiQKV = EpiQKVT<false>;

// Single-stream linear1: columns [0, 3D) are Q/K/V, the rest the GELU MLP branch.
template <bool AMAX>
struct EpiLinear1T {
  static constexpr bool kTrackAmax = AMAX;
  EpiQKVT<AMAX> qkv; EpiGeluBf16 gelu; int n_qkv;
  __device__ __forceinline__ unsigned int* amax_ptr() const { return qkv.amax; }
  __device__ __forceinline__ int slot(int r, int c) const { return c < n_qkv ? qkv.slot(r, c) : -1; }
  __device__ __forceinline__ int slot_span(int r0, int r1, int c) const {
    return c < n_qkv ? qkv.slot_span(r0, r1, c) : -1;
  }
  __device__ __forceinline__ float row4(int r, int c, f32x4 v) const {
    if (c < n_qkv) return qkv.row4(r, c, v);
    gelu.row4(r, c - n_qkv, v);
    return 0.f;
  }
  template <int NR>
  __device__ __forceinline__ float rows(int r0, int rs, int c, const f32x4 (&v)[NR]) const {
    if (c < n_qkv) return qkv.template rows<NR>(r0, rs, c, v);
#pragma unroll
    for (int i = 0; i < NR; ++i) gelu.row4(r0 + i * rs, c - n_qkv, v[i]);
    return 0.f;
  }
  __device__ __forceinline__ float stored(int slot, float m) const { return qkv.stored(slot, m); }
};
using EpiLinear1 = EpiLinear1T<false>;

// ---------------------------------------------------------------- kernel

template <class Epi>
struct GemmParams {
  GemmProblem g[2];
  Epi e[2];
  int ngroups;
  int tiles[2];     // tiles per group
  int tiles_n[2];   // n-tiles per group
  const int* gate;  // launch gate (nullptr: always run)
  // tiled kernel: the groups' tiles as one grid of grid_m x grid_n (group 1's rows
  // after split_m), cut into `bands` row bands (0: per-group raster instead)
  int grid_m, grid_n, split_m, bands;
};

// Logical tile lid -> (row, column) of a grid_m x grid_n tile grid cut into
// P row bands x Q = min(8 / P, grid_n) column bands, visited region by region.
// The 8 XCDs each receive a contiguous run of logical tiles, so each one works
// through one compact region and streams the A rows and W columns of that region
// only (an XCD's L2 is its own).  Inside a region: columns of up to 16 rows, or
// for taller regions groups of 8 rows sweeping the region's columns, so the 32
// tiles an XCD runs at once share their operand blocks.
__device__ __forceinline__ void grid_tile(int lid, int grid_m, int grid_n, int P, int& tm,
                                          int& tn) {
  const int Q = min(8 / P, grid_n);
  tm = tn = 0;
  for (int c = 0; c < Q; ++c)
    for (int r = 0; r < P; ++r) {
      const int r0 = grid_m * r / P, r1 = grid_m * (r + 1) / P;
      const int c0 = grid_n * c / Q, c1 = grid_n * (c + 1) / Q;
      const int h = r1 - r0, w = c1 - c0;
      if (lid < h * w) {
        if (h <= 16) {
          tm = r0 + lid % h;
          tn = c0 + lid / h;
        } else {
          const int in_group = 8 * w, first = (lid / in_group) * 8;
          const int gsize = min(h - first, 8);
          tm = r0 + first + (lid % in_group) % gsize;
          tn = c0 + (lid % in_group) / gsize;
        }
        return;
      }
      lid -= h * w;
    }
}

template <int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(GemmParams<Epi> p) {
  if (gate_closed(p.gate)) return;
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM / 32;
  constexpr int TN = BN / WN / 32;
  constexpr int RPP = NT / 8;       // slab rows covered per pass (8 threads per 128-B row)
  constexpr int AIT = BM / RPP;     // 16-byte loads per thread for the A slab
  constexpr int BIT = BN / RPP;
  constexpr int WROWS = BM / WM;    // rows of one wave's tile
  static_assert(AIT * RPP == BM && BIT * RPP == BN, "tile / thread mismatch");
  static_assert(WM * WN * WROWS * EPI_LDS * 4 <= 2 * (BM + BN) * GEMM_LDS * 2,
                "epilogue slice does not fit in the operand LDS");
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BM + BN) * GEMM_LDS];
  bf16_t* sA = smem;                         // [2][BM * GEMM_LDS]
  bf16_t* sB = smem + 2 * BM * GEMM_LDS;     // [2][BN * GEMM_LDS]

  // XCD-aware order: the hardware deals workgroups round-robin over 8 XCDs;
  // give each XCD a contiguous range of logical tiles so neighbours share L2.
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int xq = nblk >> 3, xr = nblk & 7, xcd = bid & 7;
  int lid = xcd * xq + min(xcd, xr) + (bid >> 3);

  const bool g1 = p.ngroups > 1 && lid >= p.tiles[0];
  if (g1) lid -= p.tiles[0];
  const GemmProblem g = g1 ? p.g[1] : p.g[0];
  const int tiles_n = g1 ? p.tiles_n[1] : p.tiles_n[0];
  const int tiles_m = (g.M + BM - 1) / BM;

  // grouped raster: 8 m-tiles sweep the n-tiles together
  constexpr int GROUP_M = 8;
  const int in_group = GROUP_M * tiles_n;
  const int gid = lid / in_group;
  const int first_m = gid * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int tm_idx = first_m + (lid % in_group) % gsize;
  const int tn_idx = (lid % in_group) / gsize;
  const int m0 = tm_idx * BM;
  const int n0 = tn_idx * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // global -> register staging: thread covers row (tid/8) + RPP*i, 16-byte chunk tid%8
  const int lrow = tid >> 3;
  const int lchk = (tid & 7) * 8;
  const bf16_t* gA[AIT];
  const bf16_t* gW[BIT];
#pragma unroll
  for (int i = 0; i < AIT; ++i) {
    int m = min(m0 + lrow + RPP * i, g.M - 1);
    gA[i] = g.A + (size_t)m * g.lda + lchk;
  }
#pragma unroll
  for (int i = 0; i < BIT; ++i) {
    int n = min(n0 + lrow + RPP * i, g.N - 1);
    gW[i] = g.W + (size_t)n * g.ldw + lchk;
  }
  i32x4 ra[AIT], rb[BIT];

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = g.K / GEMM_BK;
  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  const int wrow = wm * WROWS;
  const int wcol = wn * (BN / WN);

#define GEMM_GLOAD(kt)                                                           \
  {                                                                              \
    const int ko_ = (kt) * GEMM_BK;                                              \
    _Pragma("unroll") for (int i = 0; i < AIT; ++i) ra[i] = *(const i32x4*)(gA[i] + ko_); \
    _Pragma("unroll") for (int i = 0; i < BIT; ++i) rb[i] = *(const i32x4*)(gW[i] + ko_); \
  }
#define GEMM_SSTORE(s)                                                           \
  {                                                                              \
    bf16_t* a_ = sA + (s) * BM * GEMM_LDS;                                       \
    bf16_t* b_ = sB + (s) * BN * GEMM_LDS;                                       \
    _Pragma("unroll") for (int i = 0; i < AIT; ++i)                              \
        *(i32x4*)&a_[(lrow + RPP * i) * GEMM_LDS + lchk] = ra[i];                \
    _Pragma("unroll") for (int i = 0; i < BIT; ++i)                              \
        *(i32x4*)&b_[(lrow + RPP * i) * GEMM_LDS + lchk] = rb[i];                \
  }

  GEMM_GLOAD(0);
  GEMM_SSTORE(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt & 1;
    if (kt + 1 < nk) GEMM_GLOAD(kt + 1);
    const bf16_t* a_s = sA + s * BM * GEMM_LDS;
    const bf16_t* b_s = sB + s * BN * GEMM_LDS;
#pragma unroll
    for (int kk = 0; kk < GEMM_BK / 16; ++kk) {
      bf16x8 af[TM], bw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const bf16x8*)&a_s[(wrow + i * 32 + frow) * GEMM_LDS + kk * 16 + fk];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bw[j] = *(const bf16x8*)&b_s[(wcol + j * 32 + frow) * GEMM_LDS + kk * 16 + fk];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bw[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) GEMM_SSTORE(s ^ 1);
    __syncthreads();
  }
#undef GEMM_GLOAD
#undef GEMM_SSTORE

  // ---- epilogue (the loop above ended with a barrier: operand LDS is free)
  const Epi epi = g1 ? p.e[1] : p.e[0];
  float* slice = (float*)smem + wave * WROWS * EPI_LDS;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    // accumulator element e of block (i, j): row i*32 + (e/4)*8 + (lane/32)*4 + e%4,
    // column lane%32 of the slice
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        slice[(i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3)) * EPI_LDS + (lane & 31)] =
            acc[i][j][e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int cbase = n0 + wcol + j * 32;
    // 8 lanes per row, 4 columns each
#pragma unroll
    for (int ps = 0; ps < WROWS / 8; ++ps) {
      const int rl = ps * 8 + (lane >> 3);
      const int cl = (lane & 7) * 4;
      const int row = m0 + wrow + rl;
      const int col = cbase + cl;
      if (row < g.M && col < g.N) {
        f32x4 v = *(const f32x4*)&slice[rl * EPI_LDS + cl];
        if (g.bias) v += *(const f32x4*)(g.bias + col);
        epi.row4(row, col, v);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Tiled kernel whose LDS image is written 1 KB per wave instruction: 64 lanes x
// 16 B contiguously, so a permuted (or padded) row layout is built by giving every
// lane the global chunk that belongs at its LDS slot: 8 lanes still cover one
// 128-byte row segment.  (Padded rows re-read the row's last chunk into the pad.)
// e4m3 operands (and bf16 with more than two stages) use gfx950's direct
// global->LDS loads (global_load_lds_dwordx4), with no staging registers; bf16 and
// MXFP4 with two stages load the same chunks into registers (global_load_dwordx4)
// and write them with ds_write_b128, which lets the fragment reads run ahead of
// the MFMAs with exact waits (measured 3-6% faster on the bf16 block shapes and
// 1.5-4.5% on the MXFP4 ones; for e4m3 it measured slower).
//
// Pipeline: NS stages, each holding a K slab of SLAB bytes per row for the A and
// the W tile (SLAB / 2 bf16 or SLAB e4m3 values), so NS - 1 slabs are in flight
// while one is consumed; every stage is its own LDS object so the loads into
// one never order the reads of another.
//
// FMT 1 (e4m3): operands are OCP e4m3 with per-row (A) and per-column (W) scales;
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales) takes 32 bytes of K per
// lane; the epilogue dequantises with sa[row] * sw[col].
// FMT 2 (MXFP4): operands are E2M1 codes with an E8M0 scale per 32 K values; a
// 128-byte slab is 256 K values, and the slab's scales (8 bytes per row) travel
// with it into a 4-KB tail of the stage.  The same MFMA with E2M1 operands takes
// 16 bytes (32 K values, one block) per lane and the lane's block scale, picked by
// the opsel byte index from a word holding its 4 blocks of the slab.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);   // expcnt, lgkmcnt at max
}

// Epilogue of the direct-to-LDS kernels: a wave parks its accumulators, 32
// columns by PR = WROWS / EH rows at a time, in its LDS slice, then hands
// row-contiguous quads to the epilogue functor (dequantised first for e4m3).
// Accumulator element e of block (i, j) is row i*32 + (e/4)*8 + (lane/32)*4 + e%4,
// column j*32 + lane%32 of the wave's tile.
template <int BN, int WN, int TM, int TN, int WROWS, int EH, bool F8, class Epi>
__device__ __forceinline__ void dma_epilogue(const GemmProblem& g, const Epi& epi,
                                             f32x16 (&acc)[TM][TN], float* slice, int m0, int n0,
                                             int wrow, int wcol, int lane) {
  constexpr int PR = WROWS / EH;
  constexpr bool kAmax = TracksAmax<Epi>::value;
  unsigned int* const amax_p = amax_of(epi);
  // A wave's BN / WN = 64 columns start on a multiple of 64, so with head size and
  // tensor widths multiples of 64 they lie in one tracked tensor and head (or in
  // none); its rows usually lie in one batch row.  Then one slot covers the wave's
  // whole tile and the lanes only keep a running max; otherwise every output goes
  // to memory at once.
  float am = 0.f;
  int aslot = -1;
  bool one_slot = false;
  if constexpr (kAmax) {
    static_assert(BN / WN == 64, "amax tracking assumes 64-column wave tiles");
    const int r_lo = min(m0 + wrow, g.M - 1), r_hi = min(m0 + wrow + WROWS - 1, g.M - 1);
    aslot = epi.slot_span(r_lo, r_hi, min(n0 + wcol, g.N - 1));
    one_slot = aslot != -2;
  }
#pragma clang loop unroll(full)
  for (int j = 0; j < TN; ++j) {
#pragma unroll
    for (int h = 0; h < EH; ++h) {
#pragma unroll
      for (int i = 0; i < TM / EH; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          slice[(i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3)) * EPI_LDS + (lane & 31)] =
              acc[h * (TM / EH) + i][j][e];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int cbase = n0 + wcol + j * 32;
      const int rbase = m0 + wrow + h * PR;
      // every row and column of this pass in bounds (and one amax slot, if tracked):
      // the functor gets all PR / 8 rows of a lane at once, with no branch between
      // them, so their loads are issued together
      const bool whole = rbase + PR <= g.M && cbase + 32 <= g.N && (!kAmax || one_slot);
      if (whole) {
        const int cl = (lane & 7) * 4;
        const int col = cbase + cl;
        const int row0 = rbase + (lane >> 3);
        f32x4 v[PR / 8];
#pragma unroll
        for (int ps = 0; ps < PR / 8; ++ps) {
          v[ps] = *(const f32x4*)&slice[(ps * 8 + (lane >> 3)) * EPI_LDS + cl];
          if constexpr (F8) v[ps] *= *(const f32x4*)(g.sw + col) * g.sa[row0 + ps * 8];
        }
        if (g.bias) {
          const f32x4 bv = *(const f32x4*)(g.bias + col);
#pragma unroll
          for (int ps = 0; ps < PR / 8; ++ps) v[ps] += bv;
        }
        // e4m3: two batches of rows (a single batch of 8 spills next to the 128 accumulators)
        constexpr int NB = F8 ? 2 : 1, NRB = PR / 8 / NB;
#pragma unroll
        for (int bt = 0; bt < NB; ++bt) {
          f32x4 vb[NRB];
#pragma unroll
          for (int i = 0; i < NRB; ++i) vb[i] = v[bt * NRB + i];
          const float m = epi_rows<NRB>(epi, row0 + bt * NRB * 8, 8, col, vb);
          if constexpr (kAmax) am = fmaxf(am, m);
        }
      } else {
#pragma unroll
        for (int ps = 0; ps < PR / 8; ++ps) {
          const int rl = ps * 8 + (lane >> 3);
          const int cl = (lane & 7) * 4;
          const int row = rbase + rl;
          const int col = cbase + cl;
          if (row < g.M && col < g.N) {
            f32x4 v = *(const f32x4*)&slice[rl * EPI_LDS + cl];
            if constexpr (F8) v *= *(const f32x4*)(g.sw + col) * g.sa[row];
            if (g.bias) v += *(const f32x4*)(g.bias + col);
            if constexpr (kAmax) {
              const float m = epi.row4(row, col, v);
              if (one_slot) am = fmaxf(am, m);
              else track_amax(epi, epi.slot(row, col), m, amax_p);
            } else {
              epi.row4(row, col, v);
            }
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  if constexpr (kAmax) {
    if (amax_p && one_slot && aslot >= 0) {   // one atomic per wave
      float m = am;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (lane == 0) atomicMax(amax_p + aslot, __float_as_uint(epi.stored(aslot, m)));
    }
  }
}

template <int KK>
__device__ __forceinline__ f32x16 mfma_mx4(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, KK, sa, KK, sb);
}

template <int BM, int BN, int WM, int WN, int FMT, int NS, int SLAB, class Epi>
__global__ __launch_bounds__(WM * WN * 64) void gemm_dma_kernel(GemmParams<Epi> p) {
  if (gate_closed(p.gate)) return;
  constexpr bool F8 = FMT == 1, F4 = FMT == 2;
  // bf16 and MXFP4 with two stages: global loads staged through registers and
  // written to LDS by the waves (see below); e4m3: direct-to-LDS loads
  constexpr bool VS = (FMT == 0 || FMT == 2) && NS == 2;
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32;
  constexpr int TN = BN / WN / 32;
  constexpr int WROWS = BM / WM;
  // 128-byte slabs: unpadded rows whose 16-byte chunks are permuted by
  // chunk ^ ((row >> 1) & 7), so the 16 consecutive rows that one LDS read cycle
  // serves at one chunk hit 16 distinct bank groups; other slab widths pad each
  // row by 16 bytes for the same effect
  constexpr bool SWZ = SLAB == 128;
  constexpr int ROWB = SWZ ? SLAB : SLAB + 16;  // LDS row pitch (bytes)
  constexpr int CPR = ROWB / 16;              // 16-byte chunks per LDS row
  constexpr int AB = BM * ROWB, BB = BN * ROWB, SB = AB + BB;
  constexpr int SXB = F4 ? (BM + BN) * 8 : 0; // MX block scales of a slab
  constexpr int NI = SB / 1024;               // 1-KB load instructions per stage
  constexpr int IPW = NI / NW;
  constexpr int EH = SWZ ? 2 : 1;             // epilogue passes over a wave's rows
  constexpr int PR = WROWS / EH;              // rows parked per pass
  constexpr int SLICE = PR * EPI_LDS * 4;     // bytes of one wave's parked epilogue slice
  constexpr int WPS = SB / SLICE;             // epilogue slices per stage
  static_assert(NS >= 2 && NS <= 4, "2..4 stages");
  static_assert(AB % 1024 == 0 && BB % 1024 == 0 && NI % NW == 0, "stage / wave mismatch");
  static_assert(WPS * NS >= NW, "epilogue slices must fit the stages");
  static_assert(SLAB % (F8 ? 64 : 32) == 0, "slab holds whole MFMA K steps");
  static_assert(!F4 || (SLAB == 128 && NS == 2 && BM == 256 && BN == 256 && NW >= 4),
                "MX operands: 128-byte slabs, two stages, 256 x 256 tiles");
  static_assert(SWZ || ROWB % 32 == 16, "row pitch: an odd number of 16-byte chunks");
  __shared__ __attribute__((aligned(1024))) char st0[SB + SXB];
  __shared__ __attribute__((aligned(1024))) char st1[SB + SXB];
  __shared__ __attribute__((aligned(1024))) char st2[NS > 2 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) char st3[NS > 3 ? SB : 16];
  auto stage = [&](int s) -> char* {
    return s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : st3;
  };

  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int xq = nblk >> 3, xr = nblk & 7, xcd = bid & 7;
  int lid = xcd * xq + min(xcd, xr) + (bid >> 3);
  bool g1;
  int m0, n0;
  if (p.bands > 0) {
    int tm, tn;
    grid_tile(lid, p.grid_m, p.grid_n, p.bands, tm, tn);
    g1 = tm >= p.split_m;
    m0 = (g1 ? tm - p.split_m : tm) * BM;
    n0 = tn * BN;
  } else {
    g1 = p.ngroups > 1 && lid >= p.tiles[0];
    if (g1) lid -= p.tiles[0];
    const int tiles_n = g1 ? p.tiles_n[1] : p.tiles_n[0];
    const int tiles_m = ((g1 ? p.g[1] : p.g[0]).M + BM - 1) / BM;
    constexpr int GROUP_M = 8;
    const int in_group = GROUP_M * tiles_n;
    const int first_m = (lid / in_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    m0 = (first_m + (lid % in_group) % gsize) * BM;
    n0 = ((lid % in_group) / gsize) * BN;
  }
  const GemmProblem g = g1 ? p.g[1] : p.g[0];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // byte offset of every lane's source chunk for each of this wave's load
  // instructions (an instruction lies wholly in the A or the B part of a stage)
  constexpr int ES = F8 ? 1 : 2;                    // element bytes (e4m3, bf16)
  const char* abase = F4 ? (const char*)g.A4 : F8 ? (const char*)g.A8 : (const char*)g.A;
  const char* wbase = F4 ? (const char*)g.W4 : F8 ? (const char*)g.W8 : (const char*)g.W;
  const int apitch = F4 ? g.lda / 2 : g.lda * ES;   // row pitch in bytes
  const int wpitch = F4 ? g.ldw / 2 : g.ldw * ES;
  int voff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int off = (wave * IPW + j) * 1024 + lane * 16;
    const bool isb = (wave * IPW + j) * 1024 >= AB;
    const int o2 = isb ? off - AB : off;
    const int row = o2 / ROWB;
    const int slot = SWZ ? ((o2 - row * ROWB) >> 4) ^ ((row >> 1) & 7)
                         : min((o2 - row * ROWB) >> 4, CPR - 2);
    voff[j] = isb ? min(n0 + row, g.N - 1) * wpitch + slot * 16
                  : min(m0 + row, g.M - 1) * apitch + slot * 16;
  }
  // MX scales: waves 0, 1 load the A tile's 256 rows x 8 bytes of a slab, waves 2, 3
  // the W tile's, 1 KB each (the scale arrays are padded to 256-row multiples)
  const uint8_t* xsrc = nullptr;
  if constexpr (F4) {
    if (wave < 4)
      xsrc = wave < 2 ? g.xa + ((size_t)m0 + wave * 128) * 8 + lane * 16
                      : g.xw + ((size_t)n0 + (wave - 2) * 128) * 8 + lane * 16;
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = F4 ? g.K / 256 : g.K * ES / SLAB;  // K slabs
  const int xstride = (wave < 2 ? g.pad_m : g.pad_n) * 8;   // bytes of MX scales per slab
  const int frow = lane & 31;
  const int wrow = wm * WROWS;
  const int wcol = wn * (BN / WN);
  // byte offset within an LDS row of the 16-byte chunk c of a fragment row: bf16
  // lanes 32..63 take the row's next chunk (K 8..15 of a 16-deep step), fp8 lanes
  // the next pair of chunks (K 32..63 of a 64-deep step); the fragment rows of a
  // lane are frow + multiples of 32, so their swizzle is (frow >> 1) & 7
  const int hi = lane >> 5, swz = SWZ ? (frow >> 1) & 7 : 0;
  auto xo = [&](int c) { return ((c + hi) ^ swz) << 4; };
  auto xo8 = [&](int c) { return ((c + 2 * hi) ^ swz) << 4; };

#define GEMM_DMA(stg, kt)                                                                \
  {                                                                                      \
    const int ko_ = (kt) * SLAB;                                                         \
    _Pragma("unroll") for (int j = 0; j < IPW; ++j) {                                   \
      const char* b_ = ((wave * IPW + j) * 1024 >= AB) ? wbase : abase;                  \
      __builtin_amdgcn_global_load_lds((const void*)(b_ + voff[j] + ko_),            \
                                       (void*)((stg) + (wave * IPW + j) * 1024), 16, 0, 0); \
    }                                                                                    \
    if constexpr (F4) {                                                                  \
      if (wave < 4)                                                                      \
        __builtin_amdgcn_global_load_lds((const void*)(xsrc + (size_t)(kt) * xstride),   \
                                         (void*)((stg) + SB + wave * 1024), 16, 0, 0);   \
    }                                                                                    \
  }
  // bf16: 16-deep K steps (32 bytes of a row); the fragments of step kk+1 are
  // read while the MFMAs of step kk run
#define GEMM_COMPUTE(stg)                                                                \
  {                                                                                      \
    const char* a_s = (const char*)(stg);                                                \
    const char* b_s = (const char*)(stg) + AB;                                           \
    constexpr int KS = SLAB / 32;                                                        \
    bf16x8 af[2][TM], bw[2][TN];                                                         \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
        af[0][i] = *(const bf16x8*)(a_s + (wrow + i * 32 + frow) * ROWB + xo(0));        \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                       \
        bw[0][j] = *(const bf16x8*)(b_s + (wcol + j * 32 + frow) * ROWB + xo(0));        \
    _Pragma("unroll") for (int kk = 0; kk < KS; ++kk) {                                 \
      const int cb = kk & 1, nb = cb ^ 1;                                                \
      if (kk + 1 < KS) {                                                                 \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                   \
            af[nb][i] = *(const bf16x8*)(a_s + (wrow + i * 32 + frow) * ROWB + xo(2 * kk + 2)); \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
            bw[nb][j] = *(const bf16x8*)(b_s + (wcol + j * 32 + frow) * ROWB + xo(2 * kk + 2)); \
      }                                                                                  \
      _Pragma("unroll") for (int i = 0; i < TM; ++i)                                     \
          _Pragma("unroll") for (int j = 0; j < TN; ++j)                                 \
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][i], bw[cb][j], acc[i][j], 0, 0, 0); \
    }                                                                                    \
    /* keep the fragment reads of step kk + 1 interleaved with step kk's MFMAs */       \
    if constexpr (VS) {                                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);                          \
      _Pragma("unroll") for (int kk = 0; kk < KS - 1; ++kk) {                           \
        _Pragma("unroll") for (int r = 0; r < TM + TN; ++r) {                           \
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                            \
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                            \
        }                                                                                \
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);             \
      }                                                                                  \
      __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);                          \
    }                                                                                    \
  }
  // fp8: 64-deep K steps, 32 bytes of K per lane (two 16-byte reads)
#define GEMM_COMPUTE_F8(stg)                                                             \
  {                                                                                      \
    const char* a_s = (const char*)(stg);                                                \
    const char* b_s = (const char*)(stg) + AB;                                           \
    _Pragma("unroll") for (int kk = 0; kk < SLAB / 64; ++kk) {                          \
      i32x8 af[TM], bw[TN];                                                              \
      _Pragma("unroll") for (int i = 0; i < TM; ++i) {                                   \
        const char* q_ = a_s + (wrow + i * 32 + frow) * ROWB;                            \
        const i32x4 lo_ = *(const i32x4*)(q_ + xo8(4 * kk)),                             \
                    hi_ = *(const i32x4*)(q_ + xo8(4 * kk + 1));                         \
        af[i] = i32x8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};     \
      }                                                                                  \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                   \
        const char* q_ = b_s + (wcol + j * 32 + frow) * ROWB;                            \
        const i32x4 lo_ = *(const i32x4*)(q_ + xo8(4 * kk)),                             \
                    hi_ = *(const i32x4*)(q_ + xo8(4 * kk + 1));                         \
        bw[j] = i32x8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};     \
      }                                                                                  \
      _Pragma("unroll") for (int i = 0; i < TM; ++i)                                     \
          _Pragma("unroll") for (int j = 0; j < TN; ++j)                                 \
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(               \
                  af[i], bw[j], acc[i][j], 0, 0, 0, 127, 0, 127);                        \
    }                                                                                    \
  }

  // MXFP4: four 64-deep K steps per slab, 16 bytes (one 32-value block) per lane;
  // the lane's scale word holds its blocks 2 kk + hi for kk = 0..3, byte kk
#define GEMM_MX4_STEP(KK)                                                                \
  {                                                                                      \
    i32x8 af[TM], bw[TN];                                                                \
    _Pragma("unroll") for (int i = 0; i < TM; ++i) {                                     \
      const i32x4 v_ = *(const i32x4*)(a_s + (wrow + i * 32 + frow) * ROWB + xo(2 * KK)); \
      af[i] = i32x8{v_[0], v_[1], v_[2], v_[3], 0, 0, 0, 0};                               \
    }                                                                                    \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                     \
      const i32x4 v_ = *(const i32x4*)(b_s + (wcol + j * 32 + frow) * ROWB + xo(2 * KK)); \
      bw[j] = i32x8{v_[0], v_[1], v_[2], v_[3], 0, 0, 0, 0};                               \
    }                                                                                    \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
            acc[i][j] = mfma_mx4<KK>(af[i], bw[j], acc[i][j], sa_[i], sb_[j]);            \
  }
#define GEMM_COMPUTE_F4(stg)                                                             \
  {                                                                                      \
    const char* a_s = (const char*)(stg);                                                \
    const char* b_s = (const char*)(stg) + AB;                                           \
    const char* x_s = (const char*)(stg) + SB;                                           \
    int sa_[TM], sb_[TN];                                                                \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
        sa_[i] = *(const int*)(x_s + (wrow + i * 32 + frow) * 8 + hi * 4);               \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                       \
        sb_[j] = *(const int*)(x_s + BM * 8 + (wcol + j * 32 + frow) * 8 + hi * 4);      \
    GEMM_MX4_STEP(0) GEMM_MX4_STEP(1) GEMM_MX4_STEP(2) GEMM_MX4_STEP(3)                  \
    /* register-staged: the reads of step kk + 1 go one per MFMA between those of kk */  \
    if constexpr (VS) {                                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TM + TN), 0);                    \
      _Pragma("unroll") for (int kk = 0; kk < 3; ++kk) {                                \
        _Pragma("unroll") for (int r = 0; r < TM + TN; ++r) {                           \
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                            \
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                            \
        }                                                                                \
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);             \
      }                                                                                  \
      __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);                          \
    }                                                                                    \
  }

  if constexpr (VS) {
    // Register-staged pipeline: slab kt + 2 is loaded into registers while slab kt
    // is computed, and written to LDS at the start of the next iteration.  (While
    // a direct-to-LDS load is in flight the compiler can only wait for all LDS
    // reads at once, lgkmcnt(0), so fragment reads could not run ahead of the
    // MFMAs; with ordinary loads the waits are exact.)
    i32x4 sreg[IPW];
    i32x4 xreg = {};   // MXFP4: this wave's 1 KB share of the slab's block scales
#define GEMM_LOADR(kt)                                                                    \
  {                                                                                      \
    const int ko_ = (kt) * SLAB;                                                         \
    _Pragma("unroll") for (int j = 0; j < IPW; ++j) {                                   \
      const char* b_ = ((wave * IPW + j) * 1024 >= AB) ? wbase : abase;                  \
      sreg[j] = *(const i32x4*)(b_ + voff[j] + ko_);                                     \
    }                                                                                    \
    if constexpr (F4) {                                                                  \
      if (wave < 4) xreg = *(const i32x4*)(xsrc + (size_t)(kt) * xstride);               \
    }                                                                                    \
  }
#define GEMM_STORER(stg)                                                                  \
  {                                                                                      \
    _Pragma("unroll") for (int j = 0; j < IPW; ++j)                                     \
        *(i32x4*)((stg) + (wave * IPW + j) * 1024 + lane * 16) = sreg[j];                \
    if constexpr (F4) {                                                                  \
      if (wave < 4) *(i32x4*)((stg) + SB + wave * 1024 + lane * 16) = xreg;              \
    }                                                                                    \
  }
    GEMM_LOADR(0)
    GEMM_STORER(stage(0))
    if (nk > 1) GEMM_LOADR(1)
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      // slab kt + 1 goes into the stage slab kt - 1 used (released by the last barrier)
      if (kt + 1 < nk) {
        GEMM_STORER(stage((kt + 1) & 1))
        if (kt + 2 < nk) GEMM_LOADR(kt + 2)
      }
      if constexpr (F4) GEMM_COMPUTE_F4(stage(kt & 1))
      else GEMM_COMPUTE(stage(kt & 1))
      __syncthreads();
    }
#undef GEMM_LOADR
#undef GEMM_STORER
  } else {
  // prologue: slabs 0 .. NS-2 in flight, wait for slab 0
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) GEMM_DMA(stage(s), s);
  if (nk >= NS - 1) wait_vmcnt<(NS - 2) * IPW>();
  else wait_vmcnt<0>();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    // the stage refilled here was consumed in iteration kt - 1 (before its barrier)
    const bool refill = kt + NS - 1 < nk;
    if (refill) GEMM_DMA(stage((kt + NS - 1) % NS), kt + NS - 1);
    char* cur = stage(kt % NS);
    if constexpr (F4) GEMM_COMPUTE_F4(cur)
    else if constexpr (F8) GEMM_COMPUTE_F8(cur)
    else GEMM_COMPUTE(cur)
    // slab kt + 1 has landed once at most the later slabs' loads are outstanding
    if (refill) wait_vmcnt<(NS - 2) * IPW>();
    else wait_vmcnt<0>();
    __syncthreads();
  }
  }
#undef GEMM_DMA
#undef GEMM_COMPUTE
#undef GEMM_COMPUTE_F8
#undef GEMM_COMPUTE_F4
#undef GEMM_MX4_STEP

  const Epi epi = g1 ? p.e[1] : p.e[0];
  dma_epilogue<BN, WN, TM, TN, WROWS, EH, F8>(
      g, epi, acc, (float*)(stage(wave / WPS) + (wave % WPS) * SLICE), m0, n0, wrow, wcol, lane);
}

// ---------------------------------------------------------------- fp32 path
// Reference-precision blocks (fp32 weights and activations) for small models:
// a plain LDS-tiled VALU GEMM (64 x 64 outputs, 256 threads of 4 x 4) with the
// same epilogue interface, writing fp32.

struct EpiSiluF32 {
  float* out; int ldo;
  __device__ __forceinline__ void row4(int r, int c, f32x4 v) const {
    f32x4 o;
    for (int i = 0; i < 4; ++i) o[i] = silu_f(v[i]);
    *(f32x4*)(out + (size_t)r * ldo + c) = o;
  }
};

struct EpiGeluF32 {
  float* out; int ldo; int col_off;
  __device__ __forceinline__ void row4(int r, int c, f32x4 v) const {
    f32x4 o;
    for (int i = 0; i < 4; ++i) o[i] = gelu_tanh_f(v[i]);
    *(f32x4*)(out + (size_t)r * ldo + col_off + c) = o;
  }
};

// Q, K (rotated) and V [B, H, L, d], all fp32.
struct EpiQKV32 {
  float* q; float* k; float* v; const float* rope;
  int D, H, d; RowMap map;
  __device__ __forceinline__ void row4(int r, int c, f32x4 x) const {
    const int which = c / D;
    const int cc = c - which * D;
    const int h = cc / d;
    const int dd = cc - h * d;
    int b, t; map.token(r, b, t);
    const size_t bh = (size_t)b * H + h;
    float* dst = (which == 0 ? q : which == 1 ? k : v) + (bh * map.L + t) * d + dd;
    if (which == 2) {
      *(f32x4*)dst = x;
      return;
    }
    const f32x4 cs = *(const f32x4*)(rope + ((size_t)t * (d >> 1) + (dd >> 1)) * 2);
    f32x4 o;
    o[0] = x[0] * cs[0] - x[1] * cs[1];
    o[1] = x[0] * cs[1] + x[1] * cs[0];
    o[2] = x[2] * cs[2] - x[3] * cs[3];
    o[3] = x[2] * cs[3] + x[3] * cs[2];
    *(f32x4*)dst = o;
  }
};

struct EpiLinear1F32 {
  EpiQKV32 qkv; EpiGeluF32 gelu; int n_qkv;
  __device__ __forceinline__ void row4(int r, int c, f32x4 v) const {
    if (c < n_qkv) qkv.row4(r, c, v);
    else gelu.row4(r, c - n_qkv, v);
  }
};

constexpr int G32_T = 64;    // output tile edge
constexpr int G32_K = 16;    // K chunk

template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams<Epi> p) {
  if (gate_closed(p.gate)) return;
  __shared__ float sA[G32_K][G32_T + 4];   // k-major
  __shared__ float sB[G32_K][G32_T + 4];
  int lid = blockIdx.x;
  const bool g1 = p.ngroups > 1 && lid >= p.tiles[0];
  if (g1) lid -= p.tiles[0];
  const GemmProblem g = g1 ? p.g[1] : p.g[0];
  const int tiles_n = g1 ? p.tiles_n[1] : p.tiles_n[0];
  const int m0 = (lid / tiles_n) * G32_T;
  const int n0 = (lid % tiles_n) * G32_T;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;   // loader: row of the tile, 4 K values
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += G32_K) {
    const int kk = k0 + lk;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
    if (m0 + lrow < g.M && kk < g.K) a = *(const f32x4*)(g.A32 + (size_t)(m0 + lrow) * g.lda + kk);
    if (n0 + lrow < g.N && kk < g.K) w = *(const f32x4*)(g.W32 + (size_t)(n0 + lrow) * g.ldw + kk);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sA[lk + i][lrow] = a[i];
      sB[lk + i][lrow] = w[i];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < G32_K; ++k) {
      const f32x4 av = *(const f32x4*)&sA[k][ty * 4];
      const f32x4 bv = *(const f32x4*)&sB[k][tx * 4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  const Epi epi = g1 ? p.e[1] : p.e[0];
  const int col = n0 + tx * 4;
  if (col >= g.N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= g.M) break;
    f32x4 v = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    if (g.bias) v += *(const f32x4*)(g.bias + col);
    epi.row4(row, col, v);
  }
}

template <class Epi>
static hipError_t launch32(const GemmProblem* gp, const Epi* ep, int ng, hipStream_t st, int site) {
  KTimerScope timer(site, st);
  GemmParams<Epi> p{};
  int total = 0;
  p.ngroups = ng;
  p.gate = launch_gate();
  for (int i = 0; i < ng; ++i) {
    if (gp[i].K % 4 || gp[i].N % 4 || gp[i].lda % 4 || gp[i].ldw % 4) return hipErrorInvalidValue;
    p.g[i] = gp[i];
    p.e[i] = ep[i];
    p.tiles_n[i] = (gp[i].N + G32_T - 1) / G32_T;
    p.tiles[i] = ((gp[i].M + G32_T - 1) / G32_T) * p.tiles_n[i];
    total += p.tiles[i];
  }
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_f32_kernel<Epi>, dim3(total), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t gemm32_store(const GemmProblem& g, float* out, int ldo, hipStream_t st) {
  EpiStoreF32 e{out, ldo};
  return launch32(&g, &e, 1, st, KS_GEMM_F32);
}

hipError_t gemm32_silu(const GemmProblem& g, float* out, int ldo, hipStream_t st) {
  EpiSiluF32 e{out, ldo};
  return launch32(&g, &e, 1, st, KS_GEMM_SILU);
}

hipError_t gemm32_gelu(const GemmProblem* g, int ng, float* const* out, const int* ldo,
                       hipStream_t st) {
  EpiGeluF32 e[2];
  for (int i = 0; i < ng; ++i) e[i] = EpiGeluF32{out[i], ldo[i], 0};
  return launch32(g, e, ng, st, KS_GEMM_GELU);
}

hipError_t gemm32_gated_residual(const GemmProblem* g, int ng, float* x, int D,
                                 const float* const* gate, int gate_bstride, const RowMap* map,
                                 hipStream_t st) {
  EpiGatedResidual<float> e[2];
  for (int i = 0; i < ng; ++i) e[i] = EpiGatedResidual<float>{x, D, gate[i], gate_bstride, map[i]};
  return launch32(g, e, ng, st, KS_GEMM_RESID);
}

hipError_t gemm32_qkv(const GemmProblem* g, int ng, const QKVOut32& o, const RowMap* map,
                      hipStream_t st) {
  EpiQKV32 e[2];
  for (int i = 0; i < ng; ++i) e[i] = EpiQKV32{o.q, o.k, o.v, o.rope, o.D, o.H, o.d, map[i]};
  return launch32(g, e, ng, st, KS_GEMM_QKV);
}

hipError_t gemm32_linear1(const GemmProblem& g, const QKVOut32& o, const RowMap& map, float* cat,
                          int ldcat, hipStream_t st) {
  EpiLinear1F32 e;
  e.qkv = EpiQKV32{o.q, o.k, o.v, o.rope, o.D, o.H, o.d, map};
  e.gelu = EpiGeluF32{cat, ldcat, o.D};
  e.n_qkv = 3 * o.D;
  return launch32(&g, &e, 1, st, KS_GEMM_LIN1);
}

// ---------------------------------------------------------------- launch

// Row bands of the tiled kernels' region raster (grid_tile): of 1, 2, 4 and 8 bands
// (times 8, 4, 2, 1 column bands), the split that divides the grid exactly, then the
// one with the squarest regions (smallest region rows + columns).
static int grid_bands(int gm, int gn) {
  int best = 1;
  double best_score = 1e30;
  for (int P = 1; P <= 8; P *= 2) {
    const int Q = 8 / P;
    if (P > gm || Q > gn) continue;
    const bool exact = gm % P == 0 && gn % Q == 0;
    const double score = (exact ? 0.0 : 1e9) + (double)gm / P + (double)gn / Q;
    if (score < best_score) {
      best_score = score;
      best = P;
    }
  }
  return min(best, gm);
}

// KV: 4 = MXFP4 tiled kernel, 2 = fp8 tiled kernel, 1 = bf16 tiled kernel (256 x 256
// tiles, see above), 0 = the 32 x 256 / 128 x 128 register-staged kernel; NS stages
// of SLAB bytes per row for the tiled kernels
template <int BM, int BN, int WM, int WN, int KV, int NS = 2, int SLAB = 128, class Epi>
static hipError_t launch_cfg(const GemmProblem* gp, const Epi* ep, int ng, hipStream_t st) {
  GemmParams<Epi> p{};
  int total = 0;
  p.ngroups = ng;
  p.gate = launch_gate();
  for (int i = 0; i < ng; ++i) {
    p.g[i] = gp[i];
    p.e[i] = ep[i];
    p.tiles_n[i] = (gp[i].N + BN - 1) / BN;
    p.tiles[i] = ((gp[i].M + BM - 1) / BM) * p.tiles_n[i];
    total += p.tiles[i];
  }
  if (total == 0) return hipSuccess;
  // the region raster for the bf16 and e4m3 tiled kernels; the MXFP4 kernel keeps
  // the 8-row raster (it measured 2% slower with regions)
  p.bands = 0;
  if ((KV == 1 || KV == 2) && (ng == 1 || p.tiles_n[0] == p.tiles_n[1])) {
    const int tm0 = (gp[0].M + BM - 1) / BM;
    p.grid_m = tm0 + (ng > 1 ? (gp[1].M + BM - 1) / BM : 0);
    p.grid_n = p.tiles_n[0];
    p.split_m = ng > 1 ? tm0 : p.grid_m;
    p.bands = grid_bands(p.grid_m, p.grid_n);
  }
  void (*kern)(GemmParams<Epi>);
  if constexpr (KV == 4) kern = &gemm_dma_kernel<BM, BN, WM, WN, 2, NS, SLAB, Epi>;
  else if constexpr (KV == 2) kern = &gemm_dma_kernel<BM, BN, WM, WN, 1, NS, SLAB, Epi>;
  else if constexpr (KV == 1) kern = &gemm_dma_kernel<BM, BN, WM, WN, 0, NS, SLAB, Epi>;
  else kern = &gemm_bf16_kernel<BM, BN, WM, WN, Epi>;
  hipLaunchKernelGGL(kern, dim3(total), dim3(WM * WN * 64), 0, st, p);
  return hipGetLastError();
}

template <class Epi>
static hipError_t launch(const GemmProblem* gp, const Epi* ep, int ng, hipStream_t st, int site) {
  KTimerScope timer(site, st);
  int maxM = 0, minN = 1 << 30;
  // the direct-to-LDS kernel keeps per-lane byte offsets in 32 bits
  bool offsets32 = true;
  for (int i = 0; i < ng; ++i) {
    maxM = max(maxM, gp[i].M);
    minN = min(minN, gp[i].N);
    const long long es = gp[i].A8 ? 1 : 2;
    offsets32 = offsets32 && (long long)gp[i].M * gp[i].lda * es < (1LL << 31) &&
                (long long)gp[i].N * gp[i].ldw * es < (1LL << 31);
  }
  if (gp[0].A8 && !offsets32) return hipErrorInvalidValue;
  if (gp[0].A4) {   // MXFP4 operands: the tiled kernel, byte offsets in 32 bits
    for (int i = 0; i < ng; ++i)
      if ((long long)gp[i].M * (gp[i].lda / 2) >= (1LL << 31) ||
          (long long)gp[i].N * (gp[i].ldw / 2) >= (1LL << 31) || gp[i].K % 256)
        return hipErrorInvalidValue;
    return launch_cfg<256, 256, 2, 4, 4, 2, 128>(gp, ep, ng, st);
  }
#ifndef GEMM_NS
#define GEMM_NS 2
#define GEMM_SLAB 128
#endif
  if (gp[0].A8) return launch_cfg<256, 256, 2, 4, 2, GEMM_NS, GEMM_SLAB>(gp, ep, ng, st);
  if (maxM <= 64) return launch_cfg<32, 256, 1, 4, 0>(gp, ep, ng, st);
  // large problems: 256x256 tiles, 8 waves, 128-byte K slabs in two LDS stages
  if (maxM >= 1024 && minN >= 1024 && offsets32)
    return launch_cfg<256, 256, 2, 4, 1, GEMM_NS, GEMM_SLAB>(gp, ep, ng, st);
  return launch_cfg<128, 128, 2, 2, 0>(gp, ep, ng, st);
}

// MXFP4 operands: the tiled kernel only (256 x 256 tiles, any M, N).
template <class Epi>
static hipError_t launch_mx4(const GemmProblem& g, const Epi& e, hipStream_t st) {
  KTimerScope timer(KS_GEMM_F32, st);
  if ((long long)g.M * (g.lda / 2) >= (1LL << 31) || (long long)g.N * (g.ldw / 2) >= (1LL << 31))
    return hipErrorInvalidValue;   // byte offsets are kept in 32 bits
  return launch_cfg<256, 256, 2, 4, 4, 2, 128>(&g, &e, 1, st);
}

hipError_t gemm_mx4_store_f32(const GemmProblem& g, float* out, int ldo, hipStream_t st) {
  return launch_mx4(g, EpiStoreF32{out, ldo}, st);
}

hipError_t gemm_mx4_store_bf16(const GemmProblem& g, bf16_t* out, int ldo, hipStream_t st) {
  return launch_mx4(g, EpiStoreBf16{out, ldo}, st);
}

hipError_t gemm_store_f32(const GemmProblem& g, float* out, int ldo, hipStream_t st) {
  EpiStoreF32 e{out, ldo};
  return launch(&g, &e, 1, st, KS_GEMM_F32);
}

hipError_t gemm_store_bf16(const GemmProblem& g, bf16_t* out, int ldo, hipStream_t st) {
  EpiStoreBf16 e{out, ldo};
  return launch(&g, &e, 1, st, KS_GEMM_F32);
}

hipError_t gemm_silu_bf16(const GemmProblem& g, bf16_t* out, int ldo, hipStream_t st) {
  EpiSiluBf16 e{out, ldo};
  return launch(&g, &e, 1, st, KS_GEMM_SILU);
}

hipError_t gemm_gelu_bf16(const GemmProblem* g, int ng, bf16_t* const* out, const int* ldo,
                          hipStream_t st) {
  EpiGeluBf16 e[2];
  for (int i = 0; i < ng; ++i) e[i] = EpiGeluBf16{out[i], ldo[i], 0};
  return launch(g, e, ng, st, KS_GEMM_GELU);
}

template <class XT>
hipError_t gemm_gated_residual(const GemmProblem* g, int ng, XT* x, int D,
                               const float* const* gate, int gate_bstride, const RowMap* map,
                               hipStream_t st) {
  EpiGatedResidual<XT> e[2];
  for (int i = 0; i < ng; ++i) e[i] = EpiGatedResidual<XT>{x, D, gate[i], gate_bstride, map[i]};
  return launch(g, e, ng, st, KS_GEMM_RESID);
}
template hipError_t gemm_gated_residual<float>(const GemmProblem*, int, float*, int,
                                               const float* const*, int, const RowMap*, hipStream_t);

hipError_t gemm_qkv(const GemmProblem* g, int ng, const QKVOut& o, const RowMap* map,
                    hipStream_t st) {
  if (o.amax) {
    EpiQKVT<true> e[2];
    for (int i = 0; i < ng; ++i)
      e[i] = EpiQKVT<true>{o.q, o.k, o.v, o.rope, o.D, o.H, o.d, map[i], o.amax};
    return launch(g, e, ng, st, KS_GEMM_QKV);
  }
  EpiQKV e[2];
  for (int i = 0; i < ng; ++i)
    e[i] = EpiQKV{o.q, o.k, o.v, o.rope, o.D, o.H, o.d, map[i], nullptr};
  return launch(g, e, ng, st, KS_GEMM_QKV);
}

hipError_t gemm_linear1(const GemmProblem& g, const QKVOut& o, const RowMap& map,
                        bf16_t* cat, int ldcat, hipStream_t st) {
  if (o.amax) {
    EpiLinear1T<true> e;
    e.qkv = EpiQKVT<true>{o.q, o.k, o.v, o.rope, o.D, o.H, o.d, map, o.amax};
    e.gelu = EpiGeluBf16{cat, ldcat, o.D};
    e.n_qkv = 3 * o.D;
    return launch(&g, &e, 1, st, KS_GEMM_LIN1);
  }
  EpiLinear1 e;
  e.qkv = EpiQKV{o.q, o.k, o.v, o.rope, o.D, o.H, o.d, map, nullptr};
  e.gelu = EpiGeluBf16{cat, ldcat, o.D};
  e.n_qkv = 3 * o.D;
  return launch(&g, &e, 1, st, KS_GEMM_LIN1);
}

}  // namespace dit
