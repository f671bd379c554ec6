// Flash-style joint attention, bf16, for gfx950 (MFMA + LDS-staged K/V tiles).
//
//   O[b, t, h*d + c] = sum_u softmax_u(Q[b,h,t] . K[b,h,u] * scale) V[b,h,u,c]
//
// Work split: one workgroup = 8 wave64s = 256 queries of one (b, h); each wave
// owns 32 queries, two waves share a SIMD so one wave's softmax arithmetic runs
// while the other's MFMAs do.  Scores are computed transposed, S^T = K Q^T, so
// every lane owns a query column: the softmax max is an in-lane reduction plus
// one exchange with lane ^ 32, and the row sum needs no exchange until the end.
// K rows are fed to the MFMA in the order (r with bits 2 and 3 swapped), which
// makes the 8 score registers a lane holds per 16-key chunk correspond to 8
// consecutive keys: exactly the B operand of the P V^T MFMA, so P never leaves
// registers.  V arrives pre-transposed ([B, H, d, L], written that way by the
// QKV projection epilogue), so its MFMA operand is a contiguous LDS read too.
// The P V^T product runs in fp16 (V stored as fp16, P <= 2^8 converted to
// fp16): the same MFMA rate as bf16 with three more mantissa bits on both
// operands.
//
// Softmax reference max: exp2 is taken relative to a per-query reference m that
// only moves when a tile's maximum exceeds it by more than 2^8 (in exp2 units);
// otherwise P <= 256 and the rescale of O and of the row sum is skipped.  The
// reference cancels exactly in O / l.
//
// K/V tiles of 64 keys are double-buffered in LDS, filled by direct
// global->LDS loads (each wave instruction writes 1 KB contiguously; padded rows
// are filled by giving each lane the chunk that belongs at its slot).  Keys past
// L are masked to -inf; queries past L are computed on clamped rows, not stored.
#include "common.h"
#include "kernels.h"

namespace dit {

constexpr int ATT_D = 128;          // head dim handled by this kernel
constexpr int ATT_BN = 64;          // keys per tile
constexpr int ATT_QW = 32;          // queries per wave
constexpr int ATT_WAVES = 8;
constexpr int ATT_BM = ATT_QW * ATT_WAVES;
constexpr int ATT_KS = ATT_D + 8;   // padded K row (bf16): 272 B = 17 chunks
constexpr int ATT_VS = ATT_BN + 8;  // padded V^T row (fp16): 144 B = 9 chunks
constexpr int ATT_KB = ATT_BN * ATT_KS * 2;     // K tile bytes (17 KB)
constexpr int ATT_VB = ATT_D * ATT_VS * 2;      // V^T tile bytes (18 KB)
constexpr int ATT_SB = ATT_KB + ATT_VB;         // stage bytes
constexpr int ATT_NI = ATT_SB / 1024;           // 1-KB load instructions per stage
static_assert(ATT_KB % 1024 == 0 && ATT_VB % 1024 == 0, "stage must be whole 1-KB loads");
constexpr float ATT_RESCALE_LOG2 = 8.0f;        // P stays <= 2^8 between rescales

__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__global__ __launch_bounds__(ATT_WAVES * 64) void attention_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const f16_t* __restrict__ VT,
    bf16_t* __restrict__ O, int ldo, RowMap map, int H, int L, float scale_log2,
    const int* __restrict__ gate) {
  if (gate_closed(gate)) return;
  __shared__ __attribute__((aligned(1024))) char st0[ATT_SB];
  __shared__ __attribute__((aligned(1024))) char st1[ATT_SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;           // lane group
  const int l32 = lane & 31;

  // XCD-aware: q-tiles of one (b, h) go to the same XCD so K/V stay in its L2
  const int nqt = (L + ATT_BM - 1) / ATT_BM;
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int xq = nblk >> 3, xr = nblk & 7, xcd = bid & 7;
  const int lid = xcd * xq + min(xcd, xr) + (bid >> 3);
  const int bh = lid / nqt;
  const int qt = lid - bh * nqt;
  const int b = bh / H;
  const int h = bh - b * H;

  const bf16_t* Qb = Q + (size_t)bh * L * ATT_D;
  const bf16_t* Kb = K + (size_t)bh * L * ATT_D;
  const f16_t* Vb = VT + (size_t)bh * ATT_D * L;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[q][c*16 + g*8 .. +8]
  const int q0 = qt * ATT_BM + wave * ATT_QW;
  bf16x8 qf[ATT_D / 16];
  {
    const int qr = min(q0 + l32, L - 1);
#pragma unroll
    for (int c = 0; c < ATT_D / 16; ++c)
      qf[c] = *(const bf16x8*)(Qb + (size_t)qr * ATT_D + c * 16 + g * 8);
  }

  f32x16 oacc[ATT_D / 32];   // O^T blocks, one per 32 head channels
#pragma unroll
  for (int db = 0; db < ATT_D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float mref = -INFINITY;     // reference max (raw score units)
  float lsum = 0.f;           // this lane's partial row sum, relative to mref

  // ---- direct-to-LDS loads of a K / V^T tile pair.  Chunk c of a stage: the
  // first 64*17 chunks are K rows (16 data chunks + 1 pad) = load instructions
  // 0..16, then 128*9 V^T rows = instructions 17..34.  Wave w issues
  // instructions w, w+8, ...; each lane's source offset inside a tile is fixed,
  // so it is computed once here.
  constexpr int ATT_KI = ATT_BN * 17 / 64;        // K instructions (17)
  constexpr int ATT_IPW = (ATT_NI + ATT_WAVES - 1) / ATT_WAVES;
  static_assert(ATT_BN * 17 % 64 == 0, "K part must be whole instructions");
  int doff[ATT_IPW];   // K: row*128 + slot*8 ; V^T: row*L + slot*8
  int dkv[ATT_IPW];    // K: key row in tile ; V^T: first key of the chunk in tile
#pragma unroll
  for (int j = 0; j < ATT_IPW; ++j) {
    const int inst = wave + j * ATT_WAVES;
    const int c = inst * 64 + lane;
    if (inst < ATT_KI) {
      const int row = c / 17;
      const int slot = min(c - row * 17, 15);
      doff[j] = row * ATT_D + slot * 8;
      dkv[j] = row;
    } else {
      const int c2 = c - ATT_BN * 17;
      const int row = c2 / 9;
      const int slot = min(c2 - row * 9, 7);
      doff[j] = row * L + slot * 8;
      dkv[j] = slot * 8;
    }
  }
  auto issue_tile = [&](char* stage, int kt) {
    const int kv0 = kt * ATT_BN;
    const bool full = kv0 + ATT_BN <= L;
#pragma unroll
    for (int j = 0; j < ATT_IPW; ++j) {
      const int inst = wave + j * ATT_WAVES;
      if (inst >= ATT_NI) break;
      const void* src;
      if (inst < ATT_KI) {
        src = Kb + (size_t)kv0 * ATT_D + doff[j];
        if (!full && kv0 + dkv[j] > L - 1)   // tail tile: clamp the key row
          src = Kb + (size_t)(L - 1) * ATT_D + (doff[j] - dkv[j] * ATT_D);
      } else {
        src = Vb + kv0 + doff[j];
        if (!full && kv0 + dkv[j] > L - 8)   // tail tile: clamp the key chunk
          src = Vb + (L - 8) + (doff[j] - dkv[j]);
      }
      __builtin_amdgcn_global_load_lds((const void*)src, (void*)(stage + inst * 1024), 16, 0, 0);
    }
  };

  const int ntiles = (L + ATT_BN - 1) / ATT_BN;
  const int krow_perm = swap23(l32);
  issue_tile(st0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    char* cur = (kt & 1) ? st1 : st0;
    char* nxt = (kt & 1) ? st0 : st1;
    if (kt + 1 < ntiles) issue_tile(nxt, kt + 1);
    const bf16_t* sK = (const bf16_t*)cur;
    const f16_t* sV = (const f16_t*)(cur + ATT_KB);
    const int kv0 = kt * ATT_BN;

    // S^T for 2 key blocks of 32
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
    for (int c = 0; c < ATT_D / 16; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *(const bf16x8*)&sK[(kb * 32 + krow_perm) * ATT_KS + c * 16 + g * 8];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sacc[kb], 0, 0, 0);
      }
    }

    // element e of sacc[kb] is key kv0 + kb*32 + (e/8)*16 + g*8 + e%8 of query column l32
    if (kv0 + ATT_BN > L) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kv = kv0 + kb * 32 + (e >> 3) * 16 + g * 8 + (e & 7);
          if (kv >= L) sacc[kb][e] = -INFINITY;
        }
    }

    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    // move the reference only when some query of the wave would overflow 2^8; a
    // lane's half of the keys decides that as well as the whole row does (the
    // test is wave-wide), so the two halves exchange maxima only when it moves
    if (__any((mx - mref) * scale_log2 > ATT_RESCALE_LOG2)) {
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mref, mx);
      const float alpha = fast_exp2((mref - mnew) * scale_log2);
      mref = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < ATT_D / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
    const float moff = mref * scale_log2;
    f16x8 pf[4];   // [16-key chunk]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        f16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = fast_exp2(fmaf(sacc[kb][ch * 8 + e], scale_log2, -moff));
          lsum += pv;
          t[e] = (_Float16)pv;
        }
        pf[kb * 2 + ch] = t;
      }

    // O^T += V^T P^T over the 4 chunks of 16 keys
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
      for (int db = 0; db < ATT_D / 32; ++db) {
        const f16x8 vf = *(const f16x8*)&sV[(db * 32 + l32) * ATT_VS + ch * 16 + g * 8];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[ch], oacc[db], 0, 0, 0);
      }
    }

    __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's loads of the next tile landed
    __syncthreads();
  }

  // ---- normalise and store: O^T element e of block db is
  // d = db*32 + (e/4)*8 + g*4 + e%4 of query column l32
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.0f / lt;
  const int t = q0 + l32;
  if (t < L) {
    bf16_t* orow = O + (size_t)map.stream_row(b, t) * ldo + h * ATT_D;
#pragma unroll
    for (int db = 0; db < ATT_D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int dd = db * 32 + e4 * 8 + g * 4;
        uint2 u;
        u.x = pack_bf16x2(oacc[db][e4 * 4 + 0] * inv, oacc[db][e4 * 4 + 1] * inv);
        u.y = pack_bf16x2(oacc[db][e4 * 4 + 2] * inv, oacc[db][e4 * 4 + 3] * inv);
        *(uint2*)(orow + dd) = u;
      }
  }
}

// ---------------------------------------------------------------- fp8 (e4m3)
// Same work split.  Q, K, V^T are e4m3 with one scale per (b, h) each, so the
// score scale sq * sk folds into the exp2 constant and sv into the final
// normalisation.  S^T uses v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales):
// for key block kb the MFMA row r is fed K row  g(r)*32 + kb*16 + i(r),
// g(r) = (r/4)&1, i(r) = (r/8)*4 + r%4, so a lane's 32 score registers over the
// 64-key tile are the 32 consecutive keys its lane group needs as the P operand
// of the fp8 P V^T MFMA.
//
// Softmax reference: in exp2 units the running row max is rounded up to an
// integer r, so P = 2^(t - r) <= 1 and 448 P never saturates e4m3.  When r
// moves by k, O and the row sum scale by exactly 2^-k, and the e4m3 rounding of
// 448 P is the same for every integer r (down to e4m3's subnormals): the result
// matches quantising against the final row max rounded the same way.  The row
// sum is that of the quantised P, taken by one more MFMA of the P codes against
// an all-ones operand, so the weights that multiply V sum to one.
constexpr int AF8_BN = 64;
constexpr int AF8_KRB = 144;                      // K row: 128 B + 16 pad (9 chunks)
constexpr int AF8_VRB = 80;                       // V^T row: 64 B + 16 pad (5 chunks)
constexpr int AF8_KB = AF8_BN * AF8_KRB;          // 9 KB
constexpr int AF8_VB = ATT_D * AF8_VRB;           // 10 KB
constexpr int AF8_SB = AF8_KB + AF8_VB;
constexpr int AF8_NI = AF8_SB / 1024;             // 19 load instructions per stage
constexpr int AF8_KI = AF8_KB / 1024;             // 9 of them for K
static_assert(AF8_KB % 1024 == 0 && AF8_VB % 1024 == 0, "whole 1-KB loads");

__global__ __launch_bounds__(ATT_WAVES * 64) void attention_fp8_kernel(
    const fp8_t* __restrict__ Q, const fp8_t* __restrict__ K, const fp8_t* __restrict__ VT,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    bf16_t* __restrict__ O, int ldo, RowMap map, int H, int L, float scale_log2,
    const int* __restrict__ gate) {
  if (gate_closed(gate)) return;
  __shared__ __attribute__((aligned(1024))) char st0[AF8_SB];
  __shared__ __attribute__((aligned(1024))) char st1[AF8_SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const int nqt = (L + ATT_BM - 1) / ATT_BM;
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int xq = nblk >> 3, xr = nblk & 7, xcd = bid & 7;
  const int lid = xcd * xq + min(xcd, xr) + (bid >> 3);
  const int bh = lid / nqt;
  const int qt = lid - bh * nqt;
  const int b = bh / H;
  const int h = bh - b * H;

  const fp8_t* Qb = Q + (size_t)bh * L * ATT_D;
  const fp8_t* Kb = K + (size_t)bh * L * ATT_D;
  const fp8_t* Vb = VT + (size_t)bh * ATT_D * L;
  const float cs = scale_log2 * sq[bh] * sk[bh];   // raw score -> exp2 units

  // Q fragments: lane holds Q[q][c*64 + g*32 .. +32], c = 0, 1
  const int q0 = qt * ATT_BM + wave * ATT_QW;
  i32x8 qf[2];
  {
    const int qr = min(q0 + l32, L - 1);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const i32x4 lo = *(const i32x4*)(Qb + (size_t)qr * ATT_D + c * 64 + g * 32);
      const i32x4 hi = *(const i32x4*)(Qb + (size_t)qr * ATT_D + c * 64 + g * 32 + 16);
      qf[c] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }

  f32x16 oacc[ATT_D / 32];
#pragma unroll
  for (int db = 0; db < ATT_D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float mref = -INFINITY;    // integer-valued reference, exp2 units
  // row sums of the quantised 448 P, accumulated by one more MFMA against an
  // all-ones e4m3 operand (every row of the result is the column's sum)
  f32x16 lacc;
#pragma unroll
  for (int e = 0; e < 16; ++e) lacc[e] = 0.f;
  const i32x8 ones = i32x8{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                           0x38383838, 0x38383838, 0x38383838, 0x38383838};   // e4m3 1.0

  // per-lane load offsets (bytes inside a tile): K chunk c -> row c/9, slot c%9;
  // V^T chunk c2 -> row c2/5, slot c2%5 (the last slot of a row is padding)
  constexpr int IPW = (AF8_NI + ATT_WAVES - 1) / ATT_WAVES;
  int doff[IPW], dkv[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int inst = wave + j * ATT_WAVES;
    const int c = inst * 64 + lane;
    if (inst < AF8_KI) {
      const int row = c / 9;
      const int slot = min(c - row * 9, 7);
      doff[j] = row * ATT_D + slot * 16;
      dkv[j] = row;
    } else {
      const int c2 = c - AF8_KI * 64;
      const int row = c2 / 5;
      const int slot = min(c2 - row * 5, 3);
      doff[j] = row * L + slot * 16;
      dkv[j] = slot * 16;
    }
  }
  auto issue_tile = [&](char* stage, int kt) {
    const int kv0 = kt * AF8_BN;
    const bool full = kv0 + AF8_BN <= L;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int inst = wave + j * ATT_WAVES;
      if (inst >= AF8_NI) break;
      const fp8_t* src;
      if (inst < AF8_KI) {
        src = Kb + (size_t)kv0 * ATT_D + doff[j];
        if (!full && kv0 + dkv[j] > L - 1)
          src = Kb + (size_t)(L - 1) * ATT_D + (doff[j] - dkv[j] * ATT_D);
      } else {
        src = Vb + kv0 + doff[j];
        if (!full && kv0 + dkv[j] > L - 16) src = Vb + (L - 16) + (doff[j] - dkv[j]);
      }
      __builtin_amdgcn_global_load_lds((const void*)src, (void*)(stage + inst * 1024), 16, 0, 0);
    }
  };

  const int ntiles = (L + AF8_BN - 1) / AF8_BN;
  // K row fed to MFMA row l32 of key block kb
  const int krow0 = ((l32 >> 2) & 1) * 32 + (l32 >> 3) * 4 + (l32 & 3);
  issue_tile(st0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    char* cur = (kt & 1) ? st1 : st0;
    char* nxt = (kt & 1) ? st0 : st1;
    if (kt + 1 < ntiles) issue_tile(nxt, kt + 1);
    const char* sK = cur;
    const char* sV = cur + AF8_KB;
    const int kv0 = kt * AF8_BN;

    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const char* q_ = sK + (krow0 + kb * 16) * AF8_KRB + c * 64 + g * 32;
        const i32x4 lo = *(const i32x4*)q_, hi = *(const i32x4*)(q_ + 16);
        const i32x8 kf = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[c], sacc[kb], 0, 0, 0,
                                                                   127, 0, 127);
      }
    }
    // element e of sacc[kb] is key kv0 + g*32 + kb*16 + e of query column l32
    if (kv0 + AF8_BN > L) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kv0 + g * 32 + kb * 16 + e >= L) sacc[kb][e] = -INFINITY;
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    // as in the bf16 kernel: the halves exchange maxima only when the reference moves
    if (__any(mx * cs > mref)) {
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxl = mx * cs;
      const float mnew = fmaxf(mref, ceilf(mxl));
      // 2^(mref - mnew): an exact power of two (0 before the first tile)
      const float alpha = mref == -INFINITY ? 0.f : ldexpf(1.0f, (int)(mref - mnew));
      mref = mnew;
      lacc *= alpha;
#pragma unroll
      for (int db = 0; db < ATT_D / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
    // 448 P = 2^(t - mref + log2 448): the factor rides in the exponent
    const float moff = mref - 8.807354922057604f;
    int pw[8];   // 32 e4m3 codes of P * 448, keys g*32 + 0..31
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p[e] = fast_exp2(fmaf(sacc[kb][w4 * 4 + e], cs, -moff));
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        pw[kb * 4 + w4] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
      }
    const i32x8 pf = i32x8{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
#pragma unroll
    for (int db = 0; db < ATT_D / 32; ++db) {
      const char* v_ = sV + (db * 32 + l32) * AF8_VRB + g * 32;
      const i32x4 lo = *(const i32x4*)v_, hi = *(const i32x4*)(v_ + 16);
      const i32x8 vf = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, oacc[db], 0, 0, 0, 127,
                                                                 0, 127);
    }
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lacc, 0, 0, 0, 127, 0, 127);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }

  const float inv = sv[bh] / lacc[0];
  const int t = q0 + l32;
  if (t < L) {
    bf16_t* orow = O + (size_t)map.stream_row(b, t) * ldo + h * ATT_D;
#pragma unroll
    for (int db = 0; db < ATT_D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int dd = db * 32 + e4 * 8 + g * 4;
        uint2 u;
        u.x = pack_bf16x2(oacc[db][e4 * 4 + 0] * inv, oacc[db][e4 * 4 + 1] * inv);
        u.y = pack_bf16x2(oacc[db][e4 * 4 + 2] * inv, oacc[db][e4 * 4 + 3] * inv);
        *(uint2*)(orow + dd) = u;
      }
  }
}

// ---------------------------------------------------------------- fp32
// Reference-precision attention for small models (head dim 32 or 64): one wave
// per 64 queries of one (b, h), one query per lane, 64-key K and V^T tiles in LDS
// (every lane reads the same key, so the LDS reads broadcast); online softmax in
// exp2 units with the scale folded into q.
template <int HD>
__global__ __launch_bounds__(64) void attention_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ VT,
    float* __restrict__ O, int ldo, RowMap map, int H, int L, float scale_log2,
    const int* __restrict__ gate) {
  if (gate_closed(gate)) return;
  __shared__ float sK[64][HD];
  __shared__ float sV[HD][65];
  const int lane = threadIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int t = blockIdx.x * 64 + lane;
  const int tq = min(t, L - 1);
  const float* Kb = K + (size_t)bh * L * HD;
  const float* Vb = VT + (size_t)bh * HD * L;
  float q[HD], acc[HD];
#pragma unroll
  for (int c = 0; c < HD; ++c) {
    q[c] = Q[((size_t)bh * L + tq) * HD + c] * scale_log2;
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int k0 = 0; k0 < L; k0 += 64) {
    const int kr = k0 + lane;
#pragma unroll
    for (int c = 0; c < HD; ++c) {
      sK[lane][c] = kr < L ? Kb[(size_t)kr * HD + c] : 0.f;
      sV[c][lane] = kr < L ? Vb[(size_t)c * L + kr] : 0.f;
    }
    __syncthreads();
    const int nk = min(64, L - k0);
    for (int j0 = 0; j0 < nk; j0 += 16) {     // 16 keys per softmax update
      float sc[16];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < HD; ++c) d = fmaf(q[c], sK[j0 + j][c], d);
        sc[j] = j0 + j < nk ? d : -INFINITY;
        mx = fmaxf(mx, sc[j]);
      }
      const float mnew = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mnew);
      l *= alpha;
#pragma unroll
      for (int c = 0; c < HD; ++c) acc[c] *= alpha;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pj = fast_exp2(sc[j] - mnew);
        l += pj;
#pragma unroll
        for (int c = 0; c < HD; ++c) acc[c] = fmaf(pj, sV[c][j0 + j], acc[c]);
      }
      m = mnew;
    }
    __syncthreads();
  }
  if (t < L) {
    float* orow = O + (size_t)map.stream_row(b, t) * ldo + h * HD;
    const float inv = 1.0f / l;
#pragma unroll
    for (int c = 0; c < HD; ++c) orow[c] = acc[c] * inv;
  }
}

hipError_t attention_f32(const float* q, const float* k, const float* vt, float* o, int ldo,
                         const RowMap& map, int B, int H, int L, int d, float softmax_scale,
                         hipStream_t st) {
  if ((d != 32 && d != 64) || L < 1) return hipErrorInvalidValue;
  if (B * H == 0) return hipSuccess;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  KTimerScope timer(KS_ATTENTION, st);
  const dim3 grid((L + 63) / 64, B * H);
  if (d == 64)
    hipLaunchKernelGGL(attention_f32_kernel<64>, grid, dim3(64), 0, st, q, k, vt, o, ldo, map, H,
                       L, scale_log2, launch_gate());
  else
    hipLaunchKernelGGL(attention_f32_kernel<32>, grid, dim3(64), 0, st, q, k, vt, o, ldo, map, H,
                       L, scale_log2, launch_gate());
  return hipGetLastError();
}

hipError_t attention_fp8(const fp8_t* q8, const fp8_t* k8, const fp8_t* vt8, const float* sq,
                         const float* sk, const float* sv, bf16_t* o, int ldo, const RowMap& map,
                         int B, int H, int L, int d, float softmax_scale, hipStream_t st) {
  if (d != ATT_D || L < 16 || L % 16) return hipErrorInvalidValue;
  const int nqt = (L + ATT_BM - 1) / ATT_BM;
  const int nblk = B * H * nqt;
  if (nblk == 0) return hipSuccess;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  KTimerScope timer(KS_ATTENTION, st);
  hipLaunchKernelGGL(attention_fp8_kernel, dim3(nblk), dim3(ATT_WAVES * 64), 0, st, q8, k8, vt8,
                     sq, sk, sv, o, ldo, map, H, L, scale_log2, launch_gate());
  return hipGetLastError();
}

hipError_t attention_bf16(const bf16_t* q, const bf16_t* k, const f16_t* vt, bf16_t* o,
                          int ldo, const RowMap& map, int B, int H, int L, int d,
                          float softmax_scale, hipStream_t st) {
  if (d != ATT_D || L < 8 || L % 8) return hipErrorInvalidValue;
  const int nqt = (L + ATT_BM - 1) / ATT_BM;
  const int nblk = B * H * nqt;
  if (nblk == 0) return hipSuccess;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  KTimerScope timer(KS_ATTENTION, st);
  hipLaunchKernelGGL(attention_bf16_kernel, dim3(nblk), dim3(ATT_WAVES * 64), 0, st, q, k, vt, o,
                     ldo, map, H, L, scale_log2, launch_gate());
  return hipGetLastError();
}

}  // namespace dit
