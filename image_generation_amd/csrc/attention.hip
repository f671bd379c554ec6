// Flash-style joint attention, bf16, for gfx950 (MFMA + LDS-staged K/V tiles).
//
//   O[b, t, h*d + c] = sum_u softmax_u(Q[b,h,t] . K[b,h,u] * scale) V[b,h,u,c]
//
// Work split: one workgroup = 4 wave64s = 256 queries of one (b, h); each wave
// owns 64 queries (two 32-query column blocks).  Scores are computed transposed,
// S^T = K Q^T, so that every lane owns whole query columns: the softmax max is
// one in-lane reduction plus a single exchange with lane ^ 32, and the row sum
// needs no exchange until the end.  K rows are fed to the MFMA in the order
// (r with bits 2 and 3 swapped), which makes the 8 score registers a lane holds
// per 16-key chunk correspond to 8 consecutive keys: exactly the B operand of
// the P V^T MFMA, so P never leaves registers.  V arrives pre-transposed
// ([B, H, d, L], written that way by the QKV projection epilogue), so its MFMA
// operand is a contiguous 16-byte LDS read as well.
//
// K/V tiles of 64 keys are double-buffered in LDS with the next tile's global
// loads in flight during the current tile's MFMAs.  Keys past L are masked to
// -inf; queries past L are computed on clamped rows and not stored.
#include "common.h"
#include "kernels.h"

namespace dit {

constexpr int ATT_D = 128;          // head dim handled by this kernel
constexpr int ATT_BN = 64;          // keys per tile
constexpr int ATT_QW = 64;          // queries per wave
constexpr int ATT_WAVES = 4;
constexpr int ATT_BM = ATT_QW * ATT_WAVES;
constexpr int ATT_KS = ATT_D + 8;   // padded K row (bf16): 272 B
constexpr int ATT_VS = ATT_BN + 8;  // padded V^T row (bf16): 144 B

__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__global__ __launch_bounds__(256) void attention_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ VT,
    bf16_t* __restrict__ O, int ldo, RowMap map, int H, int L, float scale_log2) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][ATT_BN * ATT_KS];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][ATT_D * ATT_VS];

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
  const bf16_t* Vb = VT + (size_t)bh * ATT_D * L;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[q][c*16 + g*8 .. +8]
  const int q0 = qt * ATT_BM + wave * ATT_QW;
  bf16x8 qf[2][ATT_D / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qr = min(q0 + qb * 32 + l32, L - 1);
#pragma unroll
    for (int c = 0; c < ATT_D / 16; ++c)
      qf[qb][c] = *(const bf16x8*)(Qb + (size_t)qr * ATT_D + c * 16 + g * 8);
  }

  f32x16 oacc[2][ATT_D / 32];   // O^T blocks: [q-block][d-block]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < ATT_D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[qb][db][e] = 0.f;
  float mrow[2] = {-INFINITY, -INFINITY};
  float lrow[2] = {0.f, 0.f};

  // ---- K/V tile staging: K tile 64 x 128 (16 threads per row), V^T tile 128 x 64
  const int k_row = tid >> 4, k_chk = (tid & 15) * 8;   // 4 passes of 16 rows
  const int v_row = tid >> 3, v_chk = (tid & 7) * 8;    // 4 passes of 32 rows
  i32x4 rk[4], rv[4];
  const int ntiles = (L + ATT_BN - 1) / ATT_BN;

  auto gload = [&](int kt) {
    const int kv0 = kt * ATT_BN;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int kr = min(kv0 + k_row + 16 * p, L - 1);
      rk[p] = *(const i32x4*)(Kb + (size_t)kr * ATT_D + k_chk);
      const int vc = min(kv0 + v_chk, L - 8);
      rv[p] = *(const i32x4*)(Vb + (size_t)(v_row + 32 * p) * L + vc);
    }
  };
  auto sstore = [&](int s) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      *(i32x4*)&sK[s][(k_row + 16 * p) * ATT_KS + k_chk] = rk[p];
      *(i32x4*)&sV[s][(v_row + 32 * p) * ATT_VS + v_chk] = rv[p];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  const int krow_perm = swap23(l32);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int s = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1);
    const int kv0 = kt * ATT_BN;

    // S^T for 2 key blocks x 2 query blocks
    f32x16 sacc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][qb][e] = 0.f;
#pragma unroll
    for (int c = 0; c < ATT_D / 16; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf =
            *(const bf16x8*)&sK[s][(kb * 32 + krow_perm) * ATT_KS + c * 16 + g * 8];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][c], sacc[kb][qb], 0, 0, 0);
      }
    }

    // element e of sacc[kb][qb] is key kv0 + kb*32 + (e/8)*16 + g*8 + e%8 of query column l32
    if (kv0 + ATT_BN > L) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kv = kv0 + kb * 32 + (e >> 3) * 16 + g * 8 + (e & 7);
          if (kv >= L) {
            sacc[kb][0][e] = -INFINITY;
            sacc[kb][1][e] = -INFINITY;
          }
        }
    }

    bf16x8 pf[2][4];   // [q-block][16-key chunk]
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = mrow[qb];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][qb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float alpha = fast_exp2((mrow[qb] - mx) * scale_log2);
      const float moff = mx * scale_log2;
      mrow[qb] = mx;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[e] = fast_exp2(fmaf(sacc[kb][qb][ch * 8 + e], scale_log2, -moff));
            ls += pv[e];
          }
          bf16x8 t;
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = (__bf16)pv[e];
          pf[qb][kb * 2 + ch] = t;
        }
      lrow[qb] = lrow[qb] * alpha + ls;
#pragma unroll
      for (int db = 0; db < ATT_D / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[qb][db][e] *= alpha;
    }

    // O^T += V^T P^T over the 4 chunks of 16 keys
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
      for (int db = 0; db < ATT_D / 32; ++db) {
        const bf16x8 vf = *(const bf16x8*)&sV[s][(db * 32 + l32) * ATT_VS + ch * 16 + g * 8];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][ch], oacc[qb][db], 0, 0, 0);
      }
    }

    if (kt + 1 < ntiles) sstore(s ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: O^T element e of block (qb, db) is
  // d = db*32 + (e/4)*8 + g*4 + e%4 of query column l32
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = lrow[qb] + __shfl_xor(lrow[qb], 32);
    const float inv = 1.0f / lt;
    const int t = q0 + qb * 32 + l32;
    if (t < L) {
      bf16_t* orow = O + (size_t)map.stream_row(b, t) * ldo + h * ATT_D;
#pragma unroll
      for (int db = 0; db < ATT_D / 32; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int dd = db * 32 + e4 * 8 + g * 4;
          uint2 u;
          u.x = pack_bf16x2(oacc[qb][db][e4 * 4 + 0] * inv, oacc[qb][db][e4 * 4 + 1] * inv);
          u.y = pack_bf16x2(oacc[qb][db][e4 * 4 + 2] * inv, oacc[qb][db][e4 * 4 + 3] * inv);
          *(uint2*)(orow + dd) = u;
        }
    }
  }
}

hipError_t attention_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* vt, bf16_t* o,
                          int ldo, const RowMap& map, int B, int H, int L, int d,
                          float softmax_scale, hipStream_t st) {
  if (d != ATT_D) return hipErrorInvalidValue;
  const int nqt = (L + ATT_BM - 1) / ATT_BM;
  const int nblk = B * H * nqt;
  if (nblk == 0) return hipSuccess;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  KTimerScope timer(KS_ATTENTION, st);
  hipLaunchKernelGGL(attention_bf16_kernel, dim3(nblk), dim3(256), 0, st, q, k, vt, o, ldo, map,
                     H, L, scale_log2);
  return hipGetLastError();
}

}  // namespace dit
