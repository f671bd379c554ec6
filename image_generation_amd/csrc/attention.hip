// Flash-style joint attention for gfx950 (MFMA + LDS-staged K/V tiles), bf16
// and e4m3, head dim 64 or 128, any sequence length.
//
//   O[b, t, h*d + c] = sum_u softmax_u(Q[b,h,t] . K[b,h,u] * scale) V[b,h,u,c]
//
// Q, K and V arrive in the same layout, [B, H, L, d] row-major.
//
// Work split: one workgroup = 8 wave64s = 256 queries of one (b, h); each wave
// owns 32 queries and two waves share a SIMD.  In the bf16 kernel the two waves
// of a SIMD run half a tile apart (see the kernel), so one's softmax arithmetic
// runs while the other's score MFMAs do.  Scores are computed transposed, S^T = K Q^T, so
// every lane owns a query column: the softmax max is an in-lane reduction plus
// one exchange with lane ^ 32, and the row sum needs no exchange until the end.
// K rows are fed to the MFMA in the order (r with bits 2 and 3 swapped), which
// makes the 8 score registers a lane holds per 16-key chunk correspond to 8
// consecutive keys: exactly the B operand of the P V^T MFMA, so P never leaves
// registers.
//
// V^T operands without a transposed copy of V: a 64-key V tile sits in LDS row
// by row (as loaded), and the A operand of O^T = V^T P^T is read with gfx950's
// transposing LDS loads.  ds_read_b64_tr_b16 works on groups of 16 lanes: lane
// 4e + q of a group supplies 8 bytes (4 values) and lane 4q + r receives value r
// of the lanes 4e + q, e = 0..3; so when lane 4e + q points at V[key0 + e]
// [d0 + 4q .. + 3], lane j of the group receives keys key0 .. key0 + 3 of column
// d0 + j, four consecutive K values of the MFMA operand row j.  The 8-bit form
// does the same with 8 lanes' bytes: lane 2e + q supplies V[key0 + e][d0 + 8q ..
// + 7] and lane 8q + r receives keys key0 .. key0 + 7 of column d0 + 8q + r.  (This
// lane layout was measured on the GPU.)  The 16-byte chunks of each V row are
// stored permuted by an XOR with a function of the key, chosen so that the 32
// lanes one LDS cycle serves (4 keys x 64 bytes for bf16, 8 keys x 32 bytes for
// e4m3) fall in 64 distinct banks.
//
// Softmax reference max (bf16): exp2 is taken relative to a per-query reference
// m that only moves when a tile's maximum exceeds it by more than 2^8 (in exp2
// units); otherwise P <= 256 and the rescale of O and of the row sum is
// skipped.  The reference cancels exactly in O / l.  P enters P V^T as bf16, and
// the row sum l adds up those same bf16 values.
//
// K/V tiles of 64 keys are double-buffered in LDS, filled by direct
// global->LDS loads (each wave instruction writes 1 KB contiguously; padded or
// permuted K rows and permuted V rows are built by giving each lane the chunk
// that belongs at its slot).  Keys past L load row L - 1 and are masked to -inf;
// queries past L are computed on clamped rows and not stored.
#include "common.h"
#include "kernels.h"

namespace dit {

constexpr int ATT_BN = 64;          // keys per tile
constexpr int ATT_QW = 32;          // queries per wave
constexpr int ATT_WAVES = 8;
constexpr int ATT_BM = ATT_QW * ATT_WAVES;
constexpr float ATT_RESCALE_LOG2 = 8.0f;        // P stays <= 2^8 between rescales

typedef short s16x4v __attribute__((vector_size(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x2v __attribute__((vector_size(8)));
typedef short s16x8v __attribute__((vector_size(16)));
#define DIT_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// Transposing LDS reads (see above); p is each lane's own 8-byte source.
__device__ __forceinline__ s16x4v lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(DIT_LDS(s16x4v, (char*)p));
}
__device__ __forceinline__ i32x2v lds_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(DIT_LDS(i32x2v, (char*)p));
}

__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Tile geometry.  ES: element bytes (2 bf16, 1 e4m3).  K rows are padded by 16
// bytes (an odd number of 16-byte chunks per 64 banks for the row-wise fragment
// reads); V rows are unpadded with permuted chunks.
template <int D, int ES>
struct AttGeo {
  static constexpr int KROW = D * ES + 16;
  static constexpr int KC = KROW / 16;
  static constexpr int VROW = D * ES;
  static constexpr int VC = VROW / 16;
  static constexpr int KB = ATT_BN * KROW;
  static constexpr int VB = ATT_BN * VROW;
  static constexpr int SB = KB + VB;
  static constexpr int KI = KB / 1024;                     // K load instructions
  static constexpr int NI = SB / 1024;                     // per stage
  static constexpr int IPW = (NI + ATT_WAVES - 1) / ATT_WAVES;
  static_assert(KB % 1024 == 0 && VB % 1024 == 0, "stage must be whole 1-KB loads");
  // chunk permutation of V row `key` (XOR on the 16-byte chunk index)
  static __device__ __forceinline__ int vswz(int key) {
    if constexpr (ES == 2) return D == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
    else return D == 128 ? 2 * ((key >> 1) & 3) : 2 * ((key >> 2) & 1);
  }
};

// Per-lane source offsets (elements) of a stage's direct-to-LDS loads: wave w issues
// load instructions w, w + 8, ...; instruction i < KI fills K rows, the rest V rows.
template <int D, int ES>
struct AttLoads {
  using G = AttGeo<D, ES>;
  int doff[G::IPW];   // row * D + chunk * (16 / ES)
  int dkv[G::IPW];    // key row inside the tile
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < G::IPW; ++j) {
      const int inst = wave + j * ATT_WAVES;
      const int c = inst * 64 + lane;
      int row, chunk;
      if (inst < G::KI) {
        row = c / G::KC;
        chunk = min(c - row * G::KC, G::VC - 1);   // the pad slot repeats the last chunk
      } else {
        const int c2 = c - G::KI * 64;
        row = c2 / G::VC;
        chunk = (c2 - row * G::VC) ^ G::vswz(row);
      }
      doff[j] = row * D + chunk * (16 / ES);
      dkv[j] = row;
    }
  }
  // K and V tile kt of one (b, h) into `stage`; rows past L load row L - 1
  template <class T>
  __device__ __forceinline__ void issue(char* stage, const T* Kb, const T* Vb, int kt, int L,
                                        int wave) const {
    const int kv0 = kt * ATT_BN;
    const bool full = kv0 + ATT_BN <= L;
#pragma unroll
    for (int j = 0; j < G::IPW; ++j) {
      const int inst = wave + j * ATT_WAVES;
      if (inst >= G::NI) break;
      const T* base = inst < G::KI ? Kb : Vb;
      const T* src = base + (size_t)kv0 * D + doff[j];
      if (!full && kv0 + dkv[j] > L - 1) src = base + (size_t)(L - 1) * D + (doff[j] - dkv[j] * D);
      __builtin_amdgcn_global_load_lds((const void*)src, (void*)(stage + inst * 1024), 16, 0, 0);
    }
  }
};

// One 64-key tile of K or V in LDS: 64 unpadded rows of D elements whose 16-byte
// chunks sit permuted by an XOR with a function of the row.  K's permutation puts
// the 16 rows that one LDS cycle serves to a fragment read (16 lanes x 16 bytes,
// one chunk of 16 different keys) in 16 distinct bank groups; V's serves the
// transposing reads (see vswz).  A tile is NI 1-KB direct-to-LDS loads, IPW per wave.
template <int D, int ES>
struct KVTile {
  static constexpr int ROW = D * ES;
  static constexpr int CPR = ROW / 16;
  static constexpr int BYTES = ATT_BN * ROW;
  static constexpr int NI = BYTES / 1024;
  static constexpr int IPW = NI / ATT_WAVES;
  static_assert(NI % ATT_WAVES == 0, "tile loads split evenly over the waves");
  // bf16 reads take rows swap23(l) (+ 32 kb): 16 consecutive rows per cycle; e4m3
  // reads take rows ((l >> 2) & 1) * 32 + (l >> 3) * 4 + (l & 3) (+ 16 kb)
  static __device__ __forceinline__ int kswz(int r) {
    if constexpr (ES == 2) return ROW == 256 ? (r & 15) : ((r >> 1) & 7);
    else return ROW == 128 ? (((r >> 1) & 3) | ((r >> 3) & 4)) : (((r >> 2) & 1) | ((r >> 4) & 2));
  }
};

// Per-lane source of a tile's direct-to-LDS loads: instruction wave + 8 j covers
// LDS chunks (wave + 8 j) * 64 + lane, i.e. row `row[j]` and the logical chunk
// whose elements start at `off[j]`.
template <int D, int ES, bool IS_K>
struct TileLoads {
  using T = KVTile<D, ES>;
  int row[T::IPW];
  int off[T::IPW];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < T::IPW; ++j) {
      const int sl = (wave + j * ATT_WAVES) * 64 + lane;
      const int r = sl / T::CPR, pc = sl - r * T::CPR;
      const int lc = pc ^ (IS_K ? T::kswz(r) : AttGeo<D, ES>::vswz(r));
      row[j] = r;
      off[j] = lc * (16 / ES);
    }
  }
  // rows kv0 .. kv0 + 63 of one (b, h) into dst; rows past L load row L - 1
  template <class E>
  __device__ __forceinline__ void issue(char* dst, const E* base, int kv0, int L, int wave) const {
#pragma unroll
    for (int j = 0; j < T::IPW; ++j) {
      const int r = min(kv0 + row[j], L - 1);
      __builtin_amdgcn_global_load_lds((const void*)(base + (size_t)r * D + off[j]),
                                       (void*)(dst + (wave + j * ATT_WAVES) * 1024), 16, 0, 0);
    }
  }
};

// s_waitcnt vmcnt(n) lgkmcnt(0) for a wave-uniform n in 0..3
__device__ __forceinline__ void wait_vm_lgkm0(int n) {
  if (n >= 3) __builtin_amdgcn_s_waitcnt(3 | 0x0070);
  else if (n == 2) __builtin_amdgcn_s_waitcnt(2 | 0x0070);
  else if (n == 1) __builtin_amdgcn_s_waitcnt(1 | 0x0070);
  else __builtin_amdgcn_s_waitcnt(0x0070);
}

// Two wave groups in ping-pong: waves 0-3 and 4-7 (one of each per SIMD) run the
// same work one segment apart.  Each tile takes two barrier-separated segments;
// in each segment one group computes a tile's scores (MFMA-bound) while the other
// turns the previous tile's scores into P and P V^T (exp2-bound, with the P V^T
// MFMAs), so a SIMD's MFMA and vector units both have work at once instead of its
// two waves queueing on the same unit.  Segment hs runs, for group r, step hs - r:
// the scores of tile (hs - r)/2 when even, its P V^T when odd.
//
// K and V each have two LDS buffers, four arrays always named statically (the
// loop is unrolled over two tiles), so the compiler knows which array a pending
// direct-to-LDS load writes and lets reads of the others proceed.  K(t) is loaded
// in segment 2t - 2, after its buffer's last reader (group 1's scores of tile
// t - 2, segment 2t - 3); V(t) in segment 2t - 1, after group 1's P V^T of tile
// t - 2.  A batch has landed by the end of the segment after the one issuing it,
// one segment before its first reader.  Segments end in a plain s_barrier after
// the wave's own waits (__syncthreads()' fence would also wait for the batch in
// flight).
template <int D>
__global__ __launch_bounds__(ATT_WAVES * 64) void attention_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    bf16_t* __restrict__ O, int ldo, RowMap map, int H, int L, float scale_log2,
    const int* __restrict__ gate) {
  using T = KVTile<D, 2>;
  using G = AttGeo<D, 2>;
  if (gate_closed(gate)) return;
  __shared__ __attribute__((aligned(1024))) char sk0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char sk1[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char sv0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char sv1[T::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp = wave >> 2;         // ping-pong group
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

  const bf16_t* Qb = Q + (size_t)bh * L * D;
  const bf16_t* Kb = K + (size_t)bh * L * D;
  const bf16_t* Vb = V + (size_t)bh * L * D;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[q][c*16 + g*8 .. +8]
  const int q0 = qt * ATT_BM + wave * ATT_QW;
  bf16x8 qf[D / 16];
  {
    const int qr = min(q0 + l32, L - 1);
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qf[c] = *(const bf16x8*)(Qb + (size_t)qr * D + c * 16 + g * 8);
  }

  f32x16 oacc[D / 32];   // O^T blocks, one per 32 head channels
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float mref = -INFINITY;     // reference max (raw score units)
  float lsum = 0.f;           // this lane's partial row sum, relative to mref

  TileLoads<D, 2, true> ldk;
  TileLoads<D, 2, false> ldv;
  ldk.init(wave, lane);
  ldv.init(wave, lane);

  // transposing V reads: lane 4e + q of its 16-lane group sources key
  // (chunk base) + e, channels db*32 + (group & 1)*16 + 4q .. + 3
  const int tg = lane >> 4, ts = lane & 15, te = ts >> 2, tq = ts & 3;
  const int vsw = G::vswz(te);   // the rows a lane sources are all = te (mod 4)
  int vbase[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
    vbase[db] = (g * 8 + te) * T::ROW +
                (((4 * db + 2 * (tg & 1) + (tq >> 1)) ^ vsw) << 4) + 8 * (tq & 1);

  const int ntiles = (L + ATT_BN - 1) / ATT_BN;
  // K fragment of key block kb, d-chunk c: row kb*32 + swap23(l32), logical
  // 16-byte chunk 2c + g, stored at chunk (2c + g) ^ kswz(row) = kc0 ^ 2c
  const int krow = swap23(l32);
  const int kbase = krow * T::ROW;
  const int kc0 = g ^ T::kswz(krow);   // the same for krow + 32

  f32x16 sacc[2];
  // ---- scores of tile kt from K buffer sK: element e of sacc[kb] is key kv0 +
  // kb*32 + (e/8)*16 + g*8 + e%8 of query column l32; then the reference max
  auto scores = [&](const char* sK, int kt) {
    const int kv0 = kt * ATT_BN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
    // reads and MFMAs interleaved a pair at a time (measured 4-7% faster here than
    // all reads of a batch first, unlike the e4m3 kernel)
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf =
            *(const bf16x8*)(sK + kbase + kb * 32 * T::ROW + ((kc0 ^ (2 * c)) << 4));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sacc[kb], 0, 0, 0);
      }
    }
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
    // lane's half of the keys decides that as well as the whole row does (the test
    // is wave-wide), so the two halves exchange maxima only when it moves
    if (__any((mx - mref) * scale_log2 > ATT_RESCALE_LOG2)) {
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mref, mx);
      const float alpha = fast_exp2((mref - mnew) * scale_log2);
      mref = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
  };
  // ---- P of the scores in sacc (bf16, the B operand of O^T += V^T P^T) and P V^T
  // over its 4 chunks of 16 keys from V buffer sV; the V^T fragment of chunk ch
  // (keys ch*16 + g*8 .. + 7 of channel db*32 + l32) is two transposing reads
  auto pv = [&](const char* sV) {
    const float moff = mref * scale_log2;
    bf16x8 pf[4];
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        bf16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          t[e] = (__bf16)fast_exp2(fmaf(sacc[kb][ch * 8 + e], scale_log2, -moff));
        // the row sum takes the same bf16 weights that multiply V (two per
        // instruction, fp32 accumulation), so the weights applied sum to one
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{t[e], t[e + 1]}, one2, lsum, false);
        pf[kb * 2 + ch] = t;
      }
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const char* vp = sV + vbase[db] + ch * 16 * T::ROW;
        const s16x4v lo = lds_tr16(vp);
        const s16x4v hi = lds_tr16(vp + 4 * T::ROW);
        const s16x8v v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), pf[ch],
                                                           oacc[db], 0, 0, 0);
      }
    }
  };
  // end of a segment: this wave's LDS reads have returned and the batch it issued
  // one segment earlier has landed (`inflight`: this segment's own batch, which
  // may stay in flight); then the barrier.  The "memory" clobber keeps the
  // compiler from moving LDS accesses across it.
  auto seg_end = [&](int inflight) {
    wait_vm_lgkm0(inflight);
    asm volatile("s_barrier" ::: "memory");
  };

  ldk.issue(sk0, Kb, 0, L, wave);
  ldv.issue(sv0, Vb, 0, L, wave);
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  __syncthreads();

  // segments 2 t0 .. 2 t0 + 3 cover tiles t0 (buffers 0) and t0 + 1 (buffers 1);
  // group 1 runs one segment behind group 0.  Each group runs its own copy of the
  // loop (both pass the same barriers in the same order).  Every segment issues
  // one batch (past the last tile it reloads the last tile into a buffer no one
  // reads again), so the outstanding-load count is the same on every path.
  const int tlast = ntiles - 1;
  if (grp == 0) {
    for (int t0 = 0; t0 <= ntiles; t0 += 2) {
      ldk.issue(sk1, Kb, min(t0 + 1, tlast) * ATT_BN, L, wave);        // hs = 2 t0
      if (t0 < ntiles) scores(sk0, t0);
      seg_end(T::IPW);
      if (2 * t0 + 1 > 2 * ntiles) break;
      ldv.issue(sv1, Vb, min(t0 + 1, tlast) * ATT_BN, L, wave);        // hs = 2 t0 + 1
      pv(sv0);
      seg_end(T::IPW);
      if (2 * t0 + 2 > 2 * ntiles) break;
      ldk.issue(sk0, Kb, min(t0 + 2, tlast) * ATT_BN, L, wave);        // hs = 2 t0 + 2
      if (t0 + 1 < ntiles) scores(sk1, t0 + 1);
      seg_end(T::IPW);
      if (2 * t0 + 3 > 2 * ntiles) break;
      ldv.issue(sv0, Vb, min(t0 + 2, tlast) * ATT_BN, L, wave);        // hs = 2 t0 + 3
      pv(sv1);
      seg_end(T::IPW);
    }
  } else {
    for (int t0 = 0; t0 <= ntiles; t0 += 2) {
      ldk.issue(sk1, Kb, min(t0 + 1, tlast) * ATT_BN, L, wave);        // hs = 2 t0
      if (t0 >= 1) pv(sv1);
      seg_end(T::IPW);
      if (2 * t0 + 1 > 2 * ntiles) break;
      ldv.issue(sv1, Vb, min(t0 + 1, tlast) * ATT_BN, L, wave);        // hs = 2 t0 + 1
      scores(sk0, t0);
      seg_end(T::IPW);
      if (2 * t0 + 2 > 2 * ntiles) break;
      ldk.issue(sk0, Kb, min(t0 + 2, tlast) * ATT_BN, L, wave);        // hs = 2 t0 + 2
      pv(sv0);
      seg_end(T::IPW);
      if (2 * t0 + 3 > 2 * ntiles) break;
      ldv.issue(sv0, Vb, min(t0 + 2, tlast) * ATT_BN, L, wave);        // hs = 2 t0 + 3
      scores(sk1, t0 + 1);
      seg_end(T::IPW);
    }
  }
  // no direct-to-LDS load may outlive the workgroup
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- normalise and store: O^T element e of block db is
  // d = db*32 + (e/4)*8 + g*4 + e%4 of query column l32
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.0f / lt;
  const int t = q0 + l32;
  if (t < L) {
    bf16_t* orow = O + (size_t)map.stream_row(b, t) * ldo + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
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
// Same work split.  Q, K, V are e4m3 with one scale per (b, h) each, so the
// score scale sq * sk folds into the exp2 constant and sv into the final
// normalisation.  S^T uses v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales):
// for key block kb the MFMA row r is fed K row  g(r)*32 + kb*16 + i(r),
// g(r) = (r/4)&1, i(r) = (r/8)*4 + r%4, so a lane's 32 score registers over the
// 64-key tile are the 32 consecutive keys its lane group needs as the P operand
// of the fp8 P V^T MFMA; that operand's V^T fragment (channel db*32 + l32, keys
// g*32 .. + 31) is four 8-bit transposing reads.
//
// Softmax reference: in exp2 units the running row max is rounded up to an
// integer r, so P = 2^(t - r) <= 1 and 448 P never saturates e4m3.  When r
// moves by k, O and the row sum scale by exactly 2^-k, and the e4m3 rounding of
// 448 P is the same for every integer r (down to e4m3's subnormals): the result
// matches quantising against the final row max rounded the same way.  The row
// sum is that of the quantised P, taken by one more MFMA of the P codes against
// an all-ones operand, so the weights that multiply V sum to one.
template <int D>
__global__ __launch_bounds__(ATT_WAVES * 64) void attention_fp8_db_kernel(
    const fp8_t* __restrict__ Q, const fp8_t* __restrict__ K, const fp8_t* __restrict__ V,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    bf16_t* __restrict__ O, int ldo, RowMap map, int H, int L, float scale_log2,
    const int* __restrict__ gate) {
  using G = AttGeo<D, 1>;
  if (gate_closed(gate)) return;
  __shared__ __attribute__((aligned(1024))) char st0[G::SB];
  __shared__ __attribute__((aligned(1024))) char st1[G::SB];

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

  const fp8_t* Qb = Q + (size_t)bh * L * D;
  const fp8_t* Kb = K + (size_t)bh * L * D;
  const fp8_t* Vb = V + (size_t)bh * L * D;
  const float cs = scale_log2 * sq[bh] * sk[bh];   // raw score -> exp2 units

  // Q fragments: lane holds Q[q][c*64 + g*32 .. +32]
  const int q0 = qt * ATT_BM + wave * ATT_QW;
  i32x8 qf[D / 64];
  {
    const int qr = min(q0 + l32, L - 1);
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      const i32x4 lo = *(const i32x4*)(Qb + (size_t)qr * D + c * 64 + g * 32);
      const i32x4 hi = *(const i32x4*)(Qb + (size_t)qr * D + c * 64 + g * 32 + 16);
      qf[c] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
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

  AttLoads<D, 1> ld;
  ld.init(wave, lane);

  // transposing V reads: lane 2e + q of its 16-lane group sources key
  // g*32 + 8t + e, channels db*32 + (group & 1)*16 + 8q .. + 7
  const int tg = lane >> 4, ts = lane & 15, te = ts >> 1, tq = ts & 1;
  const int vsw = G::vswz(te);   // the rows a lane sources are all = te (mod 8)
  int vbase[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
    vbase[db] = (g * 32 + te) * G::VROW + (((2 * db + (tg & 1)) ^ vsw) << 4) + 8 * tq;

  const int ntiles = (L + ATT_BN - 1) / ATT_BN;
  // K row fed to MFMA row l32 of key block kb
  const int krow0 = ((l32 >> 2) & 1) * 32 + (l32 >> 3) * 4 + (l32 & 3);
  ld.issue(st0, Kb, Vb, 0, L, wave);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    char* cur = (kt & 1) ? st1 : st0;
    char* nxt = (kt & 1) ? st0 : st1;
    if (kt + 1 < ntiles) ld.issue(nxt, Kb, Vb, kt + 1, L, wave);
    const char* sK = cur;
    const char* sV = cur + G::KB;
    const int kv0 = kt * ATT_BN;

    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 64; ++c) {
        const char* q_ = sK + (krow0 + kb * 16) * G::KROW + c * 64 + g * 32;
        const i32x4 lo = *(const i32x4*)q_, hi = *(const i32x4*)(q_ + 16);
        const i32x8 kf = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[c], sacc[kb], 0, 0, 0,
                                                                   127, 0, 127);
      }
    }
    // element e of sacc[kb] is key kv0 + g*32 + kb*16 + e of query column l32
    if (kv0 + ATT_BN > L) {
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
      for (int db = 0; db < D / 32; ++db)
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
    for (int db = 0; db < D / 32; ++db) {
      const char* vp = sV + vbase[db];
      const i32x2v t0 = lds_tr8(vp), t1 = lds_tr8(vp + 8 * G::VROW);
      const i32x2v t2 = lds_tr8(vp + 16 * G::VROW), t3 = lds_tr8(vp + 24 * G::VROW);
      const i32x8 vf = i32x8{t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
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
    bf16_t* orow = O + (size_t)map.stream_row(b, t) * ldo + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
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

// The e4m3 kernel for head dim 128 in the bf16 kernel's ping-pong form (see there):
// unpadded K tiles with the e4m3 row permutation, one 1-KB load per wave for each
// of K and V, four statically named LDS buffers.  (Head dim 64 has 4-KB tiles,
// fewer loads than waves, and uses the double-buffered kernel above.)
template <int D>
__global__ __launch_bounds__(ATT_WAVES * 64) void attention_fp8_kernel(
    const fp8_t* __restrict__ Q, const fp8_t* __restrict__ K, const fp8_t* __restrict__ V,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    bf16_t* __restrict__ O, int ldo, RowMap map, int H, int L, float scale_log2,
    const int* __restrict__ gate) {
  static_assert(D == 128, "head dim 128");
  using T = KVTile<D, 1>;
  using G = AttGeo<D, 1>;
  if (gate_closed(gate)) return;
  __shared__ __attribute__((aligned(1024))) char sk0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char sk1[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char sv0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char sv1[T::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp = wave >> 2;         // ping-pong group
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

  const fp8_t* Qb = Q + (size_t)bh * L * D;
  const fp8_t* Kb = K + (size_t)bh * L * D;
  const fp8_t* Vb = V + (size_t)bh * L * D;
  const float cs = scale_log2 * sq[bh] * sk[bh];   // raw score -> exp2 units

  // Q fragments: lane holds Q[q][c*64 + g*32 .. +32]
  const int q0 = qt * ATT_BM + wave * ATT_QW;
  i32x8 qf[D / 64];
  {
    const int qr = min(q0 + l32, L - 1);
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      const i32x4 lo = *(const i32x4*)(Qb + (size_t)qr * D + c * 64 + g * 32);
      const i32x4 hi = *(const i32x4*)(Qb + (size_t)qr * D + c * 64 + g * 32 + 16);
      qf[c] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
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

  TileLoads<D, 1, true> ldk;
  TileLoads<D, 1, false> ldv;
  ldk.init(wave, lane);
  ldv.init(wave, lane);

  // transposing V reads: lane 2e + q of its 16-lane group sources key
  // g*32 + 8t + e, channels db*32 + (group & 1)*16 + 8q .. + 7
  const int tg = lane >> 4, ts = lane & 15, te = ts >> 1, tq = ts & 1;
  const int vsw = G::vswz(te);   // the rows a lane sources are all = te (mod 8)
  int vbase[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
    vbase[db] = (g * 32 + te) * T::ROW + (((2 * db + (tg & 1)) ^ vsw) << 4) + 8 * tq;

  const int ntiles = (L + ATT_BN - 1) / ATT_BN;
  // K row fed to MFMA row l32 of key block kb: krow0 + 16 kb; its logical 16-byte
  // chunks 4c + 2g and 4c + 2g + 1 sit at those XOR kswz(row) (the same for both kb)
  const int krow0 = ((l32 >> 2) & 1) * 32 + (l32 >> 3) * 4 + (l32 & 3);
  const int kbase = krow0 * T::ROW;
  const int ksw = T::kswz(krow0);

  f32x16 sacc[2];
  // ---- scores of tile kt from K buffer sK: element e of sacc[kb] is key kv0 +
  // g*32 + kb*16 + e of query column l32; then the reference
  auto scores = [&](const char* sK, int kt) {
    const int kv0 = kt * ATT_BN;
    // all 8 K fragment reads of the tile before its 4 MFMAs: while a direct-to-LDS
    // load is pending the compiler can only wait for all of a wave's LDS reads at
    // once, so one wait here instead of one per MFMA (measured 1-2% faster; the
    // bf16 kernel is faster with its reads interleaved)
    i32x8 kf[2][D / 64];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < D / 64; ++c) {
        const char* r_ = sK + kbase + kb * 16 * T::ROW;
        const i32x4 lo = *(const i32x4*)(r_ + (((4 * c + 2 * g) ^ ksw) << 4));
        const i32x4 hi = *(const i32x4*)(r_ + (((4 * c + 2 * g + 1) ^ ksw) << 4));
        kf[kb][c] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 64; ++c)
        sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[kb][c], qf[c], sacc[kb], 0,
                                                                   0, 0, 127, 0, 127);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * (D / 64), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * (D / 64), 0);
    if (kv0 + ATT_BN > L) {
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
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
  };
  // ---- the e4m3 codes of 448 P = 2^(t - mref + log2 448) and P V^T from V buffer sV
  auto pv = [&](const char* sV) {
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
    for (int db = 0; db < D / 32; ++db) {
      const char* vp = sV + vbase[db];
      const i32x2v t0 = lds_tr8(vp), t1 = lds_tr8(vp + 8 * T::ROW);
      const i32x2v t2 = lds_tr8(vp + 16 * T::ROW), t3 = lds_tr8(vp + 24 * T::ROW);
      const i32x8 vf = i32x8{t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, oacc[db], 0, 0, 0, 127,
                                                                 0, 127);
    }
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lacc, 0, 0, 0, 127, 0, 127);
  };
  auto seg_end = [&]() {
    wait_vm_lgkm0(T::IPW);
    asm volatile("s_barrier" ::: "memory");
  };

  ldk.issue(sk0, Kb, 0, L, wave);
  ldv.issue(sv0, Vb, 0, L, wave);
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  __syncthreads();

  // the same segment schedule as the bf16 kernel
  const int tlast = ntiles - 1;
  if (grp == 0) {
    for (int t0 = 0; t0 <= ntiles; t0 += 2) {
      ldk.issue(sk1, Kb, min(t0 + 1, tlast) * ATT_BN, L, wave);   // hs = 2 t0
      if (t0 < ntiles) scores(sk0, t0);
      seg_end();
      if (2 * t0 + 1 > 2 * ntiles) break;
      ldv.issue(sv1, Vb, min(t0 + 1, tlast) * ATT_BN, L, wave);   // hs = 2 t0 + 1
      pv(sv0);
      seg_end();
      if (2 * t0 + 2 > 2 * ntiles) break;
      ldk.issue(sk0, Kb, min(t0 + 2, tlast) * ATT_BN, L, wave);   // hs = 2 t0 + 2
      if (t0 + 1 < ntiles) scores(sk1, t0 + 1);
      seg_end();
      if (2 * t0 + 3 > 2 * ntiles) break;
      ldv.issue(sv0, Vb, min(t0 + 2, tlast) * ATT_BN, L, wave);   // hs = 2 t0 + 3
      pv(sv1);
      seg_end();
    }
  } else {
    for (int t0 = 0; t0 <= ntiles; t0 += 2) {
      ldk.issue(sk1, Kb, min(t0 + 1, tlast) * ATT_BN, L, wave);   // hs = 2 t0
      if (t0 >= 1) pv(sv1);
      seg_end();
      if (2 * t0 + 1 > 2 * ntiles) break;
      ldv.issue(sv1, Vb, min(t0 + 1, tlast) * ATT_BN, L, wave);   // hs = 2 t0 + 1
      scores(sk0, t0);
      seg_end();
      if (2 * t0 + 2 > 2 * ntiles) break;
      ldk.issue(sk0, Kb, min(t0 + 2, tlast) * ATT_BN, L, wave);   // hs = 2 t0 + 2
      pv(sv0);
      seg_end();
      if (2 * t0 + 3 > 2 * ntiles) break;
      ldv.issue(sv0, Vb, min(t0 + 2, tlast) * ATT_BN, L, wave);   // hs = 2 t0 + 3
      scores(sk1, t0 + 1);
      seg_end();
    }
  }
  // no direct-to-LDS load may outlive the workgroup
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const float inv = sv[bh] / lacc[0];
  const int t = q0 + l32;
  if (t < L) {
    bf16_t* orow = O + (size_t)map.stream_row(b, t) * ldo + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
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
// per 64 queries of one (b, h), one query per lane, 64-key K and V tiles in LDS
// (V stored transposed there)
// (every lane reads the same key, so the LDS reads broadcast); online softmax in
// exp2 units with the scale folded into q.
template <int HD>
__global__ __launch_bounds__(64) void attention_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
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
  const float* Vb = V + (size_t)bh * L * HD;
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
      sV[c][lane] = kr < L ? Vb[(size_t)kr * HD + c] : 0.f;
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

hipError_t attention_f32(const float* q, const float* k, const float* v, float* o, int ldo,
                         const RowMap& map, int B, int H, int L, int d, float softmax_scale,
                         hipStream_t st) {
  if ((d != 32 && d != 64) || L < 1) return hipErrorInvalidValue;
  if (B * H == 0) return hipSuccess;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  KTimerScope timer(KS_ATTENTION, st);
  const dim3 grid((L + 63) / 64, B * H);
  if (d == 64)
    hipLaunchKernelGGL(attention_f32_kernel<64>, grid, dim3(64), 0, st, q, k, v, o, ldo, map, H,
                       L, scale_log2, launch_gate());
  else
    hipLaunchKernelGGL(attention_f32_kernel<32>, grid, dim3(64), 0, st, q, k, v, o, ldo, map, H,
                       L, scale_log2, launch_gate());
  return hipGetLastError();
}

hipError_t attention_fp8(const fp8_t* q8, const fp8_t* k8, const fp8_t* v8, const float* sq,
                         const float* sk, const float* sv, bf16_t* o, int ldo, const RowMap& map,
                         int B, int H, int L, int d, float softmax_scale, hipStream_t st) {
  if ((d != 64 && d != 128) || L < 1) return hipErrorInvalidValue;
  const int nqt = (L + ATT_BM - 1) / ATT_BM;
  const int nblk = B * H * nqt;
  if (nblk == 0) return hipSuccess;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  KTimerScope timer(KS_ATTENTION, st);
  auto kern = d == 128 ? attention_fp8_kernel<128> : attention_fp8_db_kernel<64>;
  hipLaunchKernelGGL(kern, dim3(nblk), dim3(ATT_WAVES * 64), 0, st, q8, k8, v8, sq, sk, sv, o, ldo,
                     map, H, L, scale_log2, launch_gate());
  return hipGetLastError();
}

hipError_t attention_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* v, bf16_t* o,
                          int ldo, const RowMap& map, int B, int H, int L, int d,
                          float softmax_scale, hipStream_t st) {
  if ((d != 64 && d != 128) || L < 1) return hipErrorInvalidValue;
  const int nqt = (L + ATT_BM - 1) / ATT_BM;
  const int nblk = B * H * nqt;
  if (nblk == 0) return hipSuccess;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  KTimerScope timer(KS_ATTENTION, st);
  auto kern = d == 128 ? attention_bf16_kernel<128> : attention_bf16_kernel<64>;
  hipLaunchKernelGGL(kern, dim3(nblk), dim3(ATT_WAVES * 64), 0, st, q, k, v, o, ldo, map, H, L,
                     scale_log2, launch_gate());
  return hipGetLastError();
}

}  // namespace dit
