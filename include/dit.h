/*
 * dit.h - C ABI of libdit, the MI355X (gfx950) DiT denoise-step library.
 *
 * What it computes.  One flow-matching Euler step of a FLUX-shaped diffusion
 * transformer over joint text + image tokens: adaLN-modulated LayerNorm, fused
 * QKV projection with 2-D RoPE, joint softmax attention, output projection and
 * GELU-tanh MLP with gated residuals, repeated over double-stream and
 * single-stream blocks; then the velocity head and the Euler (and CFG) update.
 * The First-Block-Cache test decides, after the first block, whether the
 * remaining blocks are skipped and their cached residual reused.
 *
 * Sources.  The step is the one the pages on image-generation speed keep
 * returning to: the denoising stage dominates the pipeline and attention plus
 * matrix products dominate it (devotd.net VisualGen article on FLUX Klein,
 * stage-latency table and the section on why the speed-ups differ); the
 * First-Block-Cache test is the unsloth studio diffusion.py commit "Add opt-in
 * step caching (First-Block-Cache)"; RoPE as its own step and the scheduler /
 * flow shift / solver triple come from the vflash "Optimization ledger" page
 * (table "Accepted or exposed"; section "Fewer steps require a new contract");
 * fp8 W8A8 with dynamic scales from the runinfra.ai image-gen runbook,
 * "Optimization stack" table.  The pages give no formulas: the exact
 * definitions implemented here are the readings listed in the design notes
 * shipped with the library (LN eps 1e-6 without affine, (1 + scale) modulation,
 * interleaved-pair 2-D RoPE with base 10000, tanh GELU, shifted sigmas
 * s*t / (1 + (s-1) t), rel-L1 = sum|r - a| / sum|a| with a strict "<").
 *
 * Conventions (every entry point).
 *   - The caller owns all memory.  Pointers named "device" are HIP device
 *     pointers (e.g. torch tensor data_ptr()), 16-byte aligned, contiguous,
 *     row-major.  The library allocates nothing and keeps no state between
 *     calls; scratch comes from a caller workspace sized by
 *     dit_workspace_bytes() (dit_step_at_workspace_bytes() for
 *     dit_denoise_step_at()).  (Two exceptions: the handle of a replayed loop,
 *     dit_loop_graph_create() to dit_loop_graph_destroy(); and the static
 *     device array that dit_modulation_static() uses instead of a workspace.)
 *   - stream: a hipStream_t (NULL = default stream).  Work is enqueued
 *     asynchronously; only fbcache_should_skip() and dit_denoise_step() with an
 *     enabled cache synchronise that stream, to hand the skip decision to the
 *     host, and the replayed loop's create / sync / reset calls, which move its
 *     state between host and device.
 *   - Return value: DIT_OK (0) or a negative DIT_ERR_* code.  All arguments are
 *     validated before anything is enqueued; on an error nothing has been
 *     launched (except DIT_ERR_HIP, raised by the runtime mid-way, and
 *     DIT_ERR_NONFINITE, raised after the cache test ran).  Nothing throws or
 *     aborts across the ABI.  dit_last_error() gives a message for the calling
 *     thread's last failure.
 *   - Weights follow torch.nn.Linear: W is [out, in], y = x W^T + b, with the
 *     bias always fp32 [out].
 *   - Runs only on gfx950; any other device gives DIT_ERR_UNSUPPORTED.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported symbols (the library is built with hidden default visibility). */
#define DIT_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ status */
#define DIT_OK 0
#define DIT_ERR_INVALID_ARG (-1)  /* bad pointer, shape, alignment or value        */
#define DIT_ERR_UNSUPPORTED (-2)  /* dtype / shape / device the library does not support */
#define DIT_ERR_WORKSPACE (-3)    /* workspace smaller than dit_workspace_bytes()   */
#define DIT_ERR_HIP (-4)          /* the HIP runtime reported an error              */
#define DIT_ERR_NONFINITE (-5)    /* NaN / Inf reached the First-Block-Cache test   */

/* ------------------------------------------------------------------ dtypes */
#define DIT_F32 0
#define DIT_BF16 1
#define DIT_FP8 2   /* OCP e4m3 ("e4m3fn") */
#define DIT_MXFP4 3 /* OCP MXFP4: E2M1 elements, one E8M0 scale per 32 (blocks only) */
#define DIT_MXFP4_FP8ATTN 4 /* MXFP4 block linears with e4m3 attention (blocks only) */

#define DIT_BLOCK_DOUBLE 0
#define DIT_BLOCK_SINGLE 1

/* Workspace purposes for dit_workspace_bytes(). */
#define DIT_WS_ATTENTION 0
#define DIT_WS_BLOCK 1
#define DIT_WS_STEP 2
#define DIT_WS_MODULATION 3
#define DIT_WS_FBCACHE 4

/* Token layout of one denoise problem.
 *   B       batch rows (1, or 2 for a CFG pair: row 0 positive, row 1 negative)
 *   Lt      text tokens (>= 0)
 *   grid_h, grid_w  patch grid; Li = grid_h * grid_w image tokens
 *   D, H, F hidden size, heads (head dim D / H: 64 or 128; 32 or 64 for DIT_F32),
 *           MLP hidden size
 * Joint token order is [text ; image]: token t < Lt is text, token Lt + i is
 * image patch (i / grid_w, i % grid_w). */
typedef struct dit_dims {
  int B, Lt, grid_h, grid_w, D, H, F;
} dit_dims;

/* One linear layer on the device: w [out, in], b fp32 [out].
 *   bf16 layers: w bf16, w_scale NULL.
 *   fp8 layers (DIT_FP8 blocks): w OCP e4m3 and w_scale fp32 [out], the
 *   per-output-channel scale (weight = code * w_scale[n]), as produced by
 *   dit_quantize_rows() on the bf16 weight.
 *   fp32 layers (DIT_F32 models and blocks): w fp32, w_scale NULL.
 *   MXFP4 layers (DIT_MXFP4 blocks): w E2M1 codes [out, in / 2] and w_mx their
 *   E8M0 block scales [in / 256][dit_mx_rows(out)][8], both as produced by
 *   dit_quantize_mxfp4() on the bf16 weight; in a multiple of 256. */
typedef struct dit_linear {
  const void* w;
  const float* b;
  const float* w_scale;
  const unsigned char* w_mx;
} dit_linear;

/* A transformer block.
 * Double-stream (kind DIT_BLOCK_DOUBLE): index 0 = image stream, 1 = text stream;
 *   qkv [3D, D] (rows: q then k then v, head-major inside each), proj [D, D],
 *   mlp1 [F, D], mlp2 [D, F].
 * Single-stream (kind DIT_BLOCK_SINGLE): lin1 [3D + F, D] (q, k, v, MLP-in),
 *   lin2 [D, D + F] (input: [attention out, GELU(MLP-in)]). */
typedef struct dit_block {
  int kind;
  dit_linear qkv[2], proj[2], mlp1[2], mlp2[2];
  dit_linear lin1, lin2;
} dit_block;

/* The whole model.  blocks: host array of n_double double blocks followed by
 * n_single single blocks.  mod: every modulation linear stacked row-wise into
 * one [N_mod, D] matrix, N_mod = (12 n_double + 3 n_single + 2) D, in the order
 * double block j image (shift1, scale1, gate1, shift2, scale2, gate2) then text
 * (same six), single block j (shift, scale, gate), final layer (shift, scale). */
typedef struct dit_model {
  dit_dims dims;
  int n_double, n_single;
  const dit_block* blocks;
  dit_linear time1;      /* [D, 256] */
  dit_linear time2;      /* [D, D]   */
  dit_linear img_in;     /* [D, C_in] */
  dit_linear final_out;  /* [C_in, D] */
  dit_linear mod;        /* [N_mod, D] */
  int C_in;              /* patch features, <= 64 */
  float guidance;        /* CFG scale (B == 2) */
  int dtype;             /* DIT_BF16; DIT_FP8: the blocks' linears and attention run
                            in e4m3 with dynamic per-token activation scales, the
                            modulation, embedders, timestep MLP and velocity head stay
                            bf16; DIT_MXFP4: the blocks' linears W4A4 in MXFP4 (see
                            dit_block_forward), the rest as for DIT_FP8;
                            DIT_MXFP4_FP8ATTN: the same with e4m3 attention;
                            DIT_F32: every weight and activation fp32 (head dim
                            32 or 64; reference precision for small models) */
} dit_model;

/* Caller-held First-Block-Cache state; resuming a loop = passing it back. */
typedef struct dit_fbcache {
  int enabled;       /* 0: no test, every block runs, state untouched           */
  float threshold;   /* skip iff rel < threshold (0: never skip; +inf: always   */
                     /* after the first full step)                              */
  int has_anchor;    /* in/out: 0 until a fully computed step stored an anchor  */
  float* anchor;     /* device fp32 [B, Li, D]: first block's residual at the   */
                     /* last fully computed step                                */
  float* cached;     /* device fp32 [B, Li, D]: image hidden after the last     */
                     /* block minus image hidden after block 0, same step       */
  /* Skip policy on top of the rel test (>= 0 each; zero-initialised = plain test).
   * Warm-up and the cache's threshold as the tuning levers: "Optimization ledger",
   * the optimisation table (warm-up of a step cache); the VisualGen article on
   * FLUX Klein, Cache-DiT paragraph (residual-difference threshold). */
  int warmup_steps;  /* the first warmup_steps steps taken with the cache enabled  */
                     /* compute in full whatever rel is                         */
  int max_skips;     /* after max_skips consecutive skipped steps the next step  */
                     /* computes in full; 0: no limit                           */
  int steps_done;    /* in/out: steps taken with the cache enabled              */
  int skip_run;      /* in/out: consecutive skipped steps ending at the last one */
} dit_fbcache;

typedef struct dit_step_info {
  double rel;        /* relative L1 change of the first block's residual        */
                     /* (+inf when there is no anchor or the cache is disabled) */
  int skipped;       /* 1 if blocks 1.. were skipped                             */
} dit_step_info;

/* ------------------------------------------------------------------ helpers */

/* Static message for a status code. */
DIT_API const char* dit_status_string(int status);
/* Message of the calling thread's last failed call ("" if none). */
DIT_API const char* dit_last_error(void);

/* Bytes of device workspace an entry point needs.  purpose: DIT_WS_*;
 * n_steps is used by DIT_WS_MODULATION only.  Returns 0 for invalid dims. */
DIT_API size_t dit_workspace_bytes(const dit_dims* dims, int purpose, int n_steps);

/* Shifted flow-matching sigmas (host, fp64): tau_i = 1 - i/n,
 * out[i] = shift tau_i / (1 + (shift - 1) tau_i), i = 0..n (n + 1 values). */
DIT_API int dit_sigmas(int n_steps, double shift, double* out_host);

/* 2-D RoPE table, device fp32 [Lt + Li, d/2, 2] = (cos, sin) of the angle of
 * pair p at token t: pairs p < d/4 turn with the patch row, p >= d/4 with the
 * patch column, pair j of an axis at theta^(-j/(d/4)) radians per position;
 * text tokens sit at (0, 0). */
DIT_API int dit_rope_table(int grid_h, int grid_w, int Lt, int head_dim, double theta, float* table,
                   void* stream);

/* Opt-in launch timing for benchmarks.  While a timer is installed on the
 * calling thread, every kernel the library launches from a site whose bit is
 * set in site_mask is bracketed by hipEventRecord(start[i]) / (stop[i]) on the
 * launch stream, and sites[i] receives the site id, i = count++ (nothing is
 * recorded once count == capacity).  The caller creates the hipEvent_t
 * handles and reads the times after synchronising; NULL uninstalls. */
#define DIT_SITE_ATTENTION 0    /* flash attention                              */
#define DIT_SITE_GEMM_QKV 1     /* QKV projection + RoPE epilogue (double)      */
#define DIT_SITE_GEMM_RESID 2   /* proj / mlp2 / lin2 + gated residual          */
#define DIT_SITE_GEMM_GELU 3    /* mlp1 + GELU (double)                         */
#define DIT_SITE_GEMM_LIN1 4    /* single-block linear1: QKV + RoPE | GELU      */
#define DIT_SITE_GEMM_F32 5     /* plain fp32-out GEMM (modulation, final)      */
#define DIT_SITE_GEMM_SILU 6    /* timestep MLP                                 */
#define DIT_SITE_LN 7           /* LayerNorm + modulate                         */
#define DIT_SITE_FBC 8          /* First-Block-Cache reduction                  */
#define DIT_SITE_OTHER 9        /* embeddings, cache apply/commit, Euler, RoPE  */
#define DIT_SITE_QUANT 10       /* fp8 activation quantisation passes           */
typedef struct dit_kernel_timer {
  unsigned site_mask;
  int capacity;
  int count;
  int* sites;        /* host [capacity] */
  void** start;      /* host [capacity] of hipEvent_t */
  void** stop;       /* host [capacity] of hipEvent_t */
} dit_kernel_timer;
DIT_API int dit_set_kernel_timer(dit_kernel_timer* timer);

/* ------------------------------------------------------------------ entry points */

/* One linear layer: y[M, N] = x[M, K] W^T + b (bf16 operands, fp32 accumulate).
 *   x: device bf16 [M, K] (row stride K); lin->w bf16 [N, K]; lin->b fp32 [N];
 *   y: device [M, N], y_dtype DIT_F32 or DIT_BF16.  K % 64 == 0, N % 4 == 0.
 *   The same MFMA kernel as the block projections.  Workspace: none. */
DIT_API int dit_linear_forward(const void* x, int M, int K, const dit_linear* lin, int N, void* y,
                       int y_dtype, void* stream);

/* Joint softmax attention, no mask: O = softmax(Q K^T * softmax_scale) V, per
 * (batch, head) over all L tokens (the joint text + image attention of a block:
 * VisualGen article on FLUX Klein, section on why the speed-ups differ, where
 * BF16 attention is the largest part of the DiT's kernel time; cuDNN FP8
 * attention is the low-precision variant there).
 *   q, k, v: device [B, H, L, head_dim] row-major, all three the same layout;
 *   o: device [B, L, H * head_dim] (token-major), bf16 (fp32 for DIT_F32).
 *   L >= 1, any value (keys past the last tile are masked; no padding needed).
 *   dtype DIT_BF16: q, k, v bf16, head_dim 64 or 128; scales NULL.  P enters the
 *     P V product as bf16.
 *   dtype DIT_FP8: q, k, v OCP e4m3, head_dim 64 or 128, each with one fp32
 *     scale per (b, h) in q_scale / k_scale / v_scale [B * H] (value = code *
 *     scale); with t the scores in exp2 units and r the row maximum of t rounded
 *     up to an integer, P = 2^(t - r) enters P V as e4m3(448 P) / 448 and the
 *     normaliser is the sum of those quantised P.
 *   dtype DIT_F32: q, k, v, o fp32, head_dim 32 or 64 (reference precision).
 *   Softmax statistics and both products accumulate in fp32.  Workspace: none.
 *   Errors: DIT_ERR_INVALID_ARG for NULL / misaligned pointers, B, H or L < 1,
 *   a non-finite scale or missing fp8 scales; DIT_ERR_UNSUPPORTED for another
 *   head_dim or dtype.  The caller keeps ownership of every buffer. */
DIT_API int dit_attention(const void* q, const void* k, const void* v, void* o,
                          const float* q_scale, const float* k_scale, const float* v_scale,
                          int B, int H, int L, int head_dim, int dtype, float softmax_scale,
                          void* stream);

/* Dynamic per-row e4m3 quantisation (the W8A8 recipe): for each row r,
 *   scale[r] = amax_r / 448 (1 if the row is all zero),
 *   dst[r, c] = e4m3 code of src[r, c] * (448 / amax_r), round to nearest even,
 *   saturating; both factors are single correctly rounded fp32 divisions.
 *   src: device [rows, width], row stride src_ld elements, src_dtype DIT_BF16;
 *   dst: device e4m3 [rows, width], row stride dst_ld; scale: device fp32 [rows].
 *   width, src_ld, dst_ld multiples of 8.  Used offline for fp8 weights (one
 *   scale per output channel) and by the fp8 blocks for their activations. */
DIT_API int dit_quantize_rows(const void* src, int src_dtype, int src_ld, int rows, int width,
                              void* dst, int dst_ld, float* scale, void* stream);

/* MXFP4 block-scaled 4-bit quantisation of rows (the W4A4 variant next to the
 * fp8 path; OCP microscaling: E2M1 elements sharing one E8M0 scale per 32
 * consecutive elements of a row).  For each row r and block of 32:
 *   e = floor(log2(amax)) - 2, clamped to [-127, 127] (0 for an all-zero block);
 *   each element x / 2^e is rounded to the nearest E2M1 value (0, 0.5, 1, 1.5, 2,
 *   3, 4, 6 and negatives), ties to the even mantissa, beyond 6 saturating.
 *   src: device bf16 (src_dtype DIT_BF16) or fp32 (DIT_F32) [rows, src_ld];
 *   width % 256 == 0, src_ld >= width, src_ld % 8 == 0;
 *   codes: device [rows, width / 2] bytes, element 2j of a row in the low nibble
 *     of byte j;
 *   scales: device E8M0 bytes (2^(byte - 127)) in the GEMM's order
 *     [width / 256][dit_mx_rows(rows)][8]: the 8 block scales of one row in one
 *     256-wide slab, stored as blocks 0, 2, 4, 6, 1, 3, 5, 7; the padding rows
 *     are written as 127 (2^0).
 * Weights (offline) and activations use the same routine.  Workspace: none.
 * Reading of the pages: their 4-bit format is NVFP4 (VisualGen article on FLUX
 * Klein, checkpoint and speed tables; the diffusion-backend commit, precision per
 * GPU generation: nvfp4 / fp8 / mxfp8); gfx950's block-scaled FP4 MFMA takes OCP
 * MX scales, so that is the format here. */
DIT_API int dit_quantize_mxfp4(const void* src, int src_dtype, int src_ld, int rows, int width,
                               void* codes, unsigned char* scales, void* stream);
/* Rows of an MXFP4 scale array for `rows` rows: rows rounded up to 256. */
DIT_API int dit_mx_rows(int rows);

/* W4A4 linear y = x W^T + b on MXFP4 operands, both as written by
 * dit_quantize_mxfp4 (x [M, K], W [N, K]): block-scaled MFMAs
 * (v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1 operands, each lane's E8M0 block
 * scale), fp32 accumulation; b fp32 [N] or NULL; y device [M, N], DIT_F32 or
 * DIT_BF16.  K % 256 == 0, N % 4 == 0.  Workspace: none. */
DIT_API int dit_linear_mxfp4(const void* x_codes, const unsigned char* x_scales, int M, int K,
                             const void* w_codes, const unsigned char* w_scales, const float* b,
                             int N, void* y, int y_dtype, void* stream);

/* One transformer block, in place on the joint residual stream.
 *   x: device [B, Lt + Li, D], dtype x_dtype (DIT_F32 or DIT_BF16), updated;
 *      a bf16 x is carried in fp32 through both residual updates and rounded
 *      once at the end.
 *   mod: device fp32 modulation vectors for batch row b at mod + b * mod_bstride
 *        (mod_bstride = 0 shares them): double block 12 D-vectors (image
 *        shift1, scale1, gate1, shift2, scale2, gate2, then text), single 3.
 *   rope: device table from dit_rope_table() for these dims.
 *   dtype: DIT_BF16; DIT_FP8 (e4m3 linears with w_scale set, per-token
 *   activation scales, e4m3 attention with per-(b, h) scales); DIT_MXFP4 (W4A4
 *   linears with w_mx set: each linear's bf16 input is quantised to MXFP4 on the
 *   fly, 32-value blocks along the input dimension; attention in bf16; D and F
 *   multiples of 256); DIT_MXFP4_FP8ATTN (the same linears, attention in e4m3 as
 *   for DIT_FP8); DIT_F32 (fp32 weights, head dim 32 or 64).  bf16 / fp8 /
 *   MXFP4 blocks take head dim 64 or 128 and any token counts.
 *   workspace >= DIT_WS_BLOCK bytes. */
DIT_API int dit_block_forward(const dit_dims* dims, const dit_block* blk, int dtype, void* x, int x_dtype,
                      const float* mod, long mod_bstride, const float* rope, void* workspace,
                      size_t ws_bytes, void* stream);

/* Where a block leaves its intermediates in a DIT_WS_BLOCK workspace, for tests
 * and debugging (the stage-by-stage comparison of a block with a reference).
 * After dit_block_forward() the buffers hold that block's values.  Row order
 * of the [rows, *] buffers: a single-stream block uses the joint order (b, t);
 * a double-stream block puts all image rows first (batch-major), then all
 * text rows.  Pointers are into the caller's workspace; nothing is copied. */
typedef struct dit_block_views {
  void* ln;          /* bf16 [B L, D]: LN-modulate output (bf16 blocks; the      */
                     /* second LN of a double block once the block has run)      */
  void* ln8;         /* e4m3 [B L, D] and                                         */
  float* ln_scale;   /* fp32 [B L]: the same for fp8 blocks                       */
  void* q;           /* bf16 [B, H, L, d]: Q (rotated)                            */
  void* k;           /* bf16 [B, H, L, d]: K (rotated)                            */
  void* v;           /* bf16 [B, H, L, d]: V                                      */
  void* q8;          /* e4m3 [B, H, L, d] codes of Q, K, V (fp8 attention) with   */
  void* k8;
  void* v8;
  float* qkv_scale;  /* fp32 [3, B H]: one scale per (b, h) for Q, K, V           */
  void* cat;         /* bf16 [B L, D + F]: attention output | GELU hidden         */
  void* cat8;        /* e4m3 [B L, D + F]: their codes (fp8 blocks), with         */
  float* att_scale;  /* fp32 [B L]: attention-output row scales (single-stream:   */
                     /* one scale over the whole D + F row)                       */
  float* hid_scale;  /* fp32 [B L]: GELU-hidden row scales (double-stream)        */
} dit_block_views;
DIT_API int dit_block_views_of(const dit_dims* dims, void* workspace, size_t ws_bytes,
                               dit_block_views* out);

/* Modulation vectors of the whole model for n sigmas at once:
 *   out[i] = mod.W SiLU(c_i) + mod.b,  c_i = time2(SiLU(time1(emb(sigma_i)))),
 *   emb(t) = [cos(1000 t w_k), sin(1000 t w_k)], w_k = 10000^(-k/128), k < 128.
 *   sigmas_host: n fp64 values; out: device fp32 [n, N_mod].
 *   workspace >= DIT_WS_MODULATION bytes (for n). */
DIT_API int dit_modulation(const dit_model* m, const double* sigmas_host, int n, float* out,
                   void* workspace, size_t ws_bytes, void* stream);

/* dit_modulation with no workspace argument and no allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same kernels and results as
 * dit_modulation; their intermediates (the n x 256 timestep sinusoids and two
 * n x D activations) live in a static device array of DIT_MOD_STATIC_BYTES
 * that the library holds on each GPU it runs on until the process ends.
 *   n steps need dit_workspace_bytes(dims, DIT_WS_MODULATION, n) bytes of it
 *   (about n (256 + 2 D) 4 bytes: 327 steps at D 3072); a larger n returns
 *   DIT_ERR_WORKSPACE before anything is enqueued.
 *   Calls on one GPU share that GPU's array: calls that overlap on one GPU (on
 *   different streams, or from several threads, before the earlier one's kernels
 *   have finished) race and must be serialised by the caller.  Every
 *   intermediate is written in full before it is read, so nothing carries over
 *   from an earlier call.  The first call on a device looks up that device's
 *   copy of the array (hipGetSymbolAddress); no call allocates or frees. */
#define DIT_MOD_STATIC_BYTES (8u << 20)
DIT_API int dit_modulation_static(const dit_model* m, const double* sigmas_host, int n,
                                  float* out, void* stream);

/* First-Block-Cache test.
 *   x_after: device fp32 joint stream [B, Lt + Li, D] after the first block
 *            (Lt may be 0 for a plain image tensor);
 *   x_before: device fp32 [B, Li, D], image hidden before the first block;
 *   anchor: device fp32 [B, Li, D] (ignored when has_anchor == 0);
 *   staging: device fp32 [B, Li, D], receives r = x_after(image) - x_before.
 *   rel = sum|r - anchor| / sum|anchor| (fp64, fixed-order reduction: the same
 *   inputs always give the same rel); skip = has_anchor && rel < threshold,
 *   with a NaN rel or a zero denominator never skipping.  Synchronises the
 *   stream and writes rel_out / skip_out on the host.  Returns
 *   DIT_ERR_NONFINITE (with skip 0) if a NaN or Inf reached the sums.
 *   workspace >= DIT_WS_FBCACHE bytes. */
DIT_API int fbcache_should_skip(const float* x_after, const float* x_before, const float* anchor,
                        float* staging, int B, int Lt, int Li, int D, float threshold,
                        int has_anchor, void* workspace, size_t ws_bytes, void* stream,
                        double* rel_out, int* skip_out);

/* One Euler step of the whole model:
 *   latents <- latents + (sigma_next - sigma) v,  v the velocity of the model at
 *   t = sigma (CFG pair: v = v_neg + guidance (v_pos - v_neg)).
 *   mod_step: device fp32 [N_mod], this sigma's row of dit_modulation().
 *   txt: device [B, Lt, D], bf16 (fp32 for a DIT_F32 model); latents: device fp32
 *   [Li, C_in], in place
 *   (shared by a CFG pair).  cache: NULL or a dit_fbcache (state updated).
 *   info_out: optional host pointer.  workspace >= DIT_WS_STEP bytes. */
DIT_API int dit_denoise_step(const dit_model* m, const float* mod_step, const void* txt, float* latents,
                     double sigma, double sigma_next, dit_fbcache* cache, void* workspace,
                     size_t ws_bytes, void* stream, dit_step_info* info_out);

/* One Euler step addressed by its place in the schedule: step `step` of
 * `num_steps` (0 <= step < num_steps), with sigma = sigmas_host[step] and
 * sigma_next = sigmas_host[step + 1] from a host table of num_steps + 1 entries
 * (dit_sigmas()).  This step's adaLN modulation vectors are computed here by the
 * kernels of dit_modulation() (timestep MLP, then one pass over the stacked
 * modulation weights; the per-row arithmetic is the same, so the row equals row
 * `step` of dit_modulation() over the table), then the step runs exactly as
 * dit_denoise_step().  Calling this once per step reads the modulation weights
 * once per step; precomputing every row once with dit_modulation() and calling
 * dit_denoise_step() (or the replayed loop) reads them once per loop.
 *   latents, txt, cache, info_out: as dit_denoise_step();
 *   workspace >= dit_step_at_workspace_bytes(m) bytes (device), 16-byte aligned.
 * Sources: the loop calls the transformer once per scheduler step, with the cache
 * deciding per step (unsloth studio diffusion.py commit log, commit "Add opt-in
 * step caching (First-Block-Cache)"); the sigma table is the flow-shift
 * schedule (vflash "Optimization ledger", section "Fewer steps require a new
 * contract"). */
DIT_API int dit_denoise_step_at(const dit_model* m, float* latents, const void* txt, int step,
                                int num_steps, const double* sigmas_host, dit_fbcache* cache,
                                void* workspace, size_t ws_bytes, void* stream,
                                dit_step_info* info_out);

/* Device workspace bytes dit_denoise_step_at() needs for this model (the step's
 * own workspace, one modulation row and the modulation scratch); 0 for NULL or
 * invalid dimensions. */
DIT_API size_t dit_step_at_workspace_bytes(const dit_model* m);

/* ------------------------------------------------------------------ replayed loop
 *
 * The denoise loop as one captured HIP graph per step, replayed with no host
 * synchronisation: the step index, the sigma step, the modulation row and the
 * First-Block-Cache decision (with its warm-up / max-skips policy) live in
 * device memory, and every kernel of blocks 1.. reads the decision on entry and
 * returns at once on a skipped step (HIP graphs have no conditional nodes here,
 * so the skip is a gate inside the kernels).  The per-step host sync of
 * dit_denoise_step() and its per-launch host work go away.  Sources: recording
 * and replaying the step's kernel launches more than halved the 8-GPU denoise
 * time once per-GPU work had shrunk (VisualGen article on FLUX Klein, section on
 * why the speed-ups differ); the First-Block-Cache commit notes that the cache's
 * per-step decision breaks a whole-step compiled graph, which a decision kept on
 * the device avoids.
 *
 * Results equal the eager loop's bit for bit (same kernels, same inputs).  One
 * difference: a NaN / Inf in the cache test does not stop the loop; that step
 * computes in full and dit_loop_graph_sync() reports DIT_ERR_NONFINITE.
 *
 * Memory: the caller owns the workspace (DIT_WS_STEP bytes) and the loop state
 * (dit_loop_state_bytes()); the graph keeps their addresses and those of
 * mod_all, txt, latents and the cache buffers, which must stay valid and must not
 * be used by other work while replays are pending.  The handle itself (the
 * instantiated graph) is host memory the library allocates at create and frees
 * at destroy: the one exception to "allocates nothing". */
typedef struct dit_loop_graph dit_loop_graph;

/* Device bytes of a loop's own state for n_steps steps (state, sigma table,
 * per-step log, the running step's modulation row).  0 for bad arguments. */
DIT_API size_t dit_loop_state_bytes(const dit_model* m, int n_steps);

/* Capture one step of m into a graph.  mod_all: device fp32 [n_steps, N_mod],
 * row i from dit_modulation() at sigmas_host[i]; sigmas_host: n_steps + 1 host
 * values (copied); txt, latents as for dit_denoise_step(); cache: NULL or an
 * enabled / disabled state, whose policy fields and counters seed the device
 * state (its anchor / cached buffers are baked in).  The device state is set to
 * step 0 (stream is synchronised).  *out receives the handle. */
DIT_API int dit_loop_graph_create(const dit_model* m, const float* mod_all, const void* txt,
                                  float* latents, const double* sigmas_host, int n_steps,
                                  const dit_fbcache* cache, void* workspace, size_t ws_bytes,
                                  void* loop_state, size_t state_bytes, void* stream,
                                  dit_loop_graph** out);
/* Enqueue n replays (n steps, from the device's next step) on stream; no sync.
 * DIT_ERR_INVALID_ARG if the loop would pass n_steps or the current device is
 * not the one the graph was created on. */
DIT_API int dit_loop_graph_run(dit_loop_graph* g, int n, void* stream);
/* Synchronise stream and read back: info[i] (i < n_info) = step i's rel and skip
 * (steps not run hold earlier contents); cache (optional, the create-time one)
 * gets has_anchor / steps_done / skip_run; *steps_run (optional) = steps
 * completed.  DIT_ERR_NONFINITE if a completed step met a NaN / Inf in the test. */
DIT_API int dit_loop_graph_sync(dit_loop_graph* g, dit_fbcache* cache, dit_step_info* info,
                                int n_info, void* stream, int* steps_run);
/* Restart at first_step (0..n_steps) with the counters of cache (same buffers and
 * enabled flag as at create; threshold and policy may change).  Synchronises. */
DIT_API int dit_loop_graph_reset(dit_loop_graph* g, const dit_fbcache* cache, int first_step,
                                 void* stream);
/* Free the handle (NULL is a no-op).  Replays must have finished. */
DIT_API int dit_loop_graph_destroy(dit_loop_graph* g);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H */
