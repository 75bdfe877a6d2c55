/*
 * vitenc.h - C ABI of the MI355X (gfx950) encoder for DeepSeek-V4-Flash-Vision images.
 *
 * The library computes the hot path of the vision encoder described on the NeMo
 * Automodel API page "nemo_automodel.components.models.deepseek_v4.vision":
 * patch embedding (DeepseekV4VisionPatchEmbed), a stack of pre-norm blocks
 * (DeepseekV4VisionBlock: fp32-scale RMSNorm, wqkv, half-split 2D rotary, full
 * bidirectional patch attention, out-projection, bias-free SwiGLU MLP), the final
 * RMSNorm (DeepseekV4VisionTransformer.norm) and the 2x2 spatial-downsampling
 * aligner (DeepseekV4VisionAligner), as chained by DeepseekV4Model.encode_image on
 * the "...deepseek_v4.model" page.  Batches of images of different grids are
 * concatenated as in that page's ``pixel_values`` / ``image_grid_hws`` arguments.
 *
 * Conventions shared by every entry point
 *  - Device pointers are HIP device addresses; "host" marks the few host arrays.
 *  - Matrices are row-major with a PyTorch-style weight layout [out, in].
 *  - Activations and weights are bfloat16 (VIT_BF16) or float32 (VIT_F32) as
 *    chosen by vit_config.dtype; norm scales are always float32.
 *  - The caller owns every buffer (inputs, weights, outputs, workspace).  The
 *    library never allocates or frees device memory, never writes inputs or
 *    weights, and enqueues all work asynchronously on ``stream`` (a hipStream_t;
 *    NULL = the null stream).  Host arrays are read before the call returns.
 *  - Errors are returned as vit_status; no exception crosses the ABI.
 *    vit_last_error() gives a human-readable detail of the last failure on the
 *    calling thread.  NaN in gives NaN out (no NaN checks).
 *  - Results are deterministic: no floating-point atomics.
 *  - Calls on different streams must use different workspaces.
 */
#ifndef VITENC_H
#define VITENC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VIT_OK = 0,
  VIT_E_ARG = -1,        /* null pointer or invalid enum/flag */
  VIT_E_SHAPE = -2,      /* inconsistent or unsupported dimensions */
  VIT_E_ODD_GRID = -3,   /* aligner requested on a grid not divisible by merge */
  VIT_E_WORKSPACE = -4,  /* workspace smaller than vit_workspace_bytes() */
  VIT_E_HIP = -5,        /* a HIP launch or runtime call failed */
} vit_status;

typedef enum { VIT_BF16 = 0, VIT_F32 = 1 } vit_dtype;

/* flags for vit_encode / vit_encode_varlen / vit_workspace_bytes */
enum {
  VIT_NO_ALIGNER = 1,  /* stop after the final norm: out is [sum P, vision_dim] */
  VIT_OUT_NLAYOUT = 2, /* aligner rows land at their newline-layout slots (see
                          vit_aligner_layout); sentinel rows are not written */
  VIT_IN_PIXELS = 4,   /* `in` holds pixel images instead of patches: image i is
                          [3, ps*grid_h, ps*grid_w] (C order, ps = patch size with
                          patch_dim = 3*ps^2), images back to back; the library cuts
                          them into patches (DeepseekV4VisionTransformer.forward
                          takes [n_h*n_w, 3, ps, ps] patches of the image) */
  VIT_ALIGN_PAD = 8,   /* odd grids with the aligner: zero-pad to even (a zero patch
                          row below, a zero patch column on the right) before the
                          2x2 merge, giving ceil(grid_h/2)*ceil(grid_w/2) merged
                          tokens and a newline layout over that merged grid.  The
                          release handles odd grids (PR #3772 validation: 27x37,
                          37x27, 112x7) by a rule the pages do not give; without
                          this flag odd grids are rejected (VIT_E_ODD_GRID) */
};

/* Upper bound on images per varlen call (descriptors travel as kernel args). */
#define VIT_MAX_IMAGES 128

/* Encoder shape.  head_dim must equal vision_dim / n_heads (the page's
 * DeepseekV4VisionAttention.head_dim) and be a multiple of 4 (two halves, each
 * split in rotate_half quarters); bf16 mode supports head_dim 64 and 72.
 * patch_dim = 3 * patch_size^2 (588 for 14x14 RGB patches).  merge is the
 * aligner's downsample_ratio (2).  rms_eps is 1e-6 on the page's
 * DeepseekV4VisionRMSNorm.  rope_theta is DeepseekV4VisionTransformer.rope_theta. */
typedef struct {
  int32_t vision_dim;
  int32_t n_heads;
  int32_t head_dim;
  int32_t mlp_hidden;
  int32_t n_blocks;
  int32_t patch_dim;
  int32_t merge;
  int32_t llm_dim;
  float rope_theta;
  float rms_eps;
  int32_t dtype; /* vit_dtype */
} vit_config;

/* Weights (device pointers; the per-block arrays are HOST arrays of n_blocks
 * device pointers).  dtype = cfg.dtype except the norm scales (float32).
 *   patch_embed [d, patch_dim]     DeepseekV4VisionPatchEmbed.proj
 *   wqkv[b]     [3d, d]            rows [q; k; v], each head-major
 *   wo[b]       [d, d]             attention out-projection
 *   w_gate[b], w_up[b] [h, d]      SwiGLU gate and up
 *   w_down[b]   [d, h]
 *   norm1[b], norm2[b], final_norm [d] float32
 *   aligner     [llm_dim, merge^2 * d] (may be NULL with VIT_NO_ALIGNER) */
typedef struct {
  const void* patch_embed;
  const void* const* wqkv;
  const void* const* wo;
  const void* const* w_gate;
  const void* const* w_up;
  const void* const* w_down;
  const float* const* norm1;
  const float* const* norm2;
  const float* final_norm;
  const void* aligner;
} vit_weights;

/* Text for a status code (static storage). */
const char* vit_status_str(int32_t status);
/* Detail of the last failing call on this thread ("" if none). */
const char* vit_last_error(void);

/* Workspace bytes needed by vit_encode_varlen (and vit_encode, n_images = 1) for
 * these grids (host array [n_images, 2] of (rows, cols)).  Returns 0 when the
 * arguments are invalid. */
size_t vit_workspace_bytes(const vit_config* cfg, const int32_t* grid_hw_host, int32_t n_images,
                           int32_t flags);

/* Encode one image: DeepseekV4Model.encode_image on the "...deepseek_v4.model" page
 * (vision tower, then aligner unless VIT_NO_ALIGNER).
 *   in   [grid_h * grid_w, patch_dim] patches, row-major over the grid, each patch
 *        flattened in [3, ps, ps] C order (DeepseekV4VisionTransformer.forward);
 *        with VIT_IN_PIXELS the pixel image [3, ps*grid_h, ps*grid_w] instead
 *        (patch_dim must then be 3*ps^2; VIT_E_SHAPE otherwise).
 *   out  aligner on: [h'*w', llm_dim] with h' = grid_h/merge, w' = grid_w/merge
 *        (rounded up with VIT_ALIGN_PAD), merged tokens row-major over the merged
 *        grid (or newline-layout rows with VIT_OUT_NLAYOUT: [(h'*(w'+1)+2), llm_dim]);
 *        aligner off: [grid_h*grid_w, vision_dim].  dtype = cfg.dtype.
 *   ws   device workspace of ws_bytes >= vit_workspace_bytes(); contents scratch.
 * Errors: VIT_E_ARG (null pointer), VIT_E_SHAPE (dims), VIT_E_ODD_GRID (aligner
 * on an odd grid without VIT_ALIGN_PAD), VIT_E_WORKSPACE, VIT_E_HIP.  out must not
 * alias in or ws. */
vit_status vit_encode(const vit_config* cfg, const vit_weights* w, const void* in, int32_t grid_h,
                      int32_t grid_w, int32_t flags, void* out, void* ws, size_t ws_bytes,
                      void* stream);

/* Encode a batch of images packed back to back (the page's pixel_values with
 * image_grid_hws [n_images, 2]).  Each image attends only to itself (block-
 * diagonal attention) with rotary positions restarting at (0, 0).  Outputs are
 * concatenated in image order with the per-image layouts of vit_encode.
 * grid_hw_host is a HOST array [n_images, 2]; 1 <= n_images <= VIT_MAX_IMAGES. */
vit_status vit_encode_varlen(const vit_config* cfg, const vit_weights* w, const void* in,
                             const int32_t* grid_hw_host, int32_t n_images, int32_t flags,
                             void* out, void* ws, size_t ws_bytes, void* stream);

/* vit_encode_varlen for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and output, with the workspace taken from a fixed array that
 * the library holds on every GPU it runs on (VIT_NOALLOC_WORKSPACE_MAX bytes,
 * from the library's load until the process ends) instead of a caller buffer.
 * The call itself allocates nothing and launches the same kernels.
 *   Limits: calls whose vit_workspace_bytes() exceeds the maximum return
 *   VIT_E_WORKSPACE (with a message naming both sizes) and enqueue nothing.
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps the last
 *   call's contents (each call initialises what it needs); calls that overlap on
 *   one GPU (other streams or threads) race and must be serialised by the caller.
 *   The stream must belong to the calling thread's current device.
 * Other arguments and errors as vit_encode_varlen. */
#define VIT_NOALLOC_WORKSPACE_MAX ((size_t)160 << 20)
vit_status vit_encode_varlen_noalloc(const vit_config* cfg, const vit_weights* w, const void* in,
                                     const int32_t* grid_hw_host, int32_t n_images,
                                     int32_t flags, void* out, void* stream);
/* VIT_NOALLOC_WORKSPACE_MAX as built into the library. */
size_t vit_noalloc_workspace_limit(void);

/* Index arrays of one image's aligner layout (the "permutation" and "N-layout"
 * columns of the PR #3772 parity table).  All device int32:
 *   perm    [grid_h*grid_w]: slot 4t+s of merged token t holds patch perm[4t+s];
 *           token t = i*(grid_w/2)+j covers rows 2i..2i+1, cols 2j..2j+1 in the
 *           order TL, TR, BL, BR.
 *   nl_type [h'*(w'+1)+2]: 0 START, 1 IMAGE, 2 NEWLINE, 3 END for the span
 *           [START] + per merged row (w' IMAGE, NEWLINE) + [END].
 *   nl_src  [same]: merged token index of IMAGE slots, -1 for sentinels.
 * Any of the three pointers may be NULL (skipped).  merge must be 2. */
vit_status vit_aligner_layout(int32_t grid_h, int32_t grid_w, int32_t merge, int32_t* perm,
                              int32_t* nl_type, int32_t* nl_src, void* stream);

/* ---------------------------------------------------------------------------
 * Step entry points: the single steps of the path, for per-step parity tests.
 * ------------------------------------------------------------------------- */

/* RMSNorm (DeepseekV4VisionRMSNorm): out[r] = w * x[r] / sqrt(mean(x[r]^2) + eps),
 * computed in fp32.  x [rows, dim] float32, w [dim] float32, out [rows, dim] of
 * out_dtype.  dim must be a multiple of 4. */
vit_status vit_rmsnorm(const float* x, const float* w, float eps, int64_t rows, int32_t dim,
                       int32_t out_dtype, void* out, void* stream);

/* Rotary table for a batch of grids (get_vision_cos_sin on the vision page):
 * table [sum P, head_dim/2] of float2 (cos, sin); entries k < head_dim/4 use the
 * patch row angle row * theta^(-k/(head_dim/4)), the rest the column angle.
 * head_dim a multiple of 4, at most 128 (VIT_E_SHAPE otherwise). */
vit_status vit_rope_table(const int32_t* grid_hw_host, int32_t n_images, int32_t head_dim,
                          float theta, void* table, void* stream);

/* Half-split 2D rotary (apply_vision_rotary) in place on the q and k parts of a
 * packed qkv buffer [P, 3*n_heads*head_dim] of dtype, fp32 math, using a table
 * from vit_rope_table. */
vit_status vit_rope(int32_t dtype, void* qkv, const void* table, int64_t P, int32_t n_heads,
                    int32_t head_dim, void* stream);

/* Full bidirectional attention per image and head (DeepseekV4VisionAttention):
 * out[p, h*D:(h+1)*D] = softmax(q k^T / sqrt(D)) v over the patches of p's image.
 * qkv [P, 3*n_heads*D] (rows [q|k|v], rotary already applied), out [P, n_heads*D].
 * bf16 first packs V transposed per head into ws (size from
 * vit_attention_workspace_bytes); fp32 needs none and accepts NULL. */
size_t vit_attention_workspace_bytes(int32_t dtype, const int32_t* grid_hw_host,
                                     int32_t n_images, int32_t n_heads, int32_t head_dim);
vit_status vit_attention_varlen(int32_t dtype, const void* qkv, const int32_t* grid_hw_host,
                                int32_t n_images, int32_t n_heads, int32_t head_dim, void* out,
                                void* ws, size_t ws_bytes, void* stream);

/* GEMM epilogues for vit_gemm */
enum {
  VIT_EPI_STORE = 0,     /* C (dtype)   = A B^T                      */
  VIT_EPI_STORE_F32 = 1, /* C (float32) = A B^T                      */
  VIT_EPI_ADD_F32 = 2,   /* C (float32) += A B^T (residual, in place)  */
  VIT_EPI_SWIGLU = 3,    /* C (dtype)   = silu(A B^T) * (A B2^T)      */
  VIT_EPI_BIAS = 4,      /* C (bf16)    = A B^T + bias       (vit_gemm_bias) */
  VIT_EPI_BIAS_GELU = 5, /* C (bf16)    = gelu(A B^T + bias) (vit_gemm_bias) */
};

/* C[M, N] = epilogue(A[M, K] . B[N, K]^T): the bias-free linear maps of the block
 * (wqkv, out-projection, SwiGLU gate/up, down) and of the aligner.  Leading
 * dimensions are in elements.  bf16: K, lda, ldb multiple of 8 and 16-byte aligned
 * A/B.  B2 is only read by VIT_EPI_SWIGLU. */
vit_status vit_gemm(int32_t dtype, int32_t epilogue, const void* A, int64_t lda, const void* B,
                    const void* B2, int64_t ldb, void* C, int64_t ldc, int64_t M, int64_t N,
                    int64_t K, void* stream);

/* 2x2 aligner gather for a batch: G[t_i + t, s*d:(s+1)*d] = x[off_i + perm_i[4t+s]]
 * with x [sum P, d] and G [sum P/4, 4d] of dtype (DeepseekV4VisionAligner). */
vit_status vit_aligner_gather(int32_t dtype, const void* x, const int32_t* grid_hw_host,
                              int32_t n_images, int32_t d, void* G, void* stream);

/* ---------------------------------------------------------------------------
 * PatchMerger projector (DeepSeek-V4-Flash-Vision-NVFP4 model page): an
 * alternative to the aligner that merges every 2x2 group of encoder patches
 * and maps the 4*dim features to the LLM width through two biased linear maps.
 * The page gives the shapes (1152-dim patches, 4608 -> 4096) and the parameter
 * count, 40,119,040 = norm weight and bias (2*1152) + Linear(4608, 4608) with
 * bias + Linear(4608, 4096) with bias; the activation between the linear maps
 * is not named and is taken as GELU (erf form), the norm as LayerNorm.
 *   out = gelu(G W1^T + b1) W2^T + b2,  G[t] = concat over the 2x2 group of
 *   merged token t (order TL, TR, BL, BR, as the aligner) of LayerNorm(x[p]).
 * bf16 only: x [sum P, dim], w1 [hidden, 4*dim], w2 [out_dim, hidden] and out
 * [sum P/4, out_dim] bf16 (16-byte aligned); ln_w, ln_b [dim], b1 [hidden],
 * b2 [out_dim] float32 (16-byte aligned).  dim % 16 == 0 and dim <= 4096,
 * hidden % 64 == 0, out_dim % 8 == 0.  Grids must be even (VIT_E_ODD_GRID).
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t dim;     /* encoder width d (1152 on the page)  */
  int32_t hidden;  /* first linear's width (4608)         */
  int32_t out_dim; /* LLM width (4096)                    */
  float eps;       /* LayerNorm eps (1e-6)                */
  const float* ln_w;
  const float* ln_b;
  const void* w1;
  const float* b1;
  const void* w2;
  const float* b2;
} vit_merger;

/* Workspace of vit_patch_merger: G [sum P/4, 4*dim] and the GELU output
 * [sum P/4, hidden], bf16.  0 on bad arguments (see vit_last_error). */
size_t vit_patch_merger_workspace_bytes(const vit_merger* m, const int32_t* grid_hw_host,
                                        int32_t n_images);
vit_status vit_patch_merger(const vit_merger* m, const void* x, const int32_t* grid_hw_host,
                            int32_t n_images, void* out, void* ws, size_t ws_bytes, void* stream);

/* Step entry points of the projector, for per-step parity tests:
 * the LayerNorm + 2x2 gather into G [sum P/4, 4*dim] bf16, and the bias GEMMs
 * C [M, N] bf16 = A . B^T + bias (VIT_EPI_BIAS) or gelu(A . B^T + bias)
 * (VIT_EPI_BIAS_GELU), A [M, K] and B [N, K] bf16 with K % 64 == 0, bias [N]
 * float32. */
vit_status vit_layernorm_gather(const void* x, const int32_t* grid_hw_host, int32_t n_images,
                                int32_t dim, const float* ln_w, const float* ln_b, float eps,
                                void* G, void* stream);
vit_status vit_gemm_bias(int32_t epilogue, const void* A, int64_t lda, const void* B, int64_t ldb,
                         const float* bias, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                         void* stream);

/* ---------------------------------------------------------------------------
 * Backward of the MLP half of an encoder block (DeepseekV4VisionBlock on the
 * vision page: y = x + mlp(norm2(x)), mlp the bias-free SwiGLU; PR #3772 lists
 * backward over ragged grids among its tested paths).  Given dy = dL/dy,
 * computes dL/dx, dL/dnorm_w, dL/dW_gate, dL/dW_up and dL/dW_down, the exact
 * chain rule of the forward (the SwiGLU pre-activations are recomputed from x).
 * Rows are independent (patches of any images).  bf16 GEMM operands (x's
 * normalised rows, dy, the activations and their gradients are rounded to
 * bf16), fp32 accumulation and fp32 outputs.  dim a multiple of 64 and at most
 * 2048, hidden a multiple of 16 (4304 for the 1152-wide tower).  Every pointer
 * 16-byte aligned, all device memory.
 * ------------------------------------------------------------------------- */
typedef struct {
  int64_t rows;        /* sum of patches                                  */
  int32_t dim;         /* vision_dim d                                    */
  int32_t hidden;      /* MLP hidden h                                    */
  float eps;           /* RMSNorm eps                                     */
  const float* x;      /* [rows, dim] fp32: input of the MLP half         */
  const float* norm_w; /* [dim] fp32: norm2 scale                         */
  const void* w_gate;  /* [hidden, dim] bf16                              */
  const void* w_up;    /* [hidden, dim] bf16                              */
  const void* w_down;  /* [dim, hidden] bf16                              */
  const float* dy;     /* [rows, dim] fp32: gradient of y                 */
  float* dx;           /* [rows, dim] fp32 out: gradient of x (dy + ...)  */
  float* d_norm_w;     /* [dim] fp32 out                                  */
  float* d_w_gate;     /* [hidden, dim] fp32 out                          */
  float* d_w_up;       /* [hidden, dim] fp32 out                          */
  float* d_w_down;     /* [dim, hidden] fp32 out                          */
} vit_mlp_grad;

/* Workspace bytes of vit_mlp_backward (0 on bad sizes). */
size_t vit_mlp_backward_workspace_bytes(int64_t rows, int32_t dim, int32_t hidden);
vit_status vit_mlp_backward(const vit_mlp_grad* a, void* ws, size_t ws_bytes, void* stream);

/* Backward of the attention half of an encoder block (DeepseekV4VisionBlock:
 * y = x + attn(norm1(x)), attn = wqkv, half-split 2D rotary on q and k, full
 * bidirectional attention per image and head, out-projection wo).  Given dy,
 * computes dL/dx, dL/dnorm_w, dL/dwqkv and dL/dwo by the chain rule; q, k, v
 * and each query's softmax log-sum-exp are recomputed by a forward pass.  bf16
 * GEMM and attention operands, fp32 accumulation and outputs; head_dim 64 or
 * 72 (dim = 64 or 72 times n_heads), dim a multiple of 64 and at most 2048.
 * Images as in vit_encode_varlen (rows of x / dy concatenated in image order).
 * Every pointer 16-byte aligned, device. */
typedef struct {
  int32_t dim;         /* vision_dim d = head_dim (64 or 72) * n_heads    */
  int32_t n_heads;
  float rope_theta;
  float eps;           /* RMSNorm eps                                     */
  const float* x;      /* [sum P, dim] fp32: input of the attention half  */
  const float* norm_w; /* [dim] fp32: norm1 scale                         */
  const void* wqkv;    /* [3*dim, dim] bf16, rows [q; k; v]               */
  const void* wo;      /* [dim, dim] bf16                                 */
  const float* dy;     /* [sum P, dim] fp32: gradient of y                */
  float* dx;           /* [sum P, dim] fp32 out                           */
  float* d_norm_w;     /* [dim] fp32 out                                  */
  float* d_wqkv;       /* [3*dim, dim] fp32 out                           */
  float* d_wo;         /* [dim, dim] fp32 out                             */
} vit_attn_grad;

size_t vit_attn_backward_workspace_bytes(const vit_attn_grad* a, const int32_t* grid_hw_host,
                                         int32_t n_images);
vit_status vit_attn_backward(const vit_attn_grad* a, const int32_t* grid_hw_host,
                             int32_t n_images, void* ws, size_t ws_bytes, void* stream);

/* Backward of the whole tower (DeepseekV4VisionTransformer.forward on the vision
 * page: patch embedding, blocks, final norm; PR #3772 lists backward over ragged
 * grids among its tested paths).  Given dy = dL/d(out) for the tower's output
 * (the final norm's, as vit_encode_varlen with VIT_NO_ALIGNER returns it),
 * computes the gradient of every weight: the forward is run once, keeping the
 * fp32 residual stream at the input of each residual branch; then the final
 * norm's gradient, the blocks in reverse (each as vit_mlp_backward then
 * vit_attn_backward) and the patch embedding's weight gradient dx0^T . patches.
 * bf16 weights and patches, fp32 gradients; head_dim 64 or 72, vision_dim a
 * multiple of 64 and at most 2048, mlp_hidden a multiple of 16, patch_dim a
 * multiple of 4.  Images as in
 * vit_encode_varlen (patches [sum P, patch_dim], rows of dy in the same order).
 * The per-block arrays are HOST arrays of n_blocks device pointers (as in
 * vit_weights).  Every device pointer 16-byte aligned; the workspace must not
 * alias any argument.  Errors as vit_encode_varlen, VIT_E_ARG for a NULL
 * gradient pointer. */
typedef struct {
  float* d_patch_embed;       /* [d, patch_dim] */
  float* const* d_wqkv;       /* [3d, d] per block */
  float* const* d_wo;         /* [d, d] */
  float* const* d_w_gate;     /* [h, d] */
  float* const* d_w_up;       /* [h, d] */
  float* const* d_w_down;     /* [d, h] */
  float* const* d_norm1;      /* [d] */
  float* const* d_norm2;      /* [d] */
  float* d_final_norm;        /* [d] */
} vit_tower_grads;

size_t vit_tower_backward_workspace_bytes(const vit_config* cfg, const int32_t* grid_hw_host,
                                          int32_t n_images);
vit_status vit_tower_backward(const vit_config* cfg, const vit_weights* w, const void* patches,
                              const int32_t* grid_hw_host, int32_t n_images, const float* dy,
                              const vit_tower_grads* grads, void* ws, size_t ws_bytes,
                              void* stream);

/* Measured dense bf16 MFMA peak (a measurement aid beside the encoder, used to
 * report its kernels against the throughput the chip sustains as well as against
 * the published 2.5 PFLOP/s): one 8-wave workgroup per CU issues `iters` rounds
 * of 8 back-to-back v_mfma_f32_32x32x16_bf16 on register operands, no memory
 * traffic in the loop.  *flops (host) receives the call's FLOP count; time the
 * call with events on `stream`.  out: device float buffer of
 * vit_mfma_peak_out_floats() elements (receives the accumulator sums, so the
 * work is not optimised away).  VIT_E_ARG for NULL pointers or iters outside
 * [1, 2^24]. */
int64_t vit_mfma_peak_out_floats(void);
vit_status vit_mfma_peak(int32_t iters, float* out, double* flops, void* stream);

/* Image tokens into the LLM input stream (DeepSeek-V4 model page,
 * DeepseekV4Model.merge_image_embeddings): for each position p of a text
 * embedding stream embeds [positions, hidden] (in place, dtype):
 *   types[p] == 1 (IMAGE)     row p = tokens[t], t = IMAGE positions before p;
 *   types[p] == 0 / 2 / 3     row p = sentinels[0 / 1 / 2] (image_start,
 *                             image_newline, image_end);
 *   any other value (-1 text) row p is left as it is.
 * types is device int32 [positions] with the codes of vit_aligner_layout's
 * nl_type, so an image's span is its nl_type array and its tokens are the
 * aligner output in order; several images simply follow one another.
 * tokens [n_tokens, hidden] and sentinels [3, hidden] are device, dtype, rows
 * 16-byte aligned (hidden * sizeof(dtype) % 16 == 0).  IMAGE positions beyond
 * n_tokens are left unchanged; n_image (device int32, may be NULL) receives the
 * number of IMAGE positions so the caller can check it against n_tokens.
 * ws: device scratch of vit_merge_workspace_bytes(positions) bytes (0 is returned
 * only for positions outside [0, 2^31)).  The rows of
 * embeds must not overlap tokens or sentinels.  Asynchronous on stream. */
size_t vit_merge_workspace_bytes(int64_t positions);
vit_status vit_merge_image_embeddings(int32_t dtype, void* embeds, int64_t positions,
                                      int32_t hidden, const int32_t* types, const void* tokens,
                                      int64_t n_tokens, const void* sentinels, int32_t* n_image,
                                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Kernel timing with HIP events (for measurement tools).  When enabled for a
 * kernel class, every launch of that class inside vit_encode(_varlen),
 * vit_merge_image_embeddings, vit_patch_merger, vit_mlp_backward and
 * vit_attn_backward is bracketed by events on the call's stream;
 * vit_profile_read synchronises them and returns the summed duration and the
 * launch count, then resets.
 * ------------------------------------------------------------------------- */
enum {
  VIT_K_EMBED = 0,
  VIT_K_RMSNORM = 1,
  VIT_K_QKV = 2,
  VIT_K_ROPE = 3,
  VIT_K_ATTN = 4,
  VIT_K_OUTPROJ = 5,
  VIT_K_GATEUP = 6,
  VIT_K_DOWN = 7,
  VIT_K_GATHER = 8,
  VIT_K_ALIGNER = 9,
  VIT_K_MERGE = 10,     /* the row copies of vit_merge_image_embeddings */
  VIT_K_LNGATHER = 11,  /* vit_patch_merger: LayerNorm + 2x2 gather */
  VIT_K_PROJ1 = 12,     /* vit_patch_merger: first linear (bias, GELU) */
  VIT_K_PROJ2 = 13,     /* vit_patch_merger: second linear (bias) */
  VIT_K_BWD_GEMM = 14,  /* vit_mlp_backward: every GEMM */
  VIT_K_BWD_DN = 15,    /* vit_mlp_backward: the GEMM of the normed rows' gradient */
  VIT_K_BWD_PASS = 16,  /* vit_mlp_backward: norm, casts, transposes, SwiGLU gradient */
  VIT_K_BWD_ATTN = 17,  /* vit_attn_backward: the dQ and dK/dV kernels */
  VIT_K_COUNT = 18,
};
vit_status vit_profile_enable(int32_t kernel_class, int32_t on);
vit_status vit_profile_read(int32_t kernel_class, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* VITENC_H */
