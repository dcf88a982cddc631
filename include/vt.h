/*
 * vt.h -- C ABI of the tiled ViT vision tower for AMD MI355X (gfx950).
 *
 * The library computes the forward pass of a CLIP-style ViT vision tower of
 * the MiniMax-M3 shape (MiniMax-M3-Vision README, "Architecture" table:
 * 32 layers, hidden 1280, 16 heads, MLP 5120, patch 14, Conv3d patch embed,
 * 3D RoPE, GELU; 2x2 spatial merge, temporal patch 2; projector
 * Linear(1280,6144) GELU Linear(6144,6144), flatten four 6144-wide patches,
 * Linear(24576,6144) GELU Linear(6144,6144)).  Attention is computed tiled
 * with an online softmax: no [seq, seq] buffer exists at any point, so memory
 * is linear in the number of patches (the quadratic score buffer is what caps
 * image size in "init.rs (VisionEncoder::new)", doc comment of
 * CEILING_MAX_PATCHES).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.    Every device pointer is owned by the caller.  The library never
 *            allocates or frees device memory; scratch comes from the caller's
 *            workspace (`ws`, `ws_bytes`), sized by the *_workspace_size
 *            functions -- except vt_attention_varlen_noalloc, whose scratch is
 *            a fixed array inside the library.  Host arrays (the grid list)
 *            are read during the call and not kept.
 * Dtypes.    "bf16" tensors are uint16 bit patterns of bfloat16.  Weights are
 *            bf16 in PyTorch Linear layout [out, in] (row-major, the input
 *            dimension contiguous).  The residual stream is fp32.
 * Alignment. Every device pointer must be 16-byte aligned; the workspace
 *            256-byte aligned.
 * Tokens.    Inside the library, and at every boundary that says "token
 *            order", the tokens of one item are stored per temporal patch
 *            tt in 2x2-window order: with w2 = w/2, token
 *            tt*h*w + 4*(R*w2 + C) + 2*dr + dc is the patch at (tt, 2R+dr,
 *            2C+dc).  The four patches of merged token tt*h*w/4 + R*w2 + C
 *            are therefore adjacent and the 2x2 merge is a reshape.  Items
 *            follow each other in grid-list order.  Outputs documented as
 *            "raster" use (tt, row, col) row-major patch order instead.
 * Streams.   `stream` is a hipStream_t (NULL = the default stream).  Calls
 *            only enqueue work; they return before it finishes.  Inputs must
 *            stay valid until the stream reaches that point.
 * Errors.    Arguments are validated on the host before any launch, in every
 *            build; a failing call launches nothing and returns a status
 *            code, with details in vt_last_error() (thread-local).  Launch
 *            failures return VT_ERR_HIP.  Nothing is clamped silently; the
 *            one clamp, of RoPE coordinates, is stated at
 *            vt_attention_varlen.
 * Range.     Attention runs its matrix products on fp16 operands (fp32
 *            accumulation): the rotated q times log2(e)/sqrt(head_dim), the
 *            rotated k and v must stay below 65504 in magnitude, else the
 *            result holds infinities or NaN.  Stated again at each entry
 *            point that runs attention.
 * Threads.   Calls are reentrant; there is no global mutable state other
 *            than the thread-local error string, and the per-GPU scratch
 *            array of vt_attention_varlen_noalloc (with its device address,
 *            cached per GPU under a lock).
 */
#ifndef VT_H
#define VT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vt_status {
  VT_OK = 0,
  VT_ERR_INVALID_ARG = 1,   /* NULL, negative/zero size, odd grid, misaligned pointer */
  VT_ERR_UNSUPPORTED = 2,   /* valid request outside what the kernels implement */
  VT_ERR_WORKSPACE = 3,     /* ws_bytes below the *_workspace_size() value */
  VT_ERR_HIP = 4            /* a HIP launch or runtime call failed */
} vt_status;

typedef enum vt_dtype { VT_BF16 = 0, VT_FP32 = 1 } vt_dtype;

/* Row order of a [tokens, width] tensor at the boundary. */
typedef enum vt_order { VT_ORDER_WINDOW = 0, VT_ORDER_RASTER = 1 } vt_order;

/* Epilogue of vt_linear (y = x W^T + b, fp32 accumulation). */
typedef enum vt_epilogue {
  VT_EPI_BF16 = 0,          /* out bf16 = y                                   */
  VT_EPI_GELU_TANH_BF16 = 1,/* out bf16 = gelu_tanh(y)                        */
  VT_EPI_GELU_ERF_BF16 = 2, /* out bf16 = gelu_erf(y)                         */
  VT_EPI_RESID_F32 = 3,     /* out fp32 += y   (residual update, in place)    */
  VT_EPI_F32 = 4,           /* out fp32 = y                                   */
  VT_EPI_SPLITK_PARTIALS_F32 = 5 /* out fp32 [splits, M, N]: the split-K partial
                               products x[:, Kz] W[:, Kz]^T of the K ranges the
                               library splits this shape into, no bias, not
                               summed (kernel-level measurement and tests) */
} vt_epilogue;

/* One item: t temporal patches x h x w patches (README Architecture: temporal
 * patch 2).  t == 1 is a still image, whose single frame is repeated to fill
 * the temporal patch ("v2_loaders FINDINGS", section 3); t > 1 is a clip of
 * 2t frames, temporal patch tt covering frames 2tt and 2tt+1.  h and w must
 * be even (2x2 merge, applied within each temporal patch). */
typedef struct vt_grid_thw { int32_t t, h, w; } vt_grid_thw;

/* Tower shape.  vt_config_default() fills the MiniMax-M3 shape; the kernels
 * implement head_dim 80, patch 14, temporal patch 2, merge 2; other widths
 * must be multiples of 64 (hidden, mlp, proj_*) and hidden = heads*head_dim. */
typedef struct vt_config {
  int32_t layers;           /* 32 */
  int32_t hidden;           /* 1280 */
  int32_t heads;            /* 16 */
  int32_t head_dim;         /* 80 */
  int32_t mlp;              /* 5120 */
  int32_t patch;            /* 14 */
  int32_t t_patch;          /* 2 */
  int32_t merge;            /* 2 */
  int32_t proj_hidden;      /* 6144 */
  int32_t proj_out;         /* 6144 */
  float ln_eps;             /* 1e-6 */
  float rope_theta;         /* 10000 */
  int32_t rope_pairs[3];    /* rotation pairs on the t, h, w axes: 8, 16, 16 */
  int32_t rope_shared_ladder; /* 0: per-axis ladder theta^(-k/n_axis); 1: theta^(-2j/head_dim) */
  int32_t gelu_erf_projector; /* 0: GELU(tanh) in the projector (default); 1: exact erf GELU */
} vt_config;

/* Weights of one pre-LN block.  W_qkv rows are [Q | K | V], each head-major
 * (heads x head_dim).  Biases may be NULL (read as zero); LN gamma/beta may not. */
typedef struct vt_block_weights {
  const uint16_t *ln1_g, *ln1_b;
  const uint16_t *w_qkv, *b_qkv;   /* [3*hidden, hidden], [3*hidden] */
  const uint16_t *w_o, *b_o;       /* [hidden, hidden], [hidden]     */
  const uint16_t *ln2_g, *ln2_b;
  const uint16_t *w_fc1, *b_fc1;   /* [mlp, hidden], [mlp]           */
  const uint16_t *w_fc2, *b_fc2;   /* [hidden, mlp], [hidden]        */
} vt_block_weights;

/* Projector (MiniMax-M3-Vision README, Architecture table, Projector row). */
typedef struct vt_projector_weights {
  const uint16_t *w1, *b1;   /* [proj_hidden, hidden]                       */
  const uint16_t *w2, *b2;   /* [proj_hidden, proj_hidden]                  */
  const uint16_t *w3, *b3;   /* [proj_out, 4*proj_hidden]  (24576 wide)     */
  const uint16_t *w4, *b4;   /* [proj_out, proj_out]                        */
} vt_projector_weights;

typedef struct vt_tower_weights {
  const uint16_t *w_patch;   /* [hidden, 3*2*14*14] = Conv3d [hidden,3,2,14,14] flattened */
  const uint16_t *b_patch;   /* [hidden] or NULL */
  const vt_block_weights *blocks; /* host array of cfg->layers blocks */
  vt_projector_weights proj;
} vt_tower_weights;

/* ---------------------------------------------------------------- basics */
void vt_config_default(vt_config* cfg);
const char* vt_status_string(vt_status s);
/* Detail of the last failed call on this thread ("" if none).  Never NULL. */
const char* vt_last_error(void);
/* Library version string. */
const char* vt_version(void);

/* Workspace bytes for vt_tower_forward / vt_patch_embed / vt_merge_project on
 * this grid list.  Affine in the token count (no term grows with seq^2), plus
 * a fixed 86 MB of attention partial records once a call is large enough for
 * the lean attention kernels, and up to 64 MB of GEMM partial sums whose
 * presence depends on how a call's GEMM tiles fill the CUs.
 * Returns 0 and sets vt_last_error() if the arguments are invalid. */
size_t vt_tower_workspace_size(const vt_config* cfg, const vt_grid_thw* grid, int32_t n_img);

/* Workspace bytes for vt_block_forward and vt_attention_varlen.
 * Returns 0 and sets vt_last_error() if the arguments are invalid. */
size_t vt_block_workspace_size(const vt_config* cfg, int32_t total_tokens, int32_t n_img,
                               int32_t max_seqlen);

/* ---------------------------------------------------------------- metadata
 * Integer maps of a grid list, written on the device ("v2_loaders FINDINGS",
 * section 3: grid_thw; section 1: per-image native-resolution grids).
 *   cu_seqlens   [n_img+1] int32: cu[0] = 0, cu[i+1] = cu[i] + t*h*w.
 *   pos_thw      [N, 3] int32 in token order: (tt, row, col) patch coordinates,
 *                restarting at 0 for each item.
 *   raster_index [N] int32 in token order, or NULL: global raster index
 *                (cu[i] + tt*h*w + row*w + col) of each token. */
vt_status vt_build_metadata(const vt_grid_thw* grid, int32_t n_img, int32_t* cu_seqlens,
                            int32_t* pos_thw, int32_t* raster_index, void* stream);

/* ---------------------------------------------------------------- steps */
/* Patchify + patch embed (README Architecture: patch 14, Conv3d patch embed,
 * temporal patch 2; FINDINGS s.3: a still frame is repeated to fill it).
 *   pixels    bf16, the items one after another: [3, 14h, 14w] row-major for a
 *             still image (t == 1), [2t, 3, 14h, 14w] for a clip (t > 1).
 *   resid_out fp32 [N, hidden] in token order: X W_patch^T + b_patch, where
 *             row X[j] = (channel, tau, py, px) of token j's 3x2x14x14 block. */
vt_status vt_patch_embed(const vt_config* cfg, const uint16_t* pixels, const vt_grid_thw* grid,
                         int32_t n_img, const uint16_t* w_patch, const uint16_t* b_patch,
                         float* resid_out, void* ws, size_t ws_bytes, void* stream);

/* Tiled varlen non-causal attention with 3D RoPE on Q and K.
 *   qkv        bf16 [N, 3, heads, head_dim] (the QKV Linear output).
 *   cu_seqlens [n_img+1] int32 on the device; image i attends only to its own
 *              tokens cu[i] .. cu[i+1]-1 (block-diagonal, no padding tokens).
 *   pos_thw    [N, 3] int32 on the device: the RoPE positions of each token.
 *              Coordinates lie in [0, max_seqlen); the device reads them
 *              during the call, so they are not validated on the host: a
 *              coordinate outside that range is clamped into it for the
 *              angle-table lookup (the result is that of the clamped
 *              position; no memory outside the table is read).
 *   out        [N, heads*head_dim], bf16 or fp32 by out_dtype:
 *              softmax(RoPE(q) RoPE(k)^T / sqrt(head_dim)) v per image and head.
 *   max_seqlen must be >= every image's token count; total_tokens = cu[n_img].
 * Range: the products run on fp16 operands with fp32 accumulation, so
 * |RoPE(q)| log2(e)/sqrt(head_dim), |RoPE(k)| and |v| must stay below 65504
 * (larger values give infinities or NaN; they are not clamped).  bf16 q, k,
 * v inside that range are represented exactly or to fp16 rounding (2^-11).
 * No [n, n] buffer is formed: memory is O(total_tokens).
 * Rounding: a call's results are deterministic.  On large calls the work
 * that would leave the GPU's workgroups partly idle in the last round is cut
 * by key tiles across all of them and the pieces merged; where an image's
 * rows are cut depends on the whole call (the other images packed into it,
 * the GPU's CU count), so the same image in another batch can differ in its
 * last bits. */
vt_status vt_attention_varlen(const vt_config* cfg, const uint16_t* qkv, const int32_t* cu_seqlens,
                              const int32_t* pos_thw, int32_t n_img, int32_t total_tokens,
                              int32_t max_seqlen, void* out, vt_dtype out_dtype, void* ws,
                              size_t ws_bytes, void* stream);

/* vt_attention_varlen in its two parts, for callers that time them apart or
 * run the attention on prepared operands more than once.  Same operation,
 * same kernels: vt_attention_pack then vt_attention_packed on one workspace
 * give vt_attention_varlen's output bit for bit.
 * vt_attention_pack: the per-call schedule (which queries and key tiles each
 *   workgroup takes), the RoPE angle table, q rotated, scaled by
 *   log2(e)/sqrt(head_dim) and rounded to fp16, and k, v as fp16 key-tile
 *   images, all written into ws (arguments, range and clamp as
 *   vt_attention_varlen; ws sized by vt_block_workspace_size).
 * vt_attention_packed: the attention kernels alone (the step the tower runs
 *   after its QKV Linear, whose epilogue does the packing itself) on what the
 *   last vt_attention_pack left in ws, writing out as vt_attention_varlen.
 *   ws and the sizes (cfg, n_img, total_tokens, max_seqlen, ws_bytes) must be
 *   those of that vt_attention_pack, ordered after it (same stream, or
 *   otherwise synchronized); ws is read, not consumed, so the call may be
 *   repeated.  The sizes are validated as for vt_attention_varlen; the
 *   contents of ws are not (they are device data): a workspace not prepared
 *   by vt_attention_pack with the same sizes gives undefined results,
 *   including out-of-bounds device accesses.
 *   host_seqlens: optional (NULL), host memory, n_img int32: the images'
 *   token counts in cu_seqlens order, each in [1, max_seqlen], adding up to
 *   total_tokens (else VT_ERR_INVALID_ARG).  Given them, the call forms on
 *   the host the plan that decides whether the last round of workgroups is
 *   split across key tiles, and launches neither the split's extra
 *   workgroups nor its merge when nothing is split.  A performance hint
 *   only: counts that pass these checks but do not match cu_seqlens can cost
 *   time, never change the result (the device forms its own plan whenever a
 *   split is launched). */
vt_status vt_attention_pack(const vt_config* cfg, const uint16_t* qkv, const int32_t* cu_seqlens,
                            const int32_t* pos_thw, int32_t n_img, int32_t total_tokens,
                            int32_t max_seqlen, void* ws, size_t ws_bytes, void* stream);
vt_status vt_attention_packed(const vt_config* cfg, int32_t n_img, int32_t total_tokens,
                              int32_t max_seqlen, const int32_t* host_seqlens, void* out,
                              vt_dtype out_dtype, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- no allocation
 * For callers that can neither allocate device memory nor pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  vt_attention_varlen_noalloc computes what vt_attention_varlen
 * computes, with the same kernels, except that it never cuts the last round
 * across workgroups (the merge's partial records do not fit the array): its
 * results equal vt_attention_varlen's bit for bit when that call does not
 * cut (for example 7 images of 448x448), and to rounding otherwise.  Its
 * scratch -- the attention schedule, the rotated fp16 Q, the K/V tile images
 * and the RoPE table, about 8.5 KB per token plus 384 KB per image at 16
 * heads -- in one fixed device array of VT_NOALLOC_SCRATCH_BYTES inside the
 * library.  Each GPU the library runs on holds its own copy of that array
 * from the first use of the library on that GPU until the process ends.
 *   Arguments, layouts and errors as vt_attention_varlen, without ws.
 *   A call whose scratch would exceed the array returns VT_ERR_WORKSPACE
 *   (one image fits up to about 7,300 tokens; 448x448 images, up to 7 per
 *   call).
 * The call enqueues kernels only: no hipMalloc, hipFree or memset.  Its
 * first call on each GPU resolves the array's device address
 * (hipGetSymbolAddress); make that first call outside graph capture.
 * Every call on one GPU uses the same array and leaves its contents there;
 * nothing in it needs to start at zero.  Calls that overlap on one GPU
 * (on different streams, or from threads without ordering) race on it. */
#define VT_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
vt_status vt_attention_varlen_noalloc(const vt_config* cfg, const uint16_t* qkv,
                                      const int32_t* cu_seqlens, const int32_t* pos_thw,
                                      int32_t n_img, int32_t total_tokens, int32_t max_seqlen,
                                      void* out, vt_dtype out_dtype, void* stream);

/* Gradient of vt_attention_varlen with respect to its qkv input ("v2_loaders
 * FINDINGS", section 3: the towers are differentiable; the probe's backward
 * pass).  Per image and head, with P = softmax(q k^T / sqrt(head_dim)) of the
 * rotated q, k and D_i = sum_d dO_id O_id:
 *   dv = P^T dO,  dS = P * (dO v^T - D),  dq = dS k / sqrt(head_dim),
 *   dk = dS^T q / sqrt(head_dim),
 * then dq and dk rotated back by the opposite RoPE angle.
 *   qkv, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen: as in
 *              vt_attention_varlen (the forward is recomputed inside; its
 *              output and per-query log-sum-exp stay in the workspace).
 *   dout       bf16 [N, heads*head_dim]: dL/d(out), out as vt_attention_varlen's.
 *   dqkv       [N, 3, heads, head_dim], bf16 or fp32 by dqkv_dtype: dL/d(qkv).
 *              Every element is written; it may not overlap qkv or dout.
 *   ws         device workspace of vt_attention_backward_workspace_size bytes
 *              (about 36 KB per token at 16 heads, affine in the token count).
 * Pointers are 16-byte aligned device memory owned by the caller; ws 256-byte
 * aligned.  Errors, the RoPE-coordinate clamp and the fp16 operand range
 * (which here covers dO as well) as for vt_attention_varlen; nothing is
 * launched on error. */
vt_status vt_attention_backward(const vt_config* cfg, const uint16_t* qkv, const int32_t* cu_seqlens,
                                const int32_t* pos_thw, int32_t n_img, int32_t total_tokens,
                                int32_t max_seqlen, const uint16_t* dout, void* dqkv,
                                vt_dtype dqkv_dtype, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for vt_attention_backward.
 * Returns 0 and sets vt_last_error() if the arguments are invalid. */
size_t vt_attention_backward_workspace_size(const vt_config* cfg, int32_t total_tokens,
                                            int32_t n_img, int32_t max_seqlen);

/* One pre-LN block on the fp32 residual, in place:
 *   R += O(attention(RoPE(LN1(R) W_qkv^T + b_qkv)))  with O(a) = a W_o^T + b_o
 *   R += GELU_tanh(LN2(R) W_fc1^T + b_fc1) W_fc2^T + b_fc2
 * LayerNorm: biased variance over hidden, eps inside the square root.
 * Arguments as in vt_attention_varlen; resid is [total_tokens, hidden].  The
 * attention inside keeps vt_attention_varlen's RoPE-coordinate clamp and fp16
 * operand range (on the q, k, v this block computes). */
vt_status vt_block_forward(const vt_config* cfg, float* resid, const vt_block_weights* w,
                           const int32_t* cu_seqlens, const int32_t* pos_thw, int32_t n_img,
                           int32_t total_tokens, int32_t max_seqlen, void* ws, size_t ws_bytes,
                           void* stream);

/* Gradients of one block's parameters, fp32, each shaped like its weight in
 * vt_block_weights ([out, in] for the linears, [hidden] for LN gamma/beta).
 * A NULL member is not formed. */
typedef struct vt_block_grads {
  float *ln1_g, *ln1_b;
  float *w_qkv, *b_qkv;
  float *w_o, *b_o;
  float *ln2_g, *ln2_b;
  float *w_fc1, *b_fc1;
  float *w_fc2, *b_fc2;
} vt_block_grads;

/* Backward pass of vt_block_forward ("v2_loaders FINDINGS", section 3: the
 * towers are differentiable): given the block's input and dL/d(output), form
 * dL/d(input) and the parameter gradients.  The block's forward is
 * recomputed from resid_in; per linear y = x W^T + b: dx = dy W, dW = dy^T x,
 * db = column sums of dy; GELU(tanh) and LayerNorm by their derivatives;
 * attention as in vt_attention_backward.  Activations and dL/d(activation)
 * enter the products as bf16 (the forward's precision), accumulate in fp32.
 *   resid_in  fp32 [N, hidden]: the block's input (not modified).
 *   dresid    fp32 [N, hidden]: in, dL/d(block output); out, dL/d(resid_in).
 *   grads     host struct of device pointers (members may be NULL); each
 *             formed gradient is overwritten, not accumulated.
 *   other arguments as in vt_block_forward (with its clamp and fp16 operand
 *             range); hidden <= 2048.
 *   ws        vt_block_backward_workspace_size bytes (about 120 KB per token
 *             at the MiniMax-M3 shape, affine in the token count).
 * Errors as for vt_block_forward; nothing is launched on error. */
vt_status vt_block_backward(const vt_config* cfg, const float* resid_in, const vt_block_weights* w,
                            const int32_t* cu_seqlens, const int32_t* pos_thw, int32_t n_img,
                            int32_t total_tokens, int32_t max_seqlen, float* dresid,
                            const vt_block_grads* grads, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for vt_block_backward.
 * Returns 0 and sets vt_last_error() if the arguments are invalid. */
size_t vt_block_backward_workspace_size(const vt_config* cfg, int32_t total_tokens, int32_t n_img,
                                        int32_t max_seqlen);

/* Gradients of the tower's parameters (fp32): the patch embed and a host
 * array of cfg->layers block gradients.  NULL members are not formed. */
typedef struct vt_tower_grads {
  float *w_patch, *b_patch;          /* [hidden, 1176], [hidden] */
  const vt_block_grads* blocks;      /* host array of cfg->layers entries */
} vt_tower_grads;

/* Backward pass of the tower -- patch embed and cfg->layers blocks -- from
 * dL/d(tower output) ("v2_loaders FINDINGS", section 3: the probe mean-pools
 * the tower output and runs a backward pass through the tower).  Runs the
 * forward of vt_tower_forward keeping each block's input, then
 * vt_block_backward from the last block to the first, then the patch
 * embed's dW = dR0^T X and db = column sums of dR0.  The bf16 rounding of the
 * tower output is passed through as the identity.
 *   pixels, grid, n_img, w: as vt_tower_forward (w->proj is not read).
 *   d_tower   fp32 [N, hidden], raster order per item (the order of
 *             vt_tower_forward's tower_out): dL/d(tower output).
 *   grads     host struct; every formed gradient is overwritten.
 *   ws        vt_tower_backward_workspace_size bytes (about 320 KB per token at
 *             32 layers: each block's fp32 input is kept).
 * Errors, the clamp and the fp16 operand range as for vt_tower_forward;
 * hidden <= 2048; nothing is launched on error. */
vt_status vt_tower_backward(const vt_config* cfg, const uint16_t* pixels, const vt_grid_thw* grid,
                            int32_t n_img, const vt_tower_weights* w, const float* d_tower,
                            const vt_tower_grads* grads, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for vt_tower_backward; 0 (and vt_last_error()) if invalid. */
size_t vt_tower_backward_workspace_size(const vt_config* cfg, const vt_grid_thw* grid, int32_t n_img);

/* 2x2 merge + projector (README Architecture, Projector row).
 *   tower      bf16 [N, hidden] tower tokens, rows in `order`.
 *   merged_raw bf16 [N/4, 4*hidden] or NULL: the 2x2 gather of the tower
 *              tokens (the "5120-wide merged tokens"), merged raster order.
 *   out        bf16 [N/4, proj_out], merged raster order per image:
 *              Y = GELU(T W1^T + b1) W2^T + b2 per token; Z[m] = the four Y
 *              rows of merged token m in slot order 2*dr+dc (24576 wide);
 *              out = GELU(Z W3^T + b3) W4^T + b4. */
vt_status vt_merge_project(const vt_config* cfg, const uint16_t* tower, vt_order order,
                           const vt_grid_thw* grid, int32_t n_img, const vt_projector_weights* w,
                           uint16_t* merged_raw, uint16_t* out, void* ws, size_t ws_bytes,
                           void* stream);

/* The whole forward pass: patch embed, cfg->layers blocks, then (if `out` is
 * not NULL) merge + projector.
 *   tower_out  bf16 [N, hidden] raster order, or NULL (last_hidden_state).
 *   merged_raw bf16 [N/4, 4*hidden] or NULL.
 *   out        bf16 [N/4, proj_out] or NULL.  At least one output is needed.
 * Positions come from the grid list, so the RoPE clamp never applies; the
 * attention of every block keeps vt_attention_varlen's fp16 operand range on
 * the q, k, v the blocks compute (|RoPE(q)| below about 4.06e5 before its
 * log2(e)/sqrt(head_dim) scale, |RoPE(k)| and |v| below 65504). */
vt_status vt_tower_forward(const vt_config* cfg, const uint16_t* pixels, const vt_grid_thw* grid,
                           int32_t n_img, const vt_tower_weights* w, uint16_t* tower_out,
                           uint16_t* merged_raw, uint16_t* out, void* ws, size_t ws_bytes,
                           void* stream);

/* ---------------------------------------------------------------- planning
 * Host-only: no device work, no stream. */

/* Patches one call can hold in a workspace budget: the analogue of the pages'
 * derive_max_patches ("init.rs (VisionEncoder::new)": patches = area /
 * patch^2, clamped to what memory affords, the clamp reported).  Scratch here
 * is O(tokens), so the limit is the budget, not a fixed ceiling.
 *   budget_bytes workspace bytes available to one call.
 *   n_img        items per call.
 *   max_pixels   an area bound in pixels per call, or 0 for none.
 *   patches      out: min(max_pixels / patch^2, the largest token count, a
 *                multiple of 4, that fits for any grid of n_img items).
 *   wanted       out: max_pixels / patch^2 when that was clamped, else 0.
 * VT_ERR_WORKSPACE if not even 4 tokens per item fit. */
vt_status vt_plan_patches(const vt_config* cfg, size_t budget_bytes, int32_t n_img,
                          int64_t max_pixels, int64_t* patches, int64_t* wanted);

/* Greedy packing of the items, in list order, into calls whose workspace
 * (vt_tower_workspace_size of the call's items) fits budget_bytes: a call
 * takes items until the next one would not fit.
 *   batch      out, [n_img] host array: call index of each item (0, 1, ...).
 *   n_batches  out: number of calls.
 * VT_ERR_WORKSPACE, naming the item, if one item alone does not fit (nothing
 * is dropped or clamped). */
vt_status vt_pack_items(const vt_config* cfg, const vt_grid_thw* grid, int32_t n_img,
                        size_t budget_bytes, int32_t* batch, int32_t* n_batches);

/* Mean-pooled feature ("v2_loaders FINDINGS" section 3: the tower's output
 * sequence mean-pooled to (1, 1280) per image).
 *   tower      bf16 [N, hidden] tower tokens in token or raster order (the
 *              mean does not depend on the order inside an item).
 *   cu_seqlens [n_img+1] int32 on the device (vt_build_metadata).
 *   out        fp32 [n_img, hidden]: the mean of each item's rows, summed in
 *              fp32 in a fixed order (deterministic).
 * hidden must be a multiple of 128.  No workspace. */
vt_status vt_mean_pool(const uint16_t* tower, const int32_t* cu_seqlens, int32_t n_img,
                       int32_t hidden, float* out, void* stream);

/* ---------------------------------------------------------------- kernels
 * The two non-attention kernels of the path, exposed on their own.
 * vt_linear: y = x W^T + b with x bf16 [M, K], W bf16 [N, K], b bf16 [N] or
 * NULL, fp32 accumulation, then the epilogue (see vt_epilogue); out is bf16
 * or fp32 [M, N].  K must be a multiple of 8; N a multiple of 64.
 * ws: at least vt_linear_workspace_size(M, N, K) bytes (may be 0).
 * Shapes with few output tiles split K: the fp32 partial products go to ws,
 * vt_linear_workspace_size(M, N, K) = splits * M * N * 4 bytes, and a second
 * kernel sums them in split order.  VT_EPI_SPLITK_PARTIALS_F32 stops before
 * that sum: out receives the partials themselves (it must hold
 * vt_linear_workspace_size(M, N, K) bytes), bias must be NULL, ws is unused;
 * a shape that is not split returns VT_ERR_UNSUPPORTED. */
size_t vt_linear_workspace_size(int32_t M, int32_t N, int32_t K);
vt_status vt_linear(const uint16_t* x, int32_t M, int32_t K, const uint16_t* w, int32_t N,
                    const uint16_t* bias, vt_epilogue epi, void* out, void* ws, size_t ws_bytes,
                    void* stream);

/* The residual step of a pre-LN block (README Architecture: the attention
 * output projection followed by LN2, and the second MLP Linear followed by
 * the next block's LN1), as the blocks run it:
 *   R   += x W^T + b          (R fp32 [M, N], in place; b bf16 [N] or NULL)
 *   out  = LN(R) * g + beta   (bf16 [M, N]; biased variance, eps inside the
 *                              square root)
 * When the shape splits K, the partial products are summed in split order,
 * the bias and the old R added and the LayerNorm taken in one kernel; else
 * the GEMM updates R in its epilogue and a LayerNorm kernel follows.
 *   x bf16 [M, K], W bf16 [N, K]; K a multiple of 8; N a multiple of 256, at
 *   most 4096.  ws: vt_linear_workspace_size(M, N, K) bytes. */
vt_status vt_linear_residual_ln(const uint16_t* x, int32_t M, int32_t K, const uint16_t* w, int32_t N,
                                const uint16_t* bias, float* R, const uint16_t* g, const uint16_t* beta,
                                float eps, uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* vt_layer_norm: out bf16 [rows, width] = LN(x) * g + b over fp32 x [rows, width];
 * width must be a multiple of 256 and at most 4096. */
vt_status vt_layer_norm(const float* x, int32_t rows, int32_t width, const uint16_t* g,
                        const uint16_t* b, float eps, uint16_t* out, void* stream);

/* ---------------------------------------------------------------- measurement
 * vt_clock_probe: the core clock while other work runs (not part of the
 * path; the benchmark uses it to state each roofline fraction also against
 * the clock the chip actually ran at, since the published bf16 peak assumes
 * the 2.4 GHz peak engine clock).  Enqueues on `stream` one wavefront that
 * reads the shader-clock counter and the constant-rate real-time counter,
 * waits until wait_us microseconds of real time have passed (a wait on a
 * counter that always advances), and reads both again.
 *   wait_us      1 .. 10,000,000.
 *   out          device, 8-byte aligned, 4 x uint64 written when the kernel
 *                ends: clock ticks at start and end, real-time ticks at
 *                start and end.
 *   realtime_hz  host, written during the call: the real-time counter rate.
 * Core clock (Hz) = (out[1] - out[0]) / (out[3] - out[2]) * realtime_hz.
 * Launch it on a second stream just before the work to be measured. */
vt_status vt_clock_probe(int64_t wait_us, unsigned long long* out, int64_t* realtime_hz,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VT_H */
