// Host-side launchers of the gfx950 kernels.  Each returns hipSuccess or the
// launch error; shapes are validated by the caller (vt_api.cpp) before any
// launcher runs.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vt {

// ---- metadata (meta.hip)
constexpr int kMetaChunk = 128;  // images per metadata launch (kernel-argument table)
struct ImgInfo {                 // one item (image or clip) as the device kernels see it
  int32_t t, h, w;               // temporal patches and patch grid; t == 1: one still frame
  int64_t pix_off;               // first pixel of the item in the packed pixel array
};
struct MetaChunk {
  int32_t first, count;          // items [first, first+count)
  int32_t t[kMetaChunk], h[kMetaChunk], w[kMetaChunk], cu[kMetaChunk];
  int64_t pix_off[kMetaChunk];
};
hipError_t launch_metadata(const MetaChunk& c, int32_t max_tokens_in_chunk, int32_t* cu_seqlens,
                           ImgInfo* info, int32_t* pos_thw, int32_t* raster_index,
                           int32_t* tok_img, hipStream_t s);
hipError_t launch_cu_last(int32_t* cu_seqlens, int32_t n_img, int32_t total, hipStream_t s);

// Attention work schedule: images ordered by token count (largest first),
// tile_start[r] = first q-tile of the image of rank r; ktile_start[i] = first
// 64-key tile of image i (image order) in the packed K/V tile images.
// qdesc[t] = (first query, image begin, image end, first key tile of the
// image) of q-tile slot t < max_qtiles; kdesc[T] = (first token, image end)
// of key-tile slot T < max_ktiles; unused slots have .x = -1.  qkpre, when
// not null, receives max_qtiles + 1 entries: qkpre[t] = the key tiles of the
// q-tile slots before t (a q-tile's key tiles are those of its image; unused
// slots count 0).
hipError_t launch_attn_schedule(const int32_t* cu_seqlens, int32_t n_img, int32_t q_tile,
                                int32_t k_tile, int32_t max_qtiles, int32_t max_ktiles,
                                int32_t* order, int32_t* tile_start, int32_t* ktile_start,
                                int4* qdesc, int2* kdesc, hipStream_t s, int32_t* qkpre = nullptr);
// RoPE table cs[pos][j] = (cos, sin)(pos * inv_freq[j]), pos < n_pos, j < 40.
struct RopeFreq { double inv_freq[64]; int32_t pairs; };
hipError_t launch_rope_table(const RopeFreq& f, int32_t n_pos, float2* cs, hipStream_t s);

// ---- permutations (permute.hip)
hipError_t launch_patchify(const uint16_t* pixels, const ImgInfo* info, const int32_t* cu_seqlens,
                           const int32_t* tok_img, int32_t total_tokens, uint16_t* X,
                           hipStream_t s);
// dst[raster_index[j]] = src[j] (scatter == true) or dst[j] = src[raster_index[j]].
// out[i] = mean of rows cu[i] .. cu[i+1]-1 of T (bf16 [N, hidden]), fp32; hidden % 128 == 0.
hipError_t launch_mean_pool(const uint16_t* T, const int32_t* cu_seqlens, int32_t n_img,
                            int32_t hidden, float* out, hipStream_t s);
hipError_t launch_clock_probe(uint64_t ticks, unsigned long long* out, hipStream_t s);
hipError_t launch_row_permute(const uint16_t* src, uint16_t* dst, const int32_t* raster_index,
                              int32_t rows, int32_t width, bool scatter, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t s);

// ---- LayerNorm (layernorm.hip)
hipError_t launch_layer_norm(const float* x, int32_t rows, int32_t width, const uint16_t* g,
                             const uint16_t* b, float eps, uint16_t* out, hipStream_t s);
// R += sum_z part[z] (z = 0..splits-1 in order) + bias, then out = LN(R; g, b, eps);
// part is [splits][rows][width] fp32 (the split-K partials of launch_gemm_partials).
hipError_t launch_resid_ln(const float* part, int32_t splits, int32_t rows, int32_t width,
                           const uint16_t* bias, float* R, const uint16_t* g, const uint16_t* b,
                           float eps, uint16_t* out, hipStream_t s);

// ---- GEMM (gemm.hip)
enum Epi : int { kEpiBf16 = 0, kEpiGeluTanh = 1, kEpiGeluErf = 2, kEpiResid = 3, kEpiF32 = 4,
                 kEpiQkvPack = 5 };
struct GemmPlan {
  int bm, bn;        // tile
  int splits;        // split-K factor (1 = none)
  int kper;          // K elements per split (multiple of 64)
  // Stream-K tail (256 x 256 tiles only): the first n_whole tiles run whole,
  // one workgroup each (whole rounds of the GPU's workgroups); the K steps of
  // the rest are shared evenly by sk_wgs workgroups (0: no tail split).
  int n_whole = 0;
  int sk_wgs = 0;
  // Partial last round without a stream-K tail (256 x 256 tiles only): the
  // first n_whole tiles run whole and the last tail128 tiles run as four
  // 128 x 128 quadrants each (0: none).
  int tail128 = 0;
};
// Which tiles a gemm_dl_kernel launch covers: its blocks map to the first npid
// tiles (XCD-contiguous); with a stream-K tail, the tail kernel's sk_wgs blocks
// share the K steps of the tiles from n_whole on.
struct TileSched {
  int npid;
  int n_whole;
  int sk_wgs;
  int tail_of = -1;  // >= 0 (128 x 128 launches): the quadrants of 256 x 256 tiles tail_of, tail_of + 1, ...
};
GemmPlan plan_gemm(int M, int N, int K);
size_t gemm_workspace_bytes(int M, int N, int K);
hipError_t launch_gemm(const uint16_t* A, int M, int K, const uint16_t* B, int N,
                       const uint16_t* bias, int epi, void* out, void* ws, hipStream_t s);
// Split-K GEMMs only: writes the fp32 partials part[z][M][N] of plan_gemm's
// splits (> 1) to ws, no bias and no epilogue (launch_resid_ln finishes them).
hipError_t launch_gemm_partials(const uint16_t* A, int M, int K, const uint16_t* B, int N, void* ws,
                                hipStream_t s);
// The QKV Linear of a block (N = 3 * d, head_dim 80) with the attention's
// pack step as its epilogue: y = x W_qkv^T + b rounded to bf16 (the values
// the pack kernel would read), then 3D RoPE on q and k (pairs (j, j+40) of
// a head), q scaled by q_scale, both rounded to fp16: Q rows into qpk
// [N, heads, 80], K rows and V^T columns into the tile images of kv at the
// slots given by kslot (launch_attn_image_init).  W_qkv rows are read in an
// order that puts both halves of every rotation pair in one output tile.
struct QkvPack {
  uint16_t* qpk;
  uint16_t* kv;
  const int32_t* pos;     // [N, 3] positions (t, row, col)
  const int32_t* kslot;   // [N]
  const float2* rope;     // [n_pos, 40] (cos, sin)
  int32_t n_pos, axis_code, heads, d;
  float q_scale;
};
hipError_t launch_gemm_qkv_pack(const uint16_t* A, int M, int K, const uint16_t* B, const uint16_t* bias,
                                const QkvPack& pk, hipStream_t s);

// ---- attention (attention.hip)
constexpr int kAttnKTile = 64;         // keys per tile
constexpr int kAttnTileBytes = 24576;  // one (head, key tile) image: K [64][88] + V^T [81][72] fp16 + pad
constexpr int kAttnKRow = 88;          // fp16 per K row of an image (dims 0..79 + pad)
constexpr int kAttnVRow = 72;          // fp16 per V^T row of an image (64 key slots + pad)
// Attention kernel variants, chosen by the size of the call:
//   kAttnSmall  attention_kernel, two key groups of 2 wavefronts, 64 queries
//               per workgroup (few query tiles: every CU gets work);
//   kAttnLean4  attention_lean_kernel, 4 wavefronts = 128 queries, three
//               workgroups per CU;
//   kAttnLean8  attention_lean_kernel, 8 wavefronts = 256 queries, two
//               workgroups per CU (many query tiles).
enum AttnVariant : int { kAttnSmall = 0, kAttnLean4 = 1, kAttnLean8 = 2 };
inline int attn_q_tile(int variant) {
  return variant == kAttnSmall ? 64 : variant == kAttnLean4 ? 128 : 256;
}
// The split tail of the lean kernels.  Work items are (q-tile, head) pairs,
// q-tile major, in the schedule's order; one workgroup runs each.  When the
// items do not fill a whole number of rounds of the workgroups the GPU holds
// at once (S of them), the last, partial round is instead spread evenly over
// S workgroups by key tiles: workgroup k of the tail takes key tiles
// [k T / S, (k+1) T / S) of the tail's T (item after item, each item's
// key tiles in order), and an item cut between workgroups leaves unnormalized
// partial results (O, running max, row sum) that a merge kernel combines.
// qkpre / nq: launch_attn_schedule's qkpre and q-tile count (tile_start[n_img]);
// part: attn_tail_records(variant) records of attn_tail_record_floats(variant)
// floats (attn_tail_part_floats() covers either lean variant), or null for no
// split.
struct AttnTail {
  const int32_t* qkpre = nullptr;
  const int32_t* nq = nullptr;
  float* part = nullptr;
  // Optional, host memory: the images' token counts, when the caller knows
  // them; a call whose plan (formed here on the host as on the device) has no
  // split then launches neither the extra workgroups nor the merge.
  const int64_t* host_tokens = nullptr;
  int32_t host_n_img = 0;
};
constexpr int kAttnTailMinTiles = 8;       // no split when a tail workgroup would get fewer key tiles
constexpr int kAttnTailMinItemTiles = 64;  // ... or when the tail's longest item has fewer
inline int attn_tail_max_wgs(int variant) { return variant == kAttnLean4 ? 768 : 512; }
inline int64_t attn_tail_records(int variant) { return variant == kAttnSmall ? 0 : 2 * attn_tail_max_wgs(variant); }
inline int64_t attn_tail_record_floats(int variant) { return int64_t(attn_q_tile(variant)) * 82; }
inline int64_t attn_tail_part_floats() {
  const int64_t a = attn_tail_records(kAttnLean4) * attn_tail_record_floats(kAttnLean4);
  const int64_t b = attn_tail_records(kAttnLean8) * attn_tail_record_floats(kAttnLean8);
  return a > b ? a : b;
}

// qpk: [N, heads, 80] fp16 rotated+scaled Q; kv: max_ktiles x heads tile
// images.  qdesc / kdesc come from launch_attn_schedule with
// attn_q_tile(variant) and the same max_qtiles / max_ktiles.  lse, when
// not null, receives [N, heads] fp32: the log2-domain log-sum-exp of each
// query's scaled scores (max + log2 of the row sum).
hipError_t launch_attention(const uint16_t* qkv, const int32_t* pos_thw, const int4* qdesc,
                            const int2* kdesc, int32_t max_qtiles, int32_t max_ktiles,
                            int32_t heads, int32_t n_pos, int32_t axis_code, const float2* rope_cs,
                            float q_scale_log2, int32_t variant, uint16_t* qpk, uint16_t* kv,
                            void* out, bool out_f32, float* lse, hipStream_t s,
                            const AttnTail& tail = AttnTail());

// The pack kernel alone: rotated, scaled fp16 Q into qpk and the K/V tile
// images into kv, from bf16 qkv [N, 3, heads, 80] (the first step of
// launch_attention).
hipError_t launch_attn_pack(const uint16_t* qkv, const int32_t* pos_thw, const int2* kdesc, int32_t max_ktiles,
                            int32_t heads, int32_t n_pos, int32_t axis_code, const float2* rope_cs,
                            float q_scale_log2, uint16_t* qpk, uint16_t* kv, hipStream_t s);

// The attention kernel alone, on Q and tile images already packed (by the
// pack kernel inside launch_attention, or by the QKV GEMM epilogue).
hipError_t launch_attention_packed(const uint16_t* qpk, const uint16_t* kv, const int4* qdesc,
                                   int32_t max_qtiles, int32_t heads, int32_t variant, void* out,
                                   bool out_f32, float* lse, hipStream_t s, const AttnTail& tail = AttnTail());
// Layer-independent parts of the tile images (V^T ones rows, zero padding
// keys) and kslot[tok] = 64 * key tile + slot of every token (int32 [N]),
// from launch_attn_schedule's kdesc; run once before launch_gemm_qkv_pack.
hipError_t launch_attn_image_init(const int2* kdesc, int32_t max_ktiles, int32_t heads, uint16_t* kv,
                                  int32_t* kslot, hipStream_t s);

// ---- block backward helpers (backward.hip)
// 64 x 64-tiled transpose of in [M, C] (fp32 or bf16; C a multiple of 4, Mp
// a multiple of 64, Mp >= M) with v = op(in): op 0 identity, 1 GELU(tanh), 2 in * GELU'(aux)
// (aux bf16 [M, C]; fp32 input only with op 0).  Optional outputs: copy
// [M, C] bf16(v), outT [C, Mp] bf16(v)^T (rows M.. zero), colsum [C] = the
// column sums of bf16(v), formed per 64-row tile in colpart [Mp/64][C] and
// summed in tile order (reproducible bit for bit).
hipError_t launch_transpose(const void* in, bool in_f32, int op, const uint16_t* aux, int32_t M,
                            int32_t C, int32_t Mp, uint16_t* copy, uint16_t* outT, float* colsum,
                            float* colpart, hipStream_t s);
// dx = dres + LayerNorm'(x; g)^T dy per row (width = 256 k, k <= 8); dg, db =
// the gamma / beta gradients, summed per block into part
// [ln_backward_blocks(rows)][2][width] and then in block order.  dx may alias dres.
constexpr int kLnBwdMaxBlocks = 256;
int ln_backward_blocks(int32_t rows);
hipError_t launch_ln_backward(const float* x, const uint16_t* g, const float* dy, const float* dres,
                              int32_t rows, int32_t width, float eps, float* dx, float* dg,
                              float* db, float* part, hipStream_t s);
// out [C, R] = in [R, C]^T, fp32.
hipError_t launch_transpose_f32(const float* in, int32_t R, int32_t C, float* out, hipStream_t s);

// ---- attention backward (attention_bwd.hip)
// Tile images of 64 tokens of one head: the key side (K, V, K^T) and the
// query side (Q, dO, Q^T, dO^T, log-sum-exp, D).
constexpr int kAttnBwdKBytes = 36864;
constexpr int kAttnBwdQBytes = 49152;
constexpr int kAttnBwdTile = 128;  // queries (dQ pass) or keys (dK/dV pass) per workgroup
// o: the forward output [N, heads*80] fp32; lse: its [N, heads] log-sum-exp;
// dout: [N, heads*80] bf16.  kdesc from launch_attn_schedule (key tiles of
// 64), bdesc from a schedule with q_tile = kAttnBwdTile (max_btiles slots).
// kdesc256, when not null, is a schedule with q_tile = kAttnBwdWideTile
// (max_ktiles256 slots): the dK/dV pass then runs 8 wavefronts of 256 keys
// (attn_bwd_wide decides).  dqkv: [N, 3, heads, 80], bf16 or fp32.
constexpr int kAttnBwdWideTile = 256;
inline bool attn_bwd_wide(int64_t N, int32_t n_img, int32_t heads) {
  return ((N + kAttnBwdWideTile - 1) / kAttnBwdWideTile + n_img) * heads >= 1024;
}
hipError_t launch_attention_backward(const uint16_t* qkv, const uint16_t* dout, const float* o,
                                     const float* lse, const int32_t* pos_thw, const int2* kdesc,
                                     const int4* bdesc, int32_t max_ktiles, int32_t max_btiles,
                                     int32_t heads, int32_t n_pos, int32_t axis_code,
                                     const float2* rope_cs, float q_scale_log2, char* qimg,
                                     char* kimg, void* dqkv, bool out_f32, const int4* kdesc256,
                                     int32_t max_ktiles256, hipStream_t s);

}  // namespace vt
