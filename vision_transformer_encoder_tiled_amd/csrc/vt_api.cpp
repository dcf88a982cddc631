// C ABI of the tiled ViT vision tower: argument validation, workspace
// planning (linear in the token count), and launch sequencing on the
// caller's stream.  Every check runs before the first launch, in every
// build; a failing call launches nothing and records the reason in a
// thread-local string.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/vt.h"
#include "vt_kernels.h"

#define VT_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_err;

vt_status fail(vt_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define VT_TRY_HIP(expr)                                                                   \
  do {                                                                                     \
    hipError_t _e = (expr);                                                                \
    if (_e != hipSuccess) return fail(VT_ERR_HIP, "%s: %s", #expr, hipGetErrorString(_e)); \
  } while (0)

constexpr int64_t kMaxTokens = int64_t(1) << 26;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

vt_status check_config(const vt_config* c) {
  if (!c) return fail(VT_ERR_INVALID_ARG, "cfg is NULL");
  if (c->hidden <= 0 || c->heads <= 0 || c->head_dim <= 0 || c->mlp <= 0 || c->layers < 0 ||
      c->proj_hidden <= 0 || c->proj_out <= 0)
    return fail(VT_ERR_INVALID_ARG, "config sizes must be positive (layers >= 0)");
  if (c->hidden != c->heads * c->head_dim)
    return fail(VT_ERR_INVALID_ARG, "hidden %d != heads %d * head_dim %d", c->hidden, c->heads,
                c->head_dim);
  if (!(c->ln_eps > 0.f) || !(c->rope_theta > 0.f))
    return fail(VT_ERR_INVALID_ARG, "ln_eps and rope_theta must be > 0");
  if (c->rope_pairs[0] < 0 || c->rope_pairs[1] < 0 || c->rope_pairs[2] < 0 ||
      c->rope_pairs[0] + c->rope_pairs[1] + c->rope_pairs[2] != c->head_dim / 2)
    return fail(VT_ERR_INVALID_ARG, "rope_pairs must be >= 0 and sum to head_dim/2");
  if (c->head_dim != 80)
    return fail(VT_ERR_UNSUPPORTED, "attention kernel implements head_dim 80 (got %d)", c->head_dim);
  if (c->patch != 14 || c->t_patch != 2 || c->merge != 2)
    return fail(VT_ERR_UNSUPPORTED, "kernels implement patch 14, temporal patch 2, merge 2");
  if (c->rope_pairs[0] % 8 || c->rope_pairs[1] % 8 || c->rope_pairs[2] % 8)
    return fail(VT_ERR_UNSUPPORTED, "rope_pairs must be multiples of 8");
  if (c->hidden % 256 || c->hidden > 4096)
    return fail(VT_ERR_UNSUPPORTED, "hidden must be a multiple of 256, at most 4096");
  if (c->mlp % 64 || c->proj_hidden % 64 || c->proj_out % 64)
    return fail(VT_ERR_UNSUPPORTED, "mlp, proj_hidden and proj_out must be multiples of 64");
  if (c->heads > 1024) return fail(VT_ERR_UNSUPPORTED, "at most 1024 heads");
  return VT_OK;
}

struct GridInfo {
  int64_t tokens = 0;
  int32_t max_hw = 0;     // largest t, h or w: RoPE positions lie in [0, max_hw)
  int32_t max_seq = 0;    // largest image token count
  int64_t pixels = 0;
};

// Token counts t*h*w of the items of a grid list.
std::vector<int64_t> grid_tokens(const vt_grid_thw* grid, int32_t n_img) {
  std::vector<int64_t> n(n_img);
  for (int i = 0; i < n_img; ++i) n[i] = int64_t(grid[i].t) * grid[i].h * grid[i].w;
  return n;
}

// Frames stored per item: one still frame for t = 1, 2t frames for a clip.
int64_t frames_of(int32_t t) { return t == 1 ? 1 : 2 * int64_t(t); }

vt_status check_grid(const vt_grid_thw* grid, int32_t n_img, GridInfo* gi) {
  if (!grid) return fail(VT_ERR_INVALID_ARG, "grid is NULL");
  if (n_img <= 0) return fail(VT_ERR_INVALID_ARG, "n_img must be >= 1 (got %d)", n_img);
  GridInfo g;
  for (int i = 0; i < n_img; ++i) {
    const vt_grid_thw& x = grid[i];
    if (x.t <= 0 || x.h <= 0 || x.w <= 0)
      return fail(VT_ERR_INVALID_ARG, "image %d: t, h, w must be positive (got %d, %d, %d)", i,
                  x.t, x.h, x.w);
    if (x.h % 2 || x.w % 2)
      return fail(VT_ERR_INVALID_ARG, "image %d: h and w must be even for the 2x2 merge (got %d x %d)",
                  i, x.h, x.w);
    const int64_t n = int64_t(x.t) * x.h * x.w;
    if (n > kMaxTokens)
      return fail(VT_ERR_UNSUPPORTED, "image %d: more than %lld tokens", i, (long long)kMaxTokens);
    g.tokens += n;
    if (g.tokens > kMaxTokens)
      return fail(VT_ERR_UNSUPPORTED, "more than %lld tokens in one call", (long long)kMaxTokens);
    g.max_hw = std::max(g.max_hw, std::max(x.t, std::max(x.h, x.w)));
    g.max_seq = std::max<int32_t>(g.max_seq, int32_t(n));
    g.pixels += int64_t(frames_of(x.t)) * x.h * x.w * 3 * 196;
  }
  *gi = g;
  return VT_OK;
}

// ---- workspace carving
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

struct Dims {
  int32_t N, n_img, d, mlp, heads, P, Pout;
  bool ws_upper = false;  // size split-K partials at their bound for any M (capacity planning)
};

// Split-K partials never exceed 256 tiles of 256 x 256 fp32: tiles x splits
// is kept <= 256 (gemm.hip plan_gemm).
constexpr size_t kPartialsBound = size_t(256) * 256 * 256 * sizeof(float);

// Buffers of one block, used by vt_block_forward and vt_tower_forward.
struct BlockBufs {
  int32_t* order;
  int32_t* tile_start;
  int32_t* ktile_start;
  int4* qdesc;     // per q-tile slot (max_q_tiles at 64 queries)
  int32_t* qkpre;  // key tiles before each q-tile slot (max_q_tiles at 64 queries, + 1)
  float* part;     // partial records of the lean kernel's split tail (null: no split)
  int2* kdesc;     // per key-tile slot
  const int64_t* host_tokens = nullptr;  // the images' token counts when the host knows them
  int32_t host_n_img = 0;
  uint16_t* qpk;   // [N, heads, 80] fp16 rotated, scaled Q
  uint16_t* kv;    // max_ktiles x heads K/V tile images (fp16)
  int32_t* kslot;  // [N] tile image and slot of each token's key
  float2* rope;
  uint16_t* xn;    // [N, d] LayerNorm output
  uint16_t* act;   // [N, max(4d, mlp)]: qkv [N,3d] then attn [N,d]; later the MLP hidden [N, mlp]
  void* gemm_ws;   // split-K partials
};

size_t block_gemm_ws(int N, int d, int mlp) {
  size_t w = vt::gemm_workspace_bytes(N, d, 1176);  // patch embed shares this buffer
  w = std::max(w, vt::gemm_workspace_bytes(N, 3 * d, d));
  w = std::max(w, vt::gemm_workspace_bytes(N, d, d));
  w = std::max(w, vt::gemm_workspace_bytes(N, mlp, d));
  w = std::max(w, vt::gemm_workspace_bytes(N, d, mlp));
  return w;
}

int32_t max_k_tiles(int64_t N, int32_t n_img) {
  return int32_t((N + vt::kAttnKTile - 1) / vt::kAttnKTile + n_img);
}

int32_t max_q_tiles(int64_t N, int32_t n_img, int32_t q_tile) {
  return int32_t((N + q_tile - 1) / q_tile + n_img);
}

int32_t attn_variant(int64_t N, int32_t n_img, int32_t heads);

// The attention step's buffers (schedule, packed Q, tile images, RoPE table,
// and with split_tail the lean kernel's partial records).
void carve_attention(Carver& c, const Dims& D, int32_t n_pos, BlockBufs* b, bool split_tail = true) {
  b->order = c.take<int32_t>(D.n_img);
  b->tile_start = c.take<int32_t>(D.n_img + 1);
  b->ktile_start = c.take<int32_t>(D.n_img + 1);
  b->qdesc = c.take<int4>(max_q_tiles(D.N, D.n_img, vt::attn_q_tile(vt::kAttnSmall)));
  b->qkpre = c.take<int32_t>(max_q_tiles(D.N, D.n_img, vt::attn_q_tile(vt::kAttnSmall)) + 1);
  const int32_t var = attn_variant(D.N, D.n_img, D.heads);
  // one size for both lean variants, so the workspace stays affine in the
  // token count across the switch between them
  b->part = split_tail && var != vt::kAttnSmall ? c.take<float>(size_t(vt::attn_tail_part_floats())) : nullptr;
  b->kdesc = c.take<int2>(max_k_tiles(D.N, D.n_img));
  b->qpk = c.take<uint16_t>(size_t(D.N) * D.d);
  b->kv = reinterpret_cast<uint16_t*>(
      c.take<char>(size_t(D.heads) * max_k_tiles(D.N, D.n_img) * vt::kAttnTileBytes));
  b->kslot = c.take<int32_t>(D.N);
  b->rope = c.take<float2>(size_t(n_pos) * 40);
}

void carve_block(Carver& c, const Dims& D, int32_t n_pos, BlockBufs* b) {
  carve_attention(c, D, n_pos, b);
  b->xn = c.take<uint16_t>(size_t(D.N) * D.d);
  b->act = c.take<uint16_t>(size_t(D.N) * std::max(4 * D.d, D.mlp));
  b->gemm_ws = c.take<char>(D.ws_upper ? kPartialsBound : block_gemm_ws(D.N, D.d, D.mlp));
}

struct TowerBufs {
  int32_t *cu, *pos, *ridx, *tok_img;
  vt::ImgInfo* info;
  float* R;        // [N, d] fp32 residual
  uint16_t* X;     // [N, 1176] patches (aliases the block's act region)
  uint16_t* T;     // [N, d] bf16 tower tokens, token order
  uint16_t *Y1, *Y2, *U;
  void* proj_ws;
  BlockBufs blk;
};

size_t proj_gemm_ws(int N, int d, int P, int Pout) {
  size_t w = 0;
  w = std::max(w, vt::gemm_workspace_bytes(N, P, d));
  w = std::max(w, vt::gemm_workspace_bytes(N, P, P));
  w = std::max(w, vt::gemm_workspace_bytes(N / 4, Pout, 4 * P));
  w = std::max(w, vt::gemm_workspace_bytes(N / 4, Pout, Pout));
  return w;
}

void carve_tower(Carver& c, const Dims& D, int32_t n_pos, TowerBufs* t) {
  t->cu = c.take<int32_t>(D.n_img + 1);
  t->info = c.take<vt::ImgInfo>(D.n_img);
  t->pos = c.take<int32_t>(size_t(D.N) * 3);
  t->ridx = c.take<int32_t>(D.N);
  t->tok_img = c.take<int32_t>(D.N);
  t->R = c.take<float>(size_t(D.N) * D.d);
  t->T = c.take<uint16_t>(size_t(D.N) * D.d);
  carve_block(c, D, n_pos, &t->blk);
  // Patches are only live before the first block: they share the act region
  // when it is large enough, else get their own buffer.
  if (size_t(std::max(4 * D.d, D.mlp)) >= 1176)
    t->X = t->blk.act;
  else
    t->X = c.take<uint16_t>(size_t(D.N) * 1176);
  t->Y1 = c.take<uint16_t>(size_t(D.N) * D.P);
  t->Y2 = c.take<uint16_t>(size_t(D.N) * D.P);
  t->U = c.take<uint16_t>(size_t(D.N / 4) * D.Pout);
  t->proj_ws = c.take<char>(D.ws_upper ? kPartialsBound : proj_gemm_ws(D.N, D.d, D.P, D.Pout));
}

Dims dims_of(const vt_config* cfg, int64_t N, int32_t n_img) {
  return Dims{int32_t(N), n_img, cfg->hidden, cfg->mlp, cfg->heads, cfg->proj_hidden,
              cfg->proj_out};
}

vt::RopeFreq rope_freq(const vt_config* cfg, int32_t* axis_code) {
  vt::RopeFreq f{};
  const int half = cfg->head_dim / 2;
  f.pairs = half;
  int j = 0, code = 0;
  for (int a = 0; a < 3; ++a) {
    const int n = cfg->rope_pairs[a];
    for (int k = 0; k < n; ++k, ++j) {
      // per-axis ladder theta^(-2k / (2n)); shared ladder theta^(-2j / head_dim)
      f.inv_freq[j] = cfg->rope_shared_ladder
                          ? std::pow(double(cfg->rope_theta), -2.0 * j / cfg->head_dim)
                          : std::pow(double(cfg->rope_theta), -2.0 * k / (2.0 * n));
      if (j % 8 == 0) code |= a << (2 * (j / 8));
    }
  }
  *axis_code = code;
  return f;
}

vt_status launch_meta(const vt_grid_thw* grid, int32_t n_img, int64_t total, int32_t* cu,
                      vt::ImgInfo* info, int32_t* pos, int32_t* ridx, int32_t* tok_img,
                      hipStream_t s) {
  int64_t tok = 0, pix = 0;
  for (int first = 0; first < n_img; first += vt::kMetaChunk) {
    vt::MetaChunk c{};
    c.first = first;
    c.count = std::min(vt::kMetaChunk, n_img - first);
    int32_t maxn = 0;
    for (int i = 0; i < c.count; ++i) {
      const vt_grid_thw& g = grid[first + i];
      c.t[i] = g.t;
      c.h[i] = g.h;
      c.w[i] = g.w;
      c.cu[i] = int32_t(tok);
      c.pix_off[i] = pix;
      const int64_t n = int64_t(g.t) * g.h * g.w;
      maxn = std::max<int32_t>(maxn, int32_t(n));
      tok += n;
      pix += frames_of(g.t) * g.h * g.w * 3 * 196;
    }
    VT_TRY_HIP(vt::launch_metadata(c, maxn, cu, info, pos, ridx, tok_img, s));
  }
  if (cu) VT_TRY_HIP(vt::launch_cu_last(cu, n_img, int32_t(total), s));
  return VT_OK;
}

// Attention kernel variant (vt_kernels.h): 64-query workgroups with two key
// groups when 128-query tiles would not give every CU a workgroup; 256-query
// workgroups when those still fill the chip twice over at two per CU; else
// 128-query workgroups.  A function of the call's sizes only, so the
// schedule and the launch agree.
int32_t attn_variant(int64_t N, int32_t n_img, int32_t heads) {
  const int64_t tiles128 = (N + 127) / 128 + n_img, tiles256 = (N + 255) / 256 + n_img;
  if (tiles128 * heads <= 256) return vt::kAttnSmall;
  return tiles256 * heads >= 1024 ? vt::kAttnLean8 : vt::kAttnLean4;
}

// The per-call attention prologue: LPT schedule and RoPE cos/sin table; for
// the blocks (whose QKV GEMM packs Q and the tile images itself) also the
// layer-independent parts of the tile images and the token -> slot map.
vt_status attn_prologue(const vt_config* cfg, const int32_t* cu, int32_t n_img, int64_t N,
                        int32_t n_pos, const BlockBufs& b, int32_t* axis_code, hipStream_t s,
                        bool for_blocks = false) {
  const int q_tile = vt::attn_q_tile(attn_variant(N, n_img, cfg->heads));
  VT_TRY_HIP(vt::launch_attn_schedule(cu, n_img, q_tile, vt::kAttnKTile,
                                      max_q_tiles(N, n_img, q_tile), max_k_tiles(N, n_img),
                                      b.order, b.tile_start, b.ktile_start, b.qdesc, b.kdesc, s,
                                      b.qkpre));
  const vt::RopeFreq f = rope_freq(cfg, axis_code);
  VT_TRY_HIP(vt::launch_rope_table(f, n_pos, b.rope, s));
  if (for_blocks)
    VT_TRY_HIP(vt::launch_attn_image_init(b.kdesc, max_k_tiles(N, n_img), cfg->heads, b.kv, b.kslot, s));
  return VT_OK;
}

float q_scale_log2(const vt_config* cfg) {
  return float(1.4426950408889634 / std::sqrt(double(cfg->head_dim)));
}

// The images' token counts on the host when the sizes alone fix them: n_img
// images of at most max_seqlen tokens that add up to n_img * max_seqlen all
// have max_seqlen.  Then the attention's split-tail plan is formed on the
// host too and a call without a split launches no merge.  Else empty.
std::vector<int64_t> uniform_tokens(int32_t n_img, int64_t total, int32_t max_seqlen) {
  if (int64_t(n_img) * max_seqlen != total) return {};
  return std::vector<int64_t>(size_t(n_img), int64_t(max_seqlen));
}

vt_status run_attention(const vt_config* cfg, const uint16_t* qkv, const int32_t* cu,
                        const int32_t* pos, int32_t n_img, int64_t N, int32_t n_pos,
                        int32_t axis_code, const BlockBufs& b, void* out, bool f32,
                        hipStream_t s, float* lse = nullptr) {
  const int32_t var = attn_variant(N, n_img, cfg->heads);
  VT_TRY_HIP(vt::launch_attention(qkv, pos, b.qdesc, b.kdesc, max_q_tiles(N, n_img, vt::attn_q_tile(var)),
                                  max_k_tiles(N, n_img), cfg->heads, n_pos, axis_code, b.rope,
                                  q_scale_log2(cfg), var, b.qpk, b.kv, out, f32, lse, s,
                                  vt::AttnTail{b.qkpre, b.tile_start + n_img, b.part}));
  return VT_OK;
}

// One block.  LN1 is skipped when the previous block already wrote LN1(R)
// into xn (*xn_ready).  When a residual GEMM runs split-K, its reduction is
// fused with the LayerNorm that follows it: LN2 of this block after O, LN1 of
// the next block (next_ln1_g/b, when given) after FC2.
vt_status run_block(const vt_config* cfg, float* R, const vt_block_weights* w, const int32_t* cu,
                    const int32_t* pos, int32_t n_img, int64_t N, int32_t n_pos, int32_t axis_code,
                    const BlockBufs& b, const uint16_t* next_ln1_g, const uint16_t* next_ln1_b,
                    bool* xn_ready, hipStream_t s) {
  const int d = cfg->hidden, mlp = cfg->mlp, M = int(N);
  uint16_t* qkv = b.act;
  uint16_t* att = b.act + size_t(N) * 3 * d;
  if (!*xn_ready)
    VT_TRY_HIP(vt::launch_layer_norm(R, M, d, w->ln1_g, w->ln1_b, cfg->ln_eps, b.xn, s));
  // QKV with RoPE, the fp16 conversion and the tile-image writes in its
  // epilogue (the images' constant parts come from attn_prologue), then the
  // attention kernel on what it packed.
  const vt::QkvPack pk{b.qpk, b.kv, pos, b.kslot, b.rope, n_pos, axis_code, cfg->heads, d, q_scale_log2(cfg)};
  const hipError_t e = vt::launch_gemm_qkv_pack(b.xn, M, d, w->w_qkv, w->b_qkv, pk, s);
  if (e == hipSuccess) {
    const int32_t var = attn_variant(N, n_img, cfg->heads);
    VT_TRY_HIP(vt::launch_attention_packed(b.qpk, b.kv, b.qdesc, max_q_tiles(N, n_img, vt::attn_q_tile(var)),
                                           cfg->heads, var, att, false, nullptr, s,
                                           vt::AttnTail{b.qkpre, b.tile_start + n_img, b.part, b.host_tokens,
                                                        b.host_n_img}));
  } else if (e == hipErrorInvalidValue) {  // a shape the pack epilogue does not take (nothing launched)
    (void)hipGetLastError();
    VT_TRY_HIP(vt::launch_gemm(b.xn, M, d, w->w_qkv, 3 * d, w->b_qkv, vt::kEpiBf16, qkv, b.gemm_ws, s));
    vt_status st = run_attention(cfg, qkv, cu, pos, n_img, N, n_pos, axis_code, b, att, false, s);
    if (st != VT_OK) return st;
  } else {
    return fail(VT_ERR_HIP, "QKV pack GEMM: %s", hipGetErrorString(e));
  }
  const float* part = reinterpret_cast<const float*>(b.gemm_ws);
  if (vt::plan_gemm(M, d, d).splits > 1) {
    VT_TRY_HIP(vt::launch_gemm_partials(att, M, d, w->w_o, d, b.gemm_ws, s));
    VT_TRY_HIP(vt::launch_resid_ln(part, vt::plan_gemm(M, d, d).splits, M, d, w->b_o, R, w->ln2_g,
                                   w->ln2_b, cfg->ln_eps, b.xn, s));
  } else {
    VT_TRY_HIP(vt::launch_gemm(att, M, d, w->w_o, d, w->b_o, vt::kEpiResid, R, b.gemm_ws, s));
    VT_TRY_HIP(vt::launch_layer_norm(R, M, d, w->ln2_g, w->ln2_b, cfg->ln_eps, b.xn, s));
  }
  VT_TRY_HIP(vt::launch_gemm(b.xn, M, d, w->w_fc1, mlp, w->b_fc1, vt::kEpiGeluTanh, b.act, b.gemm_ws, s));
  *xn_ready = false;
  const int fc2_splits = vt::plan_gemm(M, d, mlp).splits;
  if (fc2_splits > 1 && next_ln1_g) {
    VT_TRY_HIP(vt::launch_gemm_partials(b.act, M, mlp, w->w_fc2, d, b.gemm_ws, s));
    VT_TRY_HIP(vt::launch_resid_ln(part, fc2_splits, M, d, w->b_fc2, R, next_ln1_g, next_ln1_b,
                                   cfg->ln_eps, b.xn, s));
    *xn_ready = true;
  } else {
    VT_TRY_HIP(vt::launch_gemm(b.act, M, mlp, w->w_fc2, d, w->b_fc2, vt::kEpiResid, R, b.gemm_ws, s));
  }
  return VT_OK;
}

vt_status check_block_weights(const vt_block_weights* w, int layer) {
  if (!w) return fail(VT_ERR_INVALID_ARG, "block weights %d are NULL", layer);
  const void* req[] = {w->ln1_g, w->ln1_b, w->w_qkv, w->w_o, w->ln2_g, w->ln2_b, w->w_fc1, w->w_fc2};
  const char* names[] = {"ln1_g", "ln1_b", "w_qkv", "w_o", "ln2_g", "ln2_b", "w_fc1", "w_fc2"};
  for (int i = 0; i < 8; ++i) {
    if (!req[i]) return fail(VT_ERR_INVALID_ARG, "block %d: %s is NULL", layer, names[i]);
    if (!aligned16(req[i]))
      return fail(VT_ERR_INVALID_ARG, "block %d: %s is not 16-byte aligned", layer, names[i]);
  }
  const void* opt[] = {w->b_qkv, w->b_o, w->b_fc1, w->b_fc2};
  for (const void* p : opt)
    if (p && !aligned16(p)) return fail(VT_ERR_INVALID_ARG, "block %d: a bias is not 16-byte aligned", layer);
  return VT_OK;
}

vt_status check_proj_weights(const vt_projector_weights* w) {
  if (!w) return fail(VT_ERR_INVALID_ARG, "projector weights are NULL");
  const void* req[] = {w->w1, w->w2, w->w3, w->w4};
  for (int i = 0; i < 4; ++i) {
    if (!req[i]) return fail(VT_ERR_INVALID_ARG, "projector w%d is NULL", i + 1);
    if (!aligned16(req[i])) return fail(VT_ERR_INVALID_ARG, "projector w%d is not 16-byte aligned", i + 1);
  }
  const void* opt[] = {w->b1, w->b2, w->b3, w->b4};
  for (const void* p : opt)
    if (p && !aligned16(p)) return fail(VT_ERR_INVALID_ARG, "a projector bias is not 16-byte aligned");
  return VT_OK;
}

vt_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need && !ws) return fail(VT_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (ws && (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)))
    return fail(VT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(VT_ERR_WORKSPACE, "workspace of %zu bytes is too small: %zu needed", ws_bytes, need);
  return VT_OK;
}

vt_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(VT_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(VT_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return VT_OK;
}

size_t block_ws_bytes(const vt_config* cfg, int64_t N, int32_t n_img, int32_t n_pos) {
  Carver c(nullptr);
  BlockBufs b;
  carve_block(c, dims_of(cfg, N, n_img), n_pos, &b);
  return c.off;
}

// The attention step's own buffers (schedule, packed Q, tile images, RoPE
// table; no split-tail records): what vt_attention_varlen_noalloc carves from
// its fixed array.
size_t attn_ws_bytes(const vt_config* cfg, int64_t N, int32_t n_img, int32_t n_pos) {
  Carver c(nullptr);
  BlockBufs b;
  carve_attention(c, dims_of(cfg, N, n_img), n_pos, &b, false);
  return c.off;
}

size_t tower_ws_bytes(const vt_config* cfg, const GridInfo& gi, int32_t n_img) {
  Carver c(nullptr);
  TowerBufs t;
  carve_tower(c, dims_of(cfg, gi.tokens, n_img), gi.max_hw, &t);
  return c.off;
}

// A bound on tower_ws_bytes over every grid list of n_img items with N tokens
// in all: the RoPE table sized for positions up to N and the split-K
// partials at their bound.  Non-decreasing in N.
size_t tower_ws_upper(const vt_config* cfg, int64_t N, int32_t n_img) {
  Carver c(nullptr);
  TowerBufs t;
  Dims D = dims_of(cfg, N, n_img);
  D.ws_upper = true;
  carve_tower(c, D, int32_t(N), &t);
  return c.off;
}

// Everything after the last block: bf16 cast, optional outputs, projector.
vt_status run_tail(const vt_config* cfg, const TowerBufs& t, const uint16_t* T, int64_t N,
                   const vt_projector_weights* pw, uint16_t* merged_raw, uint16_t* out,
                   hipStream_t s) {
  const int d = cfg->hidden, P = cfg->proj_hidden, Po = cfg->proj_out, M = int(N);
  if (merged_raw)
    VT_TRY_HIP(hipMemcpyAsync(merged_raw, T, size_t(N) * d * sizeof(uint16_t),
                              hipMemcpyDeviceToDevice, s));
  if (out) {
    const int e1 = cfg->gelu_erf_projector ? vt::kEpiGeluErf : vt::kEpiGeluTanh;
    VT_TRY_HIP(vt::launch_gemm(T, M, d, pw->w1, P, pw->b1, e1, t.Y1, t.proj_ws, s));
    VT_TRY_HIP(vt::launch_gemm(t.Y1, M, P, pw->w2, P, pw->b2, vt::kEpiBf16, t.Y2, t.proj_ws, s));
    // token order keeps the four patches of a merged token adjacent: Y2 viewed
    // as [N/4, 4P] is the flattened 2x2 group, slot k = 2*dr + dc.
    VT_TRY_HIP(vt::launch_gemm(t.Y2, M / 4, 4 * P, pw->w3, Po, pw->b3, e1, t.U, t.proj_ws, s));
    VT_TRY_HIP(vt::launch_gemm(t.U, M / 4, Po, pw->w4, Po, pw->b4, vt::kEpiBf16, out, t.proj_ws, s));
  }
  return VT_OK;
}

}  // namespace

// =================================================================== ABI
VT_API void vt_config_default(vt_config* c) {
  if (!c) return;
  c->layers = 32;
  c->hidden = 1280;
  c->heads = 16;
  c->head_dim = 80;
  c->mlp = 5120;
  c->patch = 14;
  c->t_patch = 2;
  c->merge = 2;
  c->proj_hidden = 6144;
  c->proj_out = 6144;
  c->ln_eps = 1e-6f;
  c->rope_theta = 10000.f;
  c->rope_pairs[0] = 8;
  c->rope_pairs[1] = 16;
  c->rope_pairs[2] = 16;
  c->rope_shared_ladder = 0;
  c->gelu_erf_projector = 0;
}

VT_API const char* vt_status_string(vt_status s) {
  switch (s) {
    case VT_OK: return "VT_OK";
    case VT_ERR_INVALID_ARG: return "VT_ERR_INVALID_ARG";
    case VT_ERR_UNSUPPORTED: return "VT_ERR_UNSUPPORTED";
    case VT_ERR_WORKSPACE: return "VT_ERR_WORKSPACE";
    case VT_ERR_HIP: return "VT_ERR_HIP";
  }
  return "VT_ERR_UNKNOWN";
}

VT_API const char* vt_last_error(void) { return g_err.c_str(); }

VT_API const char* vt_version(void) { return "vt 0.1 gfx950"; }

VT_API size_t vt_tower_workspace_size(const vt_config* cfg, const vt_grid_thw* grid, int32_t n_img) {
  if (check_config(cfg) != VT_OK) return 0;
  GridInfo gi;
  if (check_grid(grid, n_img, &gi) != VT_OK) return 0;
  return tower_ws_bytes(cfg, gi, n_img);
}

VT_API size_t vt_block_workspace_size(const vt_config* cfg, int32_t total_tokens, int32_t n_img,
                                      int32_t max_seqlen) {
  if (check_config(cfg) != VT_OK) return 0;
  if (total_tokens <= 0 || n_img <= 0 || max_seqlen <= 0) {
    fail(VT_ERR_INVALID_ARG, "total_tokens, n_img and max_seqlen must be positive");
    return 0;
  }
  return block_ws_bytes(cfg, total_tokens, n_img, max_seqlen);
}

VT_API vt_status vt_build_metadata(const vt_grid_thw* grid, int32_t n_img, int32_t* cu_seqlens,
                                   int32_t* pos_thw, int32_t* raster_index, void* stream) {
  GridInfo gi;
  vt_status st = check_grid(grid, n_img, &gi);
  if (st != VT_OK) return st;
  if (!cu_seqlens || !pos_thw) return fail(VT_ERR_INVALID_ARG, "cu_seqlens and pos_thw are required");
  return launch_meta(grid, n_img, gi.tokens, cu_seqlens, nullptr, pos_thw, raster_index, nullptr,
                     static_cast<hipStream_t>(stream));
}

VT_API vt_status vt_patch_embed(const vt_config* cfg, const uint16_t* pixels, const vt_grid_thw* grid,
                                int32_t n_img, const uint16_t* w_patch, const uint16_t* b_patch,
                                float* resid_out, void* ws, size_t ws_bytes, void* stream) {
  vt_status st = check_config(cfg);
  if (st != VT_OK) return st;
  GridInfo gi;
  if ((st = check_grid(grid, n_img, &gi)) != VT_OK) return st;
  if ((st = check_ptr(pixels, "pixels")) != VT_OK) return st;
  if ((st = check_ptr(w_patch, "w_patch")) != VT_OK) return st;
  if (b_patch && !aligned16(b_patch)) return fail(VT_ERR_INVALID_ARG, "b_patch is not 16-byte aligned");
  if ((st = check_ptr(resid_out, "resid_out")) != VT_OK) return st;
  const size_t need = tower_ws_bytes(cfg, gi, n_img);
  if ((st = check_ws(ws, ws_bytes, need)) != VT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  TowerBufs t;
  carve_tower(c, dims_of(cfg, gi.tokens, n_img), gi.max_hw, &t);
  st = launch_meta(grid, n_img, gi.tokens, t.cu, t.info, t.pos, t.ridx, t.tok_img, s);
  if (st != VT_OK) return st;
  VT_TRY_HIP(vt::launch_patchify(pixels, t.info, t.cu, t.tok_img, int32_t(gi.tokens), t.X, s));
  VT_TRY_HIP(vt::launch_gemm(t.X, int(gi.tokens), 1176, w_patch, cfg->hidden, b_patch, vt::kEpiF32,
                             resid_out, t.blk.gemm_ws, s));
  return VT_OK;
}

static vt_status check_varlen(const vt_config* cfg, const int32_t* cu_seqlens, const int32_t* pos_thw,
                              int32_t n_img, int32_t total_tokens, int32_t max_seqlen) {
  vt_status st = check_config(cfg);
  if (st != VT_OK) return st;
  if (!cu_seqlens || !pos_thw) return fail(VT_ERR_INVALID_ARG, "cu_seqlens and pos_thw are required");
  if (n_img <= 0 || total_tokens <= 0 || max_seqlen <= 0)
    return fail(VT_ERR_INVALID_ARG, "n_img, total_tokens and max_seqlen must be positive");
  if (max_seqlen > total_tokens)
    return fail(VT_ERR_INVALID_ARG, "max_seqlen %d exceeds total_tokens %d", max_seqlen, total_tokens);
  if (total_tokens > kMaxTokens)
    return fail(VT_ERR_UNSUPPORTED, "more than %lld tokens in one call", (long long)kMaxTokens);
  return VT_OK;
}

// The two halves of vt_attention_varlen, on the workspace layout of
// vt_block_forward (carve_block): the pack (schedule, RoPE table, rotated Q,
// tile images) and the attention kernels on what it left there.
static vt_status attention_pack_into(const vt_config* cfg, const uint16_t* qkv, const int32_t* cu_seqlens,
                                     const int32_t* pos_thw, int32_t n_img, int32_t total_tokens,
                                     int32_t max_seqlen, const BlockBufs& b, hipStream_t s) {
  int32_t axis_code = 0;
  vt_status st = attn_prologue(cfg, cu_seqlens, n_img, total_tokens, max_seqlen, b, &axis_code, s);
  if (st != VT_OK) return st;
  VT_TRY_HIP(vt::launch_attn_pack(qkv, pos_thw, b.kdesc, max_k_tiles(total_tokens, n_img), cfg->heads, max_seqlen,
                                  axis_code, b.rope, q_scale_log2(cfg), b.qpk, b.kv, s));
  return VT_OK;
}

static vt_status attention_on_packed(const vt_config* cfg, int32_t n_img, int32_t total_tokens, int32_t max_seqlen,
                                     const BlockBufs& b, void* out, bool f32, hipStream_t s,
                                     const int32_t* host_seqlens = nullptr) {
  const int32_t var = attn_variant(total_tokens, n_img, cfg->heads);
  std::vector<int64_t> tok = uniform_tokens(n_img, total_tokens, max_seqlen);
  if (host_seqlens && tok.empty()) tok.assign(host_seqlens, host_seqlens + n_img);
  VT_TRY_HIP(vt::launch_attention_packed(b.qpk, b.kv, b.qdesc,
                                         max_q_tiles(total_tokens, n_img, vt::attn_q_tile(var)), cfg->heads,
                                         var, out, f32, nullptr, s,
                                         vt::AttnTail{b.qkpre, b.tile_start + n_img, b.part,
                                                      tok.empty() ? nullptr : tok.data(), n_img}));
  return VT_OK;
}

VT_API vt_status vt_attention_varlen(const vt_config* cfg, const uint16_t* qkv,
                                     const int32_t* cu_seqlens, const int32_t* pos_thw,
                                     int32_t n_img, int32_t total_tokens, int32_t max_seqlen,
                                     void* out, vt_dtype out_dtype, void* ws, size_t ws_bytes,
                                     void* stream) {
  vt_status st = check_varlen(cfg, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen);
  if (st != VT_OK) return st;
  if ((st = check_ptr(qkv, "qkv")) != VT_OK) return st;
  if ((st = check_ptr(out, "out")) != VT_OK) return st;
  if (out_dtype != VT_BF16 && out_dtype != VT_FP32) return fail(VT_ERR_INVALID_ARG, "bad out_dtype");
  const size_t need = block_ws_bytes(cfg, total_tokens, n_img, max_seqlen);
  if ((st = check_ws(ws, ws_bytes, need)) != VT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  BlockBufs b;
  carve_block(c, dims_of(cfg, total_tokens, n_img), max_seqlen, &b);
  if ((st = attention_pack_into(cfg, qkv, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen, b, s)) != VT_OK)
    return st;
  return attention_on_packed(cfg, n_img, total_tokens, max_seqlen, b, out, out_dtype == VT_FP32, s);
}

VT_API vt_status vt_attention_pack(const vt_config* cfg, const uint16_t* qkv, const int32_t* cu_seqlens,
                                   const int32_t* pos_thw, int32_t n_img, int32_t total_tokens,
                                   int32_t max_seqlen, void* ws, size_t ws_bytes, void* stream) {
  vt_status st = check_varlen(cfg, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen);
  if (st != VT_OK) return st;
  if ((st = check_ptr(qkv, "qkv")) != VT_OK) return st;
  const size_t need = block_ws_bytes(cfg, total_tokens, n_img, max_seqlen);
  if ((st = check_ws(ws, ws_bytes, need)) != VT_OK) return st;
  Carver c(ws);
  BlockBufs b;
  carve_block(c, dims_of(cfg, total_tokens, n_img), max_seqlen, &b);
  return attention_pack_into(cfg, qkv, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen, b,
                             static_cast<hipStream_t>(stream));
}

VT_API vt_status vt_attention_packed(const vt_config* cfg, int32_t n_img, int32_t total_tokens, int32_t max_seqlen,
                                     const int32_t* host_seqlens, void* out, vt_dtype out_dtype, void* ws,
                                     size_t ws_bytes, void* stream) {
  vt_status st = check_config(cfg);
  if (st != VT_OK) return st;
  if (n_img <= 0 || total_tokens <= 0 || max_seqlen <= 0)
    return fail(VT_ERR_INVALID_ARG, "n_img, total_tokens and max_seqlen must be positive");
  if (max_seqlen > total_tokens)
    return fail(VT_ERR_INVALID_ARG, "max_seqlen %d exceeds total_tokens %d", max_seqlen, total_tokens);
  if (total_tokens > kMaxTokens)
    return fail(VT_ERR_UNSUPPORTED, "more than %lld tokens in one call", (long long)kMaxTokens);
  if ((st = check_ptr(out, "out")) != VT_OK) return st;
  if (out_dtype != VT_BF16 && out_dtype != VT_FP32) return fail(VT_ERR_INVALID_ARG, "bad out_dtype");
  if (host_seqlens) {
    int64_t sum = 0;
    for (int32_t i = 0; i < n_img; ++i) {
      if (host_seqlens[i] < 1 || host_seqlens[i] > max_seqlen)
        return fail(VT_ERR_INVALID_ARG, "host_seqlens[%d] = %d is outside [1, max_seqlen]", i, host_seqlens[i]);
      sum += host_seqlens[i];
    }
    if (sum != total_tokens)
      return fail(VT_ERR_INVALID_ARG, "host_seqlens add up to %lld, not total_tokens %d", (long long)sum, total_tokens);
  }
  const size_t need = block_ws_bytes(cfg, total_tokens, n_img, max_seqlen);
  if ((st = check_ws(ws, ws_bytes, need)) != VT_OK) return st;
  Carver c(ws);
  BlockBufs b;
  carve_block(c, dims_of(cfg, total_tokens, n_img), max_seqlen, &b);
  return attention_on_packed(cfg, n_img, total_tokens, max_seqlen, b, out, out_dtype == VT_FP32,
                             static_cast<hipStream_t>(stream), host_seqlens);
}

// ---- vt_attention_varlen without a workspace argument
// Its scratch is one file-scope device array, of which each GPU the library
// runs on holds its own copy (from the first use of the library's code on
// that GPU until the process ends).  In host code `scratch` names a host-side
// stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, resolved once per device on the first call with that
// device current, and only that address is passed to kernels.
static __device__ __align__(256) char scratch[VT_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices] = {};

static vt_status noalloc_scratch(void** out) {
  int dev = 0;
  VT_TRY_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VT_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    VT_TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || (reinterpret_cast<uintptr_t>(p) & (kAlign - 1)))
      return fail(VT_ERR_HIP, "device %d: the scratch array has no 256-byte aligned address", dev);
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return VT_OK;
}

VT_API vt_status vt_attention_varlen_noalloc(const vt_config* cfg, const uint16_t* qkv,
                                             const int32_t* cu_seqlens, const int32_t* pos_thw,
                                             int32_t n_img, int32_t total_tokens, int32_t max_seqlen,
                                             void* out, vt_dtype out_dtype, void* stream) {
  vt_status st = check_varlen(cfg, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen);
  if (st != VT_OK) return st;
  if ((st = check_ptr(qkv, "qkv")) != VT_OK) return st;
  if ((st = check_ptr(out, "out")) != VT_OK) return st;
  if (out_dtype != VT_BF16 && out_dtype != VT_FP32) return fail(VT_ERR_INVALID_ARG, "bad out_dtype");
  const size_t need = attn_ws_bytes(cfg, total_tokens, n_img, max_seqlen);
  if (need > size_t(VT_NOALLOC_SCRATCH_BYTES))
    return fail(VT_ERR_WORKSPACE, "%d tokens in %d images need %zu bytes of attention scratch, more than "
                "the %zu bytes of the fixed array", total_tokens, n_img, need,
                size_t(VT_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != VT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Every buffer carved here is written in full by this call before it is
  // read (schedule, packed Q, tile images with their padding and ones rows,
  // RoPE table), so nothing left by an earlier call needs clearing.
  Carver c(ws);
  BlockBufs b;
  carve_attention(c, dims_of(cfg, total_tokens, n_img), max_seqlen, &b, false);
  int32_t axis_code = 0;
  if ((st = attn_prologue(cfg, cu_seqlens, n_img, total_tokens, max_seqlen, b, &axis_code, s)) != VT_OK)
    return st;
  return run_attention(cfg, qkv, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen, axis_code, b, out,
                       out_dtype == VT_FP32, s);
}

// Buffers of vt_attention_backward: the forward's attention buffers, its
// fp32 output and log-sum-exp, the 128-token schedule and both tile images.
struct AttnBwdBufs {
  BlockBufs fwd;
  int4* bdesc;
  int4* bdesc256;  // 256-key schedule of the wide dK/dV pass
  float* o;
  float* lse;
  char* qimg;
  char* kimg;
};

void carve_attn_bwd(Carver& c, const Dims& D, int32_t n_pos, AttnBwdBufs* a) {
  carve_attention(c, D, n_pos, &a->fwd);
  const size_t kt = size_t(max_k_tiles(D.N, D.n_img)) * D.heads;
  a->bdesc = c.take<int4>(max_q_tiles(D.N, D.n_img, vt::kAttnBwdTile));
  a->bdesc256 = c.take<int4>(max_q_tiles(D.N, D.n_img, vt::kAttnBwdWideTile));
  a->o = c.take<float>(size_t(D.N) * D.d);
  a->lse = c.take<float>(size_t(D.N) * D.heads);
  a->qimg = c.take<char>(kt * vt::kAttnBwdQBytes);
  a->kimg = c.take<char>(kt * vt::kAttnBwdKBytes);
}

// The backward kernels' schedules (128-token tiles; 256-key tiles for the
// wide dK/dV pass) after attn_prologue: kdesc is rewritten unchanged.
vt_status attn_bwd_schedule(const int32_t* cu, int32_t n_img, int64_t N, int32_t heads,
                            const AttnBwdBufs& a, hipStream_t s) {
  const BlockBufs& b = a.fwd;
  VT_TRY_HIP(vt::launch_attn_schedule(cu, n_img, vt::kAttnBwdTile, vt::kAttnKTile,
                                      max_q_tiles(N, n_img, vt::kAttnBwdTile), max_k_tiles(N, n_img),
                                      b.order, b.tile_start, b.ktile_start, a.bdesc, b.kdesc, s));
  if (vt::attn_bwd_wide(N, n_img, heads))
    VT_TRY_HIP(vt::launch_attn_schedule(cu, n_img, vt::kAttnBwdWideTile, vt::kAttnKTile,
                                        max_q_tiles(N, n_img, vt::kAttnBwdWideTile),
                                        max_k_tiles(N, n_img), b.order, b.tile_start, b.ktile_start,
                                        a.bdesc256, b.kdesc, s));
  return VT_OK;
}

// Packs, dQ and dK/dV passes of the attention backward (forward already run
// into a.o and a.lse).
vt_status run_attn_bwd(const vt_config* cfg, const uint16_t* qkv, const uint16_t* dout,
                       const int32_t* pos, int32_t n_img, int64_t N, int32_t n_pos, int32_t axis_code,
                       const AttnBwdBufs& a, void* dqkv, bool f32, hipStream_t s) {
  const bool wide = vt::attn_bwd_wide(N, n_img, cfg->heads);
  VT_TRY_HIP(vt::launch_attention_backward(
      qkv, dout, a.o, a.lse, pos, a.fwd.kdesc, a.bdesc, max_k_tiles(N, n_img),
      max_q_tiles(N, n_img, vt::kAttnBwdTile), cfg->heads, n_pos, axis_code, a.fwd.rope,
      q_scale_log2(cfg), a.qimg, a.kimg, dqkv, f32, wide ? a.bdesc256 : nullptr,
      max_q_tiles(N, n_img, vt::kAttnBwdWideTile), s));
  return VT_OK;
}

size_t attn_bwd_ws_bytes(const vt_config* cfg, int64_t N, int32_t n_img, int32_t n_pos) {
  Carver c(nullptr);
  AttnBwdBufs a;
  carve_attn_bwd(c, dims_of(cfg, N, n_img), n_pos, &a);
  return c.off;
}

VT_API size_t vt_attention_backward_workspace_size(const vt_config* cfg, int32_t total_tokens,
                                                   int32_t n_img, int32_t max_seqlen) {
  if (check_config(cfg) != VT_OK) return 0;
  if (total_tokens <= 0 || n_img <= 0 || max_seqlen <= 0) {
    fail(VT_ERR_INVALID_ARG, "total_tokens, n_img and max_seqlen must be positive");
    return 0;
  }
  return attn_bwd_ws_bytes(cfg, total_tokens, n_img, max_seqlen);
}

VT_API vt_status vt_attention_backward(const vt_config* cfg, const uint16_t* qkv,
                                       const int32_t* cu_seqlens, const int32_t* pos_thw,
                                       int32_t n_img, int32_t total_tokens, int32_t max_seqlen,
                                       const uint16_t* dout, void* dqkv, vt_dtype dqkv_dtype,
                                       void* ws, size_t ws_bytes, void* stream) {
  vt_status st = check_varlen(cfg, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen);
  if (st != VT_OK) return st;
  if ((st = check_ptr(qkv, "qkv")) != VT_OK) return st;
  if ((st = check_ptr(dout, "dout")) != VT_OK) return st;
  if ((st = check_ptr(dqkv, "dqkv")) != VT_OK) return st;
  if (dqkv_dtype != VT_BF16 && dqkv_dtype != VT_FP32) return fail(VT_ERR_INVALID_ARG, "bad dqkv_dtype");
  const size_t need = attn_bwd_ws_bytes(cfg, total_tokens, n_img, max_seqlen);
  if ((st = check_ws(ws, ws_bytes, need)) != VT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  AttnBwdBufs a;
  const int64_t N = total_tokens;
  carve_attn_bwd(c, dims_of(cfg, N, n_img), max_seqlen, &a);
  const BlockBufs& b = a.fwd;
  int32_t axis_code = 0;
  if ((st = attn_prologue(cfg, cu_seqlens, n_img, N, max_seqlen, b, &axis_code, s)) != VT_OK) return st;
  if ((st = attn_bwd_schedule(cu_seqlens, n_img, N, cfg->heads, a, s)) != VT_OK) return st;
  if ((st = run_attention(cfg, qkv, cu_seqlens, pos_thw, n_img, N, max_seqlen, axis_code, b, a.o, true,
                          s, a.lse)) != VT_OK)
    return st;
  return run_attn_bwd(cfg, qkv, dout, pos_thw, n_img, N, max_seqlen, axis_code, a, dqkv,
                      dqkv_dtype == VT_FP32, s);
}

// ---- one block's backward pass
int32_t pad64(int64_t n) { return int32_t((n + 63) / 64 * 64); }

// Buffers of vt_block_backward: the recomputed forward activations, the
// backward activations, their token-major transposes (rows padded to 64
// tokens, zero), one transposed weight at a time, and the GEMM partials.
struct BlockBwdBufs {
  AttnBwdBufs at;
  uint16_t *x1, *qkv, *a, *x2, *h, *dh, *gb, *da, *dqkv;
  float *R1, *dx;
  uint16_t *gT, *hT, *xT, *dqkvT, *wT;
  float* ln_scratch;  // gamma / beta gradients the caller did not ask for
  float* part;        // per-tile / per-block partial sums of the bias and LN gradients
  void* gemm_ws;
};

size_t block_bwd_gemm_ws(int N, int d, int mlp) {
  const int Np = pad64(N);
  const int shapes[][3] = {{N, 3 * d, d}, {N, d, d}, {N, mlp, d}, {d, mlp, Np}, {mlp, d, Np},
                           {N, d, mlp}, {d, d, Np}, {3 * d, d, Np}, {N, d, 3 * d}};
  size_t w = 0;
  for (const auto& x : shapes) w = std::max(w, vt::gemm_workspace_bytes(x[0], x[1], x[2]));
  return w;
}

void carve_block_bwd(Carver& c, const Dims& D, int32_t n_pos, BlockBwdBufs* b) {
  carve_attn_bwd(c, D, n_pos, &b->at);
  const size_t N = D.N, d = D.d, mlp = D.mlp, Np = pad64(D.N);
  b->x1 = c.take<uint16_t>(N * d);
  b->qkv = c.take<uint16_t>(N * 3 * d);
  b->a = c.take<uint16_t>(N * d);
  b->x2 = c.take<uint16_t>(N * d);
  b->h = c.take<uint16_t>(N * mlp);
  b->dh = c.take<uint16_t>(N * mlp);
  b->gb = c.take<uint16_t>(N * d);
  b->da = c.take<uint16_t>(N * d);
  b->dqkv = c.take<uint16_t>(N * 3 * d);
  b->R1 = c.take<float>(N * d);
  b->dx = c.take<float>(N * d);
  b->gT = c.take<uint16_t>(d * Np);
  b->hT = c.take<uint16_t>(mlp * Np);
  b->xT = c.take<uint16_t>(d * Np);
  b->dqkvT = c.take<uint16_t>(3 * d * Np);
  b->wT = c.take<uint16_t>(std::max(mlp * d, 3 * d * d));
  b->ln_scratch = c.take<float>(4 * d);
  b->part = c.take<float>(size_t(Np / 64) * std::max(mlp, 3 * d) + size_t(vt::kLnBwdMaxBlocks) * 2 * d);
  b->gemm_ws = c.take<char>(D.ws_upper ? kPartialsBound : block_bwd_gemm_ws(D.N, D.d, D.mlp));
}

size_t block_bwd_ws_bytes(const vt_config* cfg, int64_t N, int32_t n_img, int32_t n_pos) {
  Carver c(nullptr);
  BlockBwdBufs b;
  carve_block_bwd(c, dims_of(cfg, N, n_img), n_pos, &b);
  return c.off;
}

vt_status run_block_backward(const vt_config* cfg, const float* R, const vt_block_weights* w,
                             const int32_t* cu, const int32_t* pos, int32_t n_img, int64_t N,
                             int32_t n_pos, float* dR, const vt_block_grads* g, const BlockBwdBufs& B,
                             hipStream_t s) {
  const int d = cfg->hidden, mlp = cfg->mlp, M = int(N), Np = pad64(N);
  const float eps = cfg->ln_eps;
  void* ws = B.gemm_ws;
  float* ln1g = g->ln1_g ? g->ln1_g : B.ln_scratch;
  float* ln1b = g->ln1_b ? g->ln1_b : B.ln_scratch + d;
  float* ln2g = g->ln2_g ? g->ln2_g : B.ln_scratch + 2 * d;
  float* ln2b = g->ln2_b ? g->ln2_b : B.ln_scratch + 3 * d;

  // ---- the block's forward, keeping what the backward reads
  const AttnBwdBufs& at = B.at;
  VT_TRY_HIP(vt::launch_layer_norm(R, M, d, w->ln1_g, w->ln1_b, eps, B.x1, s));
  VT_TRY_HIP(vt::launch_gemm(B.x1, M, d, w->w_qkv, 3 * d, w->b_qkv, vt::kEpiBf16, B.qkv, ws, s));
  int32_t axis_code = 0;
  vt_status st = attn_prologue(cfg, cu, n_img, N, n_pos, at.fwd, &axis_code, s);
  if (st != VT_OK) return st;
  if ((st = attn_bwd_schedule(cu, n_img, N, cfg->heads, at, s)) != VT_OK) return st;
  if ((st = run_attention(cfg, B.qkv, cu, pos, n_img, N, n_pos, axis_code, at.fwd, at.o, true, s,
                          at.lse)) != VT_OK)
    return st;
  VT_TRY_HIP(vt::launch_f32_to_bf16(at.o, B.a, size_t(N) * d, s));
  VT_TRY_HIP(hipMemcpyAsync(B.R1, R, size_t(N) * d * sizeof(float), hipMemcpyDeviceToDevice, s));
  VT_TRY_HIP(vt::launch_gemm(B.a, M, d, w->w_o, d, w->b_o, vt::kEpiResid, B.R1, ws, s));
  VT_TRY_HIP(vt::launch_layer_norm(B.R1, M, d, w->ln2_g, w->ln2_b, eps, B.x2, s));
  VT_TRY_HIP(vt::launch_gemm(B.x2, M, d, w->w_fc1, mlp, w->b_fc1, vt::kEpiBf16, B.h, ws, s));

  // ---- MLP: dR holds dL/d(output) = dR2
  VT_TRY_HIP(vt::launch_transpose(dR, true, 0, nullptr, M, d, Np, B.gb, B.gT, g->b_fc2, B.part, s));
  VT_TRY_HIP(vt::launch_transpose(w->w_fc2, false, 0, nullptr, d, mlp, d, nullptr, B.wT, nullptr, nullptr, s));
  VT_TRY_HIP(vt::launch_gemm(B.gb, M, d, B.wT, mlp, nullptr, vt::kEpiBf16, B.dh, ws, s));  // du
  if (g->w_fc2) {  // dW_fc2 = dR2^T GELU(h)
    VT_TRY_HIP(vt::launch_transpose(B.h, false, 1, nullptr, M, mlp, Np, nullptr, B.hT, nullptr, nullptr, s));
    VT_TRY_HIP(vt::launch_gemm(B.gT, d, Np, B.hT, mlp, nullptr, vt::kEpiF32, g->w_fc2, ws, s));
  }
  // dh = du * GELU'(h), in place, with its transpose and column sums
  VT_TRY_HIP(vt::launch_transpose(B.dh, false, 2, B.h, M, mlp, Np, B.dh, B.hT, g->b_fc1, B.part, s));
  if (g->w_fc1) {  // dW_fc1 = dh^T x2
    VT_TRY_HIP(vt::launch_transpose(B.x2, false, 0, nullptr, M, d, Np, nullptr, B.xT, nullptr, nullptr, s));
    VT_TRY_HIP(vt::launch_gemm(B.hT, mlp, Np, B.xT, d, nullptr, vt::kEpiF32, g->w_fc1, ws, s));
  }
  VT_TRY_HIP(vt::launch_transpose(w->w_fc1, false, 0, nullptr, mlp, d, mlp, nullptr, B.wT, nullptr, nullptr, s));
  VT_TRY_HIP(vt::launch_gemm(B.dh, M, mlp, B.wT, d, nullptr, vt::kEpiF32, B.dx, ws, s));  // dx2
  VT_TRY_HIP(vt::launch_ln_backward(B.R1, w->ln2_g, B.dx, dR, M, d, eps, dR, ln2g, ln2b, B.part, s));

  // ---- attention: dR now holds dR1
  VT_TRY_HIP(vt::launch_transpose(dR, true, 0, nullptr, M, d, Np, B.gb, B.gT, g->b_o, B.part, s));
  if (g->w_o) {  // dW_o = dR1^T a
    VT_TRY_HIP(vt::launch_transpose(B.a, false, 0, nullptr, M, d, Np, nullptr, B.xT, nullptr, nullptr, s));
    VT_TRY_HIP(vt::launch_gemm(B.gT, d, Np, B.xT, d, nullptr, vt::kEpiF32, g->w_o, ws, s));
  }
  VT_TRY_HIP(vt::launch_transpose(w->w_o, false, 0, nullptr, d, d, d, nullptr, B.wT, nullptr, nullptr, s));
  VT_TRY_HIP(vt::launch_gemm(B.gb, M, d, B.wT, d, nullptr, vt::kEpiBf16, B.da, ws, s));
  if ((st = run_attn_bwd(cfg, B.qkv, B.da, pos, n_img, N, n_pos, axis_code, at, B.dqkv, false, s)) != VT_OK)
    return st;
  VT_TRY_HIP(vt::launch_transpose(B.dqkv, false, 0, nullptr, M, 3 * d, Np, nullptr, B.dqkvT, g->b_qkv,
                                  B.part, s));
  if (g->w_qkv) {  // dW_qkv = dqkv^T x1
    VT_TRY_HIP(vt::launch_transpose(B.x1, false, 0, nullptr, M, d, Np, nullptr, B.xT, nullptr, nullptr, s));
    VT_TRY_HIP(vt::launch_gemm(B.dqkvT, 3 * d, Np, B.xT, d, nullptr, vt::kEpiF32, g->w_qkv, ws, s));
  }
  VT_TRY_HIP(vt::launch_transpose(w->w_qkv, false, 0, nullptr, 3 * d, d, 3 * d, nullptr, B.wT, nullptr, nullptr, s));
  VT_TRY_HIP(vt::launch_gemm(B.dqkv, M, 3 * d, B.wT, d, nullptr, vt::kEpiF32, B.dx, ws, s));  // dx1
  VT_TRY_HIP(vt::launch_ln_backward(R, w->ln1_g, B.dx, dR, M, d, eps, dR, ln1g, ln1b, B.part, s));
  return VT_OK;
}

VT_API size_t vt_block_backward_workspace_size(const vt_config* cfg, int32_t total_tokens,
                                               int32_t n_img, int32_t max_seqlen) {
  if (check_config(cfg) != VT_OK) return 0;
  if (total_tokens <= 0 || n_img <= 0 || max_seqlen <= 0) {
    fail(VT_ERR_INVALID_ARG, "total_tokens, n_img and max_seqlen must be positive");
    return 0;
  }
  return block_bwd_ws_bytes(cfg, total_tokens, n_img, max_seqlen);
}

VT_API vt_status vt_block_backward(const vt_config* cfg, const float* resid_in,
                                   const vt_block_weights* w, const int32_t* cu_seqlens,
                                   const int32_t* pos_thw, int32_t n_img, int32_t total_tokens,
                                   int32_t max_seqlen, float* dresid, const vt_block_grads* grads,
                                   void* ws, size_t ws_bytes, void* stream) {
  vt_status st = check_varlen(cfg, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen);
  if (st != VT_OK) return st;
  if (cfg->hidden > 2048) return fail(VT_ERR_UNSUPPORTED, "the backward pass supports hidden <= 2048");
  if ((st = check_ptr(resid_in, "resid_in")) != VT_OK) return st;
  if ((st = check_ptr(dresid, "dresid")) != VT_OK) return st;
  if ((st = check_block_weights(w, 0)) != VT_OK) return st;
  if (!grads) return fail(VT_ERR_INVALID_ARG, "grads is NULL (its members may be NULL)");
  const float* gp[] = {grads->ln1_g, grads->ln1_b, grads->w_qkv, grads->b_qkv, grads->w_o, grads->b_o,
                       grads->ln2_g, grads->ln2_b, grads->w_fc1, grads->b_fc1, grads->w_fc2, grads->b_fc2};
  for (const float* p : gp)
    if (p && !aligned16(p)) return fail(VT_ERR_INVALID_ARG, "a gradient buffer is not 16-byte aligned");
  const size_t need = block_bwd_ws_bytes(cfg, total_tokens, n_img, max_seqlen);
  if ((st = check_ws(ws, ws_bytes, need)) != VT_OK) return st;
  Carver c(ws);
  BlockBwdBufs B;
  carve_block_bwd(c, dims_of(cfg, total_tokens, n_img), max_seqlen, &B);
  return run_block_backward(cfg, resid_in, w, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen,
                            dresid, grads, B, static_cast<hipStream_t>(stream));
}

VT_API vt_status vt_block_forward(const vt_config* cfg, float* resid, const vt_block_weights* w,
                                  const int32_t* cu_seqlens, const int32_t* pos_thw, int32_t n_img,
                                  int32_t total_tokens, int32_t max_seqlen, void* ws,
                                  size_t ws_bytes, void* stream) {
  vt_status st = check_varlen(cfg, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen);
  if (st != VT_OK) return st;
  if ((st = check_ptr(resid, "resid")) != VT_OK) return st;
  if ((st = check_block_weights(w, 0)) != VT_OK) return st;
  const size_t need = block_ws_bytes(cfg, total_tokens, n_img, max_seqlen);
  if ((st = check_ws(ws, ws_bytes, need)) != VT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  BlockBufs b;
  carve_block(c, dims_of(cfg, total_tokens, n_img), max_seqlen, &b);
  int32_t axis_code = 0;
  if ((st = attn_prologue(cfg, cu_seqlens, n_img, total_tokens, max_seqlen, b, &axis_code, s, true)) != VT_OK)
    return st;
  bool xn_ready = false;
  const std::vector<int64_t> tok = uniform_tokens(n_img, total_tokens, max_seqlen);
  if (!tok.empty()) {
    b.host_tokens = tok.data();
    b.host_n_img = n_img;
  }
  return run_block(cfg, resid, w, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen, axis_code, b,
                   nullptr, nullptr, &xn_ready, s);
}

VT_API vt_status vt_merge_project(const vt_config* cfg, const uint16_t* tower, vt_order order,
                                  const vt_grid_thw* grid, int32_t n_img,
                                  const vt_projector_weights* w, uint16_t* merged_raw, uint16_t* out,
                                  void* ws, size_t ws_bytes, void* stream) {
  vt_status st = check_config(cfg);
  if (st != VT_OK) return st;
  GridInfo gi;
  if ((st = check_grid(grid, n_img, &gi)) != VT_OK) return st;
  if ((st = check_ptr(tower, "tower")) != VT_OK) return st;
  if (order != VT_ORDER_WINDOW && order != VT_ORDER_RASTER)
    return fail(VT_ERR_INVALID_ARG, "order must be VT_ORDER_WINDOW or VT_ORDER_RASTER");
  if (!out && !merged_raw) return fail(VT_ERR_INVALID_ARG, "out and merged_raw are both NULL");
  if (out) {
    if ((st = check_ptr(out, "out")) != VT_OK) return st;
    if ((st = check_proj_weights(w)) != VT_OK) return st;
  }
  if (merged_raw && (st = check_ptr(merged_raw, "merged_raw")) != VT_OK) return st;
  const size_t need = tower_ws_bytes(cfg, gi, n_img);
  if ((st = check_ws(ws, ws_bytes, need)) != VT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  TowerBufs t;
  carve_tower(c, dims_of(cfg, gi.tokens, n_img), gi.max_hw, &t);
  const uint16_t* T = tower;
  if (order == VT_ORDER_RASTER) {
    st = launch_meta(grid, n_img, gi.tokens, nullptr, nullptr, nullptr, t.ridx, nullptr, s);
    if (st != VT_OK) return st;
    VT_TRY_HIP(vt::launch_row_permute(tower, t.T, t.ridx, int32_t(gi.tokens), cfg->hidden, false, s));
    T = t.T;
  }
  return run_tail(cfg, t, T, gi.tokens, w, merged_raw, out, s);
}

VT_API vt_status vt_tower_forward(const vt_config* cfg, const uint16_t* pixels,
                                  const vt_grid_thw* grid, int32_t n_img, const vt_tower_weights* w,
                                  uint16_t* tower_out, uint16_t* merged_raw, uint16_t* out, void* ws,
                                  size_t ws_bytes, void* stream) {
  vt_status st = check_config(cfg);
  if (st != VT_OK) return st;
  GridInfo gi;
  if ((st = check_grid(grid, n_img, &gi)) != VT_OK) return st;
  if ((st = check_ptr(pixels, "pixels")) != VT_OK) return st;
  if (!w) return fail(VT_ERR_INVALID_ARG, "weights are NULL");
  if ((st = check_ptr(w->w_patch, "w_patch")) != VT_OK) return st;
  if (w->b_patch && !aligned16(w->b_patch)) return fail(VT_ERR_INVALID_ARG, "b_patch is not 16-byte aligned");
  if (cfg->layers > 0 && !w->blocks) return fail(VT_ERR_INVALID_ARG, "blocks is NULL");
  for (int l = 0; l < cfg->layers; ++l)
    if ((st = check_block_weights(&w->blocks[l], l)) != VT_OK) return st;
  if (!tower_out && !merged_raw && !out) return fail(VT_ERR_INVALID_ARG, "no output requested");
  if (out) {
    if ((st = check_ptr(out, "out")) != VT_OK) return st;
    if ((st = check_proj_weights(&w->proj)) != VT_OK) return st;
  }
  if (tower_out && (st = check_ptr(tower_out, "tower_out")) != VT_OK) return st;
  if (merged_raw && (st = check_ptr(merged_raw, "merged_raw")) != VT_OK) return st;
  const size_t need = tower_ws_bytes(cfg, gi, n_img);
  if ((st = check_ws(ws, ws_bytes, need)) != VT_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  TowerBufs t;
  const int64_t N = gi.tokens;
  carve_tower(c, dims_of(cfg, N, n_img), gi.max_hw, &t);
  if ((st = launch_meta(grid, n_img, N, t.cu, t.info, t.pos, t.ridx, t.tok_img, s)) != VT_OK) return st;
  int32_t axis_code = 0;
  if ((st = attn_prologue(cfg, t.cu, n_img, N, gi.max_hw, t.blk, &axis_code, s, true)) != VT_OK) return st;
  VT_TRY_HIP(vt::launch_patchify(pixels, t.info, t.cu, t.tok_img, int32_t(N), t.X, s));
  VT_TRY_HIP(vt::launch_gemm(t.X, int(N), 1176, w->w_patch, cfg->hidden, w->b_patch, vt::kEpiF32, t.R,
                             t.blk.gemm_ws, s));
  const std::vector<int64_t> tokens = grid_tokens(grid, n_img);
  t.blk.host_tokens = tokens.data();
  t.blk.host_n_img = n_img;
  bool xn_ready = false;
  for (int l = 0; l < cfg->layers; ++l) {
    const vt_block_weights* nx = l + 1 < cfg->layers ? &w->blocks[l + 1] : nullptr;
    st = run_block(cfg, t.R, &w->blocks[l], t.cu, t.pos, n_img, N, gi.max_hw, axis_code, t.blk,
                   nx ? nx->ln1_g : nullptr, nx ? nx->ln1_b : nullptr, &xn_ready, s);
    if (st != VT_OK) return st;
  }
  VT_TRY_HIP(vt::launch_f32_to_bf16(t.R, t.T, size_t(N) * cfg->hidden, s));
  if (tower_out)
    VT_TRY_HIP(vt::launch_row_permute(t.T, tower_out, t.ridx, int32_t(N), cfg->hidden, true, s));
  return run_tail(cfg, t, t.T, N, &w->proj, merged_raw, out, s);
}

// ---- the tower's backward pass
// Buffers of vt_tower_backward: metadata, patches, the running residual and
// every block's input, the forward block buffers, the block backward's
// buffers, dL/dR, and the patch-weight gradient's operands.
struct TowerBwdBufs {
  int32_t *cu, *pos, *ridx, *tok_img;
  vt::ImgInfo* info;
  uint16_t* X;      // [N, 1176] patches
  float* R;         // [N, d] running residual
  float* Rsave;     // [layers, N, d] the input of each block
  float* dR;        // [N, d]
  uint16_t* XT;     // [1176, Np]
  float* dwT;       // [1176, d]
  BlockBufs blk;
  BlockBwdBufs bb;
  void* patch_ws;
};

void carve_tower_bwd(Carver& c, const vt_config* cfg, const Dims& D, int32_t n_pos, TowerBwdBufs* t) {
  const size_t N = D.N, d = D.d, Np = pad64(D.N);
  t->cu = c.take<int32_t>(D.n_img + 1);
  t->info = c.take<vt::ImgInfo>(D.n_img);
  t->pos = c.take<int32_t>(N * 3);
  t->ridx = c.take<int32_t>(N);
  t->tok_img = c.take<int32_t>(N);
  t->X = c.take<uint16_t>(N * 1176);
  t->R = c.take<float>(N * d);
  t->Rsave = c.take<float>(size_t(std::max(cfg->layers, 1)) * N * d);
  t->dR = c.take<float>(N * d);
  t->XT = c.take<uint16_t>(1176 * Np);
  t->dwT = c.take<float>(1176 * d);
  carve_block(c, D, n_pos, &t->blk);
  carve_block_bwd(c, D, n_pos, &t->bb);
  t->patch_ws = c.take<char>(D.ws_upper ? kPartialsBound : vt::gemm_workspace_bytes(1176, D.d, int(Np)));
}

size_t tower_bwd_ws_bytes(const vt_config* cfg, const GridInfo& gi, int32_t n_img) {
  Carver c(nullptr);
  TowerBwdBufs t;
  carve_tower_bwd(c, cfg, dims_of(cfg, gi.tokens, n_img), gi.max_hw, &t);
  return c.off;
}

VT_API size_t vt_tower_backward_workspace_size(const vt_config* cfg, const vt_grid_thw* grid,
                                               int32_t n_img) {
  if (check_config(cfg) != VT_OK) return 0;
  GridInfo gi;
  if (check_grid(grid, n_img, &gi) != VT_OK) return 0;
  return tower_bwd_ws_bytes(cfg, gi, n_img);
}

VT_API vt_status vt_tower_backward(const vt_config* cfg, const uint16_t* pixels,
                                   const vt_grid_thw* grid, int32_t n_img, const vt_tower_weights* w,
                                   const float* d_tower, const vt_tower_grads* grads, void* ws,
                                   size_t ws_bytes, void* stream) {
  vt_status st = check_config(cfg);
  if (st != VT_OK) return st;
  if (cfg->hidden > 2048) return fail(VT_ERR_UNSUPPORTED, "the backward pass supports hidden <= 2048");
  GridInfo gi;
  if ((st = check_grid(grid, n_img, &gi)) != VT_OK) return st;
  if ((st = check_ptr(pixels, "pixels")) != VT_OK) return st;
  if ((st = check_ptr(d_tower, "d_tower")) != VT_OK) return st;
  if (!w) return fail(VT_ERR_INVALID_ARG, "weights are NULL");
  if ((st = check_ptr(w->w_patch, "w_patch")) != VT_OK) return st;
  if (w->b_patch && !aligned16(w->b_patch)) return fail(VT_ERR_INVALID_ARG, "b_patch is not 16-byte aligned");
  if (cfg->layers > 0 && !w->blocks) return fail(VT_ERR_INVALID_ARG, "blocks is NULL");
  for (int l = 0; l < cfg->layers; ++l)
    if ((st = check_block_weights(&w->blocks[l], l)) != VT_OK) return st;
  if (!grads) return fail(VT_ERR_INVALID_ARG, "grads is NULL (its members may be NULL)");
  if (cfg->layers > 0 && !grads->blocks) return fail(VT_ERR_INVALID_ARG, "grads->blocks is NULL");
  if ((grads->w_patch && !aligned16(grads->w_patch)) || (grads->b_patch && !aligned16(grads->b_patch)))
    return fail(VT_ERR_INVALID_ARG, "a patch gradient buffer is not 16-byte aligned");
  for (int l = 0; l < cfg->layers; ++l) {
    const vt_block_grads& g = grads->blocks[l];
    const float* gp[] = {g.ln1_g, g.ln1_b, g.w_qkv, g.b_qkv, g.w_o, g.b_o,
                         g.ln2_g, g.ln2_b, g.w_fc1, g.b_fc1, g.w_fc2, g.b_fc2};
    for (const float* p : gp)
      if (p && !aligned16(p)) return fail(VT_ERR_INVALID_ARG, "block %d: a gradient buffer is not 16-byte aligned", l);
  }
  const size_t need = tower_bwd_ws_bytes(cfg, gi, n_img);
  if ((st = check_ws(ws, ws_bytes, need)) != VT_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  TowerBwdBufs t;
  const int64_t N = gi.tokens;
  const int d = cfg->hidden, M = int(N), Np = pad64(N);
  carve_tower_bwd(c, cfg, dims_of(cfg, N, n_img), gi.max_hw, &t);
  // forward, keeping each block's input
  if ((st = launch_meta(grid, n_img, N, t.cu, t.info, t.pos, t.ridx, t.tok_img, s)) != VT_OK) return st;
  int32_t axis_code = 0;
  if ((st = attn_prologue(cfg, t.cu, n_img, N, gi.max_hw, t.blk, &axis_code, s, true)) != VT_OK) return st;
  VT_TRY_HIP(vt::launch_patchify(pixels, t.info, t.cu, t.tok_img, M, t.X, s));
  VT_TRY_HIP(vt::launch_gemm(t.X, M, 1176, w->w_patch, d, w->b_patch, vt::kEpiF32, t.R, t.blk.gemm_ws, s));
  const std::vector<int64_t> tokens = grid_tokens(grid, n_img);
  t.blk.host_tokens = tokens.data();
  t.blk.host_n_img = n_img;
  bool xn_ready = false;
  const size_t plane = size_t(N) * d;
  for (int l = 0; l < cfg->layers; ++l) {
    VT_TRY_HIP(hipMemcpyAsync(t.Rsave + l * plane, t.R, plane * sizeof(float), hipMemcpyDeviceToDevice, s));
    const vt_block_weights* nx = l + 1 < cfg->layers ? &w->blocks[l + 1] : nullptr;
    st = run_block(cfg, t.R, &w->blocks[l], t.cu, t.pos, n_img, N, gi.max_hw, axis_code, t.blk,
                   nx ? nx->ln1_g : nullptr, nx ? nx->ln1_b : nullptr, &xn_ready, s);
    if (st != VT_OK) return st;
  }
  // dL/dR after the last block, in token order (rows of 2 * d 16-bit units)
  VT_TRY_HIP(vt::launch_row_permute(reinterpret_cast<const uint16_t*>(d_tower),
                                    reinterpret_cast<uint16_t*>(t.dR), t.ridx, M, 2 * d, false, s));
  for (int l = cfg->layers - 1; l >= 0; --l) {
    st = run_block_backward(cfg, t.Rsave + l * plane, &w->blocks[l], t.cu, t.pos, n_img, N, gi.max_hw,
                            t.dR, &grads->blocks[l], t.bb, s);
    if (st != VT_OK) return st;
  }
  // patch embed: dW = dR0^T X (formed as X^T dR0, then transposed), db = column sums of dR0
  if (grads->w_patch || grads->b_patch)
    VT_TRY_HIP(vt::launch_transpose(t.dR, true, 0, nullptr, M, d, Np, nullptr,
                                    grads->w_patch ? t.bb.gT : nullptr, grads->b_patch, t.bb.part, s));
  if (grads->w_patch) {
    VT_TRY_HIP(vt::launch_transpose(t.X, false, 0, nullptr, M, 1176, Np, nullptr, t.XT, nullptr, nullptr, s));
    VT_TRY_HIP(vt::launch_gemm(t.XT, 1176, Np, t.bb.gT, d, nullptr, vt::kEpiF32, t.dwT, t.patch_ws, s));
    VT_TRY_HIP(vt::launch_transpose_f32(t.dwT, 1176, d, grads->w_patch, s));
  }
  return VT_OK;
}

VT_API size_t vt_linear_workspace_size(int32_t M, int32_t N, int32_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return vt::gemm_workspace_bytes(M, N, K);
}

VT_API vt_status vt_linear(const uint16_t* x, int32_t M, int32_t K, const uint16_t* w, int32_t N,
                           const uint16_t* bias, vt_epilogue epi, void* out, void* ws,
                           size_t ws_bytes, void* stream) {
  vt_status st;
  if ((st = check_ptr(x, "x")) != VT_OK) return st;
  if ((st = check_ptr(w, "w")) != VT_OK) return st;
  if ((st = check_ptr(out, "out")) != VT_OK) return st;
  if (bias && !aligned16(bias)) return fail(VT_ERR_INVALID_ARG, "bias is not 16-byte aligned");
  if (M <= 0 || N <= 0 || K <= 0) return fail(VT_ERR_INVALID_ARG, "M, N, K must be positive");
  if (K % 8) return fail(VT_ERR_UNSUPPORTED, "K must be a multiple of 8 (got %d)", K);
  if (N % 64) return fail(VT_ERR_UNSUPPORTED, "N must be a multiple of 64 (got %d)", N);
  if (int64_t(M) * N > (int64_t(1) << 34) || int64_t(M) > kMaxTokens)
    return fail(VT_ERR_UNSUPPORTED, "M x N too large");
  if (epi < VT_EPI_BF16 || epi > VT_EPI_SPLITK_PARTIALS_F32)
    return fail(VT_ERR_INVALID_ARG, "bad epilogue %d", int(epi));
  if (epi == VT_EPI_SPLITK_PARTIALS_F32) {
    if (bias) return fail(VT_ERR_INVALID_ARG, "the split-K partials carry no bias (bias must be NULL)");
    if (vt::plan_gemm(M, N, K).splits < 2)
      return fail(VT_ERR_UNSUPPORTED, "%d x %d x %d runs without split-K: there are no partials", M, N, K);
    VT_TRY_HIP(vt::launch_gemm_partials(x, M, K, w, N, out, static_cast<hipStream_t>(stream)));
    return VT_OK;
  }
  if ((st = check_ws(ws, ws_bytes, vt::gemm_workspace_bytes(M, N, K))) != VT_OK) return st;
  VT_TRY_HIP(vt::launch_gemm(x, M, K, w, N, bias, int(epi), out, ws, static_cast<hipStream_t>(stream)));
  return VT_OK;
}

VT_API vt_status vt_linear_residual_ln(const uint16_t* x, int32_t M, int32_t K, const uint16_t* w,
                                       int32_t N, const uint16_t* bias, float* R, const uint16_t* g,
                                       const uint16_t* beta, float eps, uint16_t* out, void* ws,
                                       size_t ws_bytes, void* stream) {
  vt_status st;
  if ((st = check_ptr(x, "x")) != VT_OK) return st;
  if ((st = check_ptr(w, "w")) != VT_OK) return st;
  if ((st = check_ptr(R, "R")) != VT_OK) return st;
  if ((st = check_ptr(g, "g")) != VT_OK) return st;
  if ((st = check_ptr(beta, "beta")) != VT_OK) return st;
  if ((st = check_ptr(out, "out")) != VT_OK) return st;
  if (bias && !aligned16(bias)) return fail(VT_ERR_INVALID_ARG, "bias is not 16-byte aligned");
  if (M <= 0 || N <= 0 || K <= 0) return fail(VT_ERR_INVALID_ARG, "M, N, K must be positive");
  if (K % 8) return fail(VT_ERR_UNSUPPORTED, "K must be a multiple of 8 (got %d)", K);
  if (N % 256 || N > 4096) return fail(VT_ERR_UNSUPPORTED, "N must be a multiple of 256, at most 4096 (got %d)", N);
  if (int64_t(M) > kMaxTokens) return fail(VT_ERR_UNSUPPORTED, "M too large");
  if (!(eps > 0.f)) return fail(VT_ERR_INVALID_ARG, "eps must be > 0");
  if ((st = check_ws(ws, ws_bytes, vt::gemm_workspace_bytes(M, N, K))) != VT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int splits = vt::plan_gemm(M, N, K).splits;
  if (splits > 1) {  // the blocks' fused path (run_block)
    VT_TRY_HIP(vt::launch_gemm_partials(x, M, K, w, N, ws, s));
    VT_TRY_HIP(vt::launch_resid_ln(reinterpret_cast<const float*>(ws), splits, M, N, bias, R, g, beta, eps,
                                   out, s));
  } else {
    VT_TRY_HIP(vt::launch_gemm(x, M, K, w, N, bias, vt::kEpiResid, R, ws, s));
    VT_TRY_HIP(vt::launch_layer_norm(R, M, N, g, beta, eps, out, s));
  }
  return VT_OK;
}

VT_API vt_status vt_plan_patches(const vt_config* cfg, size_t budget_bytes, int32_t n_img,
                                 int64_t max_pixels, int64_t* patches, int64_t* wanted) {
  vt_status st;
  if ((st = check_config(cfg)) != VT_OK) return st;
  if (!patches || !wanted) return fail(VT_ERR_INVALID_ARG, "patches and wanted must not be NULL");
  if (n_img <= 0) return fail(VT_ERR_INVALID_ARG, "n_img must be >= 1 (got %d)", n_img);
  if (max_pixels < 0) return fail(VT_ERR_INVALID_ARG, "max_pixels must be >= 0");
  const int64_t per = int64_t(cfg->patch) * cfg->patch;
  // Largest multiple of 4 (whole merged tokens) whose bound fits the budget.
  int64_t lo = 0, hi = kMaxTokens / 4;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (tower_ws_upper(cfg, 4 * mid, n_img) <= budget_bytes) lo = mid; else hi = mid - 1;
  }
  const int64_t fit = 4 * lo;
  if (fit < 4 * int64_t(n_img))
    return fail(VT_ERR_WORKSPACE, "a workspace of %zu bytes holds no %d-item call (%lld bytes for 4 "
                "tokens per item)", budget_bytes, n_img, (long long)tower_ws_upper(cfg, 4 * n_img, n_img));
  const int64_t want = max_pixels > 0 ? std::max<int64_t>(1, max_pixels / per) : fit;
  *patches = std::min(want, fit);
  *wanted = want > fit ? want : 0;
  return VT_OK;
}

VT_API vt_status vt_pack_items(const vt_config* cfg, const vt_grid_thw* grid, int32_t n_img,
                               size_t budget_bytes, int32_t* batch, int32_t* n_batches) {
  vt_status st;
  if ((st = check_config(cfg)) != VT_OK) return st;
  GridInfo gi;
  if ((st = check_grid(grid, n_img, &gi)) != VT_OK) return st;
  if (!batch || !n_batches) return fail(VT_ERR_INVALID_ARG, "batch and n_batches must not be NULL");
  auto need = [&](int32_t from, int32_t to) {  // workspace of items [from, to]
    GridInfo g;
    check_grid(grid + from, to - from + 1, &g);
    return tower_ws_bytes(cfg, g, to - from + 1);
  };
  int32_t b = 0, first = 0;
  for (int32_t i = 0; i < n_img; ++i) {
    if (i > first && need(first, i) > budget_bytes) {
      ++b;
      first = i;
    }
    if (i == first && need(i, i) > budget_bytes)
      return fail(VT_ERR_WORKSPACE, "item %d (%d x %d x %d) alone needs %zu workspace bytes, "
                  "more than the %zu available", i, grid[i].t, grid[i].h, grid[i].w, need(i, i),
                  budget_bytes);
    batch[i] = b;
  }
  *n_batches = b + 1;
  return VT_OK;
}

VT_API vt_status vt_mean_pool(const uint16_t* tower, const int32_t* cu_seqlens, int32_t n_img,
                              int32_t hidden, float* out, void* stream) {
  vt_status st;
  if ((st = check_ptr(tower, "tower")) != VT_OK) return st;
  if ((st = check_ptr(cu_seqlens, "cu_seqlens")) != VT_OK) return st;
  if ((st = check_ptr(out, "out")) != VT_OK) return st;
  if (n_img <= 0 || hidden <= 0) return fail(VT_ERR_INVALID_ARG, "n_img and hidden must be positive");
  if (hidden % 128) return fail(VT_ERR_UNSUPPORTED, "hidden must be a multiple of 128 (got %d)", hidden);
  if (n_img > 65535) return fail(VT_ERR_UNSUPPORTED, "at most 65535 items per call");
  VT_TRY_HIP(vt::launch_mean_pool(tower, cu_seqlens, n_img, hidden, out, static_cast<hipStream_t>(stream)));
  return VT_OK;
}

VT_API vt_status vt_clock_probe(int64_t wait_us, unsigned long long* out, int64_t* realtime_hz,
                                void* stream) {
  vt_status st;
  if ((st = check_ptr(out, "out")) != VT_OK) return st;
  if (!realtime_hz) return fail(VT_ERR_INVALID_ARG, "realtime_hz is NULL");
  if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0)
    return fail(VT_ERR_INVALID_ARG, "out is not 8-byte aligned");
  if (wait_us <= 0 || wait_us > 10000000)
    return fail(VT_ERR_INVALID_ARG, "wait_us must be in 1 .. 10,000,000 (got %lld)", (long long)wait_us);
  int dev = 0, khz = 0;
  VT_TRY_HIP(hipGetDevice(&dev));
  VT_TRY_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev));
  if (khz <= 0) return fail(VT_ERR_UNSUPPORTED, "the device reports no real-time counter rate");
  *realtime_hz = int64_t(khz) * 1000;
  const uint64_t ticks = uint64_t(wait_us) * uint64_t(khz) / 1000u;
  VT_TRY_HIP(vt::launch_clock_probe(ticks, out, static_cast<hipStream_t>(stream)));
  return VT_OK;
}

VT_API vt_status vt_layer_norm(const float* x, int32_t rows, int32_t width, const uint16_t* g,
                               const uint16_t* b, float eps, uint16_t* out, void* stream) {
  vt_status st;
  if ((st = check_ptr(x, "x")) != VT_OK) return st;
  if ((st = check_ptr(g, "g")) != VT_OK) return st;
  if ((st = check_ptr(b, "b")) != VT_OK) return st;
  if ((st = check_ptr(out, "out")) != VT_OK) return st;
  if (rows <= 0 || width <= 0) return fail(VT_ERR_INVALID_ARG, "rows and width must be positive");
  if (width % 256 || width > 4096)
    return fail(VT_ERR_UNSUPPORTED, "width must be a multiple of 256, at most 4096 (got %d)", width);
  if (!(eps > 0.f)) return fail(VT_ERR_INVALID_ARG, "eps must be > 0");
  VT_TRY_HIP(vt::launch_layer_norm(x, rows, width, g, b, eps, out, static_cast<hipStream_t>(stream)));
  return VT_OK;
}
