// Backward pass of the tiled varlen attention with 3D RoPE (head_dim 80) on
// the gfx950 matrix cores: dL/d(qkv) from dL/d(out).
//
// The pages' towers are differentiable: their probe runs a backward pass
// through the tower and reports the gradient norm ("v2_loaders FINDINGS",
// section 3).  Per image and head, with q and k rotated by RoPE, scores
// s = q k^T / sqrt(80), P = softmax(s) row-wise and O = P v, the textbook
// gradients are
//   D_i  = sum_d dO_id O_id
//   dP   = dO v^T,   dS = P * (dP - D)            (elementwise, D per row)
//   dv   = P^T dO,   dq = dS k / sqrt(80),   dk = dS^T q / sqrt(80)
// and the rotation's gradient is the rotation by the opposite angle.  No
// [n, n] matrix is stored: P is rebuilt tile by tile from the scores and the
// forward's per-query log-sum-exp, as in the forward's online softmax.
//
// Four kernels after the forward (which keeps its fp32 output O and the
// log2-domain log-sum-exp L of every query):
//
// bwd_pack_k_kernel  per (64-key tile, head): rotated k and v in fp16 as a
//   36 KB key-side image  K [64][88] | V [64][88] | K^T [80][72]  (K^T with
//   the keys in MFMA slot order, as the forward's V^T).
// bwd_pack_q_kernel  per (64-query tile, head): a 48 KB query-side image
//   Q [64][88] | dO [64][88] | Q^T [80][72] | dO^T [80][72] | L [64] | D [64]
//   with Q rotated and scaled by log2(e)/sqrt(80) (the forward's Q), D from
//   the fp32 O.  Padding queries get L = +inf and zero rows, so their P is 0.
// bwd_dq_kernel  query-major: a workgroup owns 128 queries (4 wavefronts of
//   32) of one head and streams the image's key-side images; per tile
//     S^T  = K Q^T - L        (the MFMAs accumulate onto -L: P = 2^(S^T))
//     dP^T = V dO^T - D
//     dQ^T += K^T dS^T        (dS^T straight from the registers in slot order)
// bwd_dkv_kernel key-major: a workgroup owns 128 keys (4 wavefronts), or 256
//   (8 wavefronts sharing the stream) when the call has many key tiles, and
//   streams the image's query-side images; per tile, with L and D per
//   accumulator row loaded from LDS into the MFMA's initial value,
//     S  = Q K^T - L,  dP = dO V^T - D,  dV^T += dO^T P,  dK^T += Q^T dS.
// Both end by un-rotating (dq, dk) in registers -- the pair (j, j + 40) of a
// lane's dims always sits in the same lane -- and store dqkv rows.
//
// Precision: fp16 MFMA operands (q, k, v, dO, P, dS) with fp32 accumulation,
// as in the forward.  P <= 1 after the log-sum-exp shift.
//
// Grid of both main kernels: one workgroup per (128- or 256-token tile,
// head), head fastest, largest images first (the forward's schedule with
// that tile size).  Each image's tiles start on a fresh 64-token tile image.
#include "vt_device.h"
#include "vt_kernels.h"

namespace vt {

namespace {
constexpr int HD = 80;
constexpr int BT = kAttnKTile;              // 64 tokens per tile image
constexpr int ROW = 88;                     // fp16 per row of a [token][dim] matrix
constexpr int TROW = 72;                    // fp16 per row of a [dim][slot] matrix
constexpr int RM_BYTES = BT * ROW * 2;      // 11264
constexpr int TM_BYTES = HD * TROW * 2;     // 11520
// key side
constexpr int KS_V = RM_BYTES;
constexpr int KS_KT = 2 * RM_BYTES;
constexpr int KS_BYTES = kAttnBwdKBytes;
// query side
constexpr int QS_DO = RM_BYTES;
constexpr int QS_QT = 2 * RM_BYTES;
constexpr int QS_DOT = QS_QT + TM_BYTES;
constexpr int QS_L = QS_DOT + TM_BYTES;
constexpr int QS_D = QS_L + 4 * BT;
constexpr int QS_BYTES = kAttnBwdQBytes;
// The dim-block-2 MFMAs read [dim][slot] rows up to 95: rows 80..95 fall in
// the next matrix or the image's zero tail and only reach discarded rows.
static_assert(KS_KT + 96 * TROW * 2 <= KS_BYTES, "key-side image size");
static_assert(QS_DOT + 96 * TROW * 2 <= QS_BYTES && QS_D + 4 * BT <= QS_BYTES, "query-side image size");
static_assert(KS_BYTES % 4096 == 0 && QS_BYTES % 4096 == 0, "images are whole rounds of 4 x 1 KB copies");
constexpr int NW = 4;                       // wavefronts per workgroup
static_assert(kAttnBwdTile == 32 * NW, "tile of the main kernels");

// Rotated (r1, r2) = (x1 c - x2 s, x2 c + x1 s) of 8 pairs, times sc, as fp16.
__device__ __forceinline__ void rotate8(uint4 a, uint4 b, const float* cs, float sc, uint32_t* r) {
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x1l = bflo(aw[j]), x1h = bfhi(aw[j]), x2l = bflo(bw[j]), x2h = bfhi(bw[j]);
    const float cl = cs[4 * j], sl = cs[4 * j + 1], ch = cs[4 * j + 2], sh = cs[4 * j + 3];
    r[j] = pack_f16x2((x1l * cl - x2l * sl) * sc, (x1h * ch - x2h * sh) * sc);
    r[4 + j] = pack_f16x2((x2l * cl + x1l * sl) * sc, (x2h * ch + x1h * sh) * sc);
  }
}

__device__ __forceinline__ void load_cs16(const float2* rope_cs, const int32_t* pos, int tok, int c,
                                          int axis_code, int n_pos, float* cs) {
  const int ax = (axis_code >> (2 * c)) & 3;
  const int p = min(max(pos[3 * tok + ax], 0), n_pos - 1);
  const float4* cs4 = reinterpret_cast<const float4*>(rope_cs + int64_t(p) * 40 + 8 * c);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 v = cs4[j];
    cs[4 * j] = v.x; cs[4 * j + 1] = v.y; cs[4 * j + 2] = v.z; cs[4 * j + 3] = v.w;
  }
}

__device__ __forceinline__ void bf16x8_to_f16(uint4 a, uint32_t* r) {
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = pack_f16x2(bflo(aw[j]), bfhi(aw[j]));
}

// Thread (t, c) of a pack block holds dims 8c..8c+7 (r[0..3]) and
// 40+8c..40+8c+7 (r[4..7]) of token t as fp16 pairs: write them as row t of a
// [token][dim] matrix and as column slot(t) of a [dim][slot] LDS buffer.
__device__ __forceinline__ void put_row_and_column(char* img, int off, uint16_t* ts, int t, int c,
                                                   const uint32_t* r) {
  uint16_t* row = reinterpret_cast<uint16_t*>(img + off) + t * ROW;
  *reinterpret_cast<uint4*>(row + 8 * c) = make_uint4(r[0], r[1], r[2], r[3]);
  *reinterpret_cast<uint4*>(row + 40 + 8 * c) = make_uint4(r[4], r[5], r[6], r[7]);
  if (c == 0) *reinterpret_cast<uint4*>(row + HD) = make_uint4(0u, 0u, 0u, 0u);  // row padding
  const int s = mfma_slot16(t);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ts[(8 * c + 2 * j) * BT + s] = uint16_t(r[j] & 0xffffu);
    ts[(8 * c + 2 * j + 1) * BT + s] = uint16_t(r[j] >> 16);
    ts[(40 + 8 * c + 2 * j) * BT + s] = uint16_t(r[4 + j] & 0xffffu);
    ts[(40 + 8 * c + 2 * j + 1) * BT + s] = uint16_t(r[4 + j] >> 16);
  }
}

// Copy an LDS [80][64] transpose into the image's [80][72] rows (slot
// padding zero), by all 320 threads.
__device__ __forceinline__ void put_transpose(char* img, int off, const uint16_t* ts) {
  uint16_t* dst = reinterpret_cast<uint16_t*>(img + off);
  for (int i = threadIdx.x; i < HD * 9; i += 320) {
    const int d = i / 9, sg = i % 9;
    const uint4 v = sg < 8 ? *reinterpret_cast<const uint4*>(ts + d * BT + 8 * sg) : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(dst + d * TROW + 8 * sg) = v;
  }
}

__device__ __forceinline__ void zero_tail(char* img, int from, int to) {
  for (int i = from + 16 * threadIdx.x; i < to; i += 16 * 320)
    *reinterpret_cast<uint4*>(img + i) = make_uint4(0u, 0u, 0u, 0u);
}
}  // namespace

// ---------------------------------------------------------------- packs
__global__ void __launch_bounds__(320) bwd_pack_k_kernel(
    const uint16_t* __restrict__ qkv, const int32_t* __restrict__ pos, const int2* __restrict__ kdesc,
    int32_t heads, int32_t n_pos, const float2* __restrict__ rope_cs, int32_t axis_code,
    char* __restrict__ kimg) {
  __shared__ __align__(16) uint16_t ts[HD * BT];
  const int T = blockIdx.x / heads, head = blockIdx.x % heads;  // the heads of a tile together
  const int2 desc = kdesc[T];
  if (desc.x < 0) return;
  const int t = threadIdx.x / 5, c = threadIdx.x % 5;
  const int tok = desc.x + t;
  char* img = kimg + (int64_t(T) * heads + head) * KS_BYTES;
  uint32_t kr[8], vr[8];
  if (tok < desc.y) {
    const uint16_t* row = qkv + int64_t(tok) * 3 * heads * HD + head * HD;
    float cs[16];
    load_cs16(rope_cs, pos, tok, c, axis_code, n_pos, cs);
    const uint4* k4 = reinterpret_cast<const uint4*>(row + heads * HD);
    rotate8(k4[c], k4[c + 5], cs, 1.0f, kr);
    const uint4* v4 = reinterpret_cast<const uint4*>(row + 2 * heads * HD);
    bf16x8_to_f16(v4[c], vr);
    bf16x8_to_f16(v4[c + 5], vr + 4);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) kr[j] = vr[j] = 0u;
  }
  put_row_and_column(img, 0, ts, t, c, kr);
  uint16_t* vrow = reinterpret_cast<uint16_t*>(img + KS_V) + t * ROW;
  *reinterpret_cast<uint4*>(vrow + 8 * c) = make_uint4(vr[0], vr[1], vr[2], vr[3]);
  *reinterpret_cast<uint4*>(vrow + 40 + 8 * c) = make_uint4(vr[4], vr[5], vr[6], vr[7]);
  if (c == 0) *reinterpret_cast<uint4*>(vrow + HD) = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  put_transpose(img, KS_KT, ts);
  zero_tail(img, KS_KT + TM_BYTES, KS_BYTES);
}

__global__ void __launch_bounds__(320) bwd_pack_q_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dout, const float* __restrict__ o,
    const float* __restrict__ lse, const int32_t* __restrict__ pos, const int2* __restrict__ kdesc,
    int32_t heads, int32_t n_pos, const float2* __restrict__ rope_cs, int32_t axis_code,
    float q_scale_log2, char* __restrict__ qimg) {
  __shared__ __align__(16) uint16_t ts[2][HD * BT];
  __shared__ float dpart[BT * 5];
  const int T = blockIdx.x / heads, head = blockIdx.x % heads;  // the heads of a tile together
  const int2 desc = kdesc[T];
  if (desc.x < 0) return;
  const int t = threadIdx.x / 5, c = threadIdx.x % 5;
  const int tok = desc.x + t;
  char* img = qimg + (int64_t(T) * heads + head) * QS_BYTES;
  uint32_t qr[8], dr[8];
  float dpp = 0.f;
  if (tok < desc.y) {
    const uint16_t* row = qkv + int64_t(tok) * 3 * heads * HD + head * HD;
    float cs[16];
    load_cs16(rope_cs, pos, tok, c, axis_code, n_pos, cs);
    const uint4* q4 = reinterpret_cast<const uint4*>(row);
    rotate8(q4[c], q4[c + 5], cs, q_scale_log2, qr);
    const int64_t orow = int64_t(tok) * heads * HD + head * HD;
    const uint4* d4 = reinterpret_cast<const uint4*>(dout + orow);
    const uint4 da = d4[c], db = d4[c + 5];
    bf16x8_to_f16(da, dr);
    bf16x8_to_f16(db, dr + 4);
    // D partial over this thread's 16 dims, from the bf16 dO and the fp32 O.
    const float4* o4 = reinterpret_cast<const float4*>(o + orow);
    const uint32_t dw[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 oa = o4[(40 * h + 8 * c) / 4], ob = o4[(40 * h + 8 * c) / 4 + 1];
      dpp += bflo(dw[4 * h]) * oa.x + bfhi(dw[4 * h]) * oa.y + bflo(dw[4 * h + 1]) * oa.z +
             bfhi(dw[4 * h + 1]) * oa.w + bflo(dw[4 * h + 2]) * ob.x + bfhi(dw[4 * h + 2]) * ob.y +
             bflo(dw[4 * h + 3]) * ob.z + bfhi(dw[4 * h + 3]) * ob.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) qr[j] = dr[j] = 0u;
  }
  dpart[threadIdx.x] = dpp;
  put_row_and_column(img, 0, ts[0], t, c, qr);
  put_row_and_column(img, QS_DO, ts[1], t, c, dr);
  __syncthreads();
  put_transpose(img, QS_QT, ts[0]);
  put_transpose(img, QS_DOT, ts[1]);
  if (threadIdx.x < BT) {
    const int i = threadIdx.x, tk = desc.x + i;
    const bool valid = tk < desc.y;
    const float* dp = dpart + 5 * i;
    reinterpret_cast<float*>(img + QS_L)[i] = valid ? lse[int64_t(tk) * heads + head] : INFINITY;
    reinterpret_cast<float*>(img + QS_D)[i] = valid ? (dp[0] + dp[1]) + (dp[2] + dp[3]) + dp[4] : 0.f;
  }
  zero_tail(img, QS_D + 4 * BT, QS_BYTES);
}

namespace {
// acc[d][4g + r] holds dim 32d + 8g + 4hf + r (dims 80..95 are padding) of
// token tok in the rotated frame.  Un-rotate (when rope is set) by the
// opposite angle, scale, and store as dqkv[tok][which][head][:].
__device__ __forceinline__ void store_grad(f32x16_t (&acc)[3], int tok, int which, int head,
                                           int heads, float scale, bool rope,
                                           const int32_t* pos, int n_pos, const float2* rope_cs,
                                           int axis_code, int hf, void* out, int out_f32) {
  if (rope) {
    // Pair (j, j + 40): j = 32d + 8g + 4hf + r for (d, g) = (0, 0..3), (1, 0),
    // its partner at block d + (g + 5) / 4, group (g + 5) % 4 of the same lane.
#pragma unroll
    for (int dg = 0; dg < 5; ++dg) {
      const int d = dg / 4, g = dg % 4;
      const int d2 = d + (g + 5) / 4, g2 = (g + 5) % 4;
      const int ax = (axis_code >> (2 * dg)) & 3;  // pairs 8dg .. 8dg + 7
      const int p = min(max(pos[3 * tok + ax], 0), n_pos - 1);
      const float4* cs = reinterpret_cast<const float4*>(rope_cs + int64_t(p) * 40 + 8 * dg + 4 * hf);
      const float4 a = cs[0], b = cs[1];
      const float cv[4] = {a.x, a.z, b.x, b.z}, sv[4] = {a.y, a.w, b.y, b.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x1 = acc[d][4 * g + r], x2 = acc[d2][4 * g2 + r];
        acc[d][4 * g + r] = x1 * cv[r] + x2 * sv[r];
        acc[d2][4 * g2 + r] = x2 * cv[r] - x1 * sv[r];
      }
    }
  }
  const int64_t orow = (int64_t(tok) * 3 + which) * heads * HD + head * HD;
#pragma unroll
  for (int d = 0; d < 3; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = 32 * d + 8 * g + 4 * hf;
      if (dim >= HD) continue;
      const float o0 = acc[d][4 * g] * scale, o1 = acc[d][4 * g + 1] * scale;
      const float o2 = acc[d][4 * g + 2] * scale, o3 = acc[d][4 * g + 3] * scale;
      if (out_f32)
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + orow + dim) = make_float4(o0, o1, o2, o3);
      else
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + orow + dim) =
            make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    }
  }
}

__device__ __forceinline__ f16x8_t ld16(const char* p) { return *reinterpret_cast<const f16x8_t*>(p); }

__device__ __forceinline__ f32x16_t splat(float v) {
  f32x16_t r;
#pragma unroll
  for (int e = 0; e < 16; ++e) r[e] = v;
  return r;
}
}  // namespace

// ---------------------------------------------------------------- dQ
// Lane (ln, hf) of wavefront w: query q0 + 32w + ln; accumulator rows are
// keys (S^T, dP^T) or dims (dQ^T).  CW > 0: CW more wavefronts that only
// copy the key-side images and meet the others' per-tile barriers (with one
// multiplying wavefront per SIMD, its own copy-issue stalls would leave the
// matrix unit idle); the multiplying wavefronts then issue no copies.
template <int CW>
__global__ void __launch_bounds__(64 * (NW + CW)) bwd_dq_kernel(
    const char* __restrict__ qimg, const char* __restrict__ kimg, const int4* __restrict__ bdesc,
    int32_t heads, const int32_t* __restrict__ pos, int32_t n_pos, const float2* __restrict__ rope_cs,
    int32_t axis_code, float scale, void* __restrict__ dqkv, int32_t out_f32) {
  extern __shared__ __align__(16) char lds[];
  const int head = blockIdx.x % heads;
  const int4 desc = bdesc[blockIdx.x / heads];  // (first query, image begin, image end, first tile)
  if (desc.x < 0) return;
  const int q0 = desc.x, beg = desc.y, end = desc.z;
  const int ntiles = (end - beg + BT - 1) / BT;
  const char* src = kimg + (int64_t(desc.w) * heads + head) * KS_BYTES;
  const int64_t tile_stride = int64_t(heads) * KS_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, ln = lane & 31;
  constexpr int NCP = CW > 0 ? CW : NW;           // wavefronts that copy
  static_assert(KS_BYTES % (1024 * NCP) == 0, "whole rounds of copies");
  const int cwave = CW > 0 ? wave - NW : wave;    // index among them
  const uint32_t lds_wave = lds_offset(lds) + 1024 * cwave;
  auto issue = [&](int t) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_wave + (t & 1) * KS_BYTES);
    const char* g = src + t * tile_stride + 1024 * cwave + 16 * lane;
#pragma unroll
    for (int c = 0; c < KS_BYTES / (1024 * NCP); ++c) dma16(g + NCP * 1024 * c, base + NCP * 1024 * c);
  };
  if constexpr (CW > 0) {
    if (wave >= NW) {  // copy-only: tile t + 1 after the barrier of tile t, as below
      __builtin_amdgcn_s_setprio(1);
      issue(0);
      for (int t = 0; t < ntiles; ++t) {
        wait_vmcnt<0>();
        wg_barrier();
        if (t + 1 < ntiles) issue(t + 1);
      }
      return;
    }
  }

  const int qrow = q0 + 32 * wave + ln;
  const bool qvalid = qrow < end;
  const int qr = qvalid ? qrow : end - 1;
  const char* qi = qimg + (int64_t(desc.w + (qr - beg) / BT) * heads + head) * QS_BYTES;
  const int qrow_img = (qr - beg) % BT;
  f16x8_t qf[5], df[5];
#pragma unroll
  for (int s = 0; s < 5; ++s) {
    qf[s] = ld16(qi + qrow_img * ROW * 2 + 32 * s + 16 * hf);
    df[s] = ld16(qi + QS_DO + qrow_img * ROW * 2 + 32 * s + 16 * hf);
  }
  const f32x16_t c_l = splat(-reinterpret_cast<const float*>(qi + QS_L)[qrow_img]);
  const f32x16_t c_d = splat(-reinterpret_cast<const float*>(qi + QS_D)[qrow_img]);

  f32x16_t acc[3];
#pragma unroll
  for (int d = 0; d < 3; ++d) acc[d] = splat(0.f);

  if constexpr (CW == 0) issue(0);
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<0>();      // tile t has landed
    wait_lds_reads();     // and every wave is done with tile t - 1
    wg_barrier();
    if constexpr (CW == 0)
      if (t + 1 < ntiles) issue(t + 1);
    const char* st = lds + (t & 1) * KS_BYTES;
    const int koff = ln * ROW * 2 + 16 * hf;
    f32x16_t sc[2], dp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) { sc[b] = c_l; dp[b] = c_d; }
#pragma unroll
    for (int sl = 0; sl < 5; ++sl)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        sc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ld16(st + koff + b * 32 * ROW * 2 + 32 * sl),
                                                       qf[sl], sc[b], 0, 0, 0);
#pragma unroll
    for (int sl = 0; sl < 5; ++sl)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        dp[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            ld16(st + KS_V + koff + b * 32 * ROW * 2 + 32 * sl), df[sl], dp[b], 0, 0, 0);
    const int kt = beg + t * BT;
    if (kt + BT > end) {  // keys past the image end
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kt + 32 * b + 8 * (e >> 2) + 4 * hf + (e & 3) >= end) sc[b][e] = -INFINITY;
    }
    f16x8_t ds[4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        ds[2 * b + (e >> 3)][e & 7] = (_Float16)(__builtin_amdgcn_exp2f(sc[b][e]) * dp[b][e]);
    const int toff = KS_KT + ln * TROW * 2 + 16 * hf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int d = 0; d < 3; ++d)
        acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ld16(st + toff + 32 * d * TROW * 2 + 32 * ks),
                                                        ds[ks], acc[d], 0, 0, 0);
  }
  if (!qvalid) return;
  store_grad(acc, qrow, 0, head, heads, scale, true, pos, n_pos, rope_cs, axis_code, hf, dqkv, out_f32);
}

// ---------------------------------------------------------------- dK, dV
// Lane (ln, hf) of wavefront w: key k0 + 32w + ln; accumulator rows are
// queries (S, dP) or dims (dK^T, dV^T).  KW wavefronts (4 or 8) share one
// stream of query-side images: the 96 KB ring allows one workgroup per CU,
// so 8 wavefronts (256 keys) put two on each SIMD when the image is large.
// CW > 0: CW copy-only wavefronts, as in bwd_dq_kernel.
template <int KW, int CW>
__global__ void __launch_bounds__(64 * (KW + CW)) bwd_dkv_kernel(
    const char* __restrict__ qimg, const char* __restrict__ kimg, const int4* __restrict__ bdesc,
    int32_t heads, const int32_t* __restrict__ pos, int32_t n_pos, const float2* __restrict__ rope_cs,
    int32_t axis_code, float dk_scale, void* __restrict__ dqkv, int32_t out_f32) {
  extern __shared__ __align__(16) char lds[];
  const int head = blockIdx.x % heads;
  const int4 desc = bdesc[blockIdx.x / heads];  // (first key, image begin, image end, first tile)
  if (desc.x < 0) return;
  const int k0 = desc.x, beg = desc.y, end = desc.z;
  const int ntiles = (end - beg + BT - 1) / BT;
  const char* src = qimg + (int64_t(desc.w) * heads + head) * QS_BYTES;
  const int64_t tile_stride = int64_t(heads) * QS_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, ln = lane & 31;
  constexpr int NCP = CW > 0 ? CW : KW;           // wavefronts that copy
  static_assert(QS_BYTES % (1024 * NCP) == 0, "whole rounds of copies");
  const int cwave = CW > 0 ? wave - KW : wave;    // index among them
  const uint32_t lds_wave = lds_offset(lds) + 1024 * cwave;
  auto issue = [&](int t) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_wave + (t & 1) * QS_BYTES);
    const char* g = src + t * tile_stride + 1024 * cwave + 16 * lane;
#pragma unroll
    for (int c = 0; c < QS_BYTES / (1024 * NCP); ++c) dma16(g + NCP * 1024 * c, base + NCP * 1024 * c);
  };
  if constexpr (CW > 0) {
    if (wave >= KW) {  // copy-only: tile t + 1 after the barrier of tile t, as below
      __builtin_amdgcn_s_setprio(1);
      issue(0);
      for (int t = 0; t < ntiles; ++t) {
        wait_vmcnt<0>();
        wg_barrier();
        if (t + 1 < ntiles) issue(t + 1);
      }
      return;
    }
  }

  const int krow = k0 + 32 * wave + ln;
  const bool kvalid = krow < end;
  const int kr = kvalid ? krow : end - 1;
  const char* ki = kimg + (int64_t(desc.w + (kr - beg) / BT) * heads + head) * KS_BYTES;
  const int krow_img = (kr - beg) % BT;
  f16x8_t kf[5], vf[5];
#pragma unroll
  for (int s = 0; s < 5; ++s) {
    kf[s] = ld16(ki + krow_img * ROW * 2 + 32 * s + 16 * hf);
    vf[s] = ld16(ki + KS_V + krow_img * ROW * 2 + 32 * s + 16 * hf);
  }

  f32x16_t dv[3], dk[3];
#pragma unroll
  for (int d = 0; d < 3; ++d) { dv[d] = splat(0.f); dk[d] = splat(0.f); }

  if constexpr (CW == 0) issue(0);
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<0>();
    wait_lds_reads();
    wg_barrier();
    if constexpr (CW == 0)
      if (t + 1 < ntiles) issue(t + 1);
    const char* st = lds + (t & 1) * QS_BYTES;
    const int qoff = ln * ROW * 2 + 16 * hf;
    // Initial values: -L and -D of each accumulator row's query.
    f32x16_t sc[2], dp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int q = 32 * b + 8 * g + 4 * hf;
        const float4 l4 = *reinterpret_cast<const float4*>(st + QS_L + 4 * q);
        const float4 d4 = *reinterpret_cast<const float4*>(st + QS_D + 4 * q);
        sc[b][4 * g] = -l4.x; sc[b][4 * g + 1] = -l4.y; sc[b][4 * g + 2] = -l4.z; sc[b][4 * g + 3] = -l4.w;
        dp[b][4 * g] = -d4.x; dp[b][4 * g + 1] = -d4.y; dp[b][4 * g + 2] = -d4.z; dp[b][4 * g + 3] = -d4.w;
      }
#pragma unroll
    for (int sl = 0; sl < 5; ++sl)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        sc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ld16(st + qoff + b * 32 * ROW * 2 + 32 * sl),
                                                       kf[sl], sc[b], 0, 0, 0);
#pragma unroll
    for (int sl = 0; sl < 5; ++sl)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        dp[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            ld16(st + QS_DO + qoff + b * 32 * ROW * 2 + 32 * sl), vf[sl], dp[b], 0, 0, 0);
    // Padding queries have L = +inf: P = 2^-inf = 0 and dS = 0.
    f16x8_t pf[4], ds[4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(sc[b][e]);
        pf[2 * b + (e >> 3)][e & 7] = (_Float16)p;
        ds[2 * b + (e >> 3)][e & 7] = (_Float16)(p * dp[b][e]);
      }
    const int toff = ln * TROW * 2 + 16 * hf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ld16(st + QS_DOT + toff + 32 * d * TROW * 2 + 32 * ks),
                                                       pf[ks], dv[d], 0, 0, 0);
        dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ld16(st + QS_QT + toff + 32 * d * TROW * 2 + 32 * ks),
                                                       ds[ks], dk[d], 0, 0, 0);
      }
  }
  if (!kvalid) return;
  store_grad(dv, krow, 2, head, heads, 1.0f, false, pos, n_pos, rope_cs, axis_code, hf, dqkv, out_f32);
  store_grad(dk, krow, 1, head, heads, dk_scale, true, pos, n_pos, rope_cs, axis_code, hf, dqkv, out_f32);
}

template <class K>
static hipError_t set_lds(K kern, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_attention_backward(const uint16_t* qkv, const uint16_t* dout, const float* o,
                                     const float* lse, const int32_t* pos_thw, const int2* kdesc,
                                     const int4* bdesc, int32_t max_ktiles, int32_t max_btiles,
                                     int32_t heads, int32_t n_pos, int32_t axis_code,
                                     const float2* rope_cs, float q_scale_log2, char* qimg,
                                     char* kimg, void* dqkv, bool out_f32, const int4* kdesc256,
                                     int32_t max_ktiles256, hipStream_t s) {
  static const hipError_t a1 = set_lds(bwd_dq_kernel<0>, 2 * KS_BYTES);
  static const hipError_t a1c = set_lds(bwd_dq_kernel<4>, 2 * KS_BYTES);
  static const hipError_t a2 = set_lds(bwd_dkv_kernel<4, 4>, 2 * QS_BYTES);
  static const hipError_t a3 = set_lds(bwd_dkv_kernel<8, 0>, 2 * QS_BYTES);
  if (a1 != hipSuccess) return a1;
  if (a1c != hipSuccess) return a1c;
  if (a2 != hipSuccess) return a2;
  if (a3 != hipSuccess) return a3;
  const dim3 pack_grid(unsigned(int64_t(max_ktiles) * heads));
  hipLaunchKernelGGL(bwd_pack_k_kernel, pack_grid, dim3(320), 0, s, qkv, pos_thw, kdesc,
                     heads, n_pos, rope_cs, axis_code, kimg);
  hipLaunchKernelGGL(bwd_pack_q_kernel, pack_grid, dim3(320), 0, s, qkv, dout, o, lse,
                     pos_thw, kdesc, heads, n_pos, rope_cs, axis_code, q_scale_log2, qimg);
  const unsigned blocks = unsigned(int64_t(max_btiles) * heads);
  const float rsqrt_hd = 1.0f / sqrtf(float(HD));
  const float ln2 = 0.6931471805599453f;  // dK from the log2(e)/sqrt(80)-scaled Q: times sqrt(80)/log2(e)/sqrt(80)
  // dQ: two 72 KB workgroups fit a CU, whose registers hold 4 wavefronts
  // per SIMD of this kernel; so copy-only wavefronts (one workgroup per CU)
  // only when the grid is a single round of the 256 CUs.
  if (blocks <= 256)
    hipLaunchKernelGGL(bwd_dq_kernel<4>, dim3(blocks), dim3(64 * (NW + 4)), 2 * KS_BYTES, s, qimg, kimg, bdesc,
                       heads, pos_thw, n_pos, rope_cs, axis_code, rsqrt_hd, dqkv, out_f32 ? 1 : 0);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<0>, dim3(blocks), dim3(64 * NW), 2 * KS_BYTES, s, qimg, kimg, bdesc,
                       heads, pos_thw, n_pos, rope_cs, axis_code, rsqrt_hd, dqkv, out_f32 ? 1 : 0);
  if (kdesc256)
    hipLaunchKernelGGL((bwd_dkv_kernel<8, 0>), dim3(unsigned(int64_t(max_ktiles256) * heads)), dim3(512),
                       2 * QS_BYTES, s, qimg, kimg, kdesc256, heads, pos_thw, n_pos, rope_cs, axis_code,
                       ln2, dqkv, out_f32 ? 1 : 0);
  else
    hipLaunchKernelGGL((bwd_dkv_kernel<4, 4>), dim3(blocks), dim3(512), 2 * QS_BYTES, s, qimg, kimg, bdesc,
                       heads, pos_thw, n_pos, rope_cs, axis_code, ln2, dqkv, out_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace vt
