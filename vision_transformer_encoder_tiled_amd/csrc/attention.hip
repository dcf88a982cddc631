// Tiled varlen non-causal multi-head attention with 3D RoPE fused into the
// Q and K loads, for head_dim 80 on the gfx950 matrix cores.
//
// The pages describe the untiled form -- a per-head [seq, seq] fp32 score
// matrix, a row softmax into a bf16 [seq, seq] probability matrix, then P V
// ("init.rs (VisionEncoder::new)": build_scratch and the GEMM-based ViT SDPA
// kernel list) -- and name that quadratic buffer as the limit on image size
// (doc comment of CEILING_MAX_PATCHES).  Here the scores never leave the MFMA
// accumulators: each workgroup owns 128 queries of one head of one image and
// streams that image's keys in tiles of 64 through LDS with an online
// softmax (running max m, running sum l, rescaled output), so memory is
// O(tokens).
//
// Operand precision: the inputs are bf16, the MFMA operands fp16 (rotated
// and scaled Q, rotated K, V, and the probabilities P), accumulation fp32.
// fp16 runs at the bf16 rate on gfx950 and carries 3 more mantissa bits:
// rounding P to bf16 alone would cost up to ~2^-9 |v| per output.  bf16 V
// converts to fp16 exactly inside the fp16 range; |RoPE(q)| log2(e)/sqrt(80),
// |k| and |v| must stay below 65504 (larger values become infinite, they
// are not clamped).
//
// Work split (4 wavefronts, 32 queries each):
//   S^T = K Q^T   v_mfma_f32_32x32x16_f16, 2 key blocks x 5 dim slices of
//                 16 (head_dim 80 = 5 x 16 exactly).  The accumulator layout
//                 gives each lane one query and 16 keys of each 32-key block.
//   O^T = V^T P^T v_mfma_f32_32x32x16_f16, 4 key slices x 3 dim blocks of
//                 32 (80 padded to 96: rows 80..95 read zeros).  The P
//                 operand comes straight from the score registers: the keys
//                 of a 16-key MFMA slice are permuted (k positions 0..7 of a
//                 lane half hold keys +0..3 and +8..11), and V^T is read in
//                 the same permuted order, which leaves the sum unchanged.
// K tiles are rotated (rotate-half RoPE, pairs (j, j+40), angle
// pos[axis(j)] * inv_freq[j] from a cos/sin table) on their way from global
// memory to LDS; V tiles are written to LDS transposed ([dim][key]) so the
// V^T operand is two 8-byte reads.  Q is rotated once, scaled by
// log2(e)/sqrt(80) and kept in registers; the softmax uses exp2.
//
// Grid: one workgroup per (q-tile, head), head fastest, q-tiles of the
// largest images first (longest-processing-time order).  With 16 heads and
// round-robin dispatch over the 8 XCDs, every q-tile of one (image, head)
// lands on the same XCD, so its K/V stream is shared through that XCD's L2.
#include "vt_device.h"
#include "vt_kernels.h"

namespace vt {

namespace {
constexpr int HD = 80;      // head_dim
constexpr int BQ = kAttnQTile;  // queries per workgroup
constexpr int BKV = 64;     // keys per tile
constexpr int KROW = 88;    // LDS row stride of the K tile (fp16): 176 B, conflict-free 16-B reads
constexpr int VROW = 68;    // LDS row stride of the V^T tile (fp16): 136 B, conflict-free 8-B reads
constexpr int K_ITEMS = BKV * 5;   // (key, 8-pair chunk) items per K tile
constexpr int V_ITEMS = BKV / 2 * 10;  // (key pair, 8-dim chunk) items per V tile
}  // namespace

__global__ void __launch_bounds__(256) attention_kernel(
    const uint16_t* __restrict__ qkv, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ order,
    const int32_t* __restrict__ tile_start, int32_t n_img, int32_t heads, int32_t n_pos,
    const float2* __restrict__ rope_cs, int32_t axis_code, float q_scale_log2,
    void* __restrict__ out, int32_t out_f32) {
  __shared__ __align__(16) uint16_t sK[2][BKV * KROW];
  __shared__ __align__(16) uint16_t sV[2][HD * VROW];

  const int head = blockIdx.x % heads;
  const int tile = blockIdx.x / heads;
  if (tile >= tile_start[n_img]) return;
  int lo = 0, hi = n_img - 1;  // largest rank r with tile_start[r] <= tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int img = order[lo];
  const int kbeg = cu[img], kend = cu[img + 1];
  const int q0 = kbeg + (tile - tile_start[lo]) * BQ;
  const int qend = min(q0 + BQ, kend);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, ln = lane & 31;
  const int64_t ld = int64_t(3) * heads * HD;  // qkv row stride (elements)
  const uint16_t* Qg = qkv + head * HD;
  const uint16_t* Kg = qkv + (heads + head) * HD;
  const uint16_t* Vg = qkv + (2 * heads + head) * HD;
  const int pmax = n_pos - 1;

  // ---- Q: load the full row, rotate, scale, keep this lane's 5 MFMA B-operand fragments.
  const int qrow = q0 + wave * 32 + ln;
  const bool qvalid = qrow < qend;
  const int qr = qvalid ? qrow : qend - 1;
  f16x8_t qfrag[5];
  {
    float qf[HD];
    const uint4* src = reinterpret_cast<const uint4*>(Qg + int64_t(qr) * ld);
#pragma unroll
    for (int c = 0; c < 10; ++c) {
      const uint4 u = src[c];
      qf[8 * c + 0] = bflo(u.x); qf[8 * c + 1] = bfhi(u.x);
      qf[8 * c + 2] = bflo(u.y); qf[8 * c + 3] = bfhi(u.y);
      qf[8 * c + 4] = bflo(u.z); qf[8 * c + 5] = bfhi(u.z);
      qf[8 * c + 6] = bflo(u.w); qf[8 * c + 7] = bfhi(u.w);
    }
    int p3[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) p3[a] = min(max(pos[3 * qr + a], 0), pmax);
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      const int ax = (axis_code >> (2 * c)) & 3;
      const float2* cs = rope_cs + int64_t(p3[ax]) * 40 + 8 * c;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float2 r = cs[i];
        const float x1 = qf[8 * c + i], x2 = qf[40 + 8 * c + i];
        qf[8 * c + i] = (x1 * r.x - x2 * r.y) * q_scale_log2;
        qf[40 + 8 * c + i] = (x2 * r.x + x1 * r.y) * q_scale_log2;
      }
    }
#pragma unroll
    for (int s = 0; s < 5; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        qfrag[s][i] = (_Float16)(hf ? qf[16 * s + 8 + i] : qf[16 * s + i]);
    }
  }

  // ---- K/V tile staging (global -> registers -> LDS).
  uint4 kreg[2][2];
  float2 kcs[2][8];
  uint4 vreg[2][2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = tid + 256 * it;
      if (i < K_ITEMS) {
        const int key = i / 5, c = i - key * 5;
        const int kk = kt + key;
        if (kk < kend) {
          const uint4* src = reinterpret_cast<const uint4*>(Kg + int64_t(kk) * ld);
          kreg[it][0] = src[c];
          kreg[it][1] = src[c + 5];
          const int ax = (axis_code >> (2 * c)) & 3;
          const int p = min(max(pos[3 * kk + ax], 0), pmax);
          const float4* cs = reinterpret_cast<const float4*>(rope_cs + int64_t(p) * 40 + 8 * c);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float4 v = cs[j];
            kcs[it][2 * j] = make_float2(v.x, v.y);
            kcs[it][2 * j + 1] = make_float2(v.z, v.w);
          }
        } else {
          kreg[it][0] = kreg[it][1] = make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < 8; ++j) kcs[it][j] = make_float2(1.f, 0.f);
        }
      }
      if (i < V_ITEMS) {
        const int kp = i & 31, c = i >> 5;
        const int kk = kt + 2 * kp;
        vreg[it][0] = kk < kend ? reinterpret_cast<const uint4*>(Vg + int64_t(kk) * ld)[c]
                                : make_uint4(0, 0, 0, 0);
        vreg[it][1] = kk + 1 < kend ? reinterpret_cast<const uint4*>(Vg + int64_t(kk + 1) * ld)[c]
                                    : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = tid + 256 * it;
      if (i < K_ITEMS) {
        const int key = i / 5, c = i - key * 5;
        const uint32_t a[4] = {kreg[it][0].x, kreg[it][0].y, kreg[it][0].z, kreg[it][0].w};
        const uint32_t b[4] = {kreg[it][1].x, kreg[it][1].y, kreg[it][1].z, kreg[it][1].w};
        uint32_t ra[4], rb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x1l = bflo(a[j]), x1h = bfhi(a[j]);
          const float x2l = bflo(b[j]), x2h = bfhi(b[j]);
          const float2 cl = kcs[it][2 * j], ch = kcs[it][2 * j + 1];
          ra[j] = pack_f16x2(x1l * cl.x - x2l * cl.y, x1h * ch.x - x2h * ch.y);
          rb[j] = pack_f16x2(x2l * cl.x + x1l * cl.y, x2h * ch.x + x1h * ch.y);
        }
        uint16_t* dst = sK[buf] + key * KROW;
        *reinterpret_cast<uint4*>(dst + 8 * c) = make_uint4(ra[0], ra[1], ra[2], ra[3]);
        *reinterpret_cast<uint4*>(dst + 40 + 8 * c) = make_uint4(rb[0], rb[1], rb[2], rb[3]);
      }
      if (i < V_ITEMS) {
        const int kp = i & 31, c = i >> 5;
        const uint32_t a[4] = {vreg[it][0].x, vreg[it][0].y, vreg[it][0].z, vreg[it][0].w};
        const uint32_t b[4] = {vreg[it][1].x, vreg[it][1].y, vreg[it][1].z, vreg[it][1].w};
        uint16_t* dst = sV[buf] + (8 * c) * VROW + 2 * kp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // dims 8c+2j (low halves) and 8c+2j+1 (high halves) of keys 2kp, 2kp+1, as fp16
          *reinterpret_cast<uint32_t*>(dst + (2 * j) * VROW) = pack_f16x2(bflo(a[j]), bflo(b[j]));
          *reinterpret_cast<uint32_t*>(dst + (2 * j + 1) * VROW) = pack_f16x2(bfhi(a[j]), bfhi(b[j]));
        }
      }
    }
  };

  f32x16_t acc[3];
#pragma unroll
  for (int d = 0; d < 3; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[d][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  gload(kbeg);
  lstore(0);
  __syncthreads();
  const int ntiles = (kend - kbeg + BKV - 1) / BKV;
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kt = kbeg + t * BKV;
    if (t + 1 < ntiles) gload(kt + BKV);

    // S^T = K Q^T for 64 keys: two 32-key blocks.
    f32x16_t s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[b][e] = 0.f;
    const uint16_t* kb = sK[buf] + ln * KROW + 8 * hf;
#pragma unroll
    for (int sl = 0; sl < 5; ++sl) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const f16x8_t a = *reinterpret_cast<const f16x8_t*>(kb + b * 32 * KROW + 16 * sl);
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qfrag[sl], s[b], 0, 0, 0);
      }
    }
    // s[b][4g + r] is key kt + 32b + 8g + 4hf + r of query ln.
    if (kt + BKV > kend) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kt + 32 * b + 8 * (e >> 2) + 4 * hf + (e & 3) >= kend) s[b][e] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[b][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
    f16x8_t pf[4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(s[b][e] - m_new);
        lsum += p;
        pf[2 * b + (e >> 3)][e & 7] = (_Float16)p;
      }
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int d = 0; d < 3; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[d][e] *= alpha;

    // O^T += V^T P^T over 4 slices of 16 keys.
    const uint16_t* vb = sV[buf];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb0 = 16 * ks + 4 * hf;
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        const int dim = 32 * d + ln;
        f16x8_t a;
        if (d < 2 || dim < HD) {
          const uint2 lo4 = *reinterpret_cast<const uint2*>(vb + dim * VROW + kb0);
          const uint2 hi4 = *reinterpret_cast<const uint2*>(vb + dim * VROW + kb0 + 8);
          a = __builtin_bit_cast(f16x8_t, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
        } else {
          a = __builtin_bit_cast(f16x8_t, make_uint4(0, 0, 0, 0));
        }
        acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], acc[d], 0, 0, 0);
      }
    }

    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: acc[d][4g + r] is dim 32d + 8g + 4hf + r of query ln.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (!qvalid) return;
  const int64_t orow = int64_t(qrow) * heads * HD + head * HD;
#pragma unroll
  for (int d = 0; d < 3; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = 32 * d + 8 * g + 4 * hf;
      if (dim >= HD) continue;
      const float o0 = acc[d][4 * g] * inv, o1 = acc[d][4 * g + 1] * inv;
      const float o2 = acc[d][4 * g + 2] * inv, o3 = acc[d][4 * g + 3] * inv;
      if (out_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + orow + dim) =
            make_float4(o0, o1, o2, o3);
      } else {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + orow + dim) =
            make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      }
    }
  }
}

hipError_t launch_attention(const uint16_t* qkv, const int32_t* cu_seqlens, const int32_t* pos_thw,
                            const int32_t* order, const int32_t* tile_start, int32_t n_img,
                            int32_t max_tiles, int32_t heads, int32_t n_pos, int32_t axis_code,
                            const float2* rope_cs, float q_scale_log2, void* out, bool out_f32,
                            hipStream_t s) {
  const int64_t blocks = int64_t(max_tiles) * heads;
  hipLaunchKernelGGL(attention_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, qkv, cu_seqlens,
                     pos_thw, order, tile_start, n_img, heads, n_pos, rope_cs, axis_code,
                     q_scale_log2, out, out_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace vt
