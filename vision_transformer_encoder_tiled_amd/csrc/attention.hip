// Tiled varlen non-causal multi-head attention with 3D RoPE, head_dim 80,
// on the gfx950 matrix cores.
//
// The pages describe the untiled form -- a per-head [seq, seq] fp32 score
// matrix, a row softmax into a bf16 [seq, seq] probability matrix, then P V
// ("init.rs (VisionEncoder::new)": build_scratch and the GEMM-based ViT SDPA
// kernel list) -- and name that quadratic buffer as the limit on image size
// (doc comment of CEILING_MAX_PATCHES).  Here the scores never leave the MFMA
// accumulators: a workgroup owns 128 queries of one head of one image and
// streams that image's keys in tiles of 64 through LDS with an online
// softmax, so memory is O(tokens).
//
// Three kernels:
//
// attn_pack_kernel (the Q/K/V load stage, once per token and head):
//   rotate q and k with 3D RoPE (rotate-half pairs (j, j+40), angle
//   pos[axis(j)] * inv_freq[j] from a (cos, sin) table built in double),
//   scale q by log2(e)/sqrt(80), convert q, k, v to fp16, and write K and V
//   as 24 KB "tile images", one per (head, 64-key tile of an image): the
//   exact bytes the attention kernel wants in LDS.
//     K   [64 keys][88]  fp16, 16-byte padded rows (conflict-free 16-byte
//                        fragment reads of 32 consecutive keys);
//     V^T [81 dims][72]  fp16, dims as rows; inside each group of 16 keys
//                        the key slots are ordered 0-3, 8-11, 4-7, 12-15 so
//                        that the 8 keys one lane feeds to an MFMA k slice
//                        are adjacent (one 16-byte read); row 80 is all ones.
//   Each image's keys start on a fresh tile; the padding keys are zero.
//   Rotating here, once, rather than per (query tile, key tile) keeps all
//   RoPE and conversion work out of the inner loop, which is VALU-bound at
//   head_dim 80.
//
// attention_kernel (calls with few query tiles): 4 wavefronts, each with 32
//   queries, in two key groups (KG = 2): 64 queries per workgroup, two
//   groups of 2 wavefronts take alternate key tiles and merge at the end, so
//   that small images still give every CU a workgroup.  (KG = 1, one group
//   of 128 queries, is the same code with the merge left out.)
// attention_lean_kernel (calls with many query tiles): the same arithmetic
//   per tile without the score pipelining described below, in fewer
//   registers, so that 3 or 4 wavefronts share each SIMD (see there).
//   S^T = K Q^T   v_mfma_f32_32x32x16_f16, 2 key blocks x 5 dim slices of
//                 16 (head_dim 80 = 5 x 16 exactly).  Each lane holds one
//                 query and 16 keys of each 32-key block.
//   O^T = V^T P^T v_mfma_f32_32x32x16_f16, 4 key slices x 3 dim blocks of
//                 32.  P comes straight from the score registers (the key
//                 order inside a slice matches the V^T slot order).  Dims
//                 80..95 of the third block are padding: the all-ones row
//                 80 makes that MFMA row the softmax denominator l = sum(P),
//                 from the same fp16 P as the numerator; rows 81..95 are
//                 never stored.
//   Online softmax in the log2 domain with lazy rescaling: the reference max
//   m of a query is set by the first key tile and only raised (O and l
//   rescaled) when some row's max grows by more than 8, decided once per
//   wavefront; P is then at most 2^8, well inside fp16.  The score MFMAs
//   accumulate onto -m, so the exponentials need no subtraction.  The two
//   lane halves of a query combine their maxima with v_permlane32_swap.
//   Tile images stream global -> LDS by direct DMA (global_load_lds) into a
//   ring of 3 stages: the copy of tile t+2 is in flight while tile t is
//   processed.  Scores are software-pipelined one tile ahead: the MFMAs of
//   tile t+1's S^T are issued between tile t's row max and its
//   exponentials.  One workgroup barrier per tile.
//
// Operand precision: fp16 operands, fp32 accumulation.  fp16 runs at the
// bf16 rate on gfx950 with 3 more mantissa bits; rounding P to bf16 would
// cost up to ~2^-9 |v| per output.  |RoPE(q)| log2(e)/sqrt(80), |k| and |v|
// must stay below 65504 (not clamped: larger values become infinite).
//
// Grid: one workgroup per (q-tile, head), head fastest, q-tiles of the
// largest images first (longest-processing-time order).  With 16 heads and
// round-robin dispatch over the 8 XCDs, every q-tile of one (image, head)
// lands on the same XCD, so its K/V stream is shared through one L2.
#include <algorithm>
#include <vector>

#include "vt_device.h"
#include "vt_kernels.h"

namespace vt {

namespace {
constexpr int HD = 80;              // head_dim
constexpr int BKV = kAttnKTile;     // keys per tile
constexpr int KROW = kAttnKRow;     // fp16 per K row (176 B)
constexpr int VROW = kAttnVRow;     // fp16 per V^T row (144 B)
constexpr int K_BYTES = BKV * KROW * 2;          // 11264
constexpr int V_ROWS = HD + 1;                   // dims 0..79 and the ones row
constexpr int IMG_BYTES = kAttnTileBytes;        // 24576: K + V^T rows 0..80 + pad
constexpr int STAGE_BYTES = K_BYTES + 96 * VROW * 2;  // 25088: the MFMA reads V^T rows up to 95
constexpr float kLazy = 8.0f;       // log2 growth of the row max tolerated before rescaling
static_assert(K_BYTES + V_ROWS * VROW * 2 <= IMG_BYTES, "tile image size");

}  // namespace

// ---------------------------------------------------------------- pack
// Block per (key tile, head), 320 threads = 64 keys x 5 chunks with the
// chunk fastest, so a wavefront reads runs of 80 contiguous bytes of each
// token's q, k and v.  Thread (k, c) handles rotation pairs 8c..8c+7, i.e.
// dims 8c..8c+7 and 40+8c..40+8c+7 of q, k and v of key k.  V is
// transposed through LDS so that every V^T row leaves as 128 contiguous
// bytes.
__global__ void __launch_bounds__(320) attn_pack_kernel(
    const uint16_t* __restrict__ qkv, const int32_t* __restrict__ pos,
    const int2* __restrict__ kdesc, int32_t heads, int32_t n_pos,
    const float2* __restrict__ rope_cs, int32_t axis_code, float q_scale_log2,
    uint16_t* __restrict__ qpk, uint16_t* __restrict__ kv) {
  __shared__ __align__(16) uint16_t vs[HD * BKV];  // V^T [dim][slot], 128 B rows
  // Block b = (key tile b / heads, head b % heads): the heads of one tile go
  // out together, so the 128-byte lines that two heads' 160-byte q/k/v
  // segments share are read from memory once.
  const int T = blockIdx.x / heads, head = blockIdx.x % heads;
  const int2 desc = kdesc[T];
  if (desc.x < 0) return;
  const int k = threadIdx.x / 5, c = threadIdx.x % 5;
  const int tok = desc.x + k;
  const bool valid = tok < desc.y;
  char* img = reinterpret_cast<char*>(kv) + (int64_t(T) * heads + head) * IMG_BYTES;
  uint32_t kr[8], vt[8];  // rotated k (fp16 pairs) and v (fp16 pairs)
  if (valid) {
    const int64_t ld = int64_t(3) * heads * HD;
    const uint16_t* row = qkv + int64_t(tok) * ld + head * HD;
    const int ax = (axis_code >> (2 * c)) & 3;
    const int p = min(max(pos[3 * tok + ax], 0), n_pos - 1);
    const float4* cs4 = reinterpret_cast<const float4*>(rope_cs + int64_t(p) * 40 + 8 * c);
    float cs[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = cs4[j];
      cs[4 * j] = v.x; cs[4 * j + 1] = v.y; cs[4 * j + 2] = v.z; cs[4 * j + 3] = v.w;
    }
#pragma unroll
    for (int which = 0; which < 2; ++which) {  // 0: q, 1: k
      const uint4 a = reinterpret_cast<const uint4*>(row + which * heads * HD)[c];
      const uint4 b = reinterpret_cast<const uint4*>(row + which * heads * HD)[c + 5];
      uint4 o1, o2;
      rope8_f16(a, b, cs, which == 0 ? q_scale_log2 : 1.0f, &o1, &o2);
      if (which == 0) {
        uint16_t* q = qpk + (int64_t(tok) * heads + head) * HD;
        reinterpret_cast<uint4*>(q)[c] = o1;
        reinterpret_cast<uint4*>(q)[c + 5] = o2;
      } else {
        kr[0] = o1.x; kr[1] = o1.y; kr[2] = o1.z; kr[3] = o1.w;
        kr[4] = o2.x; kr[5] = o2.y; kr[6] = o2.z; kr[7] = o2.w;
      }
    }
    const uint4 a = reinterpret_cast<const uint4*>(row + 2 * heads * HD)[c];
    const uint4 b = reinterpret_cast<const uint4*>(row + 2 * heads * HD)[c + 5];
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vt[j] = pack_f16x2(bflo(aw[j]), bfhi(aw[j]));
      vt[4 + j] = pack_f16x2(bflo(bw[j]), bfhi(bw[j]));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) kr[j] = vt[j] = 0u;
  }
  // K rows: dims 8c..8c+7 and 40+8c..40+8c+7 of key k (padding keys are zero).
  uint16_t* kimg = reinterpret_cast<uint16_t*>(img);
  *reinterpret_cast<uint4*>(kimg + k * KROW + 8 * c) = make_uint4(kr[0], kr[1], kr[2], kr[3]);
  *reinterpret_cast<uint4*>(kimg + k * KROW + 40 + 8 * c) = make_uint4(kr[4], kr[5], kr[6], kr[7]);
  // V^T through LDS: element (dim, slot of key k).
  const int s = mfma_slot16(k);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vs[(8 * c + 2 * j) * BKV + s] = uint16_t(vt[j] & 0xffffu);
    vs[(8 * c + 2 * j + 1) * BKV + s] = uint16_t(vt[j] >> 16);
    vs[(40 + 8 * c + 2 * j) * BKV + s] = uint16_t(vt[4 + j] & 0xffffu);
    vs[(40 + 8 * c + 2 * j + 1) * BKV + s] = uint16_t(vt[4 + j] >> 16);
  }
  __syncthreads();
  // Rows 0..79 from LDS and row 80 = fp16 1.0, 16 bytes (8 slots) per thread.
  // Row padding (K dims 80..87, V^T slots 64..71) and the tail of the image
  // are never read for rows that reach the output.
  uint16_t* vimg = reinterpret_cast<uint16_t*>(img + K_BYTES);
  for (int i = threadIdx.x; i < V_ROWS * (BKV / 8); i += 320) {
    const int d = i >> 3, sg = i & 7;
    const uint4 v = d < HD ? *reinterpret_cast<const uint4*>(vs + d * BKV + 8 * sg)
                           : make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
    *reinterpret_cast<uint4*>(vimg + d * VROW + 8 * sg) = v;
  }
}

// ---------------------------------------------------------------- image init
// The parts of the K/V tile images that do not depend on the layer, for the
// path where the QKV GEMM's epilogue writes the rotated Q and the images'
// key rows itself (launch_gemm_qkv_pack): per (key tile, head), the V^T
// ones row (row 80) and, past the image end in its last tile, zero K rows
// and zero V^T slots; and, from the head-0 workgroups, kslot[tok] = 64 T + s,
// the tile T and slot s that token tok's key occupies.  Block per (key tile,
// head) like the pack kernel, 256 threads.
__global__ void __launch_bounds__(256) attn_image_init_kernel(const int2* __restrict__ kdesc,
                                                              int32_t heads, uint16_t* __restrict__ kv,
                                                              int32_t* __restrict__ kslot) {
  const int T = blockIdx.x / heads, head = blockIdx.x % heads;
  const int2 desc = kdesc[T];
  if (desc.x < 0) return;
  const int valid = min(BKV, desc.y - desc.x);
  const int t = threadIdx.x;
  if (head == 0 && t < valid) kslot[desc.x + t] = T * BKV + t;
  char* img = reinterpret_cast<char*>(kv) + (int64_t(T) * heads + head) * IMG_BYTES;
  uint16_t* kimg = reinterpret_cast<uint16_t*>(img);
  uint16_t* vimg = reinterpret_cast<uint16_t*>(img + K_BYTES);
  if (t < BKV / 8) {  // the ones row: 8 slots per thread
    *reinterpret_cast<uint4*>(vimg + HD * VROW + 8 * t) =
        make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  }
  // padding keys: K rows (10 chunks of 16 bytes each) and V^T slots (80 dims)
  for (int i = t; i < (BKV - valid) * 10; i += 256) {
    const int k = valid + i / 10, c = i % 10;
    *reinterpret_cast<uint4*>(kimg + k * KROW + 8 * c) = make_uint4(0u, 0u, 0u, 0u);
  }
  for (int i = t; i < (BKV - valid) * HD; i += 256) {
    const int k = valid + i / HD, dim = i % HD;
    vimg[dim * VROW + mfma_slot16(k)] = 0;
  }
}

hipError_t launch_attn_image_init(const int2* kdesc, int32_t max_ktiles, int32_t heads, uint16_t* kv,
                                  int32_t* kslot, hipStream_t s) {
  hipLaunchKernelGGL(attn_image_init_kernel, dim3(unsigned(int64_t(max_ktiles) * heads)), dim3(256), 0, s,
                     kdesc, heads, kv, kslot);
  return hipGetLastError();
}

// ---------------------------------------------------------------- attention
// KG = key groups.  The 4 wavefronts form KG groups of 4/KG; a group owns
// all the workgroup's 32 * 4/KG queries and every KG-th key tile of the
// image (tile r*KG + g in round r).  With KG = 2 a workgroup holds 64
// queries, so small images give twice as many workgroups; the groups'
// partial (max, O, l) are merged through LDS at the end.
//
// CW > 0: CW more wavefronts that only copy the tile images (a wavefront
// that issues copies stalls for ~100 cycles per 1 KB copy instruction, and
// with one multiplying wavefront per SIMD nothing else runs meanwhile).  They
// wait for their copies and meet every workgroup barrier of the others, in
// the same order, then leave; the multiplying wavefronts issue no copies.
template <int NW, int KG, int NST, int CW = 0>
__global__ void __launch_bounds__(64 * (NW + CW)) attention_kernel(
    const uint16_t* __restrict__ qpk, const uint16_t* __restrict__ kv,
    const int4* __restrict__ qdesc, int32_t heads, void* __restrict__ out, int32_t out_f32,
    float* __restrict__ lse) {
  static_assert(NST == 3 || (NST == 4 && KG == 1), "stage ring");
  constexpr int QW = NW / KG;             // query wavefronts per group
  constexpr int NCW = CW > 0 ? CW : NW;   // wavefronts that copy
  constexpr int COPIES = IMG_BYTES / (1024 * NCW);  // 1 KB DMA pieces per copying wave per tile
  static_assert(COPIES * NCW * 1024 == IMG_BYTES, "tile image must be whole rounds of copies");
  constexpr int WQ = 32 * QW;             // queries per workgroup
  constexpr int STAGE = KG * STAGE_BYTES; // one round: KG tiles
  extern __shared__ __align__(16) char lds[];

  const int head = blockIdx.x % heads;
  const int4 desc = qdesc[blockIdx.x / heads];  // (first query, image begin, image end, first key tile)
  if (desc.x < 0) return;
  const int q0 = desc.x, kbeg = desc.y, kend = desc.z;
  const int qend = min(q0 + WQ, kend);
  const int ntiles = (kend - kbeg + BKV - 1) / BKV;
  const int rounds = (ntiles + KG - 1) / KG;
  // Tile t of this (image, head) is image (desc.w + t) * heads + head.
  const char* src = reinterpret_cast<const char*>(kv) + (int64_t(desc.w) * heads + head) * IMG_BYTES;
  const int64_t tile_stride = int64_t(heads) * IMG_BYTES;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave / QW, qw = wave % QW;
  const int hf = lane >> 5, ln = lane & 31;
  const int cwave = CW > 0 ? wave - NW : wave;  // index among the copying wavefronts
  const uint32_t lds_wave = lds_offset(lds) + 1024 * cwave;

  // Round r -> stage r % 3: tile r*KG + j at offset j * STAGE_BYTES; each
  // copying wavefront copies COPIES 1 KB pieces of every tile that exists.
  auto issue = [&](int r) {
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      const int t = r * KG + j;
      if (t < ntiles) {
        const uint32_t base =
            __builtin_amdgcn_readfirstlane(lds_wave + (r % NST) * STAGE + j * STAGE_BYTES);
        const char* g = src + t * tile_stride + 1024 * cwave + 16 * lane;
#pragma unroll
        for (int c = 0; c < COPIES; ++c) dma16(g + NCW * 1024 * c, base + NCW * 1024 * c);
      }
    }
  };

  if constexpr (CW > 0) {
    if (wave >= NW) {
      // The copy-only wavefronts: the first NST - 1 rounds, the barrier after
      // them, then per round the barrier of body() (everything issued so far,
      // i.e. rounds <= r + 1, has landed) followed by the copy of round
      // r + NST - 1 into the stage round r - 1 used; with KG = 2 the two
      // barriers of the group merge.  The ring is idle once they leave.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int r = 0; r < NST - 1; ++r)
        if (r < rounds) issue(r);
      wait_vmcnt<0>();
      wg_barrier();
      for (int r = 0; r < rounds; ++r) {
        wait_vmcnt<0>();
        wg_barrier();
        if (r + NST - 1 < rounds) issue(r + NST - 1);
      }
      if constexpr (KG == 2) {
        wg_barrier();
        __syncthreads();
      }
      return;
    }
  }

  // Q fragments (B operand of S^T = K Q^T): dims 16s + 8hf .. +7 of this lane's query.
  const int qrow = q0 + qw * 32 + ln;
  const bool qvalid = qrow < qend;
  const int qr = qvalid ? qrow : qend - 1;
  f16x8_t qfrag[5];
  {
    const uint4* q = reinterpret_cast<const uint4*>(qpk + (int64_t(qr) * heads + head) * HD);
#pragma unroll
    for (int s = 0; s < 5; ++s) qfrag[s] = __builtin_bit_cast(f16x8_t, q[2 * s + hf]);
  }

  // Per-lane LDS offsets inside this group's tile of a stage.
  const int koff = grp * STAGE_BYTES + ln * KROW * 2 + 16 * hf;            // + 32 b KROW*2 + 32 sl
  const int voff = grp * STAGE_BYTES + K_BYTES + ln * VROW * 2 + 16 * hf;  // + (32 d) VROW*2 + 32 ks

  f16x8_t kf[10];
  auto load_k = [&](int r) {
    const char* st = lds + (r % NST) * STAGE + koff;
#pragma unroll
    for (int sl = 0; sl < 5; ++sl)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        kf[2 * sl + b] = *reinterpret_cast<const f16x8_t*>(st + b * 32 * KROW * 2 + 32 * sl);
  };

  f32x16_t acc[3];
#pragma unroll
  for (int d = 0; d < 3; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[d][e] = 0.f;

  // S^T for one tile; the accumulation starts from c0 (all entries -m for the
  // lane's query), so the scores come out already relative to the running max.
  auto qk = [&](f32x16_t (&sc)[2], const f32x16_t& c0) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
      sc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[b], qfrag[0], c0, 0, 0, 0);
#pragma unroll
    for (int sl = 1; sl < 5; ++sl)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        sc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[2 * sl + b], qfrag[sl], sc[b], 0, 0, 0);
  };
  // Keys past the image end (last tile only) get -inf scores.
  auto mask = [&](f32x16_t (&sc)[2], int t) {
    const int kt = kbeg + t * BKV;
    if (kt + BKV > kend) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kt + 32 * b + 8 * (e >> 2) + 4 * hf + (e & 3) >= kend) sc[b][e] = -INFINITY;
    }
  };
  // Row max over this lane's 32 scores, combined with the other lane half.
  auto rowmax = [&](const f32x16_t (&sc)[2]) {
    float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
    for (int e = 2; e < 16; ++e) mx = fmaxf(mx, sc[0][e]);
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[1][e]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };

  if constexpr (CW == 0) {
#pragma unroll
    for (int r = 0; r < NST - 1; ++r)
      if (r < rounds) issue(r);
  }
  wait_vmcnt<0>();
  wg_barrier();

  // The group's first tile fixes the reference max m (per query): its scores
  // are computed from zero and shifted once; later tiles accumulate onto -m.
  // A group with no tile (one-tile image, KG = 2) keeps m = -inf and O = 0.
  f32x16_t sa[2], sb[2], negm;
  float m_use = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) negm[e] = 0.f;
  if (grp < ntiles) {
    load_k(0);
    qk(sa, negm);
    mask(sa, grp);
    m_use = rowmax(sa);
#pragma unroll
    for (int e = 0; e < 16; ++e) negm[e] = -m_use;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) sa[b][e] -= m_use;
  }

  // One round; `cur` holds the scores of the group's tile tc relative to m.
  // The group's next tile's score MFMAs are issued before this tile's
  // exponentials so they run underneath.
  auto body = [&](int r, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) {
    // Every wave is done reading round r-1 (V) and round r (K); round r+1 has
    // landed (with 4 stages round r+2 may still be in flight).
    if (NST == 4 && r + 2 < rounds) wait_vmcnt<(NST - 3) * COPIES * KG>();
    else wait_vmcnt<0>();
    wait_lds_reads();
    wg_barrier();
    if constexpr (CW == 0)
      if (r + NST - 1 < rounds) issue(r + NST - 1);  // into the stage round r-1 used
    const int tc = r * KG + grp, tn = tc + KG;
    if (tn < ntiles) load_k(r + 1);
    if (tc >= ntiles) return;

    if (r > 0) {
      mask(cur, tc);
      const float mx = rowmax(cur);  // relative to m
      // Lazy rescale: raise m only when some row's max grew by more than kLazy.
      if (__any(mx > kLazy)) {
        const float delta = fmaxf(mx, 0.f);
        m_use += delta;
        const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
        for (int d = 0; d < 3; ++d)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[d][e] *= alpha;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) cur[b][e] -= delta;
#pragma unroll
        for (int e = 0; e < 16; ++e) negm[e] = -m_use;
      }
    }

    if (tn < ntiles) qk(nxt, negm);  // next tile's scores, in flight during the exponentials

    // V^T fragments of this tile: one 16-byte read per (key slice, dim block),
    // in two halves to bound the live registers.
    const char* vst = lds + (r % NST) * STAGE + voff;
    f16x8_t vf[6];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int d = 0; d < 3; ++d)
        vf[3 * ks + d] = *reinterpret_cast<const f16x8_t*>(vst + 32 * d * VROW * 2 + 32 * ks);

    f16x8_t pf[4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        pf[2 * b + (e >> 3)][e & 7] = (_Float16)__builtin_amdgcn_exp2f(cur[b][e]);

    // O^T += V^T P^T over 4 slices of 16 keys.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int d = 0; d < 3; ++d)
        acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[3 * ks + d], pf[ks], acc[d], 0, 0, 0);
#pragma unroll
    for (int ks = 2; ks < 4; ++ks)
#pragma unroll
      for (int d = 0; d < 3; ++d)
        vf[3 * (ks - 2) + d] = *reinterpret_cast<const f16x8_t*>(vst + 32 * d * VROW * 2 + 32 * ks);
#pragma unroll
    for (int ks = 2; ks < 4; ++ks)
#pragma unroll
      for (int d = 0; d < 3; ++d)
        acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[3 * (ks - 2) + d], pf[ks], acc[d], 0, 0, 0);
  };
  int r = 0;
  for (; r + 1 < rounds; r += 2) {
    body(r, sa, sb);
    body(r + 1, sb, sa);
  }
  if (r < rounds) body(r, sa, sb);

  if constexpr (KG == 2) {
    // Merge group 1 into group 0: O = O0 2^(m0-m) + O1 2^(m1-m), m = max(m0, m1),
    // the row sum l (the ones-row element) included.  Exchange slots are
    // [element][query wave][lane] floats, conflict-free.
    float* xs = reinterpret_cast<float*>(lds);
    wait_lds_reads();
    wg_barrier();  // the ring is idle
    const int slot = qw * 64 + lane;
    if (grp == 1) {
      xs[48 * 64 * QW + slot] = m_use;
#pragma unroll
      for (int d = 0; d < 3; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) xs[(16 * d + e) * 64 * QW + slot] = acc[d][e];
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xs[48 * 64 * QW + slot];
    const float m = fmaxf(m_use, m1);
    const float s0 = __builtin_amdgcn_exp2f(m_use - m), s1 = __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
    for (int d = 0; d < 3; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[d][e] = acc[d][e] * s0 + xs[(16 * d + e) * 64 * QW + slot] * s1;
    m_use = m;
  }

  // ---- normalise and store: acc[d][4g + r] is dim 32d + 8g + 4hf + r of query ln;
  // the row sum l (dim 80) is acc[2][8] in the lanes with hf == 0.
  const float l_half0 = __shfl(acc[2][8], ln, 64);
  const float inv = 1.0f / l_half0;
  if (!qvalid) return;
  // log2-domain log-sum-exp of the query's scaled scores, for the backward pass.
  if (lse && hf == 0) lse[int64_t(qrow) * heads + head] = m_use + log2f(l_half0);
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

// ---------------------------------------------------------------- lean attention
// The kernel for calls with many query tiles: the same per-tile arithmetic
// as attention_kernel with one key group (S^T onto -m, lazy rescale, P from
// the score registers, the ones row for l), but register-lean so that more
// wavefronts share each SIMD and hide one another's latencies: one set of
// scores (no one-tile-ahead pipelining), K and V^T fragments read just ahead
// of use (each K fragment one product ahead), -m written into the score
// accumulators before each tile's first MFMA (16 moves instead of a
// loop-carried 16-register C operand), and a 2-stage ring (50 KB of LDS):
// 126 VGPRs.  4 wavefronts = 128 queries, three workgroups per CU
// (LDS-bound), or 8 wavefronts = 256 queries sharing one K/V stream, two
// workgroups per CU: four wavefronts per SIMD.  WPE is the wavefronts per
// SIMD the register budget is set for.  A wavefront raises its issue
// priority (s_setprio) over its two MFMA sections, so that of the wavefronts
// sharing a SIMD, one with a matrix product ready goes ahead of one in the
// softmax arithmetic and the matrix unit idles less (about 1% at 20,736
// tokens; scheduling only, the results are the same bits).
//
// Work split (AttnTail in vt_kernels.h): block b < n_whole runs item b --
// q-tile b / heads, head b % heads -- over all its key tiles; with a split
// tail, block n_whole + k runs key tiles [k T / S, (k+1) T / S) of the tail,
// one piece per item it touches, and an item it does not run whole goes to
// partial record 2k (the range's first piece) or 2k + 1 (its last).
namespace {
struct TailPlan {
  int32_t n_whole;  // items run whole, one per block
  int32_t qt_tail;  // first q-tile of the split tail
  int64_t T;        // key tiles of the tail over all heads (0: no split)
};
__device__ __forceinline__ TailPlan tail_plan(int nq, int heads, int S, const int32_t* qkpre) {
  TailPlan p{nq * heads, nq, 0};
  if (S <= 0) return p;
  const int n_items = nq * heads;
  const int nw = (n_items / S) * S / heads * heads;  // whole rounds, cut at a q-tile boundary
  if (nw >= n_items) return p;
  const int qt = nw / heads;
  // Short tail items (a mixed batch's smallest images, last in the schedule)
  // leave little idle time under the hardware's dynamic dispatch; the split
  // pays only for long ones.
  if (qkpre[qt + 1] - qkpre[qt] < kAttnTailMinItemTiles) return p;
  const int64_t T = int64_t(heads) * (qkpre[nq] - qkpre[qt]);
  if (T < int64_t(S) * kAttnTailMinTiles) return p;
  p.n_whole = nw;
  p.qt_tail = nw / heads;
  p.T = T;
  return p;
}
}  // namespace

template <int NW, int NST, int WPE>
__global__ void __launch_bounds__(64 * NW, WPE) attention_lean_kernel(
    const uint16_t* __restrict__ qpk, const uint16_t* __restrict__ kv,
    const int4* __restrict__ qdesc, int32_t heads, void* __restrict__ out, int32_t out_f32,
    float* __restrict__ lse, const int32_t* __restrict__ qkpre, const int32_t* __restrict__ nq_ptr,
    int32_t tail_wgs, float* __restrict__ part) {
  constexpr int COPIES = IMG_BYTES / (1024 * NW);
  constexpr int WQ = 32 * NW;
  constexpr int REC = WQ * 82;  // partial record: O [WQ][80], m [WQ], l [WQ] (fp32)
  extern __shared__ __align__(16) char lds[];
  const int64_t tile_stride = int64_t(heads) * IMG_BYTES;

  // ---- this block's work: one whole item, or a range of the split tail.
  // Every quantity here is uniform over the block; readfirstlane keeps it in
  // scalar registers.
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  const int b = blockIdx.x;
  TailPlan plan{0, 0, 0};
  int nq = 0;
  if (tail_wgs > 0) {
    nq = uni(*nq_ptr);
    plan = tail_plan(nq, heads, tail_wgs, qkpre);
  }
  const bool in_tail = plan.T > 0 && b >= plan.n_whole;
  // With a tail allowance the grid runs past the schedule's q-tile slots:
  // blocks past the last whole item that are not tail blocks have no work.
  if (tail_wgs > 0 && !in_tail && b >= plan.n_whole) return;
  // tail positions (key tiles over all heads) fit in 32 bits; only the
  // products k T need 64
  int lo = 0, hi = 0, pos = 0, tbase = 0, qt = b / heads, k = 0;
  if (in_tail) {
    k = b - plan.n_whole;
    if (k >= tail_wgs) return;
    lo = uni(int(int64_t(k) * plan.T / tail_wgs));
    hi = uni(int(int64_t(k + 1) * plan.T / tail_wgs));
    pos = lo;
    tbase = uni(qkpre[plan.qt_tail]);
    int a = plan.qt_tail, z = nq - 1;  // the q-tile holding position lo
    while (a < z) {
      const int mid = (a + z + 1) >> 1;
      if (heads * (uni(qkpre[mid]) - tbase) <= lo) a = mid; else z = mid - 1;
    }
    qt = uni(a);
  }

  for (bool first = true;; first = false) {
    int head, j0, j1, slot;
    if (in_tail) {
      if (pos >= hi) break;
      while (heads * (uni(qkpre[qt + 1]) - tbase) <= pos) ++qt;
      const int kq = uni(qkpre[qt]);
      const int n = uni(qkpre[qt + 1]) - kq;
      const int off = pos - heads * (kq - tbase);
      head = uni(off / n);
      j0 = uni(off - head * n);
      j1 = uni(min(n, j0 + (hi - pos)));
      slot = (j0 == 0 && j1 == n) ? -1 : (pos == lo ? 2 * k : 2 * k + 1);
      pos += j1 - j0;
    } else {
      if (!first) break;
      head = b % heads;
      j0 = 0;
      j1 = -1;  // all key tiles
      slot = -1;
    }
    // Lane quantities are formed anew for each piece (tid passes through an
    // empty asm statement): hoisted above the piece loop they would stay live
    // across the whole kernel and push the tile loop past its register budget.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int hf = lane >> 5, ln = lane & 31;
    const uint32_t lds_wave = lds_offset(lds) + 1024 * wave;
    const int koff = ln * KROW * 2 + 16 * hf;
    const int voff = K_BYTES + ln * VROW * 2 + 16 * hf;
    const int4 desc = qdesc[qt];
    if (desc.x < 0) return;
    const int q0 = uni(desc.x), kbeg = uni(desc.y), kend = uni(desc.z);
    const int qend = min(q0 + WQ, kend);
    if (j1 < 0) j1 = (kend - kbeg + BKV - 1) / BKV;
    const int ntiles = j1 - j0;
    const char* src = reinterpret_cast<const char*>(kv) + (int64_t(uni(desc.w)) * heads + head) * IMG_BYTES +
                      int64_t(j0) * tile_stride;
    if (!first) {  // the previous piece's waves are done with the ring
      wait_lds_reads();
      wg_barrier();
    }
    auto issue = [&](int t) {
      const uint32_t base = __builtin_amdgcn_readfirstlane(lds_wave + (t % NST) * STAGE_BYTES);
      const char* g = src + t * tile_stride + 1024 * wave + 16 * lane;
#pragma unroll
      for (int c = 0; c < COPIES; ++c) dma16(g + NW * 1024 * c, base + NW * 1024 * c);
    };
    const int qrow = q0 + wave * 32 + ln;
    const bool qvalid = qrow < qend;
    const int qr = qvalid ? qrow : qend - 1;
    f16x8_t qfrag[5];
    {
      const uint4* q = reinterpret_cast<const uint4*>(qpk + (int64_t(qr) * heads + head) * HD);
#pragma unroll
      for (int s = 0; s < 5; ++s) qfrag[s] = __builtin_bit_cast(f16x8_t, q[2 * s + hf]);
    }
    f32x16_t acc[3];
#pragma unroll
    for (int d = 0; d < 3; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[d][e] = 0.f;
    float m_use = 0.f;
#pragma unroll
    for (int r = 0; r < NST - 1; ++r)
      if (r < ntiles) issue(r);
    for (int t = 0; t < ntiles; ++t) {
      wait_vmcnt<0>();
      wait_lds_reads();
      wg_barrier();
      if (t + NST - 1 < ntiles) issue(t + NST - 1);
      const char* st = lds + (t % NST) * STAGE_BYTES;
      f32x16_t sc[2];
      __builtin_amdgcn_s_setprio(1);
      {
        // K fragment i = (key block i & 1, dim slice i >> 1), read one
        // product ahead of its use.
        const char* kp = st + koff;
        auto kfrag = [&](int i) {
          return *reinterpret_cast<const f16x8_t*>(kp + (i & 1) * 32 * KROW * 2 + 32 * (i >> 1));
        };
        f16x8_t kf[2] = {kfrag(0), kfrag(1)};
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[0][e] = sc[1][e] = -m_use;
#pragma unroll
        for (int i = 0; i < 10; ++i) {
          sc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[i & 1], qfrag[i >> 1], sc[i & 1], 0, 0, 0);
          if (i + 2 < 10) kf[i & 1] = kfrag(i + 2);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      const int kt = kbeg + (j0 + t) * BKV;
      if (kt + BKV > kend) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (kt + 32 * bb + 8 * (e >> 2) + 4 * hf + (e & 3) >= kend) sc[bb][e] = -INFINITY;
      }
      float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
      for (int e = 2; e < 16; ++e) mx = fmaxf(mx, sc[0][e]);
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[1][e]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      if (t == 0 || __any(mx > kLazy)) {
        const float delta = t == 0 ? mx : fmaxf(mx, 0.f);
        m_use += delta;
        if (t > 0) {
          const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
          for (int d = 0; d < 3; ++d)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[d][e] *= alpha;
        }
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int e = 0; e < 16; ++e) sc[bb][e] -= delta;
      }
      const char* vst = st + voff;
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        f16x8_t pf[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) pf[e >> 3][e & 7] = (_Float16)__builtin_amdgcn_exp2f(sc[bb][e]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int d = 0; d < 3; ++d)
            acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                *reinterpret_cast<const f16x8_t*>(vst + 32 * d * VROW * 2 + 32 * (2 * bb + h)), pf[h], acc[d],
                0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    // acc[d][4g + r] is dim 32d + 8g + 4hf + r of query ln; the row sum l
    // (dim 80) is acc[2][8] in the lanes with hf == 0.
    const float l_half0 = __shfl(acc[2][8], ln, 64);
    if (slot >= 0) {
      // A piece of an item: unnormalized O, the running max and the row sum.
      float* rec = part + int64_t(slot) * REC;
      const int ql = wave * 32 + ln;
      if (hf == 0) {
        rec[WQ * 80 + ql] = m_use;
        rec[WQ * 81 + ql] = l_half0;
      }
#pragma unroll
      for (int d = 0; d < 3; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = 32 * d + 8 * g + 4 * hf;
          if (dim < HD)
            *reinterpret_cast<float4*>(rec + ql * HD + dim) =
                make_float4(acc[d][4 * g], acc[d][4 * g + 1], acc[d][4 * g + 2], acc[d][4 * g + 3]);
        }
      continue;
    }
    const float inv = 1.0f / l_half0;
    if (qvalid) {
      if (lse && hf == 0) lse[int64_t(qrow) * heads + head] = m_use + log2f(l_half0);
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
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + orow + dim) = make_float4(o0, o1, o2, o3);
          } else {
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + orow + dim) =
                make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
          }
        }
      }
    }
  }
}

// Combines the partial records of the split tail's cut items: block (u, g)
// takes queries 32g .. 32g+31 of tail item n_whole + u, one thread per
// (query, 16-byte chunk of its output row), so that consecutive threads read
// consecutive chunks of a record row.  (Launched only when a split is
// possible; callers that know their images' sizes skip it when none is cut.)  With the pieces' maxima m_p, row sums
// l_p and unnormalized outputs O_p of a query: m = max m_p,
// l = sum l_p 2^(m_p - m), out = sum O_p 2^(m_p - m) / l, lse = m + log2 l.
constexpr int kMergeQ = 32;                 // queries per merge block
constexpr int kMergeThreads = kMergeQ * HD / 4;  // 640
template <int WQ>
__global__ void __launch_bounds__(kMergeThreads) attn_tail_merge_kernel(
    const int4* __restrict__ qdesc, const int32_t* __restrict__ qkpre, const int32_t* __restrict__ nq_ptr,
    int32_t heads, int32_t tail_wgs, const float* __restrict__ part, void* __restrict__ out, int32_t out_f32,
    float* __restrict__ lse) {
  constexpr int REC = WQ * 82;
  constexpr int CH = HD / 4;  // 16-byte chunks per output row
  const int nq = *nq_ptr;
  const TailPlan plan = tail_plan(nq, heads, tail_wgs, qkpre);
  if (plan.T == 0) return;
  const int item = plan.n_whole + blockIdx.x;
  if (item >= nq * heads) return;
  const int qt = item / heads, head = item % heads;
  const int n = qkpre[qt + 1] - qkpre[qt];
  const int64_t P0 = int64_t(heads) * (qkpre[qt] - qkpre[plan.qt_tail]) + int64_t(head) * n;
  // The tail workgroup whose range holds position p: the largest k with k T / S <= p.
  auto wg_of = [&](int64_t p) { return int(((p + 1) * tail_wgs - 1) / plan.T); };
  const int kA = wg_of(P0), kB = wg_of(P0 + n - 1);
  if (kA == kB) return;  // run whole by one workgroup
  const int4 desc = qdesc[qt];
  const int nvalid = min(WQ, desc.z - desc.x);
  auto rec_of = [&](int k) {
    const int64_t klo = int64_t(k) * plan.T / tail_wgs;
    return part + int64_t(klo >= P0 ? 2 * k : 2 * k + 1) * REC;
  };
  const int ql = blockIdx.y * kMergeQ + threadIdx.x / CH, c = threadIdx.x % CH;
  if (ql < nvalid) {
  float m = -INFINITY;
  for (int k = kA; k <= kB; ++k) m = fmaxf(m, rec_of(k)[WQ * 80 + ql]);
  float l = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = kA; k <= kB; ++k) {
    const float* r = rec_of(k);
    const float w = __builtin_amdgcn_exp2f(r[WQ * 80 + ql] - m);
    l += r[WQ * 81 + ql] * w;
    const float4 v = reinterpret_cast<const float4*>(r + ql * HD)[c];
    o.x += v.x * w;
    o.y += v.y * w;
    o.z += v.z * w;
    o.w += v.w * w;
  }
  const float inv = 1.0f / l;
  const int q = desc.x + ql;
  if (lse && c == 0) lse[int64_t(q) * heads + head] = m + log2f(l);
  const float4 v = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  const int64_t at = int64_t(q) * heads * HD + head * HD + 4 * c;
  if (out_f32)
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + at) = v;
  else
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + at) =
        make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  }
}

template <int NW, int KG, int NST, int CW>
static hipError_t launch_attention_kernel(const uint16_t* qpk, const uint16_t* kv,
                                          const int4* qdesc, int32_t max_qtiles, int32_t heads,
                                          void* out, bool out_f32, float* lse, hipStream_t s) {
  const size_t lds = size_t(NST) * KG * STAGE_BYTES;
  auto kern = attention_kernel<NW, KG, NST, CW>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (attr != hipSuccess) return attr;
  const int64_t blocks = int64_t(max_qtiles) * heads;
  hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(64 * (NW + CW)), lds, s, qpk, kv, qdesc, heads,
                     out, out_f32 ? 1 : 0, lse);
  return hipGetLastError();
}

// tail_plan on the host, from the images' token counts: the schedule's
// q-tiles (images largest first, ties in image order) and their key tiles.
static bool host_tail_splits(const int64_t* tokens, int n_img, int WQ, int heads, int S) {
  std::vector<int> idx(n_img);
  for (int i = 0; i < n_img; ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return tokens[a] > tokens[b]; });
  std::vector<int64_t> kt;  // key tiles of each q-tile, in schedule order
  for (int i : idx)
    for (int64_t q = 0; q < (tokens[i] + WQ - 1) / WQ; ++q) kt.push_back((tokens[i] + BKV - 1) / BKV);
  const int64_t nq = int64_t(kt.size()), n_items = nq * heads;
  const int64_t nw = (n_items / S) * S / heads * heads;
  if (nw >= n_items) return false;
  if (kt[nw / heads] < kAttnTailMinItemTiles) return false;
  int64_t T = 0;
  for (int64_t q = nw / heads; q < nq; ++q) T += heads * kt[q];
  return T >= int64_t(S) * kAttnTailMinTiles;
}

// Workgroups of kern the GPU holds at once (blocks per CU x CUs), per device
// (one cache per VARIANT: the lean kernels share a function type).
template <int VARIANT, class K>
static int resident_wgs(K kern, int threads, size_t lds) {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), threads,
                                                     lds) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev] = std::max(per_cu * cus, 1);
  }
  return cached[dev];
}

template <int NW, int WPE, int VARIANT>
static hipError_t launch_lean(const uint16_t* qpk, const uint16_t* kv, const int4* qdesc,
                              int32_t max_qtiles, int32_t heads, void* out, bool out_f32, float* lse,
                              hipStream_t s, const AttnTail& tail) {
  const size_t lds = size_t(2) * STAGE_BYTES;
  auto kern = attention_lean_kernel<NW, 2, WPE>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (attr != hipSuccess) return attr;
  int S = 0;
  if (tail.part && tail.qkpre && tail.nq)
    S = std::min(resident_wgs<VARIANT>(kern, 64 * NW, lds), attn_tail_max_wgs(VARIANT));
  if (S > 0 && tail.host_tokens && !host_tail_splits(tail.host_tokens, tail.host_n_img, 32 * NW, heads, S))
    S = 0;
  const int64_t blocks = int64_t(max_qtiles) * heads + S;
  hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(64 * NW), lds, s, qpk, kv, qdesc, heads, out,
                     out_f32 ? 1 : 0, lse, tail.qkpre, tail.nq, S, tail.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 0) return e;
  // at most S + heads - 1 items are in a split tail
  hipLaunchKernelGGL(attn_tail_merge_kernel<32 * NW>, dim3(unsigned(S + heads), NW), dim3(kMergeThreads), 0, s, qdesc,
                     tail.qkpre, tail.nq, heads, S, tail.part, out, out_f32 ? 1 : 0, lse);
  return hipGetLastError();
}

hipError_t launch_attn_pack(const uint16_t* qkv, const int32_t* pos_thw, const int2* kdesc, int32_t max_ktiles,
                            int32_t heads, int32_t n_pos, int32_t axis_code, const float2* rope_cs,
                            float q_scale_log2, uint16_t* qpk, uint16_t* kv, hipStream_t s) {
  hipLaunchKernelGGL(attn_pack_kernel, dim3(unsigned(int64_t(max_ktiles) * heads)), dim3(320), 0, s,
                     qkv, pos_thw, kdesc, heads, n_pos, rope_cs, axis_code, q_scale_log2, qpk, kv);
  return hipGetLastError();
}

hipError_t launch_attention(const uint16_t* qkv, const int32_t* pos_thw, const int4* qdesc,
                            const int2* kdesc, int32_t max_qtiles, int32_t max_ktiles,
                            int32_t heads, int32_t n_pos, int32_t axis_code, const float2* rope_cs,
                            float q_scale_log2, int32_t variant, uint16_t* qpk, uint16_t* kv,
                            void* out, bool out_f32, float* lse, hipStream_t s, const AttnTail& tail) {
  const hipError_t e =
      launch_attn_pack(qkv, pos_thw, kdesc, max_ktiles, heads, n_pos, axis_code, rope_cs, q_scale_log2, qpk, kv, s);
  if (e != hipSuccess) return e;
  return launch_attention_packed(qpk, kv, qdesc, max_qtiles, heads, variant, out, out_f32, lse, s, tail);
}

hipError_t launch_attention_packed(const uint16_t* qpk, const uint16_t* kv, const int4* qdesc,
                                   int32_t max_qtiles, int32_t heads, int32_t variant, void* out,
                                   bool out_f32, float* lse, hipStream_t s, const AttnTail& tail) {
  switch (variant) {
    case kAttnSmall:
      return launch_attention_kernel<4, 2, 3, 4>(qpk, kv, qdesc, max_qtiles, heads, out, out_f32, lse, s);
    case kAttnLean4:
      return launch_lean<4, 3, kAttnLean4>(qpk, kv, qdesc, max_qtiles, heads, out, out_f32, lse, s, tail);
    case kAttnLean8:
      return launch_lean<8, 4, kAttnLean8>(qpk, kv, qdesc, max_qtiles, heads, out, out_f32, lse, s, tail);
  }
  return hipErrorInvalidValue;
}

}  // namespace vt
