// bf16 GEMM on the gfx950 matrix cores: C[M,N] = A[M,K] B[N,K]^T (+ bias,
// + epilogue), fp32 accumulation.  A holds tokens (activations, row-major),
// B holds a PyTorch Linear weight [out, in]; both are K-contiguous, which is
// the operand layout v_mfma_f32_32x32x16_bf16 reads (8 consecutive k per
// lane).  The MFMA "A" operand is the weight tile and the "B" operand the
// token tile, so each lane ends with one token and 4 runs of 4 consecutive
// output features: epilogue stores are 8-byte (bf16) or 16-byte (fp32).
//
// Two kernels.  gemm_dl_kernel (K a multiple of 32, every GEMM of the
// blocks and the projector) copies tiles global -> LDS directly; it is
// described where it is defined.  gemm_kernel handles any K (the patch
// embedding, K = 1176): 256 threads = 4 wavefronts in a 2x2 grid over a
// BM x BN tile, K stepped by 64, tiles staged global -> registers -> LDS
// (rows padded by 16 bytes so that the 16-byte fragment reads of 16
// consecutive rows hit distinct banks), double buffered, one barrier per
// K step.
//
// Epilogues (the bias/GELU/residual work of the blocks and the projector,
// MiniMax-M3-Vision README Architecture table): bf16 out, GELU(tanh|erf) bf16
// out, fp32 residual update in place, fp32 out.  Split-K writes fp32 partial
// tiles to the workspace and a second kernel sums them in split order (no
// atomics: results are deterministic).
#include <algorithm>
#include <type_traits>

#include "vt_device.h"
#include "vt_kernels.h"

namespace vt {

constexpr int kBK = 64;
constexpr int kLdsRow = kBK + 8;  // bf16 elements per LDS row (128 B data + 16 B pad)

template <int EPI>
__device__ __forceinline__ void epi_store4(void* out, int64_t off, float v0, float v1, float v2,
                                           float v3) {
  if constexpr (EPI == kEpiResid) {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + off);
    float4 r = *p;
    r.x += v0; r.y += v1; r.z += v2; r.w += v3;
    *p = r;
  } else if constexpr (EPI == kEpiF32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + off) = make_float4(v0, v1, v2, v3);
  } else {
    if constexpr (EPI == kEpiGeluTanh) {
      v0 = gelu_tanh(v0); v1 = gelu_tanh(v1); v2 = gelu_tanh(v2); v3 = gelu_tanh(v3);
    } else if constexpr (EPI == kEpiGeluErf) {
      v0 = gelu_erf(v0); v1 = gelu_erf(v1); v2 = gelu_erf(v2); v3 = gelu_erf(v3);
    }
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + off) =
        make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
  }
}

// SPLIT: write raw fp32 partial sums of K range [z*kper, (z+1)*kper) to
// part[z][M][N]; bias and epilogue are applied by splitk_reduce_kernel.
template <int BM, int BN, int EPI, bool SPLIT>
__global__ void __launch_bounds__(256) gemm_kernel(const uint16_t* __restrict__ A, int M, int K,
                                                   const uint16_t* __restrict__ B, int N,
                                                   const uint16_t* __restrict__ bias,
                                                   void* __restrict__ out,
                                                   float* __restrict__ part, int kper) {
  constexpr int WM = BM / 2, WN = BN / 2;  // per-wave tile (tokens x features)
  constexpr int TB = WM / 32, FB = WN / 32;
  constexpr int AV = BM * 8 / 256, BV = BN * 8 / 256;  // 16-byte vectors per thread
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* sA = lds;                          // [2][BM][kLdsRow]
  uint16_t* sB = lds + 2 * BM * kLdsRow;       // [2][BN][kLdsRow]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (N + BN - 1) / BN;
  const int pid = blockIdx.x;
  const int m0 = (pid / tiles_n) * BM, n0 = (pid % tiles_n) * BN;
  const int kbeg = SPLIT ? blockIdx.y * kper : 0;
  const int kend = SPLIT ? min(K, kbeg + kper) : K;
  const int nk = (kend - kbeg + kBK - 1) / kBK;

  uint4 ra[AV], rb[BV];
  auto gload = [&](int k0) {
#pragma unroll
    for (int v = 0; v < AV; ++v) {
      const int idx = tid + 256 * v, r = idx >> 3, c = (idx & 7) * 8;
      const int gr = m0 + r, gk = k0 + c;
      ra[v] = (gr < M && gk < kend)
                  ? *reinterpret_cast<const uint4*>(A + int64_t(gr) * K + gk)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int idx = tid + 256 * v, r = idx >> 3, c = (idx & 7) * 8;
      const int gr = n0 + r, gk = k0 + c;
      rb[v] = (gr < N && gk < kend)
                  ? *reinterpret_cast<const uint4*>(B + int64_t(gr) * K + gk)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int v = 0; v < AV; ++v) {
      const int idx = tid + 256 * v, r = idx >> 3, c = (idx & 7) * 8;
      *reinterpret_cast<uint4*>(sA + (buf * BM + r) * kLdsRow + c) = ra[v];
    }
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int idx = tid + 256 * v, r = idx >> 3, c = (idx & 7) * 8;
      *reinterpret_cast<uint4*>(sB + (buf * BN + r) * kLdsRow + c) = rb[v];
    }
  };

  f32x16_t acc[FB][TB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][t][e] = 0.f;

  const int fr = lane & 31, fk = (lane >> 5) * 8;
  if (nk > 0) {
    gload(kbeg);
    lstore(0);
  }
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    if (it + 1 < nk) gload(kbeg + (it + 1) * kBK);
    const uint16_t* a_base = sA + (buf * BM + wm * WM + fr) * kLdsRow + fk;
    const uint16_t* b_base = sB + (buf * BN + wn * WN + fr) * kLdsRow + fk;
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      bf16x8_t bw[FB], at[TB];
#pragma unroll
      for (int f = 0; f < FB; ++f)
        bw[f] = *reinterpret_cast<const bf16x8_t*>(b_base + f * 32 * kLdsRow + kk);
#pragma unroll
      for (int t = 0; t < TB; ++t)
        at[t] = *reinterpret_cast<const bf16x8_t*>(a_base + t * 32 * kLdsRow + kk);
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int t = 0; t < TB; ++t)
          acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[f], at[t], acc[f][t], 0, 0, 0);
    }
    if (it + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  acc[f][t][4g + r] = C[token][feature] with
  // token = tile row wm*WM + 32t + lane%32, feature = wn*WN + 32f + 8g + 4(lane/32) + r.
  const int h = lane >> 5;
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int tok = m0 + wm * WM + t * 32 + fr;
    if (tok >= M) continue;
#pragma unroll
    for (int f = 0; f < FB; ++f) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn * WN + f * 32 + g * 8 + h * 4;
        if (col >= N) continue;
        float v0 = acc[f][t][4 * g + 0], v1 = acc[f][t][4 * g + 1];
        float v2 = acc[f][t][4 * g + 2], v3 = acc[f][t][4 * g + 3];
        if constexpr (SPLIT) {
          *reinterpret_cast<float4*>(part + (int64_t(blockIdx.y) * M + tok) * N + col) =
              make_float4(v0, v1, v2, v3);
        } else {
          if (bias) {
            const uint2 bb = *reinterpret_cast<const uint2*>(bias + col);
            v0 += bflo(bb.x); v1 += bfhi(bb.x); v2 += bflo(bb.y); v3 += bfhi(bb.y);
          }
          epi_store4<EPI>(out, int64_t(tok) * N + col, v0, v1, v2, v3);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Direct-load variant (K a multiple of 32): tiles go from global memory
// straight into LDS with global_load_lds_dwordx4 (gfx950), so no VGPRs stage
// them and three K steps stay in flight while one is multiplied.  Lane i of
// a load instruction lands at LDS base + 16 i, so the layout is chosen by
// which global chunk each lane fetches: XOR-swizzled rows (swz4 below) keep
// the MFMA fragment reads free of bank conflicts without padding.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs; block
// b is remapped so that each XCD runs a contiguous range of tiles, walked in
// groups of 4 tile rows (GROUP_M): the ~32 tiles an XCD runs at once share
// 4 activation panels and 8 weight panels through its L2.
// Tile of linear index pid: groups of GM tile rows, walked column by column.
__device__ __forceinline__ void group_tile(int pid, int tiles_m, int tiles_n, int* tm, int* tn) {
  constexpr int GM = 4;
  const int per_group = GM * tiles_n;
  const int gid = pid / per_group, first = gid * GM;
  const int gsz = min(tiles_m - first, GM);
  const int in_g = pid - gid * per_group;
  *tm = first + in_g % gsz;
  *tn = in_g / gsz;
}
// Linear tile index of block b when npid tiles are spread over the 8 XCDs as
// contiguous ranges (block b runs on XCD b mod 8).
__device__ __forceinline__ int xcd_pid(int npid, int b) {
  const int q = npid / 8, r = npid % 8, x = b % 8, l = b / 8;
  return (x < r) ? x * (q + 1) + l : r * (q + 1) + (x - r) * q + l;
}

// 64-byte rows (K step 32 = 4 chunks of 16 B): logical chunk c of row r
// lives in physical chunk c ^ swz4(r), a function of r mod 16 chosen so that
// 16 aligned consecutive rows read at one logical chunk fall in 16 distinct
// 16-byte bank groups (64 banks) and any 8 aligned rows in 8 (32 banks).
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// LDS layout of one K step of gemm_dl_kernel: BM rows of A, then BN rows of
// B, 2 BK bytes each, copied in groups of 1 KB (one copy instruction).
constexpr int dl_stage_bytes(int bm, int bn, int bk) { return (bm + bn) * 2 * bk; }

// Chunk swizzle of the LDS rows: 64-byte rows (BK = 32) use swz4; 128-byte
// rows (8 chunks) use (r mod 8) ^ bit 3 of r, so that 8 aligned consecutive
// rows read at one logical chunk fall in 8 distinct 16-byte bank groups and
// 16 aligned rows (two per 128-byte bank line) in 16.
template <int BK>
__device__ __forceinline__ int dl_swz(int r) {
  if constexpr (BK == 32) return swz4(r);
  else return (r & 7) ^ ((r >> 3) & 1);
}

// Token rows of the C tile staged per epilogue pass: BM halved until a pass
// fits the LDS ring.
constexpr int pass_rows(int bm, int row_bytes, int ring) {
  int r = bm;
  while (r > 1 && r * row_bytes > ring) r /= 2;
  return r;
}

// ---- the QKV Linear with the attention's pack step as its epilogue
// Output tile columns -> W_qkv rows.  The q and k parts (features [0, 2d))
// are read pair-major: tile column c of a BN-wide tile covers rotation pair
// p = (tile start)/2 + c mod BN/2 of its part, its first half (x_j, j = p mod
// 40 of head p / 40) for c < BN/2 and its partner x_{j+40} otherwise, so both
// halves of every pair are in one tile.  v columns keep their order.
template <int BN>
__device__ __forceinline__ int qkv_feature(int n, int d) {
  if (n >= 2 * d) return n;
  const int part = n >= d;
  const int local = n - part * d;
  const int c = local % BN, p = (local - c) / 2 + c % (BN / 2);
  return part * d + (p / 40) * 80 + p % 40 + 40 * (c / (BN / 2));
}

// Store phase of the pack epilogue: the tile (bias added, rounded to bf16,
// staged row-major in LDS as for a bf16 output) leaves as rotated fp16 Q
// rows, rotated fp16 K rows of the tile images, or fp16 V^T columns of the
// tile images.  q/k: one item per (row, chunk of 8 pairs) -- the two halves
// are chunks q and BN/16 + q of the row, rotated with the position of the
// chunk's axis (rope8_f16, the pack kernel's arithmetic).  v: lane = token
// row within a group of 64, so a store instruction writes one V^T row's
// slots; two adjacent columns (dims of one head) per LDS read.
template <int BN, int ROWS, int NT>
__device__ __forceinline__ void qkv_pack_store(const char* cs, const QkvPack& pk, int r0, int M, int n0,
                                               int tid) {
  constexpr int ROWB = BN * 2, CHUNKS = ROWB / 16;
  constexpr int IMG = kAttnTileBytes / 2, KOFF = kAttnKTile * kAttnKRow;  // in fp16 units
  const int d = pk.d;
  if (n0 < 2 * d) {
    const int part = n0 >= d;
    const int p0 = (n0 - part * d) / 2;
    constexpr int QCH = BN / 16;
    const float sc = part == 0 ? pk.q_scale : 1.0f;
    for (int i = tid; i < ROWS * QCH; i += NT) {
      const int r = i / QCH, q = i % QCH;
      const int tok = r0 + r;
      if (tok >= M) continue;
      const uint4 a = *reinterpret_cast<const uint4*>(cs + r * ROWB + ((q + (r & 15)) % CHUNKS) * 16);
      const uint4 b = *reinterpret_cast<const uint4*>(cs + r * ROWB + ((QCH + q + (r & 15)) % CHUNKS) * 16);
      const int p = p0 + 8 * q, head = p / 40, j0 = p % 40;
      const int ax = (pk.axis_code >> (2 * (j0 >> 3))) & 3;
      const int ps = min(max(pk.pos[3 * tok + ax], 0), pk.n_pos - 1);
      const float4* cs4 = reinterpret_cast<const float4*>(pk.rope + int64_t(ps) * 40 + j0);
      float csv[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v = cs4[j];
        csv[4 * j] = v.x; csv[4 * j + 1] = v.y; csv[4 * j + 2] = v.z; csv[4 * j + 3] = v.w;
      }
      uint4 o1, o2;
      rope8_f16(a, b, csv, sc, &o1, &o2);
      uint16_t* dst;
      if (part == 0) {
        dst = pk.qpk + (int64_t(tok) * pk.heads + head) * 80 + j0;
      } else {
        const int ks = pk.kslot[tok];
        dst = pk.kv + (int64_t(ks >> 6) * pk.heads + head) * IMG + (ks & 63) * kAttnKRow + j0;
      }
      *reinterpret_cast<uint4*>(dst) = o1;
      *reinterpret_cast<uint4*>(dst + 40) = o2;
    }
  } else {
    constexpr int RG = ROWS / 64, NWAVE = NT / 64, CSTEP = 2 * NWAVE / RG;
    static_assert(ROWS % 64 == 0 && NWAVE % RG == 0, "V store groups");
    const int wave = tid >> 6, lane = tid & 63;
    const int r = (wave % RG) * 64 + lane, tok = r0 + r;
    if (tok < M) {
      const int ks = pk.kslot[tok];
      uint16_t* vb = pk.kv + int64_t(ks >> 6) * pk.heads * IMG + KOFF + mfma_slot16(ks & 63);
      const int f0 = n0 - 2 * d;
      for (int c = 2 * (wave / RG); c < BN; c += CSTEP) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(
            cs + r * ROWB + (((c >> 3) + (r & 15)) % CHUNKS) * 16 + (c & 7) * 2);
        const int f = f0 + c, head = f / 80, dim = f % 80;  // dims dim, dim + 1 of one head
        uint16_t* v = vb + int64_t(head) * IMG + dim * kAttnVRow;
        v[0] = __builtin_bit_cast(uint16_t, (_Float16)bflo(w));
        v[kAttnVRow] = __builtin_bit_cast(uint16_t, (_Float16)bfhi(w));
      }
    }
  }
}

// GWM x GWN multiplying wavefronts, each owning a (BM/GWM) x (BN/GWN) block
// of C, plus CW wavefronts that only copy (and help store the tile).
// K is consumed in steps of BK (32 or 64) through a ring of NST LDS stages,
// one workgroup barrier per step.  BK = 32: 64-byte rows, NST - 1 steps in
// flight while one is multiplied.  BK = 64: 128-byte rows (a copy reads whole
// 128-byte lines), each step multiplied as two halves of 32 with the barrier
// between them, NST - 1 steps in flight.  The finished tile is staged through
// the (then idle) ring so that every global store writes whole 16-byte pieces
// of contiguous rows.
//
// SK (stream-K tail, with SPLIT): the grid is ts.sk_wgs workgroups that share
// the K steps of the tiles past the first ts.n_whole evenly: workgroup k takes
// positions [k T / S, (k+1) T / S) of the T = (tiles - n_whole) x (K / BK)
// (tile, K step) pairs, tile after tile -- at most two pieces, since a range
// is no longer than one tile's steps -- and writes each piece's raw fp32 sums
// to record k (its first piece) or S + k (its second), BM x BN floats each;
// streamk_reduce_kernel adds a tile's pieces in K order and applies the
// epilogue.  (plan_gemm cuts only where every range is one aligned piece, so
// records S.. are not used and the workspace holds S.)
template <int BM, int BN, int GWM, int GWN, int NST, int EPI, bool SPLIT, int BK = 32, int CW = 0,
          bool SK = false, bool SR = false, bool CO = false>
__global__ void __launch_bounds__(64 * (GWM * GWN + CW)) gemm_dl_kernel(
    const uint16_t* __restrict__ A, int M, int K, const uint16_t* __restrict__ B, int N,
    const uint16_t* __restrict__ bias, void* __restrict__ out, float* __restrict__ part, int kper,
    QkvPack pk, TileSched ts) {
  static_assert(!SK || (SPLIT && BK == 32 && CW == 0), "the stream-K tail writes partial sums");
  constexpr int NW = GWM * GWN;  // wavefronts that multiply
  constexpr int NWC = NW + CW;   // all wavefronts (they all store the finished tile)
  // CO: only the CW copy-only wavefronts issue the K loop's copies.  A
  // wavefront stalls ~100 cycles per 1 KB copy instruction it issues; with one
  // multiplying wavefront per SIMD, stalls of its own leave the matrix unit idle.
  constexpr int NCP = CO ? CW : NWC;  // wavefronts that issue copies
  static_assert(!CO || (CW > 0 && !SK && !SR), "copy-only issue");
  constexpr int WM = BM / GWM, WN = BN / GWN;
  constexpr int TB = WM / 32, FB = WN / 32;
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(CW == 0 || BK == 64, "copy-only wavefronts with K steps of 64 only");
  constexpr int RB = 2 * BK, CH = RB / 16, RPG = 1024 / RB;  // row bytes, chunks per row, rows per copy
  // Copy groups of one K step (RPG rows, 1 KB, one copy instruction): BM/RPG
  // of A, then BN/RPG of B; group g is copied by copying wavefront g % NCP, so
  // the first G % NCP of them copy one group more (CP_HI against CP_LO) when G
  // is not a multiple of NCP.  A wavefront issues copies at a limited rate
  // (~21 GB/s each, up to ~140 GB/s per CU from 8 wavefronts), so tiles with
  // 4 multiplying wavefronts add CW = 4 that only copy.
  constexpr int GA = BM / RPG, G = (BM + BN) / RPG;
  constexpr int CP_HI = (G + NCP - 1) / NCP, CP_LO = G / NCP;
  constexpr int A_BYTES = BM * RB, STAGE = dl_stage_bytes(BM, BN, BK);
  // SR (split ring, K steps of 64): the A and B parts of a step have slots of
  // their own, 2 for A and 3 for B; step s's A lives in slot s mod 2 and its
  // B in slot s mod 3, so B (the weights, which may come from HBM) is copied
  // two steps ahead and A (activations, usually in L2) one step ahead.
  constexpr int B_BYTES = BN * RB, RING = SR ? 2 * A_BYTES + 3 * B_BYTES : NST * STAGE;
  constexpr int CPA = GA / NCP, CPB = (G - GA) / NCP;  // SR: A and B copies per wavefront per step
  static_assert(!SR || (BK == 64 && CW == 0 && !SK && GA % NCP == 0 && (G - GA) % NCP == 0), "split ring");
  static_assert(WM % 32 == 0 && WN % 32 == 0 && BM % 16 == 0 && BN % 16 == 0, "tiling");
  static_assert(RING <= 160 * 1024, "LDS");
  static_assert(SR || NST >= 3, "ring depth");
  extern __shared__ __align__(16) uint16_t lds[];
  const char* smem = reinterpret_cast<const char*>(lds);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;

  // Stream-K tail: this workgroup's range of (tail tile, K step) positions.
  const int nks = K / BK;
  int sk_lo = 0, sk_hi = 0, sk_pos = 0;
  if constexpr (SK) {
    const int64_t T = int64_t(tiles_m * tiles_n - ts.n_whole) * nks;
    sk_lo = int(int64_t(blockIdx.x) * T / ts.sk_wgs);
    sk_hi = int(int64_t(blockIdx.x + 1) * T / ts.sk_wgs);
    sk_pos = sk_lo;
  }
  for (int piece = 0;; ++piece) {
  int tm, tn, kbeg, kend, slot = 0;
  if constexpr (SK) {
    if (sk_pos >= sk_hi) break;
    const int u = sk_pos / nks, s0 = sk_pos - u * nks, s1 = min(nks, s0 + (sk_hi - sk_pos));
    group_tile(ts.n_whole + u, tiles_m, tiles_n, &tm, &tn);
    kbeg = s0 * BK;
    kend = s1 * BK;
    slot = sk_pos == sk_lo ? int(blockIdx.x) : ts.sk_wgs + int(blockIdx.x);
    sk_pos += s1 - s0;
    if (piece > 0) __syncthreads();  // the previous piece's epilogue is done with the LDS
  } else {
    if (piece > 0) break;
    if (BM == 128 && BN == 128 && ts.tail_of >= 0) {
      // Quadrant blockIdx.x % 4 of 256 x 256 tile tail_of + blockIdx.x / 4
      // (in that tiling's order); quadrants wholly past M or N have no work.
      int t2m, t2n;
      group_tile(ts.tail_of + int(blockIdx.x >> 2), (M + 255) / 256, (N + 255) / 256, &t2m, &t2n);
      tm = 2 * t2m + int((blockIdx.x >> 1) & 1);
      tn = 2 * t2n + int(blockIdx.x & 1);
      if (tm * BM >= M || tn * BN >= N) return;
    } else {
      group_tile(xcd_pid(ts.npid, blockIdx.x), tiles_m, tiles_n, &tm, &tn);
    }
    kbeg = SPLIT ? blockIdx.y * kper : 0;
    kend = SPLIT ? min(K, kbeg + kper) : K;
  }
  // With pieces, lane quantities are formed anew for each (tid passes
  // through an empty asm statement), so that nothing lane-dependent is
  // hoisted above the piece loop and kept live across the whole kernel.
  int tid = threadIdx.x;
  if constexpr (SK) asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const bool mw = CW == 0 || wave < NW;  // a multiplying wavefront
  // Copy-only wavefronts issue at raised priority: the copies set the pace
  // of these tiles, and each shares its SIMD with one multiplying wavefront
  // (FC1 at 1,024 tokens: 22.3 -> 21.9 us; scheduling only, same bits).
  if (!mw) __builtin_amdgcn_s_setprio(1);
  const int wm = wave / GWN, wn = wave % GWN;
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = (kend - kbeg) / BK;

  // Copy j of this lane: group g = cw + NCP j (cw: the wavefront's index among
  // the copying ones), i.e. row RPG g + lane / CH of
  // the stage (an A row while g < GA, else B row RPG (g - GA) + lane / CH),
  // logical chunk (lane % CH) ^ swz(row), landing in physical chunk lane % CH
  // of LDS bytes 1024 g + RB (lane / CH) of the stage.  Rows past M (N) read
  // the last valid row; their results are never stored.
  const int lq = lane / CH;
  const int cw = CO ? max(wave - NW, 0) : wave;  // index among the copying wavefronts
  const bool hi = cw < G % NCP;  // copies CP_HI groups (else CP_LO)
  const uint16_t* src[CP_HI];
#pragma unroll
  for (int j = 0; j < CP_HI; ++j) {
    const int g = min(cw + NCP * j, G - 1);
    const int lchunk = (lane % CH) ^ dl_swz<BK>(RPG * g + lq);
    int brow = min(n0 + RPG * (g - GA) + lq, N - 1);
    if constexpr (EPI == kEpiQkvPack) brow = qkv_feature<BN>(brow, pk.d);
    src[j] = g < GA ? A + int64_t(min(m0 + RPG * g + lq, M - 1)) * K + kbeg + 8 * lchunk
                    : B + int64_t(brow) * K + kbeg + 8 * lchunk;
  }
  const uint32_t lds0 = lds_offset(lds) + 1024 * cw;

  auto issue = [&](int it) {
    if (CO && mw) return;  // the multiplying wavefronts issue no copies
    const uint32_t sa = __builtin_amdgcn_readfirstlane(lds0 + (it % NST) * STAGE);
#pragma unroll
    for (int j = 0; j < CP_LO; ++j) dma16(src[j] + it * BK, sa + 1024 * NCP * j);
    if constexpr (CP_HI > CP_LO)
      if (hi) dma16(src[CP_LO] + it * BK, sa + 1024 * NCP * CP_LO);
  };
  // Split ring: copy j < CPA of every wavefront is an A group, the rest B.
  auto issue_a = [&](int it) {
    const uint32_t sa = __builtin_amdgcn_readfirstlane(lds0 + (it % 2) * A_BYTES);
#pragma unroll
    for (int j = 0; j < CPA; ++j) dma16(src[j] + it * BK, sa + 1024 * NCP * j);
  };
  auto issue_b = [&](int it) {
    const uint32_t sb = __builtin_amdgcn_readfirstlane(lds0 + 2 * A_BYTES + (it % 3) * B_BYTES - 1024 * GA);
#pragma unroll
    for (int j = CPA; j < CPA + CPB; ++j) dma16(src[j] + it * BK, sb + 1024 * NCP * j);
  };
  // vmcnt <= the copies of the newest `steps` issued steps.
  auto wait_steps = [&](auto steps) {
    constexpr int n = decltype(steps)::value;
    if constexpr (CP_HI > CP_LO) {
      if (hi) wait_vmcnt<n * CP_HI>();
      else wait_vmcnt<n * CP_LO>();
    } else {
      wait_vmcnt<n * CP_LO>();
    }
  };
  using None = std::integral_constant<int, 0>;

  f32x16_t acc[FB][TB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][t][e] = 0.f;

  const int fr = lane & 31, h = lane >> 5;
  const int sw = dl_swz<BK>(fr);
  // bf16-output epilogues of the 128 x 128 and 128 x 160 tiles: this lane's
  // bias values (features 32f + 8g + 4h .. + 3 of its wavefront's columns),
  // loaded before the K loop so that their latency is hidden behind it (the
  // wider tiles have no registers to spare and load them in the epilogue).
  constexpr bool F32OUT = SPLIT || EPI == kEpiResid || EPI == kEpiF32;
  constexpr bool PRE = !F32OUT && BM == 128 && BN <= 160;
  // Bias element of output column n (and the 3 after it): the W_qkv row read
  // for it in the pack epilogue (4 consecutive columns are 4 consecutive
  // features there too), else n itself.
  auto bias_col = [&](int n) {
    if constexpr (EPI == kEpiQkvPack) return qkv_feature<BN>(n, pk.d);
    else return min(n, N - 4);
  };
  uint2 bpre[PRE ? FB : 1][4];
  if constexpr (PRE) {
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        bpre[f][g] = (bias && mw) ? *reinterpret_cast<const uint2*>(
                                        bias + bias_col(n0 + wn * WN + 32 * f + 8 * g + 4 * h))
                                  : make_uint2(0, 0);
  }

  // Fragments of 32 of K (two MFMA k slices of 16): half u of step `step`
  // (u = 0 for BK = 32).  Slice q of half u is logical chunk 4u + 2q + h.
  struct Frags {
    bf16x8_t w0[FB], t0[TB], w1[FB], t1[TB];
  };
  auto load_frags = [&](Frags& F, int step, int u) {
    const char* st = smem + (step % NST) * STAGE;
    const char* a_base = (SR ? smem + (step % 2) * A_BYTES : st) + (wm * WM + fr) * RB;
    const char* b_base = (SR ? smem + 2 * A_BYTES + (step % 3) * B_BYTES : st + A_BYTES) + (wn * WN + fr) * RB;
    const int choff0 = 16 * ((4 * u + h) ^ sw), choff1 = 16 * ((4 * u + 2 + h) ^ sw);
#pragma unroll
    for (int f = 0; f < FB; ++f) F.w0[f] = *reinterpret_cast<const bf16x8_t*>(b_base + f * 32 * RB + choff0);
#pragma unroll
    for (int t = 0; t < TB; ++t) F.t0[t] = *reinterpret_cast<const bf16x8_t*>(a_base + t * 32 * RB + choff0);
#pragma unroll
    for (int f = 0; f < FB; ++f) F.w1[f] = *reinterpret_cast<const bf16x8_t*>(b_base + f * 32 * RB + choff1);
#pragma unroll
    for (int t = 0; t < TB; ++t) F.t1[t] = *reinterpret_cast<const bf16x8_t*>(a_base + t * 32 * RB + choff1);
  };
  auto mma = [&](const Frags& F) {
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int t = 0; t < TB; ++t)
        acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.w0[f], F.t0[t], acc[f][t], 0, 0, 0);
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int t = 0; t < TB; ++t)
        acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.w1[f], F.t1[t], acc[f][t], 0, 0, 0);
  };
  // The MFMAs of one half interleaved with the next half's fragment reads.
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < 2 * (FB + TB); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * FB * TB - 2 * (FB + TB), 0);
  };

  if constexpr (SR) {
    // As the BK = 64 ring below, with A_{it+1} and B_{it+2} issued at the
    // start of step it (A first), into the slots of A_{it-1} and B_{it-1},
    // whose reads were done at step it-1's barrier.  At step it's barrier
    // everything but B_{it+2} must have landed: vmcnt <= CPB.
    issue_a(0);
    issue_b(0);
    if (1 < nk) issue_b(1);
    if (nk > 0) {
      if (1 < nk) wait_vmcnt<CPB>();  // step 0 landed
      else wait_vmcnt<0>();
      wg_barrier();
      Frags F0, F1;
      load_frags(F0, 0, 0);
      for (int it = 0; it < nk; ++it) {
        if (it + 1 < nk) issue_a(it + 1);
        if (it + 2 < nk) issue_b(it + 2);
        load_frags(F1, it, 1);
        mma(F0);
        interleave();
        if (it + 2 < nk) wait_vmcnt<CPB>();
        else wait_vmcnt<0>();
        wait_lds_reads();
        wg_barrier();
        load_frags(F0, it + 1, 0);  // on the last step a stale, never used slot
        mma(F1);
        interleave();
      }
      wait_lds_reads();
      wg_barrier();
    }
  } else if constexpr (BK == 32) {
    using InFlight = std::integral_constant<int, NST - 3>;
    // One K step: copies for step it+NST-1 go out, step it+1's fragments are
    // read while step it's are multiplied; then step it+2's copies must have
    // landed (by every wave) before the next step reads them.
    // The fragment reads are unconditional (on the last step they read a
    // stale, never used stage): a branch around them makes the compiler wait
    // for every outstanding LDS read before the first MFMA of the step.
    auto step = [&](int it, const Frags& cur, Frags& nxt) {
      if (it + NST - 1 < nk) issue(it + NST - 1);  // into the stage step it-1 used
      load_frags(nxt, it + 1, 0);
      mma(cur);
      interleave();
      if (it + NST - 1 < nk) wait_steps(InFlight{});  // step it+2 has landed
      else wait_steps(None{});
      wait_lds_reads();
      wg_barrier();
    };

#pragma unroll
    for (int i = 0; i < NST - 1; ++i)
      if (i < nk) issue(i);
    if (nk > 0) {
      if (NST - 1 < nk) wait_steps(InFlight{});  // steps 0 and 1 landed
      else wait_steps(None{});
      wg_barrier();
      Frags F0, F1;
      load_frags(F0, 0, 0);
      int it = 0;
      for (; it + 1 < nk; it += 2) {
        step(it, F0, F1);
        step(it + 1, F1, F0);
      }
      if (it < nk) step(it, F0, F1);
    }
  } else {
    using InFlight = std::integral_constant<int, NST - 2>;
#pragma unroll
    for (int i = 0; i < NST - 1; ++i)
      if (i < nk) issue(i);
    if (nk > 0) {
      if (NST - 1 <= nk) wait_steps(InFlight{});  // step 0 landed
      else wait_steps(None{});
      wg_barrier();
      Frags F0, F1;
      if (mw) load_frags(F0, 0, 0);
      for (int it = 0; it < nk; ++it) {
        // First half of step it.  The copies for step it+NST-1 go into the
        // stage of step it-1, whose last reads (its second half) came before
        // the previous barrier.
        if (it + NST - 1 < nk) issue(it + NST - 1);
        if (mw) {
          load_frags(F1, it, 1);
          mma(F0);
          interleave();
        }
        // Step it+1 must have landed (by every wave) before the second half
        // reads its first fragments; the barrier also releases step it's
        // stage, all of whose reads are done.
        if (it + NST - 1 < nk) wait_steps(InFlight{});
        else wait_steps(None{});
        wait_lds_reads();
        wg_barrier();
        // Second half of step it (on the last step the read is of a stale,
        // never used stage).
        if (mw) {
          load_frags(F0, it + 1, 0);
          mma(F1);
          interleave();
        }
      }
      // The epilogue reuses the ring: every wave's reads must be done.
      wait_lds_reads();
      wg_barrier();
    }
  }

  // ---- epilogue.  acc[f][t][4g + r] = C[token][feature] with token =
  // wm*WM + 32t + lane%32 and feature = wn*WN + 32f + 8g + 4(lane/32) + r.
  // Bias and the activation are applied in registers; the tile is written
  // row-major into LDS (16-byte chunk c of row r at chunk (c + r % 16) mod
  // CHUNKS, which spreads the 32 rows one write instruction touches over the
  // banks), then
  // every thread moves whole 16-byte chunks to global memory, PASS_ROWS token
  // rows at a time.  The ring is idle: the last step waited for every copy
  // and, at its barrier, for every wave's fragment reads.
  constexpr int ESZ = F32OUT ? 4 : 2;
  constexpr int ROWB = BN * ESZ, CHUNKS = ROWB / 16, EPC = 16 / ESZ;
  constexpr int PASS_ROWS = pass_rows(BM, ROWB, RING);
  static_assert(CHUNKS >= 16 && PASS_ROWS % WM == 0 && BM % PASS_ROWS == 0, "epilogue staging");
  char* cs = reinterpret_cast<char*>(lds);
#pragma unroll
  for (int pass = 0; pass < BM / PASS_ROWS; ++pass) {
    if (pass > 0) __syncthreads();  // the previous pass's reads are done
    if (mw && wm * WM / PASS_ROWS == pass) {
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        const int r = wm * WM + 32 * t + fr - pass * PASS_ROWS;
#pragma unroll
        for (int f = 0; f < FB; ++f) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v0 = acc[f][t][4 * g + 0], v1 = acc[f][t][4 * g + 1];
            float v2 = acc[f][t][4 * g + 2], v3 = acc[f][t][4 * g + 3];
            const int c = (wn * WN + 32 * f + 8 * g) / EPC;  // logical chunk of feature 8g
            if constexpr (F32OUT) {
              // 4 fp32 = one chunk; h selects the next chunk
              const int pc = (c + h + (r & 15)) % CHUNKS;
              *reinterpret_cast<float4*>(cs + r * ROWB + pc * 16) = make_float4(v0, v1, v2, v3);
            } else {
              if (bias) {
                uint2 bb;
                if constexpr (PRE) bb = bpre[f][g];
                else bb = *reinterpret_cast<const uint2*>(bias + bias_col(n0 + wn * WN + 32 * f + 8 * g + 4 * h));
                v0 += bflo(bb.x); v1 += bfhi(bb.x); v2 += bflo(bb.y); v3 += bfhi(bb.y);
              }
              if constexpr (EPI == kEpiGeluTanh) {
                v0 = gelu_tanh(v0); v1 = gelu_tanh(v1); v2 = gelu_tanh(v2); v3 = gelu_tanh(v3);
              } else if constexpr (EPI == kEpiGeluErf) {
                v0 = gelu_erf(v0); v1 = gelu_erf(v1); v2 = gelu_erf(v2); v3 = gelu_erf(v3);
              }
              const int pc = (c + (r & 15)) % CHUNKS;
              *reinterpret_cast<uint2*>(cs + r * ROWB + pc * 16 + 8 * h) =
                  make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
            }
          }
        }
      }
    }
    __syncthreads();
    constexpr int TOTAL = PASS_ROWS * CHUNKS;
    constexpr int PER = (TOTAL + 64 * NWC - 1) / (64 * NWC);  // chunks per thread per pass
    if constexpr (EPI == kEpiQkvPack) {
      qkv_pack_store<BN, PASS_ROWS, 64 * NWC>(cs, pk, m0 + pass * PASS_ROWS, M, n0, tid);
      continue;
    }
    if constexpr (EPI == kEpiResid && !SPLIT) {
      // Residual update: every old value this thread needs is loaded first,
      // so the loads are in flight together rather than one store apart.
      float4 old[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = tid + j * 64 * NWC;
        const int r = i / CHUNKS, c = i % CHUNKS;
        const int tok = m0 + pass * PASS_ROWS + r, col = n0 + c * EPC;
        if (i < TOTAL && tok < M && col < N)
          old[j] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(out) +
                                                    int64_t(tok) * N + col);
      }
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = tid + j * 64 * NWC;
        const int r = i / CHUNKS, c = i % CHUNKS;
        const int tok = m0 + pass * PASS_ROWS + r, col = n0 + c * EPC;
        if (i >= TOTAL || tok >= M || col >= N) continue;
        float4 a = *reinterpret_cast<const float4*>(cs + r * ROWB + ((c + (r & 15)) % CHUNKS) * 16);
        if (bias) {
          const uint2 bb = *reinterpret_cast<const uint2*>(bias + col);
          a.x += bflo(bb.x); a.y += bfhi(bb.x); a.z += bflo(bb.y); a.w += bfhi(bb.y);
        }
        a.x = old[j].x + a.x; a.y = old[j].y + a.y; a.z = old[j].z + a.z; a.w = old[j].w + a.w;
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + int64_t(tok) * N + col) = a;
      }
      continue;
    }
#pragma unroll
    for (int i = tid; i < TOTAL; i += 64 * NWC) {
      const int r = i / CHUNKS, c = i % CHUNKS;
      const int tok = m0 + pass * PASS_ROWS + r, col = n0 + c * EPC;
      if (tok >= M || col >= N) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(cs + r * ROWB + ((c + (r & 15)) % CHUNKS) * 16);
      if constexpr (SK) {
        *reinterpret_cast<uint4*>(part + (int64_t(slot) * BM + (tok - m0)) * BN + (col - n0)) = v;
      } else if constexpr (SPLIT) {
        *reinterpret_cast<uint4*>(part + (int64_t(blockIdx.y) * M + tok) * N + col) = v;
      } else if constexpr (EPI == kEpiResid || EPI == kEpiF32) {
        float4 a = __builtin_bit_cast(float4, v);
        if (bias) {
          const uint2 bb = *reinterpret_cast<const uint2*>(bias + col);
          a.x += bflo(bb.x); a.y += bfhi(bb.x); a.z += bflo(bb.y); a.w += bfhi(bb.y);
        }
        float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + int64_t(tok) * N + col);
        if constexpr (EPI == kEpiResid) {
          const float4 r0 = *o;
          a.x += r0.x; a.y += r0.y; a.z += r0.z; a.w += r0.w;
        }
        *o = a;
      } else {
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + int64_t(tok) * N + col) = v;
      }
    }
  }
  }  // pieces
}

// out = epilogue(sum_z part[z] + bias), summed in split order.  The loads of
// up to 4 partials are issued together (indices clamped to the last split,
// so they stay in bounds) before the valid ones are added in order.
template <int EPI>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int M, int N,
                                                            const uint16_t* __restrict__ bias,
                                                            void* __restrict__ out) {
  const int64_t n4 = int64_t(M) * N / 4;
  const float4* p4 = reinterpret_cast<const float4*>(part);
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += int64_t(gridDim.x) * blockDim.x) {
    float4 s = p4[i];
    for (int z0 = 1; z0 < splits; z0 += 4) {
      float4 q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) q[j] = p4[int64_t(min(z0 + j, splits - 1)) * n4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (z0 + j < splits) { s.x += q[j].x; s.y += q[j].y; s.z += q[j].z; s.w += q[j].w; }
    }
    const int64_t off = i * 4;
    if (bias) {
      const int col = int(off % N);
      const uint2 bb = *reinterpret_cast<const uint2*>(bias + col);
      s.x += bflo(bb.x); s.y += bfhi(bb.x); s.z += bflo(bb.y); s.w += bfhi(bb.y);
    }
    epi_store4<EPI>(out, off, s.x, s.y, s.z, s.w);
  }
}

// out = epilogue(sum of the pieces + bias) for the tiles of a stream-K tail:
// block (i, u) takes float4 i of tail tile u (tile n_whole + u); the tile's
// pieces are those of the tail workgroups whose ranges meet its K steps
// [u nks, (u+1) nks), added in K order (deterministic).
template <int EPI, int BM, int BN>
__global__ void __launch_bounds__(256) streamk_reduce_kernel(const float* __restrict__ part, int M, int N,
                                                             int nks, TileSched ts,
                                                             const uint16_t* __restrict__ bias,
                                                             void* __restrict__ out) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int u = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= BM * BN / 4) return;
  const int r = idx / (BN / 4), c = 4 * (idx % (BN / 4));
  int tm, tn;
  group_tile(ts.n_whole + u, tiles_m, tiles_n, &tm, &tn);
  const int tok = tm * BM + r, col = tn * BN + c;
  if (tok >= M || col >= N) return;
  const int64_t T = int64_t(tiles_m * tiles_n - ts.n_whole) * nks;
  const int64_t P0 = int64_t(u) * nks;
  // The tail workgroup whose range holds position p: the largest k with k T / S <= p.
  auto wg_of = [&](int64_t p) { return int(((p + 1) * ts.sk_wgs - 1) / T); };
  const int kA = wg_of(P0), kB = wg_of(P0 + nks - 1);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = kA; k <= kB; ++k) {
    const int64_t klo = int64_t(k) * T / ts.sk_wgs;
    const int slot = klo >= P0 ? k : ts.sk_wgs + k;
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t(slot) * BM + r) * BN + c);
    if (k == kA) acc = v;
    else { acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w; }
  }
  if (bias) {
    const uint2 bb = *reinterpret_cast<const uint2*>(bias + col);
    acc.x += bflo(bb.x); acc.y += bfhi(bb.x); acc.z += bflo(bb.y); acc.w += bfhi(bb.y);
  }
  epi_store4<EPI>(out, int64_t(tok) * N + col, acc.x, acc.y, acc.z, acc.w);
}

// Tiles of a 256 x 256 tiling's partial last round to run as 128 x 128
// quadrants instead (0: none): a last round of at most half the CUs' tiles.
// Its quadrants (up to 512 workgroups, two per CU) take well under a whole
// tile's time: O at 16,384 tokens (64 tail tiles) 99.9 -> 81.3 us, QKV-shaped
// 34,852 x 3840 x 1280 (7) 383 -> 361 us; fuller last rounds were slower
// this way (173 of 256: 170 -> 189 us), so they keep whole tiles.
static int tail_quadrant_tiles(int t256, int K) {
  constexpr int kCUs = 256, kMaxTail = 128;
  if (t256 <= kCUs || K % 32 != 0) return 0;
  const int n_tail = t256 % kCUs;
  return n_tail <= kMaxTail ? n_tail : 0;
}

GemmPlan plan_gemm(int M, int N, int K) {
  auto cdiv = [](long a, long b) { return int((a + b - 1) / b); };
  GemmPlan p{256, 256, 1, K};
  const int t256 = cdiv(M, 256) * cdiv(N, 256);
  if (t256 >= 192) {
    // One 256 x 256 workgroup per CU.  Past whole rounds of the 256 CUs, a
    // partial last round would leave CUs idle for a whole tile's time; with
    // long K (the residual FC2 and the projector's wide Linears) its tiles'
    // K steps are shared over the CUs instead.  Only when the tail tiles
    // divide the CUs, so that every workgroup takes one aligned piece of one
    // tile (16 x 448x448: 64 tiles in quarters): cut points that fall inside
    // workgroup ranges (two pieces each, 2 x 256 KB of partial sums per
    // workgroup) measured slower than the idle CUs at 2016x2016.
    constexpr int kCUs = 256;
    if (t256 > kCUs && t256 % kCUs != 0 && K >= 2048 && K % 32 == 0) {
      const int n_whole = t256 / kCUs * kCUs, n_tail = t256 - n_whole, nks = K / 32;
      if (kCUs % n_tail == 0 && nks >= 8 * (kCUs / n_tail)) {
        p.n_whole = n_whole;
        p.sk_wgs = kCUs;
      }
    }
    if (p.sk_wgs == 0) {
      p.tail128 = tail_quadrant_tiles(t256, K);
      if (p.tail128 > 0) p.n_whole = t256 - p.tail128;
    }
    return p;
  }
  if (M <= 512 && K % 32 == 0) {
    // Few rows, large weights (the merged MLP of a small image): 256 x 256
    // tiles read each weight panel once; split K to fill the CUs.
    const int sp = std::min(256 / t256, K / 512);
    if (t256 * sp >= 192) {
      p.kper = cdiv(cdiv(K, sp), 64) * 64;
      p.splits = cdiv(K, p.kper);
      return p;
    }
  }
  p.bm = 128;
  p.bn = 128;
  const int tm = cdiv(M, 128);
  const int t128 = tm * cdiv(N, 128);
  if (t128 > 256 && K % 32 == 0) {
    // One round of wider tiles when N allows it (e.g. 1024 x 5120: 8 x 32 tiles of 128 x 160).
    for (int bn : {160, 192})
      if (N % bn == 0 && tm * (N / bn) <= 256 && K % 64 == 0) {
        p.bn = bn;
        return p;
      }
    return p;
  }
  if (t128 >= 200) return p;
  // Split K so that the workgroups fill the 256 CUs once (one round), each
  // split keeping at least 384 of K.
  int splits = 256 / t128;
  const int max_splits = K / 384;
  if (splits > max_splits) splits = max_splits;
  if (splits > 1) {
    p.splits = splits;
    p.kper = cdiv(cdiv(K, splits), kBK) * kBK;
    p.splits = cdiv(K, p.kper);
  }
  return p;
}

size_t gemm_workspace_bytes(int M, int N, int K) {
  const GemmPlan p = plan_gemm(M, N, K);
  if (p.sk_wgs > 0) return size_t(p.sk_wgs) * p.bm * p.bn * sizeof(float);  // one piece per workgroup
  return p.splits > 1 ? size_t(p.splits) * M * N * sizeof(float) : 0;
}

template <int BM, int BN, int EPI, bool SPLIT, int BK, bool SK = false>
static hipError_t launch_dl(const uint16_t* A, int M, int K, const uint16_t* B, int N,
                            const uint16_t* bias, void* out, float* part, const GemmPlan& p,
                            int tiles, hipStream_t s, const QkvPack& pk = QkvPack{}, int tail_of = -1) {
  // 256 x 256: 8 wavefronts (2 per SIMD) of 128 x 64; 128 x 128: 8 of 32 x 64;
  // 128 x 160 and 128 x 192: 4 of 32 x BN (one per SIMD) plus 4 that issue
  // every copy of the K loop (CO).  K steps of 32 go through 4 stages, K steps
  // of 64 through 3.
  constexpr int GWM = (BM == 256) ? 2 : 4, GWN = (BM == 256) ? 4 : (BN == 128 ? 2 : 1);
  constexpr int CW = (BK == 64 && GWM * GWN == 4) ? 4 : 0;
  constexpr bool CO = CW > 0;
  constexpr int NST = BK == 64 ? 3 : 4;
  // 256 x 256 with K steps of 64: the split ring (2 A + 3 B slots, 160 KB).
  constexpr bool SR = BM == 256 && BN == 256 && BK == 64;
  const size_t lds = SR ? size_t(2 * BM + 3 * BN) * 2 * BK : size_t(NST) * dl_stage_bytes(BM, BN, BK);
  auto kern = gemm_dl_kernel<BM, BN, GWM, GWN, NST, EPI, SPLIT, BK, CW, SK, SR, CO>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (attr != hipSuccess) return attr;
  // tiles: the blocks of the launch (the stream-K tail: its sk_wgs workgroups)
  const TileSched ts{tiles, p.n_whole, p.sk_wgs, tail_of};
  hipLaunchKernelGGL(kern, dim3(tiles, (SPLIT && !SK) ? p.splits : 1), dim3(64 * (GWM * GWN + CW)), lds, s,
                     A, M, K, B, N, bias, out, part, p.kper, pk, ts);
  return hipGetLastError();
}

template <int BM, int BN, int EPI, bool SPLIT>
static hipError_t launch_tile(const uint16_t* A, int M, int K, const uint16_t* B, int N,
                              const uint16_t* bias, void* out, float* part, const GemmPlan& p,
                              hipStream_t s) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const auto k_step_ok = [&](int bk) { return K % bk == 0 && (!SPLIT || p.kper % bk == 0); };
  if constexpr (BN == 160 || BN == 192) {
    // The wide tiles are planned only for one round of workgroups, K % 64 == 0.
    if (!k_step_ok(64)) return hipErrorInvalidValue;
    return launch_dl<BM, BN, EPI, SPLIT, 64>(A, M, K, B, N, bias, out, part, p, tiles, s);
  } else {
    // 128 x 128 in one round of workgroups: K steps of 64 (96 KB of LDS, one
    // workgroup per CU).  More rounds: K steps of 32 (64 KB, two per CU).
    // 256 x 256: K steps of 64 through the split ring (whole 128-byte lines
    // per copy, the weights two steps ahead).
    if constexpr (BM == 128)
      if (tiles * (SPLIT ? p.splits : 1) <= 256 && k_step_ok(64))
        return launch_dl<BM, BN, EPI, SPLIT, 64>(A, M, K, B, N, bias, out, part, p, tiles, s);
    if constexpr (BM == 256)
      if (k_step_ok(64)) return launch_dl<BM, BN, EPI, SPLIT, 64>(A, M, K, B, N, bias, out, part, p, tiles, s);
    if (k_step_ok(32))
      return launch_dl<BM, BN, EPI, SPLIT, 32>(A, M, K, B, N, bias, out, part, p, tiles, s);
    const size_t lds = size_t(2) * (BM + BN) * kLdsRow * sizeof(uint16_t);
    auto kern = gemm_kernel<BM, BN, EPI, SPLIT>;
    // Set once per instantiation (thread-safe static initialisation).
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3(tiles, SPLIT ? p.splits : 1), dim3(256), lds, s, A, M, K, B, N,
                       bias, out, part, p.kper);
    return hipGetLastError();
  }
}

// The first `tiles` 256 x 256 tiles, no split: K steps of 64 (split ring)
// when K allows, else 32.
template <int EPI>
static hipError_t launch_whole256(const uint16_t* A, int M, int K, const uint16_t* B, int N, const uint16_t* bias,
                                  void* out, const GemmPlan& p, int tiles, hipStream_t s,
                                  const QkvPack& pk = QkvPack{}) {
  if (K % 64 == 0) return launch_dl<256, 256, EPI, false, 64>(A, M, K, B, N, bias, out, nullptr, p, tiles, s, pk);
  return launch_dl<256, 256, EPI, false, 32>(A, M, K, B, N, bias, out, nullptr, p, tiles, s, pk);
}

// The first n_whole tiles of a 256 x 256 tiling whole, then its last
// n_tail tiles as four 128 x 128 quadrants each: one round of one workgroup
// per CU (K steps of 64) when the quadrants fit it, else two per CU.
template <int EPI>
static hipError_t launch_whole_then_quadrants(const uint16_t* A, int M, int K, const uint16_t* B, int N,
                                              const uint16_t* bias, void* out, const GemmPlan& p, int n_whole,
                                              int n_tail, hipStream_t s, const QkvPack& pk = QkvPack{}) {
  hipError_t e = launch_whole256<EPI>(A, M, K, B, N, bias, out, p, n_whole, s, pk);
  if (e != hipSuccess) return e;
  const GemmPlan q{128, 128, 1, K};
  if (4 * n_tail <= 256 && K % 64 == 0)
    return launch_dl<128, 128, EPI, false, 64>(A, M, K, B, N, bias, out, nullptr, q, 4 * n_tail, s, pk, n_whole);
  return launch_dl<128, 128, EPI, false, 32>(A, M, K, B, N, bias, out, nullptr, q, 4 * n_tail, s, pk, n_whole);
}

template <int EPI>
static hipError_t launch_epi(const uint16_t* A, int M, int K, const uint16_t* B, int N,
                             const uint16_t* bias, void* out, void* ws, hipStream_t s) {
  const GemmPlan p = plan_gemm(M, N, K);
  if (p.splits > 1) {
    float* part = reinterpret_cast<float*>(ws);
    hipError_t e = p.bm == 256 ? launch_tile<256, 256, EPI, true>(A, M, K, B, N, bias, out, part, p, s)
                               : launch_tile<128, 128, EPI, true>(A, M, K, B, N, bias, out, part, p, s);
    if (e != hipSuccess) return e;
    const int64_t n4 = int64_t(M) * N / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3(unsigned(blocks)), dim3(256), 0, s, part,
                       p.splits, M, N, bias, out);
    return hipGetLastError();
  }
  if (p.bm == 256 && p.sk_wgs > 0) {
    // whole rounds, then the tail's K steps over sk_wgs workgroups, then the
    // tail tiles' sums and epilogue
    float* part = reinterpret_cast<float*>(ws);
    hipError_t e = launch_whole256<EPI>(A, M, K, B, N, bias, out, p, p.n_whole, s);
    if (e != hipSuccess) return e;
    e = launch_dl<256, 256, kEpiF32, true, 32, true>(A, M, K, B, N, nullptr, nullptr, part, p, p.sk_wgs, s);
    if (e != hipSuccess) return e;
    const int n_tail = ((M + 255) / 256) * ((N + 255) / 256) - p.n_whole;
    const TileSched ts{0, p.n_whole, p.sk_wgs};
    hipLaunchKernelGGL((streamk_reduce_kernel<EPI, 256, 256>), dim3(256 * 256 / 4 / 256, n_tail), dim3(256), 0, s,
                       part, M, N, K / 32, ts, bias, out);
    return hipGetLastError();
  }
  if (p.bm == 256 && p.tail128 > 0)
    return launch_whole_then_quadrants<EPI>(A, M, K, B, N, bias, out, p, p.n_whole, p.tail128, s);
  if (p.bm == 256) return launch_tile<256, 256, EPI, false>(A, M, K, B, N, bias, out, nullptr, p, s);
  if (p.bn == 160) return launch_tile<128, 160, EPI, false>(A, M, K, B, N, bias, out, nullptr, p, s);
  if (p.bn == 192) return launch_tile<128, 192, EPI, false>(A, M, K, B, N, bias, out, nullptr, p, s);
  return launch_tile<128, 128, EPI, false>(A, M, K, B, N, bias, out, nullptr, p, s);
}

hipError_t launch_gemm(const uint16_t* A, int M, int K, const uint16_t* B, int N,
                       const uint16_t* bias, int epi, void* out, void* ws, hipStream_t s) {
  switch (epi) {
    case kEpiBf16: return launch_epi<kEpiBf16>(A, M, K, B, N, bias, out, ws, s);
    case kEpiGeluTanh: return launch_epi<kEpiGeluTanh>(A, M, K, B, N, bias, out, ws, s);
    case kEpiGeluErf: return launch_epi<kEpiGeluErf>(A, M, K, B, N, bias, out, ws, s);
    case kEpiResid: return launch_epi<kEpiResid>(A, M, K, B, N, bias, out, ws, s);
    case kEpiF32: return launch_epi<kEpiF32>(A, M, K, B, N, bias, out, ws, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_qkv_pack(const uint16_t* A, int M, int K, const uint16_t* B, const uint16_t* bias,
                                const QkvPack& pk, hipStream_t s) {
  // 256 x 256 tiles when they fill the chip (as plan_gemm), else 128 x 128;
  // never split-K (the epilogue needs whole sums).  Both tile widths divide d.
  const int N = 3 * pk.d;
  if (K % 32 || pk.d % 256) return hipErrorInvalidValue;
  auto cdiv = [](long a, long b) { return int((a + b - 1) / b); };
  const GemmPlan p{128, 128, 1, K};
  const int t256 = cdiv(M, 256) * cdiv(N, 256);
  if (t256 >= 192) {
    const int n_tail = tail_quadrant_tiles(t256, K);
    if (n_tail > 0)
      return launch_whole_then_quadrants<kEpiQkvPack>(A, M, K, B, N, bias, nullptr, p, t256 - n_tail, n_tail, s,
                                                      pk);
    return launch_whole256<kEpiQkvPack>(A, M, K, B, N, bias, nullptr, p, t256, s, pk);
  }
  const int t128 = cdiv(M, 128) * cdiv(N, 128);
  if (t128 <= 256 && K % 64 == 0)
    return launch_dl<128, 128, kEpiQkvPack, false, 64>(A, M, K, B, N, bias, nullptr, nullptr, p, t128, s, pk);
  return launch_dl<128, 128, kEpiQkvPack, false, 32>(A, M, K, B, N, bias, nullptr, nullptr, p, t128, s, pk);
}

hipError_t launch_gemm_partials(const uint16_t* A, int M, int K, const uint16_t* B, int N, void* ws,
                                hipStream_t s) {
  const GemmPlan p = plan_gemm(M, N, K);
  if (p.splits < 2) return hipErrorInvalidValue;
  float* part = reinterpret_cast<float*>(ws);
  return p.bm == 256 ? launch_tile<256, 256, kEpiResid, true>(A, M, K, B, N, nullptr, nullptr, part, p, s)
                     : launch_tile<128, 128, kEpiResid, true>(A, M, K, B, N, nullptr, nullptr, part, p, s);
}

}  // namespace vt
