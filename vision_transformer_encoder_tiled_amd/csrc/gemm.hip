// bf16 GEMM on the gfx950 matrix cores: C[M,N] = A[M,K] B[N,K]^T (+ bias,
// + epilogue), fp32 accumulation.  A holds tokens (activations, row-major),
// B holds a PyTorch Linear weight [out, in]; both are K-contiguous, which is
// the operand layout v_mfma_f32_32x32x16_bf16 reads (8 consecutive k per
// lane).  The MFMA "A" operand is the weight tile and the "B" operand the
// token tile, so each lane ends with one token and 4 runs of 4 consecutive
// output features: epilogue stores are 8-byte (bf16) or 16-byte (fp32).
//
// Workgroup: 256 threads = 4 wavefronts in a 2x2 grid over a BM x BN tile,
// K stepped by 64.  Tiles go global -> registers -> LDS (rows padded by 16
// bytes so that the 16-byte fragment reads of 16 consecutive rows hit
// distinct banks), double buffered, one barrier per K step.
//
// Epilogues (the bias/GELU/residual work of the blocks and the projector,
// MiniMax-M3-Vision README Architecture table): bf16 out, GELU(tanh|erf) bf16
// out, fp32 residual update in place, fp32 out.  Split-K writes fp32 partial
// tiles to the workspace and a second kernel sums them in split order (no
// atomics: results are deterministic).
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
// Direct-load variant (K a multiple of 64): tiles go from global memory
// straight into LDS with global_load_lds_dwordx4 (gfx950), so no VGPRs stage
// them and the next K tile's loads stay in flight while the current one is
// multiplied.  Lane i of a load instruction lands at LDS base + 16 i, so the
// layout is chosen by which global chunk each lane fetches: rows of 64 bf16
// (128 B, 8 chunks of 16 B) with logical chunk c of row r stored at
// physical chunk c ^ swz(r), swz(r) = (r' ^ r' >> 3) & 7 with r' = r mod 16.
// Sixteen aligned consecutive rows read at one logical chunk then hit 16
// distinct 16-byte bank groups (and any 8 aligned rows 8 distinct ones), so
// the MFMA fragment reads are conflict-free without padding.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs; block
// b is remapped so that each XCD runs a contiguous range of tiles, walked in
// groups of 4 tile rows (GROUP_M): the ~32 tiles an XCD runs at once share
// 4 activation panels and 8 weight panels through its L2.
// Swizzle of row r: a function of r mod 16 only, so it is unchanged by the
// 32- and 64-row steps between a lane's copies and between fragment blocks.
__device__ __forceinline__ int swz(int r) { return ((r & 15) ^ ((r & 15) >> 3)) & 7; }

// s_waitcnt immediate: vmcnt <= n, expcnt and lgkmcnt unconstrained (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until this wavefront's LDS reads have returned (lgkmcnt = 0; vmcnt and
// expcnt unconstrained).  Needed before the barrier that releases a stage for
// overwriting: the compiler may otherwise consume the last fragment reads
// (and so wait for them) only after the barrier.
__device__ __forceinline__ void wait_lds_reads() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_sched_barrier(0);
}

// LDS byte offset of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// One 16-byte global -> LDS copy per lane: lane i writes LDS [lds + 16 i].
// Issued as inline assembly so the compiler does not treat every later LDS
// read as dependent on it (it cannot tell the two pipeline stages apart and
// would wait for all outstanding copies); completion is awaited explicitly
// with wait_vmcnt before the workgroup barrier that publishes a stage.  The
// instruction has no register result; the address VGPRs are read at issue.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ void xcd_group_tile(int tiles_m, int tiles_n, int* tm, int* tn) {
  const int G = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int q = G / 8, r = G % 8, x = b % 8, l = b / 8;
  const int pid = (x < r) ? x * (q + 1) + l : r * (q + 1) + (x - r) * q + l;
  constexpr int GM = 4;
  const int per_group = GM * tiles_n;
  const int gid = pid / per_group, first = gid * GM;
  const int gsz = min(tiles_m - first, GM);
  const int in_g = pid - gid * per_group;
  *tm = first + in_g % gsz;
  *tn = in_g / gsz;
}

// GWM x GWN wavefronts; each owns a (BM/GWM) x (BN/GWN) block of C.
template <int BM, int BN, int GWM, int GWN, int EPI, bool SPLIT>
__global__ void __launch_bounds__(64 * GWM * GWN) gemm_dl_kernel(
    const uint16_t* __restrict__ A, int M, int K, const uint16_t* __restrict__ B, int N,
    const uint16_t* __restrict__ bias, void* __restrict__ out, float* __restrict__ part, int kper) {
  constexpr int NW = GWM * GWN;
  constexpr int WM = BM / GWM, WN = BN / GWN;
  constexpr int TB = WM / 32, FB = WN / 32;
  constexpr int LA = BM / (8 * NW), LB = BN / (8 * NW);  // copies per lane per K tile
  constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
  static_assert(WM % 32 == 0 && WN % 32 == 0 && LA * 8 * NW == BM && LB * 8 * NW == BN, "tiling");
  extern __shared__ __align__(16) uint16_t lds[];
  const char* smem = reinterpret_cast<const char*>(lds);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / GWN, wn = wave % GWN;
  int tm, tn;
  xcd_group_tile((M + BM - 1) / BM, (N + BN - 1) / BN, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = SPLIT ? blockIdx.y * kper : 0;
  const int kend = SPLIT ? min(K, kbeg + kper) : K;
  const int nk = (kend - kbeg) / 64;

  // Copy j of this lane: row 8 (wave + NW j) + lane / 8 of the tile, logical
  // chunk (lane % 8) ^ swz(row) -- it lands in physical chunk lane % 8 (row
  // steps of 8 NW keep swz(row) fixed).  Rows past M (N) read the last valid
  // row; their results are never stored.
  const int lrow = 8 * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ swz(lrow);
  const uint16_t* ga = A + int64_t(min(m0 + lrow, M - 1)) * K + kbeg + 8 * lchunk;
  const uint16_t* gb = B + int64_t(min(n0 + lrow, N - 1)) * K + kbeg + 8 * lchunk;
  int64_t oa[LA], ob[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j)
    oa[j] = int64_t(min(m0 + lrow + 8 * NW * j, M - 1) - min(m0 + lrow, M - 1)) * K;
#pragma unroll
  for (int j = 0; j < LB; ++j)
    ob[j] = int64_t(min(n0 + lrow + 8 * NW * j, N - 1) - min(n0 + lrow, N - 1)) * K;
  const uint32_t lds0 = lds_offset(lds) + 1024 * wave;

  auto issue = [&](int it, int stage) {
    const uint32_t sa = __builtin_amdgcn_readfirstlane(lds0 + stage * STAGE);
#pragma unroll
    for (int j = 0; j < LA; ++j) dma16(ga + oa[j] + it * 64, sa + 1024 * NW * j);
#pragma unroll
    for (int j = 0; j < LB; ++j) dma16(gb + ob[j] + it * 64, sa + A_BYTES + 1024 * NW * j);
  };

  f32x16_t acc[FB][TB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][t][e] = 0.f;

  const int fr = lane & 31, h = lane >> 5;
  const int sw = swz(fr);
  int choff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) choff[kk] = 16 * ((2 * kk + h) ^ sw);

  if (nk > 0) issue(0, 0);
  for (int it = 0; it < nk; ++it) {
    const int stage = it & 1;
    if (it + 1 < nk) {
      issue(it + 1, stage ^ 1);
      wait_vmcnt<LA + LB>();  // this lane's copies of tile `it` have landed
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();  // ... and every other lane's
    const char* a_base = smem + stage * STAGE + (wm * WM + fr) * 128;
    const char* b_base = smem + stage * STAGE + A_BYTES + (wn * WN + fr) * 128;
    bf16x8_t bw[2][FB], at[2][TB];
#pragma unroll
    for (int f = 0; f < FB; ++f) bw[0][f] = *reinterpret_cast<const bf16x8_t*>(b_base + f * 4096 + choff[0]);
#pragma unroll
    for (int t = 0; t < TB; ++t) at[0][t] = *reinterpret_cast<const bf16x8_t*>(a_base + t * 4096 + choff[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      if (kk < 3) {
#pragma unroll
        for (int f = 0; f < FB; ++f)
          bw[nxt][f] = *reinterpret_cast<const bf16x8_t*>(b_base + f * 4096 + choff[kk + 1]);
#pragma unroll
        for (int t = 0; t < TB; ++t)
          at[nxt][t] = *reinterpret_cast<const bf16x8_t*>(a_base + t * 4096 + choff[kk + 1]);
      }
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int t = 0; t < TB; ++t)
          acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[cur][f], at[cur][t], acc[f][t], 0, 0, 0);
      if (kk < 3) {
        // interleave the next step's fragment reads with this step's MFMAs
#pragma unroll
        for (int i = 0; i < FB + TB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FB * TB - FB - TB, 0);
      }
    }
    wait_lds_reads();
    __builtin_amdgcn_s_barrier();  // stage `it` may now be overwritten
  }

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

// out = epilogue(sum_z part[z] + bias), summed in split order.
template <int EPI>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int M, int N,
                                                            const uint16_t* __restrict__ bias,
                                                            void* __restrict__ out) {
  const int64_t n4 = int64_t(M) * N / 4;
  const int64_t plane = int64_t(M) * N;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t off = i * 4;
    float4 s = *reinterpret_cast<const float4*>(part + off);
    for (int z = 1; z < splits; ++z) {
      const float4 p = *reinterpret_cast<const float4*>(part + z * plane + off);
      s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
    }
    if (bias) {
      const int col = int(off % N);
      const uint2 bb = *reinterpret_cast<const uint2*>(bias + col);
      s.x += bflo(bb.x); s.y += bfhi(bb.x); s.z += bflo(bb.y); s.w += bfhi(bb.y);
    }
    epi_store4<EPI>(out, off, s.x, s.y, s.z, s.w);
  }
}

GemmPlan plan_gemm(int M, int N, int K) {
  auto cdiv = [](long a, long b) { return int((a + b - 1) / b); };
  GemmPlan p{256, 256, 1, K};
  const int t256 = cdiv(M, 256) * cdiv(N, 256);
  if (t256 >= 192) return p;
  p.bm = 128;
  p.bn = 128;
  const int t128 = cdiv(M, 128) * cdiv(N, 128);
  if (t128 >= 200) return p;
  int splits = cdiv(256, t128);
  const int max_splits = K / 512;
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
  return p.splits > 1 ? size_t(p.splits) * M * N * sizeof(float) : 0;
}

template <int BM, int BN, int EPI, bool SPLIT>
static hipError_t launch_tile(const uint16_t* A, int M, int K, const uint16_t* B, int N,
                              const uint16_t* bias, void* out, float* part, const GemmPlan& p,
                              hipStream_t s) {
  if (K % 64 == 0) {
    // 256 x 256 tiles: 8 wavefronts (2 per SIMD, 128 x 64 each); 128 x 128: 4 (64 x 64 each)
    constexpr int GWM = 2, GWN = (BM == 256) ? 4 : 2;
    const size_t lds = size_t(2) * (BM + BN) * 128;
    auto kern = gemm_dl_kernel<BM, BN, GWM, GWN, EPI, SPLIT>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (attr != hipSuccess) return attr;
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3(tiles, SPLIT ? p.splits : 1), dim3(64 * GWM * GWN), lds, s, A, M,
                       K, B, N, bias, out, part, p.kper);
    return hipGetLastError();
  }
  const size_t lds = size_t(2) * (BM + BN) * kLdsRow * sizeof(uint16_t);
  auto kern = gemm_kernel<BM, BN, EPI, SPLIT>;
  // Set once per instantiation (thread-safe static initialisation).
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (attr != hipSuccess) return attr;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3(tiles, SPLIT ? p.splits : 1), dim3(256), lds, s, A, M, K, B, N,
                     bias, out, part, p.kper);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_epi(const uint16_t* A, int M, int K, const uint16_t* B, int N,
                             const uint16_t* bias, void* out, void* ws, hipStream_t s) {
  const GemmPlan p = plan_gemm(M, N, K);
  if (p.splits > 1) {
    float* part = reinterpret_cast<float*>(ws);
    hipError_t e = launch_tile<128, 128, EPI, true>(A, M, K, B, N, bias, out, part, p, s);
    if (e != hipSuccess) return e;
    const int64_t n4 = int64_t(M) * N / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3(unsigned(blocks)), dim3(256), 0, s, part,
                       p.splits, M, N, bias, out);
    return hipGetLastError();
  }
  if (p.bm == 256) return launch_tile<256, 256, EPI, false>(A, M, K, B, N, bias, out, nullptr, p, s);
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

}  // namespace vt
