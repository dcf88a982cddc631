// Element-wise and row kernels of one block's backward pass ("v2_loaders
// FINDINGS", section 3: the towers are differentiable).  The products of the
// backward pass run on the forward's GEMM, C = A B^T with both operands
// K-contiguous:
//   dX = dY W        A = dY [M, out],   B = W^T [in, out]
//   dW = dY^T X      A = dY^T [out, M], B = X^T [in, M]   (K = tokens)
// so activations and weights are transposed here first, in 64 x 64 tiles
// through LDS, with what else the pass needs folded into the same read:
// fp32 -> bf16 conversion, GELU (the recomputed MLP activation) or its
// derivative (dh = du * GELU'(h)), and the column sums that are the bias
// gradients.  The LayerNorm backward is one wavefront per row.
#include <algorithm>

#include "vt_device.h"
#include "vt_kernels.h"

namespace vt {

namespace {
// d/dh of 0.5 h (1 + tanh(u)), u = sqrt(2/pi) (h + 0.044715 h^3):
// 0.5 (1 + t) + 0.5 h (1 - t^2) du/dh, t = tanh(u) = 1 - 2 / (1 + e^(2u)).
__device__ __forceinline__ float gelu_tanh_grad(float h) {
  const float c = 0.7978845608028654f;
  const float u = c * fmaf(0.044715f * h * h, h, h);
  const float e = __builtin_amdgcn_exp2f(fminf(2.0f * 1.4426950408889634f * u, 126.f));
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e);
  const float du = c * fmaf(3.0f * 0.044715f, h * h, 1.0f);
  return 0.5f * (1.0f + t) + 0.5f * h * (1.0f - t * t) * du;
}

template <class T>
__device__ __forceinline__ void load4(const T* p, float* v);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* v) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float* v) {
  const uint2 x = *reinterpret_cast<const uint2*>(p);
  v[0] = bflo(x.x); v[1] = bfhi(x.x); v[2] = bflo(x.y); v[3] = bfhi(x.y);
}
}  // namespace

// One 64 x 64 tile of in [M, C] per block (256 threads; C a multiple of 4,
// the last column tile partial): v = op(in) (op 1: GELU; op 2: in *
// GELU'(aux)), rows M .. Mp-1 read as zero.  Writes, each when its pointer is
// set: copy [M, C] = bf16(v); outT [C, Mp] = bf16(v)^T; colpart[y][c] = the
// sum of bf16(v) over the tile's 64 rows (y = the row tile), summed in order
// by colsum_reduce_kernel, so column sums are reproducible bit for bit.
template <class TIN, int OP>
__global__ void __launch_bounds__(256) transpose_kernel(const TIN* in,
                                                        const uint16_t* __restrict__ aux,
                                                        int32_t M, int32_t C, int32_t Mp,
                                                        uint16_t* copy,
                                                        uint16_t* __restrict__ outT,
                                                        float* __restrict__ colpart) {
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
  const int tid = threadIdx.x, cq = 4 * (tid & 15), rq = tid >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = rq + 16 * r, m = m0 + row;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (m < M && c0 + cq < C) {
      const int64_t off = int64_t(m) * C + c0 + cq;
      load4<TIN>(in + off, v);
      if constexpr (OP == 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = gelu_tanh(v[j]);
      } else if constexpr (OP == 2) {
        float hv[4];
        load4<uint16_t>(aux + off, hv);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] *= gelu_tanh_grad(hv[j]);
      }
      const uint2 b = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      if (copy) *reinterpret_cast<uint2*>(copy + off) = b;
      // the transposed copy carries the same bf16 values as the row copy
      v[0] = bflo(b.x); v[1] = bfhi(b.x); v[2] = bflo(b.y); v[3] = bfhi(b.y);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) tile[row][cq + j] = v[j];
  }
  __syncthreads();
  if (colpart && tid < 64 && c0 + tid < C) {
    float s = 0.f;
    for (int r = 0; r < 64; ++r) s += tile[r][tid];
    colpart[int64_t(blockIdx.y) * C + c0 + tid] = s;
  }
  if (outT && c0 + (tid >> 2) < C) {
    // thread -> (column tid / 4, rows 16 (tid % 4) .. +15): two 16-byte stores
    const int c = tid >> 2, r0 = 16 * (tid & 3);
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = pack_bf16x2(tile[r0 + 2 * j][c], tile[r0 + 2 * j + 1][c]);
    uint4* dst = reinterpret_cast<uint4*>(outT + int64_t(c0 + c) * Mp + m0 + r0);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// LayerNorm backward, one wavefront per row (rows strided over the grid):
//   xh = (x - mean) rstd,  dxh = dy * g,
//   dx = dres + rstd (dxh - mean(dxh) - xh mean(dxh xh)),
//   and per block part[block] = (sum of dy xh, sum of dy) over its rows
//   (per-lane sums, then the 4 wavefronts in order), reduced in block order
//   by colsum_reduce_kernel.
// dx may alias dres (each element is read before it is written, by one lane).
template <int NV>
__global__ void __launch_bounds__(256) ln_backward_kernel(
    const float* __restrict__ x, const uint16_t* __restrict__ g, const float* __restrict__ dy,
    const float* dres, int32_t rows, float eps, float* dx, float* __restrict__ part) {
  constexpr int W = 256 * NV;
  __shared__ float red[2][W];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float gv[NV][4], sg[NV][4], sb[NV][4];
  const uint2* g2 = reinterpret_cast<const uint2*>(g);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint2 gg = g2[lane + 64 * i];
    gv[i][0] = bflo(gg.x); gv[i][1] = bfhi(gg.x); gv[i][2] = bflo(gg.y); gv[i][3] = bfhi(gg.y);
#pragma unroll
    for (int j = 0; j < 4; ++j) sg[i][j] = sb[i][j] = 0.f;
  }
  for (int row = blockIdx.x * 4 + wave; row < rows; row += gridDim.x * 4) {
    const int64_t base = int64_t(row) * W;
    float xv[NV][4], dv[NV][4];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = 4 * (lane + 64 * i);
      load4<float>(x + base + c, xv[i]);
      load4<float>(dy + base + c, dv[i]);
      s += (xv[i][0] + xv[i][1]) + (xv[i][2] + xv[i][3]);
    }
    const float mean = wave_sum(s) * (1.0f / W);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[i][j] -= mean;
        q += xv[i][j] * xv[i][j];
      }
    const float rstd = 1.0f / sqrtf(wave_sum(q) * (1.0f / W) + eps);
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float xh = xv[i][j] * rstd, d = dv[i][j];
        sg[i][j] += d * xh;
        sb[i][j] += d;
        xv[i][j] = xh;
        dv[i][j] = d * gv[i][j];
        a += dv[i][j];
        b += dv[i][j] * xh;
      }
    const float m1 = wave_sum(a) * (1.0f / W), m2 = wave_sum(b) * (1.0f / W);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = 4 * (lane + 64 * i);
      float r[4];
      load4<float>(dres + base + c, r);
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] += rstd * (dv[i][j] - m1 - xv[i][j] * m2);
      *reinterpret_cast<float4*>(dx + base + c) = make_float4(r[0], r[1], r[2], r[3]);
    }
  }
  // The block's 4 wavefronts add their partial sums into LDS in turn.
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 4 * (lane + 64 * i) + j;
          red[0][c] = w ? red[0][c] + sg[i][j] : sg[i][j];
          red[1][c] = w ? red[1][c] + sb[i][j] : sb[i][j];
        }
    }
    __syncthreads();
  }
  float* pb = part + int64_t(blockIdx.x) * 2 * W;
  for (int c = threadIdx.x; c < W; c += 256) {
    pb[c] = red[0][c];
    pb[W + c] = red[1][c];
  }
}

// sum over p < parts of part[p * ld + c]  (c < C) in a fixed order, to
// out[c] for c < split and out2[c - split] beyond: thread group g (of 4) sums
// parts g, g + 4, g + 8, ... in turn, eight loads in flight, and the four
// group sums are added in group order.
__global__ void __launch_bounds__(256) colsum_reduce_kernel(const float* __restrict__ part,
                                                            int32_t parts, int32_t ld, int32_t C,
                                                            float* __restrict__ out, int32_t split,
                                                            float* __restrict__ out2) {
  __shared__ float gs[4][64];
  const int cl = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + cl;
  float s = 0.f;
  if (c < C) {
    int p = g;
    for (; p + 28 < parts; p += 32) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = part[int64_t(p + 4 * j) * ld + c];
#pragma unroll
      for (int j = 0; j < 8; ++j) s += v[j];
    }
    for (; p < parts; p += 4) s += part[int64_t(p) * ld + c];
  }
  gs[g][cl] = s;
  __syncthreads();
  if (g == 0 && c < C) {
    const float v = ((gs[0][cl] + gs[1][cl]) + gs[2][cl]) + gs[3][cl];
    if (c < split) out[c] = v;
    else out2[c - split] = v;
  }
}

// out [C, R] = in [R, C]^T, fp32, 32 x 32 tiles through LDS (any R, C).
__global__ void __launch_bounds__(256) transpose_f32_kernel(const float* __restrict__ in, int32_t R,
                                                            int32_t C, float* __restrict__ out) {
  __shared__ float tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8)
    if (r0 + i < R && c0 + tx < C) tile[i][tx] = in[int64_t(r0 + i) * C + c0 + tx];
  __syncthreads();
  for (int i = ty; i < 32; i += 8)
    if (c0 + i < C && r0 + tx < R) out[int64_t(c0 + i) * R + r0 + tx] = tile[tx][i];
}

hipError_t launch_transpose(const void* in, bool in_f32, int op, const uint16_t* aux, int32_t M,
                            int32_t C, int32_t Mp, uint16_t* copy, uint16_t* outT, float* colsum,
                            float* colpart, hipStream_t s) {
  if (colsum && !colpart) return hipErrorInvalidValue;
  float* cp = colsum ? colpart : nullptr;
  if (C % 4 || Mp % 64 || Mp < M || (in_f32 && op != 0) || op < 0 || op > 2 || (op == 2 && !aux))
    return hipErrorInvalidValue;
  const dim3 grid((C + 63) / 64, Mp / 64);
  if (in_f32)
    hipLaunchKernelGGL((transpose_kernel<float, 0>), grid, dim3(256), 0, s,
                       static_cast<const float*>(in), aux, M, C, Mp, copy, outT, cp);
  else if (op == 0)
    hipLaunchKernelGGL((transpose_kernel<uint16_t, 0>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(in), aux, M, C, Mp, copy, outT, cp);
  else if (op == 1)
    hipLaunchKernelGGL((transpose_kernel<uint16_t, 1>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(in), aux, M, C, Mp, copy, outT, cp);
  else
    hipLaunchKernelGGL((transpose_kernel<uint16_t, 2>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(in), aux, M, C, Mp, copy, outT, cp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !colsum) return e;
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((C + 63) / 64), dim3(256), 0, s, colpart, Mp / 64, C, C,
                     colsum, C, nullptr);
  return hipGetLastError();
}

int ln_backward_blocks(int32_t rows) {
  return int(std::min<int64_t>((int64_t(rows) + 3) / 4, kLnBwdMaxBlocks));
}

hipError_t launch_ln_backward(const float* x, const uint16_t* g, const float* dy, const float* dres,
                              int32_t rows, int32_t width, float eps, float* dx, float* dg,
                              float* db, float* part, hipStream_t s) {
  const int blocks = ln_backward_blocks(rows);
  if (width % 256) return hipErrorInvalidValue;
  switch (width / 256) {
#define VT_LNB_CASE(n)                                                                            \
  case n:                                                                                         \
    hipLaunchKernelGGL(ln_backward_kernel<n>, dim3(blocks), dim3(256), 0, s, x, g, dy, dres, rows, \
                       eps, dx, part);                                                            \
    break;
    VT_LNB_CASE(1) VT_LNB_CASE(2) VT_LNB_CASE(3) VT_LNB_CASE(4) VT_LNB_CASE(5) VT_LNB_CASE(6)
    VT_LNB_CASE(7) VT_LNB_CASE(8)
#undef VT_LNB_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // part is [blocks][2][width]: the gamma sums, then the beta sums, of each block
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((2 * width + 63) / 64), dim3(256), 0, s, part, blocks,
                     2 * width, 2 * width, dg, width, db);
  return hipGetLastError();
}

hipError_t launch_transpose_f32(const float* in, int32_t R, int32_t C, float* out, hipStream_t s) {
  hipLaunchKernelGGL(transpose_f32_kernel, dim3((C + 31) / 32, (R + 31) / 32), dim3(256), 0, s, in, R,
                     C, out);
  return hipGetLastError();
}

}  // namespace vt
