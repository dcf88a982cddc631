// LayerNorm over fp32 rows -> bf16 rows, and the same LayerNorm fused behind
// a split-K residual update.
// Textbook form: biased variance over the row, eps inside the square root,
// then gamma/beta (pre-LN blocks of the tower; eps 1e-6).  Two passes over
// the row held in registers: mean, then the centred sum of squares.  One
// 64-lane wavefront per row, reduced with butterfly shuffles; the fused
// kernel at width 1280 (the tower's) takes one 320-thread workgroup per row.
#include <algorithm>

#include "vt_device.h"
#include "vt_kernels.h"

namespace vt {

// LayerNorm of one row held by a wavefront: v[i] = elements 4(lane + 64 i) .. +3.
// Each sum is taken over the wavefront per i (a float4 sum per lane, then the
// butterfly), and the NV partial sums are added in order of i: the order of
// ln_row320 below, so both give the same bits at width 1280.
template <int NV>
__device__ __forceinline__ void ln_row(float4 (&v)[NV], int lane, const uint16_t* __restrict__ g,
                                       const uint16_t* __restrict__ b, float eps,
                                       uint16_t* __restrict__ out_row) {
  constexpr int W = 256 * NV;
  float sp[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) sp[i] = wave_sum((v[i].x + v[i].y) + (v[i].z + v[i].w));
  float s = sp[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) s += sp[i];
  const float mean = s * (1.0f / W);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i].x -= mean; v[i].y -= mean; v[i].z -= mean; v[i].w -= mean;
    sp[i] = wave_sum((v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w));
  }
  float q = sp[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) q += sp[i];
  const float var = q * (1.0f / W);
  const float rstd = 1.0f / sqrtf(var + eps);
  const uint2* g2 = reinterpret_cast<const uint2*>(g);
  const uint2* b2 = reinterpret_cast<const uint2*>(b);
  uint2* o2 = reinterpret_cast<uint2*>(out_row);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    const uint2 gg = g2[c], bb = b2[c];
    const float y0 = v[i].x * rstd * bflo(gg.x) + bflo(bb.x);
    const float y1 = v[i].y * rstd * bfhi(gg.x) + bfhi(bb.x);
    const float y2 = v[i].z * rstd * bflo(gg.y) + bflo(bb.y);
    const float y3 = v[i].w * rstd * bfhi(gg.y) + bfhi(bb.y);
    o2[c] = make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
  }
}

template <int NV>  // float4 vectors per lane: width = 256 * NV
__global__ void __launch_bounds__(256) layer_norm_kernel(const float* __restrict__ x, int32_t rows,
                                                         const uint16_t* __restrict__ g,
                                                         const uint16_t* __restrict__ b, float eps,
                                                         uint16_t* __restrict__ out) {
  constexpr int W = 256 * NV;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float4* xr = reinterpret_cast<const float4*>(x + int64_t(row) * W);
  float4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = xr[lane + 64 * i];
  ln_row<NV>(v, lane, g, b, eps, out + int64_t(row) * W);
}

// Split-K residual update fused with the next LayerNorm, one wavefront per
// row: R += (sum over z in order of part[z]) + bias, exactly the arithmetic
// of the split-K reduction with the residual epilogue; then out = LN(R).
template <int NV>
__global__ void __launch_bounds__(256) resid_ln_kernel(const float* __restrict__ part,
                                                       int32_t splits, int32_t rows,
                                                       const uint16_t* __restrict__ bias,
                                                       float* __restrict__ R,
                                                       const uint16_t* __restrict__ g,
                                                       const uint16_t* __restrict__ b, float eps,
                                                       uint16_t* __restrict__ out) {
  constexpr int W = 256 * NV;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t plane4 = int64_t(rows) * W / 4;
  float4* rr = reinterpret_cast<float4*>(R + int64_t(row) * W);
  const float4* p0 = reinterpret_cast<const float4*>(part + int64_t(row) * W);
  float4 v[NV], r[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] = p0[lane + 64 * i];
    r[i] = rr[lane + 64 * i];
  }
  // Partials 1.. in groups of 4: the loads of a group are issued together
  // (indices clamped to the last split, so they stay in bounds), then the
  // valid ones are added in split order.
  for (int z0 = 1; z0 < splits; z0 += 4) {
    float4 q[4][NV];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t zz = min(z0 + j, splits - 1);
#pragma unroll
      for (int i = 0; i < NV; ++i) q[j][i] = p0[zz * plane4 + lane + 64 * i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (z0 + j < splits) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          v[i].x += q[j][i].x; v[i].y += q[j][i].y; v[i].z += q[j][i].z; v[i].w += q[j][i].w;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (bias) {
      const uint2 bb = reinterpret_cast<const uint2*>(bias)[c];
      v[i].x += bflo(bb.x); v[i].y += bfhi(bb.x); v[i].z += bflo(bb.y); v[i].w += bfhi(bb.y);
    }
    r[i].x += v[i].x; r[i].y += v[i].y; r[i].z += v[i].z; r[i].w += v[i].w;
    rr[c] = r[i];
    v[i] = r[i];
  }
  ln_row<NV>(v, lane, g, b, eps, out + int64_t(row) * W);
}

// The fused split-K residual update + LayerNorm at width 1280 (the tower's),
// one 320-thread workgroup per row and one float4 column per thread.  The
// split-K path runs only for a few thousand rows at most; there one
// wavefront per row leaves each SIMD too few wavefronts to overlap the
// SPL + 1 loads per element with the two reductions, while five per row
// keep them in flight.  The sums are taken per wavefront, then over the 5
// wavefronts in order: the order of ln_row above, so the fused path and the
// plain LayerNorm give the same bits.
__device__ __forceinline__ void ln_row320(float4 r, int t, const uint16_t* __restrict__ g,
                                          const uint16_t* __restrict__ b, float eps,
                                          uint16_t* __restrict__ out_row, float (&red)[2][5]) {
  constexpr float INV_W = 1.0f / 1280;
  const int lane = t & 63, wave = t >> 6;
  const float s = wave_sum((r.x + r.y) + (r.z + r.w));
  if (lane == 0) red[0][wave] = s;
  __syncthreads();
  const float mean = ((((red[0][0] + red[0][1]) + red[0][2]) + red[0][3]) + red[0][4]) * INV_W;
  r.x -= mean; r.y -= mean; r.z -= mean; r.w -= mean;
  const float qq = wave_sum((r.x * r.x + r.y * r.y) + (r.z * r.z + r.w * r.w));
  if (lane == 0) red[1][wave] = qq;
  __syncthreads();
  const float var = ((((red[1][0] + red[1][1]) + red[1][2]) + red[1][3]) + red[1][4]) * INV_W;
  const float rstd = 1.0f / sqrtf(var + eps);
  const uint2 gg = reinterpret_cast<const uint2*>(g)[t], bt = reinterpret_cast<const uint2*>(b)[t];
  const float y0 = r.x * rstd * bflo(gg.x) + bflo(bt.x);
  const float y1 = r.y * rstd * bfhi(gg.x) + bfhi(bt.x);
  const float y2 = r.z * rstd * bflo(gg.y) + bflo(bt.y);
  const float y3 = r.w * rstd * bfhi(gg.y) + bfhi(bt.y);
  reinterpret_cast<uint2*>(out_row)[t] = make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
}

// Rows are strided over the grid (at most kRowGrid workgroups, so that the
// launch stays far inside the 32-bit thread count); every thread of a
// workgroup walks the same rows, so the barriers inside ln_row320 are met by
// all of them, and the two barriers of one row also order the reuse of red[]
// by the next.
constexpr int32_t kRowGrid = 1 << 20;

// The split-K residual update (the arithmetic of resid_ln_kernel: partials in
// split order, then the bias, then the old R) fused with the next LayerNorm,
// width 1280.  SPL > 0: exactly SPL partials, all loads issued at once (one
// memory round trip); SPL = 0: any count, in groups of 4.
template <int SPL>
__global__ void __launch_bounds__(320) resid_ln_row_kernel(const float* __restrict__ part,
                                                           int32_t splits, int32_t rows,
                                                           const uint16_t* __restrict__ bias,
                                                           float* __restrict__ R,
                                                           const uint16_t* __restrict__ g,
                                                           const uint16_t* __restrict__ b, float eps,
                                                           uint16_t* __restrict__ out) {
  __shared__ float red[2][5];
  const int t = threadIdx.x;
  const int64_t plane4 = int64_t(rows) * 320;
  for (int32_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const float4* p0 = reinterpret_cast<const float4*>(part) + int64_t(row) * 320 + t;
    float4* rr = reinterpret_cast<float4*>(R) + int64_t(row) * 320 + t;
    float4 v = p0[0];
    float4 r = *rr;
    if constexpr (SPL > 0) {
      float4 q[SPL];
#pragma unroll
      for (int z = 1; z < SPL; ++z) q[z] = p0[z * plane4];
#pragma unroll
      for (int z = 1; z < SPL; ++z) { v.x += q[z].x; v.y += q[z].y; v.z += q[z].z; v.w += q[z].w; }
    } else {
      for (int z0 = 1; z0 < splits; z0 += 4) {
        float4 q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = p0[int64_t(min(z0 + j, splits - 1)) * plane4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (z0 + j < splits) { v.x += q[j].x; v.y += q[j].y; v.z += q[j].z; v.w += q[j].w; }
      }
    }
    if (bias) {
      const uint2 bb = reinterpret_cast<const uint2*>(bias)[t];
      v.x += bflo(bb.x); v.y += bfhi(bb.x); v.z += bflo(bb.y); v.w += bfhi(bb.y);
    }
    r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
    *rr = r;
    ln_row320(r, t, g, b, eps, out + int64_t(row) * 1280, red);
  }
}

hipError_t launch_layer_norm(const float* x, int32_t rows, int32_t width, const uint16_t* g,
                             const uint16_t* b, float eps, uint16_t* out, hipStream_t s) {
  const dim3 grid((rows + 3) / 4), block(256);
  switch (width / 256) {
#define VT_LN_CASE(n) \
  case n: hipLaunchKernelGGL(layer_norm_kernel<n>, grid, block, 0, s, x, rows, g, b, eps, out); break;
    VT_LN_CASE(1) VT_LN_CASE(2) VT_LN_CASE(3) VT_LN_CASE(4) VT_LN_CASE(5) VT_LN_CASE(6)
    VT_LN_CASE(7) VT_LN_CASE(8) VT_LN_CASE(9) VT_LN_CASE(10) VT_LN_CASE(11) VT_LN_CASE(12)
    VT_LN_CASE(13) VT_LN_CASE(14) VT_LN_CASE(15) VT_LN_CASE(16)
#undef VT_LN_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_resid_ln(const float* part, int32_t splits, int32_t rows, int32_t width,
                           const uint16_t* bias, float* R, const uint16_t* g, const uint16_t* b,
                           float eps, uint16_t* out, hipStream_t s) {
  const dim3 grid((rows + 3) / 4), block(256);
  if (width == 1280) {  // the tower's width: a workgroup per row
    const dim3 rgrid(std::min(rows, kRowGrid)), rblock(320);
    switch (splits) {
#define VT_RLN_ROW(k, n)                                                                             \
  case k:                                                                                            \
    hipLaunchKernelGGL(resid_ln_row_kernel<n>, rgrid, rblock, 0, s, part, splits, rows, bias, R, g, b, \
                       eps, out);                                                                    \
    break;
      VT_RLN_ROW(2, 2) VT_RLN_ROW(3, 3) VT_RLN_ROW(4, 4)
#undef VT_RLN_ROW
      default:
        hipLaunchKernelGGL(resid_ln_row_kernel<0>, rgrid, rblock, 0, s, part, splits, rows, bias, R, g,
                           b, eps, out);
    }
    return hipGetLastError();
  }
  switch (width / 256) {
#define VT_RLN_CASE(n)                                                                              \
  case n:                                                                                           \
    hipLaunchKernelGGL(resid_ln_kernel<n>, grid, block, 0, s, part, splits, rows, bias, R, g, b, \
                       eps, out);                                                                   \
    break;
    VT_RLN_CASE(1) VT_RLN_CASE(2) VT_RLN_CASE(3) VT_RLN_CASE(4) VT_RLN_CASE(5) VT_RLN_CASE(6)
    VT_RLN_CASE(7) VT_RLN_CASE(8) VT_RLN_CASE(9) VT_RLN_CASE(10) VT_RLN_CASE(11) VT_RLN_CASE(12)
    VT_RLN_CASE(13) VT_RLN_CASE(14) VT_RLN_CASE(15) VT_RLN_CASE(16)
#undef VT_RLN_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vt
