// LayerNorm over fp32 rows -> bf16 rows, one 64-lane wavefront per row.
// Textbook form: biased variance over the row, eps inside the square root,
// then gamma/beta (pre-LN blocks of the tower; eps 1e-6).  Two passes over
// the row held in registers: mean, then the centred sum of squares, each
// reduced across the wavefront with butterfly shuffles.
#include "vt_device.h"
#include "vt_kernels.h"

namespace vt {

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
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] = xr[lane + 64 * i];
    s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float mean = wave_sum(s) * (1.0f / W);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i].x -= mean; v[i].y -= mean; v[i].z -= mean; v[i].w -= mean;
    q += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
  }
  const float var = wave_sum(q) * (1.0f / W);
  const float rstd = 1.0f / sqrtf(var + eps);
  const uint2* g2 = reinterpret_cast<const uint2*>(g);
  const uint2* b2 = reinterpret_cast<const uint2*>(b);
  uint2* o2 = reinterpret_cast<uint2*>(out + int64_t(row) * W);
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

}  // namespace vt
