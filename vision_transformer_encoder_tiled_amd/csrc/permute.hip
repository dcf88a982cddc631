// Memory-bound permutations and reductions: patchify (pixels -> patch rows in
// token order), row permutation between token order and raster order,
// fp32 -> bf16 cast, per-item mean pool of the tower tokens.
#include "vt_device.h"
#include "vt_kernels.h"

namespace vt {

// One thread per (token, channel, py): reads the 14 pixels of that patch row
// in the two frames of its temporal patch (tau = 0 and tau = 1: frames 2tt
// and 2tt+1 of a clip; a still image's single frame is repeated to fill the
// temporal patch of 2, "v2_loaders FINDINGS" section 3).  Row layout of X is
// (channel, tau, py, px), the flattened Conv3d weight order.  Pixels of an
// item: [frames][3][14h][14w] with 1 frame for t = 1 and 2t frames for t > 1.
// Pixel rows start at even offsets (14 * col bf16), so the 14 values are read
// as 7 aligned 32-bit words.
__global__ void __launch_bounds__(256) patchify_kernel(const uint16_t* __restrict__ pix,
                                                       const ImgInfo* __restrict__ info,
                                                       const int32_t* __restrict__ cu,
                                                       const int32_t* __restrict__ tok_img,
                                                       int32_t total, uint16_t* __restrict__ X) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= int64_t(total) * 42) return;
  const int tok = int(gid / 42);
  const int rem = int(gid - int64_t(tok) * 42);
  const int ch = rem / 14, py = rem - ch * 14;
  const int img = tok_img[tok];
  const ImgInfo in = info[img];
  const int j = tok - cu[img];
  const int hw = in.h * in.w, ti = j / hw, jj = j - ti * hw;
  const int w2 = in.w >> 1;
  const int m = jj >> 2, k = jj & 3;
  const int row = 2 * (m / w2) + (k >> 1);
  const int col = 2 * (m % w2) + (k & 1);
  const int64_t W = int64_t(in.w) * 14, H = int64_t(in.h) * 14;
  // Frames 2ti and 2ti+1 of a clip; a still image's one frame serves both.
  const int64_t frame = 3 * H * W;
  const int64_t f0 = in.t == 1 ? 0 : int64_t(2 * ti) * frame;
  const int64_t f1 = in.t == 1 ? 0 : f0 + frame;
  const int64_t at = in.pix_off + int64_t(ch) * H * W + (int64_t(row) * 14 + py) * W + int64_t(col) * 14;
  const uint32_t* src0 = reinterpret_cast<const uint32_t*>(pix + at + f0);
  const uint32_t* src1 = reinterpret_cast<const uint32_t*>(pix + at + f1);
  uint32_t v0[7], v1[7];
#pragma unroll
  for (int i = 0; i < 7; ++i) v0[i] = src0[i];
  if (in.t == 1) {  // a still image: both temporal slots hold the same frame
#pragma unroll
    for (int i = 0; i < 7; ++i) v1[i] = v0[i];
  } else {
#pragma unroll
    for (int i = 0; i < 7; ++i) v1[i] = src1[i];
  }
  uint32_t* dst0 = reinterpret_cast<uint32_t*>(X + int64_t(tok) * 1176 + (ch * 2 + 0) * 196 + py * 14);
  uint32_t* dst1 = reinterpret_cast<uint32_t*>(X + int64_t(tok) * 1176 + (ch * 2 + 1) * 196 + py * 14);
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    dst0[i] = v0[i];
    dst1[i] = v1[i];
  }
}

hipError_t launch_patchify(const uint16_t* pixels, const ImgInfo* info, const int32_t* cu_seqlens,
                           const int32_t* tok_img, int32_t total_tokens, uint16_t* X,
                           hipStream_t s) {
  const int64_t n = int64_t(total_tokens) * 42;
  hipLaunchKernelGGL(patchify_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, pixels,
                     info, cu_seqlens, tok_img, total_tokens, X);
  return hipGetLastError();
}

// One workgroup per row; rows are moved as 16-byte vectors (width % 8 == 0).
__global__ void __launch_bounds__(256) row_permute_kernel(const uint16_t* __restrict__ src,
                                                          uint16_t* __restrict__ dst,
                                                          const int32_t* __restrict__ ridx,
                                                          int32_t width, int scatter) {
  const int r = blockIdx.x;
  const int other = ridx[r];
  const int64_t so = int64_t(scatter ? r : other) * width;
  const int64_t dof = int64_t(scatter ? other : r) * width;
  const uint4* s4 = reinterpret_cast<const uint4*>(src + so);
  uint4* d4 = reinterpret_cast<uint4*>(dst + dof);
  for (int i = threadIdx.x; i < width / 8; i += blockDim.x) d4[i] = s4[i];
}

hipError_t launch_row_permute(const uint16_t* src, uint16_t* dst, const int32_t* raster_index,
                              int32_t rows, int32_t width, bool scatter, hipStream_t s) {
  hipLaunchKernelGGL(row_permute_kernel, dim3(rows), dim3(256), 0, s, src, dst, raster_index,
                     width, scatter ? 1 : 0);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) f32_to_bf16_kernel(const float4* __restrict__ src,
                                                          uint2* __restrict__ dst, size_t n4) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += size_t(gridDim.x) * blockDim.x) {
    const float4 v = src[i];
    dst[i] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  }
}

hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t s) {
  const size_t n4 = n / 4;  // n % 4 == 0 (widths are multiples of 64)
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(src), reinterpret_cast<uint2*>(dst), n4);
  return hipGetLastError();
}

// Mean of each item's tower tokens ("v2_loaders FINDINGS" s.3: the sequence
// mean-pooled to (1, 1280)).  Workgroup (item, 128-column slice) of 16
// wavefronts: lane l of wave w sums columns 2l, 2l+1 of tokens w, w+16, ...
// in order (fp32), then the 16 partial sums are added in wave order, so the
// result is deterministic.
__global__ void __launch_bounds__(1024) mean_pool_kernel(const uint16_t* __restrict__ T,
                                                         const int32_t* __restrict__ cu,
                                                         int32_t hidden, float* __restrict__ out) {
  __shared__ float2 part[16][64];
  const int img = blockIdx.x, col = blockIdx.y * 128 + 2 * (threadIdx.x & 63);
  const int wave = threadIdx.x >> 6;
  const int beg = cu[img], end = cu[img + 1];
  float sx = 0.f, sy = 0.f;
  for (int r = beg + wave; r < end; r += 16) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(T + int64_t(r) * hidden + col);
    sx += bflo(v);
    sy += bfhi(v);
  }
  part[wave][threadIdx.x & 63] = make_float2(sx, sy);
  __syncthreads();
  if (threadIdx.x < 64) {
    float2 s = part[0][threadIdx.x];
    for (int w = 1; w < 16; ++w) {
      s.x += part[w][threadIdx.x].x;
      s.y += part[w][threadIdx.x].y;
    }
    const float inv = 1.0f / float(end - beg);
    *reinterpret_cast<float2*>(out + int64_t(img) * hidden + col) = make_float2(s.x * inv, s.y * inv);
  }
}

hipError_t launch_mean_pool(const uint16_t* T, const int32_t* cu_seqlens, int32_t n_img,
                            int32_t hidden, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mean_pool_kernel, dim3(n_img, hidden / 128), dim3(1024), 0, s, T, cu_seqlens,
                     hidden, out);
  return hipGetLastError();
}

}  // namespace vt
