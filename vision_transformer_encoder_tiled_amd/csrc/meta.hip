// Integer metadata of a packed image batch, on the device.
//
// For each item i with grid (t, h, w) (grid_thw of "v2_loaders FINDINGS"
// section 3; one native-resolution grid per image as in its section 1; t
// temporal patches of 2 frames for a clip, t = 1 for a still image):
//   cu_seqlens[i]  first token of the item (prefix sum of t*h*w),
//   pos_thw[j]     (tt, row, col) of token j, restarting at 0 per item,
//   raster_index[j] cu[i] + tt*h*w + row*w + col,
//   tok_img[j]     i.
// Tokens are stored per temporal patch in 2x2-window order: token
// tt*h*w + 4*(R*(w/2) + C) + 2*dr + dc of an item is the patch at
// (tt, 2R+dr, 2C+dc), so the 2x2 merge of the MiniMax-M3-Vision README
// ("Token compression" row) is a reshape.
#include "vt_device.h"
#include "vt_kernels.h"

namespace vt {

__global__ void __launch_bounds__(256) metadata_kernel(MetaChunk c, int32_t* __restrict__ cu_seqlens,
                                                       ImgInfo* __restrict__ info,
                                                       int32_t* __restrict__ pos_thw,
                                                       int32_t* __restrict__ raster_index,
                                                       int32_t* __restrict__ tok_img) {
  const int li = blockIdx.y;  // item within the chunk
  if (li >= c.count) return;
  const int img = c.first + li;
  const int t = c.t[li], h = c.h[li], w = c.w[li], base = c.cu[li];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (cu_seqlens) cu_seqlens[img] = base;
    if (info) info[img] = ImgInfo{t, h, w, c.pix_off[li]};
  }
  const int hw = h * w, n = t * hw, w2 = w >> 1;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x) {
    const int ti = j / hw, jj = j - ti * hw;
    const int m = jj >> 2, k = jj & 3;
    const int row = 2 * (m / w2) + (k >> 1);
    const int col = 2 * (m % w2) + (k & 1);
    const int tk = base + j;
    if (pos_thw) {
      pos_thw[3 * tk + 0] = ti;
      pos_thw[3 * tk + 1] = row;
      pos_thw[3 * tk + 2] = col;
    }
    if (raster_index) raster_index[tk] = base + ti * hw + row * w + col;
    if (tok_img) tok_img[tk] = img;
  }
}

hipError_t launch_metadata(const MetaChunk& c, int32_t max_tokens_in_chunk, int32_t* cu_seqlens,
                           ImgInfo* info, int32_t* pos_thw, int32_t* raster_index,
                           int32_t* tok_img, hipStream_t s) {
  int bx = (max_tokens_in_chunk + 255) / 256;
  if (bx > 64) bx = 64;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL(metadata_kernel, dim3(bx, c.count), dim3(256), 0, s, c, cu_seqlens, info,
                     pos_thw, raster_index, tok_img);
  return hipGetLastError();
}

__global__ void cu_last_kernel(int32_t* cu_seqlens, int32_t n_img, int32_t total) {
  if (threadIdx.x == 0) cu_seqlens[n_img] = total;
}

hipError_t launch_cu_last(int32_t* cu_seqlens, int32_t n_img, int32_t total, hipStream_t s) {
  hipLaunchKernelGGL(cu_last_kernel, dim3(1), dim3(64), 0, s, cu_seqlens, n_img, total);
  return hipGetLastError();
}

// Exclusive prefix sum over r < n of f(r) by one workgroup (chunked: each
// thread sums a contiguous run, thread 0 scans the run totals).
template <class F>
__device__ void block_scan(int n, F f, int32_t* out, int32_t* part) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (n + nt - 1) / nt;
  const int lo = tid * per, hi = min(n, lo + per);
  int sum = 0;
  for (int r = lo; r < hi; ++r) sum += f(r);
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < nt; ++t) {
      const int v = part[t];
      part[t] = run;
      run += v;
    }
    out[n] = run;
  }
  __syncthreads();
  int run = part[tid];
  for (int r = lo; r < hi; ++r) {
    out[r] = run;
    run += f(r);
  }
  __syncthreads();
}

// One workgroup.  rank(i) = #{j : n_j > n_i, or n_j == n_i and j < i} orders
// the images largest first (longest-processing-time first: the expensive
// q-tiles are dispatched before the cheap ones).  tile_start is the
// exclusive prefix sum of ceil(n/q_tile) in rank order, with
// tile_start[n_img] = the total number of q-tiles; ktile_start the prefix
// sum of ceil(n/k_tile) in image order.  From these, one descriptor per
// q-tile slot (qdesc, max_qtiles entries) and per key-tile slot (kdesc,
// max_ktiles entries), so that each attention / pack workgroup finds its
// work with a single load; slots past the totals are marked unused (-1).
__global__ void __launch_bounds__(1024) attn_schedule_kernel(
    const int32_t* __restrict__ cu, int32_t n_img, int32_t q_tile, int32_t k_tile,
    int32_t max_qtiles, int32_t max_ktiles, int32_t* __restrict__ order,
    int32_t* __restrict__ tile_start, int32_t* __restrict__ ktile_start,
    int4* __restrict__ qdesc, int2* __restrict__ kdesc, int32_t* __restrict__ qkpre) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int i = tid; i < n_img; i += nt) {
    const int ni = cu[i + 1] - cu[i];
    int r = 0;
    for (int j = 0; j < n_img; ++j) {
      const int nj = cu[j + 1] - cu[j];
      r += (nj > ni) || (nj == ni && j < i);
    }
    order[r] = i;
  }
  __syncthreads();
  block_scan(n_img, [&](int r) { const int i = order[r]; return (cu[i + 1] - cu[i] + q_tile - 1) / q_tile; },
             tile_start, part);
  block_scan(n_img, [&](int i) { return (cu[i + 1] - cu[i] + k_tile - 1) / k_tile; },
             ktile_start, part);
  const int nq = tile_start[n_img], nk = ktile_start[n_img];
  for (int t = tid; t < max_qtiles; t += nt) {
    int4 d = make_int4(-1, 0, 0, 0);
    if (t < nq) {
      int lo = 0, hi = n_img - 1;  // largest rank r with tile_start[r] <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_start[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const int i = order[lo];
      d = make_int4(cu[i] + (t - tile_start[lo]) * q_tile, cu[i], cu[i + 1], ktile_start[i]);
    }
    qdesc[t] = d;
  }
  for (int T = tid; T < max_ktiles; T += nt) {
    int2 d = make_int2(-1, -1);
    if (T < nk) {
      int lo = 0, hi = n_img - 1;  // image of key tile T
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ktile_start[mid] <= T) lo = mid; else hi = mid - 1;
      }
      d = make_int2(cu[lo] + (T - ktile_start[lo]) * k_tile, cu[lo + 1]);
    }
    kdesc[T] = d;
  }
  if (qkpre) {
    // Key tiles per q-tile slot (those of its image), recomputed from the
    // scans above rather than read back from qdesc.
    block_scan(max_qtiles, [&](int t) {
      if (t >= nq) return 0;
      int lo = 0, hi = n_img - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_start[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const int i = order[lo];
      return (cu[i + 1] - cu[i] + k_tile - 1) / k_tile;
    }, qkpre, part);
  }
}

hipError_t launch_attn_schedule(const int32_t* cu_seqlens, int32_t n_img, int32_t q_tile,
                                int32_t k_tile, int32_t max_qtiles, int32_t max_ktiles,
                                int32_t* order, int32_t* tile_start, int32_t* ktile_start,
                                int4* qdesc, int2* kdesc, hipStream_t s, int32_t* qkpre) {
  // block_scan's serial step runs over the thread count: keep it near n_img.
  const int threads = n_img >= 1024 ? 1024 : (n_img >= 256 ? 256 : 64);
  hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(threads), 0, s, cu_seqlens, n_img, q_tile,
                     k_tile, max_qtiles, max_ktiles, order, tile_start, ktile_start, qdesc, kdesc, qkpre);
  return hipGetLastError();
}

// cs[pos * pairs + j] = (cos, sin)(pos * inv_freq[j]), formed in double and
// rounded to fp32 (the table is small: pairs x n_pos entries).
__global__ void __launch_bounds__(256) rope_table_kernel(RopeFreq f, int32_t n_pos,
                                                         float2* __restrict__ cs) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_pos * f.pairs) return;
  const int pos = i / f.pairs, j = i - pos * f.pairs;
  const double ang = double(pos) * f.inv_freq[j];
  double sn, cn;
  sincos(ang, &sn, &cn);
  cs[i] = make_float2(float(cn), float(sn));
}

hipError_t launch_rope_table(const RopeFreq& f, int32_t n_pos, float2* cs, hipStream_t s) {
  const int n = n_pos * f.pairs;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, f, n_pos, cs);
  return hipGetLastError();
}

}  // namespace vt
