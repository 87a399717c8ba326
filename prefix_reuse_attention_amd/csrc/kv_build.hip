// Prefix KV build: scatter packed prefix keys/values into a paged pool.
//
// The Bat page ("Problem", "Why this problem is worth solving") builds a
// prefix's key/value cache once and reuses it across queries; its
// disaggregated pool ("Why it works") keeps user and item caches apart.
// This kernel is the build step: a bit-exact copy, HBM-bound (each byte read
// once and written once), with 16-byte vector accesses on both sides.
#include "common.h"

namespace bat {

// One thread moves one 16-byte chunk of one (token, head) row of K and the
// same chunk of V.  Rows of D elements are contiguous in both layouts, so a
// wave reads and writes whole rows.
template <int ELEM>
__global__ __launch_bounds__(256) void kv_build_kernel(
    const uint8_t *__restrict__ k, const uint8_t *__restrict__ v,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ bt,
    int32_t bt_stride, int32_t B, int32_t H, int32_t D, int32_t total,
    uint8_t *__restrict__ pk, uint8_t *__restrict__ pv, int32_t num_blocks,
    int32_t bs_log2, int32_t *err) {
  const int chunks_per_row = D * ELEM / 16;
  const int64_t n_chunks = (int64_t)total * H * chunks_per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n_chunks; g += stride) {
    const int c = (int)(g % chunks_per_row);
    const int64_t row = g / chunks_per_row;  // (token, head)
    const int h = (int)(row % H);
    const int tok = (int)(row / H);
    if (tok >= cu[B]) {
      if (err) atomicOr(err, kErrLength);
      continue;
    }
    // request owning this token: last r with cu[r] <= tok
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    const int t = tok - cu[lo];
    if (t < 0 || (t >> bs_log2) >= bt_stride) {  // only with a non-monotonic cu
      if (err) atomicOr(err, kErrLength);
      continue;
    }
    const int blk = bt[(int64_t)lo * bt_stride + (t >> bs_log2)];
    if (blk < 0 || blk >= num_blocks) {
      if (err) atomicOr(err, kErrBlockId);
      continue;
    }
    const int64_t dst =
        ((((int64_t)blk * H + h) << bs_log2) | (t & ((1 << bs_log2) - 1))) * (D * ELEM) + c * 16;
    const int64_t src = row * (D * ELEM) + c * 16;
    const u32x4 a = *reinterpret_cast<const u32x4 *>(k + src);
    const u32x4 b = *reinterpret_cast<const u32x4 *>(v + src);
    *reinterpret_cast<u32x4 *>(pk + dst) = a;
    *reinterpret_cast<u32x4 *>(pv + dst) = b;
  }
}

hipError_t launch_kv_build(const void *k, const void *v, const int32_t *cu,
                           const int32_t *bt, int32_t bt_stride, int32_t B,
                           int32_t H, int32_t D, int32_t total, int elem_bytes,
                           void *pk, void *pv, int32_t num_blocks, int32_t bs_log2,
                           int32_t *err, hipStream_t stream) {
  clear_stale_launch_error();
  const int64_t n_chunks = (int64_t)total * H * (D * elem_bytes / 16);
  const int threads = 256;
  int64_t blocks = (n_chunks + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
  if (blocks < 1) blocks = 1;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(kv_build_kernel<2>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint8_t *)k, (const uint8_t *)v, cu, bt, bt_stride, B, H, D,
                       total, (uint8_t *)pk, (uint8_t *)pv, num_blocks, bs_log2, err);
  else
    hipLaunchKernelGGL(kv_build_kernel<4>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint8_t *)k, (const uint8_t *)v, cu, bt, bt_stride, B, H, D,
                       total, (uint8_t *)pk, (uint8_t *)pv, num_blocks, bs_log2, err);
  return launch_result();
}

}  // namespace bat
