// Work decomposition of one prefill batch, computed on the device so the
// host never waits for the length arrays.
//
// Items are (request, head, suffix row tile, prefix chunk).  All tiles of one
// (request, head, chunk) read the same keys/values, so they form a group that
// is placed on one XCD (blockIdx % 8 picks the XCD) in consecutive slots, to
// be served from that XCD's L2.  Groups are ordered longest first (the
// largest per-item key count first) and dealt round-robin over the XCDs, so
// each XCD's queue also runs longest first, which bounds the tail.
#include "common.h"

namespace bat {

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t *__restrict__ cu_s, const int32_t *__restrict__ prefix_lens,
    int32_t B, int32_t H, int32_t bm, int32_t chunk_len, int32_t max_p, int32_t grid,
    int32_t *__restrict__ req_key,    // [B] scratch: work key, then sorted order
    int32_t *__restrict__ req_order,  // [B] scratch
    ReqMeta *__restrict__ meta, WorkItem *__restrict__ items, int32_t *hdr) {
  const int tid = threadIdx.x;
  __shared__ int64_t s_sum[kPlanThreads][kNumXcd];  // per-thread partial sums
  __shared__ int64_t s_total[kNumXcd];

  if (tid == 0) hdr[kHdrError] = 0;
  for (int64_t idx = tid; idx < grid; idx += kPlanThreads) items[idx] = WorkItem{-1, 0, 0, 0};
  // 1) per-request tiles, chunks and work key (keys per item)
  for (int r = tid; r < B; r += kPlanThreads) {
    const int n_s = cu_s[r + 1] - cu_s[r];
    const int n_p = min(max(prefix_lens[r], 0), max_p);
    int nc = 1;
    if (chunk_len > 0 && n_p > chunk_len) nc = (n_p + chunk_len - 1) / chunk_len;
    meta[r].n_chunks = nc;
    const int keys = (n_s > 0) ? (nc > 1 ? chunk_len : n_p) + n_s : -1;
    req_key[r] = keys;
  }
  __syncthreads();
  // 2) stable rank sort, largest key first (O(B^2 / threads))
  for (int r = tid; r < B; r += kPlanThreads) {
    const int kr = req_key[r];
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const int kj = req_key[j];
      rank += (kj > kr) || (kj == kr && j < r);
    }
    req_order[rank] = r;
  }
  __syncthreads();
  // 3) per request (in sorted order): groups = H * chunks, each of T tiles.
  //    Group g (global, in order) goes to XCD g % 8.  Count, per request and
  //    XCD, the slots its groups take; an exclusive scan gives the bases.
  //    Each thread owns a contiguous run of sorted requests.
  const int per = (B + kPlanThreads - 1) / kPlanThreads;
  const int k0 = min(B, tid * per), k1 = min(B, k0 + per);
  // group index of the first group of each request needs a scan of group
  // counts first
  int64_t my_groups = 0;
  for (int k = k0; k < k1; ++k) {
    const int r = req_order[k];
    const int n_s = cu_s[r + 1] - cu_s[r];
    if (n_s > 0) my_groups += (int64_t)H * meta[r].n_chunks;
  }
  s_sum[tid][0] = my_groups;
  __syncthreads();
  if (tid == 0) {
    int64_t acc = 0;
    for (int i = 0; i < kPlanThreads; ++i) {
      const int64_t t = s_sum[i][0];
      s_sum[i][0] = acc;
      acc += t;
    }
  }
  __syncthreads();
  const int64_t g0 = s_sum[tid][0];  // first global group index of my run
  __syncthreads();
  int64_t slots[kNumXcd] = {0, 0, 0, 0, 0, 0, 0, 0};
  int64_t g = g0;
  for (int k = k0; k < k1; ++k) {
    const int r = req_order[k];
    const int n_s = cu_s[r + 1] - cu_s[r];
    if (n_s <= 0) continue;
    const int T = (n_s + bm - 1) / bm;
    const int64_t ng = (int64_t)H * meta[r].n_chunks;
    for (int x = 0; x < kNumXcd; ++x) {
      // groups g .. g+ng-1 with (group % 8) == x
      const int64_t first = g + ((x - g % kNumXcd) + kNumXcd) % kNumXcd;
      const int64_t cnt = first < g + ng ? (g + ng - 1 - first) / kNumXcd + 1 : 0;
      slots[x] += cnt * T;
    }
    g += ng;
  }
  for (int x = 0; x < kNumXcd; ++x) s_sum[tid][x] = slots[x];
  __syncthreads();
  if (tid < kNumXcd) {
    int64_t acc = 0;
    for (int i = 0; i < kPlanThreads; ++i) {
      const int64_t t = s_sum[i][tid];
      s_sum[i][tid] = acc;
      acc += t;
    }
    s_total[tid] = acc;  // slots used on XCD `tid`
  }
  __syncthreads();
  // 4) write the items of my run
  g = g0;
  for (int x = 0; x < kNumXcd; ++x) slots[x] = s_sum[tid][x];
  for (int k = k0; k < k1; ++k) {
    const int r = req_order[k];
    const int n_s = cu_s[r + 1] - cu_s[r];
    if (n_s <= 0) continue;
    const int T = (n_s + bm - 1) / bm;
    const int nc = meta[r].n_chunks;
    const int64_t ng = (int64_t)H * nc;
    for (int64_t gi = 0; gi < ng; ++gi, ++g) {
      const int x = (int)(g % kNumXcd);
      const int h = (int)(gi % H), c = (int)(gi / H);
      for (int t = 0; t < T; ++t) {
        const int64_t idx = (slots[x] + t) * kNumXcd + x;
        if (idx < grid) items[idx] = WorkItem{r, h, t, c};
        else atomicOr(&hdr[kHdrError], kErrLength);  // grid bound too small
      }
      slots[x] += T;
    }
  }
  // 5) split partial offsets (exclusive scan of n_chunks * n_s over split
  //    requests, in request order) and the empty tail slots of each XCD
  if (tid == 0) {
    int64_t acc = 0;
    for (int r = 0; r < B; ++r) {
      const int nc = meta[r].n_chunks;
      meta[r].part_off = (int32_t)acc;
      if (nc > 1) acc += (int64_t)nc * (cu_s[r + 1] - cu_s[r]);
    }
    int64_t n_items = 0;
    for (int x = 0; x < kNumXcd; ++x) n_items += s_total[x];
    hdr[kHdrItems] = (int32_t)n_items;
  }
}

hipError_t launch_plan(const int32_t *cu_s, const int32_t *prefix_lens, int32_t B,
                       int32_t H, int32_t bm, int32_t chunk_len, int32_t max_p, int32_t grid,
                       int32_t *req_key, int32_t *req_order,
                       ReqMeta *meta, WorkItem *items, int32_t *hdr, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, cu_s, prefix_lens,
                     B, H, bm, chunk_len, max_p, grid, req_key, req_order, meta, items, hdr);
  return hipGetLastError();
}

}  // namespace bat
