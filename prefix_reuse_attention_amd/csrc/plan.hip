// Work decomposition of one prefill batch, computed on the device so the
// host never waits for the length arrays.
//
// Items are (request, head, suffix row tile, prefix chunk).  All tiles of one
// (request, key/value head, chunk) read the same keys/values -- with grouped
// heads, the hg query heads of a key/value head too -- so they form a group
// that is placed on one XCD (blockIdx % 8 picks the XCD) in consecutive
// slots, to be served from that XCD's L2.  Groups are ordered longest first (the
// largest per-item key count first) and dealt round-robin over the XCDs, so
// each XCD's queue also runs longest first, which bounds the tail.
//
// One workgroup of 256 threads; thread t owns a contiguous run of requests,
// and every prefix sum over requests is a block-wide scan (wave shuffles,
// then one pass over the four wave totals).  All counts fit in 32 bits: the
// host bounds the item grid and the split-partial rows below 2^31.
#include "common.h"

namespace bat {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPlanLds = 4096;  // batches up to this size keep per-request state in LDS

// Exclusive block-wide scan of NV lanes per thread; returns the totals.
template <int NV>
__device__ __forceinline__ void block_scan(int32_t (&v)[NV], int32_t (&total)[NV],
                                           int32_t (*s_wave)[kNumXcd], int32_t *s_total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t inc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) inc[i] = v[i];
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int32_t t = __shfl_up(inc[i], off);
      if (lane >= off) inc[i] += t;
    }
  }
  if (lane == kWave - 1)
#pragma unroll
    for (int i = 0; i < NV; ++i) s_wave[w][i] = inc[i];
  __syncthreads();
  if (tid < NV) {
    int32_t acc = 0;
#pragma unroll
    for (int j = 0; j < kPlanWaves; ++j) {
      const int32_t t = s_wave[j][tid];
      s_wave[j][tid] = acc;
      acc += t;
    }
    s_total[tid] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] = inc[i] - v[i] + s_wave[w][i];
    total[i] = s_total[i];
  }
  __syncthreads();  // s_wave / s_total are reused by the next scan
}

typedef __attribute__((address_space(3))) int32_t lds_i32;

// The planner body, with the per-request arrays (work key, sorted order,
// suffix length, chunk count) at req[0 .. 4*stride): in LDS for batches up
// to kPlanLds requests, else in the global scratch.  The two cases are
// separate instances so that LDS accesses compile to LDS instructions (a
// generic pointer would make every access wait for global memory too).
template <typename ReqPtr>
__device__ __forceinline__ void plan_body(
    const int32_t *__restrict__ cu_s, const int32_t *__restrict__ prefix_lens,
    const PlanBounds &bd,
    int32_t B, int32_t H, int32_t hg, int32_t bm, int32_t chunk_len, int32_t max_p, int32_t grid,
    ReqPtr req, int32_t stride, int32_t (*s_wave)[kNumXcd], int32_t *s_total,
    __attribute__((address_space(3))) int32_t *fast, ReqMeta *__restrict__ meta,
    WorkItem *__restrict__ items, int32_t *hdr) {
  const int tid = threadIdx.x;
  const int Hk = H / hg;  // key/value heads: groups per request and chunk
  ReqPtr req_key = req, req_order = req + stride, req_ns = req + 2 * stride,
         req_nc = req + 3 * stride;

  if (tid == 0) hdr[kHdrError] = 0;
  for (int idx = tid; idx < grid; idx += kPlanThreads) items[idx] = WorkItem{-1, 0, 0, 0};

  const int per = (B + kPlanThreads - 1) / kPlanThreads;
  const int k0 = min(B, tid * per), k1 = min(B, k0 + per);

  // 1) per request: chunks, work key (keys per item), split-partial rows;
  //    partial offsets are an exclusive scan in request order
  {
    int32_t part[1] = {0}, tot[1];
    for (int r = k0; r < k1; ++r) {
      const int n_s = cu_s[r + 1] - cu_s[r];
      const int n_p = prefix_lens ? min(max(prefix_lens[r], 0), max_p) : 0;
      int nc = 1;
      if (chunk_len > 0 && n_p > chunk_len) nc = (n_p + chunk_len - 1) / chunk_len;
      req_nc[r] = nc;
      req_ns[r] = n_s;
      req_key[r] = (n_s > 0) ? (nc > 1 ? chunk_len : n_p) + n_s : -1;
      if (nc > 1 && n_s > 0) part[0] += nc * n_s;
    }
    block_scan<1>(part, tot, s_wave, s_total);
    for (int r = k0; r < k1; ++r) {
      const int nc = req_nc[r], n_s = req_ns[r];
      meta[r] = ReqMeta{nc, part[0]};
      if (nc > 1 && n_s > 0) part[0] += nc * n_s;
      // lengths against the caller's bounds and table (past the scan's
      // barrier, so after the header was cleared): reported, while the
      // kernels clamp a prefix to max_p and skip rows past total_s
      bool bad = n_s < 0 || n_s > bd.max_s || cu_s[r] < 0 || cu_s[r + 1] > bd.total_s;
      if (prefix_lens) {
        const int np = prefix_lens[r];
        const int lg = (bd.prefix_mode && bd.prefix_mode[r]) ? bd.lg_item : bd.lg_user;
        bad |= np < 0 || np > max_p || (np > 0 && ((np - 1) >> lg) >= bd.bt_stride);
      }
      if (bad) atomicOr(&hdr[kHdrError], kErrLength);
    }
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
  // 3) groups of my run of sorted requests, and the first global group index
  int32_t g0[1] = {0}, ng_total[1];
  for (int k = k0; k < k1; ++k) {
    const int r = req_order[k];
    if (req_ns[r] > 0) g0[0] += Hk * req_nc[r];
  }
  block_scan<1>(g0, ng_total, s_wave, s_total);
  // 4) slots each XCD gives my groups: group g goes to XCD g % 8
  int32_t slots[kNumXcd] = {0, 0, 0, 0, 0, 0, 0, 0}, used[kNumXcd];
  int32_t g = g0[0];
  for (int k = k0; k < k1; ++k) {
    const int r = req_order[k];
    const int n_s = req_ns[r];
    if (n_s <= 0) continue;
    const int T = hg * ((n_s + bm - 1) / bm);  // items per group
    const int ng = Hk * req_nc[r];
#pragma unroll
    for (int x = 0; x < kNumXcd; ++x) {
      const int first = g + ((x - g % kNumXcd) + kNumXcd) % kNumXcd;
      const int cnt = first < g + ng ? (g + ng - 1 - first) / kNumXcd + 1 : 0;
      slots[x] += cnt * T;
    }
    g += ng;
  }
  block_scan<kNumXcd>(slots, used, s_wave, s_total);
  // 5) write the items (key/value heads fastest within a request's groups,
  // then chunks; inside a group, its query heads, each with its row tiles).
  // The j-th group of sorted request k that lands on XCD x takes slots
  // base_k(x) + j*T_k .. +T_k-1 there, base_k(x) being the per-XCD scan above.
  if (B <= kPlanThreads) {
    // One request per thread: publish each request's bases, first group,
    // row-tile count and item offset, then every thread writes items,
    // finding an item's request by binary search over the offsets.
    lds_i32 *s_base = fast, *s_g0 = fast + kNumXcd * kPlanThreads,
            *s_T = s_g0 + kPlanThreads, *s_r = s_T + kPlanThreads, *s_off = s_r + kPlanThreads;
    int32_t nit[1] = {0}, total[1];
    int T = 0, r = -1;
    if (tid < B) {
      r = req_order[tid];
      const int n_s = req_ns[r];
      if (n_s > 0) {
        T = hg * ((n_s + bm - 1) / bm);
        nit[0] = Hk * req_nc[r] * T;
      }
    }
    block_scan<1>(nit, total, s_wave, s_total);
    if (tid < B) {
#pragma unroll
      for (int x = 0; x < kNumXcd; ++x) s_base[tid * kNumXcd + x] = slots[x];
      s_g0[tid] = g0[0];
      s_T[tid] = T;
      s_r[tid] = r;
      s_off[tid] = nit[0];
    }
    __syncthreads();
    for (int i = tid; i < total[0]; i += kPlanThreads) {
      int lo = 0, hi = B - 1;  // the last request whose items start at or before i
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      const int k = lo, Tk = s_T[k], G0 = s_g0[k];
      const int local = i - s_off[k];
      const int gi = local / Tk, t = local - gi * Tk;
      const int x = (G0 + gi) % kNumXcd;
      const int first = ((x - G0 % kNumXcd) + kNumXcd) % kNumXcd;
      const int idx = (s_base[k * kNumXcd + x] + ((gi - first) / kNumXcd) * Tk + t) * kNumXcd + x;
      const int rows = Tk / hg;  // row tiles of each query head
      if (idx < grid)
        items[idx] = WorkItem{s_r[k], (gi % Hk) * hg + t / rows, t % rows, gi / Hk};
      else atomicOr(&hdr[kHdrError], kErrLength);  // grid bound too small
    }
  } else {
  g = g0[0];
  for (int k = k0; k < k1; ++k) {
    const int r = req_order[k];
    const int n_s = req_ns[r];
    if (n_s <= 0) continue;
    const int rows = (n_s + bm - 1) / bm;
    const int T = hg * rows;
    const int nc = req_nc[r];
    int hk = 0, c = 0;
    for (int gi = 0; gi < Hk * nc; ++gi, ++g) {
      const int x = g % kNumXcd;
      for (int t = 0; t < T; ++t) {
        const int idx = (slots[x] + t) * kNumXcd + x;
        if (idx < grid) items[idx] = WorkItem{r, hk * hg + t / rows, t % rows, c};
        else atomicOr(&hdr[kHdrError], kErrLength);  // grid bound too small
      }
      slots[x] += T;
      if (++hk == Hk) {
        hk = 0;
        ++c;
      }
    }
  }
  }
  if (tid == 0) {
    int32_t n = 0;
#pragma unroll
    for (int x = 0; x < kNumXcd; ++x) n += used[x];
    hdr[kHdrItems] = n;
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t *__restrict__ cu_s, const int32_t *__restrict__ prefix_lens, PlanBounds bd,
    int32_t B, int32_t H, int32_t hg, int32_t bm, int32_t chunk_len, int32_t max_p, int32_t grid,
    int32_t *__restrict__ g_scratch,  // [4 * B] used when B > kPlanLds
    ReqMeta *__restrict__ meta, WorkItem *__restrict__ items, int32_t *hdr) {
  __shared__ int32_t s_wave[kPlanWaves][kNumXcd];
  __shared__ int32_t s_total[kNumXcd];
  __shared__ int32_t s_req[4 * kPlanLds];
  __shared__ int32_t s_fast[(kNumXcd + 4) * kPlanThreads];
  if (B <= kPlanLds)
    plan_body(cu_s, prefix_lens, bd, B, H, hg, bm, chunk_len, max_p, grid, (lds_i32 *)s_req,
              kPlanLds,
              s_wave, s_total, (lds_i32 *)s_fast, meta, items, hdr);
  else
    plan_body(cu_s, prefix_lens, bd, B, H, hg, bm, chunk_len, max_p, grid, g_scratch, B, s_wave,
              s_total, (lds_i32 *)s_fast, meta, items, hdr);
}

hipError_t launch_plan(const int32_t *cu_s, const int32_t *prefix_lens, const PlanBounds &bd,
                       int32_t B, int32_t H, int32_t hg, int32_t bm, int32_t chunk_len,
                       int32_t max_p, int32_t grid, int32_t *g_scratch, ReqMeta *meta,
                       WorkItem *items, int32_t *hdr, hipStream_t stream) {
  clear_stale_launch_error();
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, cu_s, prefix_lens, bd,
                     B, H, hg, bm, chunk_len, max_p, grid, g_scratch, meta, items, hdr);
  return launch_result();
}

}  // namespace bat
