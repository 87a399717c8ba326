// Shared device-side definitions of libbat (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bat.h"

namespace bat {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin

// Workspace header (int32 words at the start of the workspace).
constexpr int kHdrError = 0;    // device validation: nonzero = violation seen
constexpr int kHdrItems = 1;    // planner: number of real work items
constexpr int kHdrWords = 64;   // 256 bytes

// Error bits reported through the workspace header / kv-build flag.
constexpr int kErrBlockId = 1;
constexpr int kErrLength = 2;

// One unit of work of the attention kernels: suffix rows
// [m_tile * BM, m_tile * BM + BM) of request r, head h, against prefix chunk
// `chunk` (and, for the last chunk, the request's own suffix).
struct WorkItem {
  int32_t r, h, m_tile, chunk;
};

// Per-request values the planner derives (device arrays in the workspace).
struct ReqMeta {
  int32_t n_chunks;   // prefix chunks (1 = not split)
  int32_t part_off;   // first partial row of this request (split only)
};

// What the planner checks the per-request lengths against (reported in the
// workspace header's error word; the host reads it under validation).
struct PlanBounds {
  int32_t max_s, total_s;        // suffix bound and cu_s[B]
  const uint8_t *prefix_mode;    // [B] or null (all user mode)
  int32_t bt_stride;             // block-table entries per request
  int32_t lg_user, lg_item;      // log2 of each pool's block size
};

// Everything the attention kernels read, passed by value.
struct AttnParams {
  const void *q, *k, *v;          // packed suffix [total_s, H, D]
  const int32_t *cu_s;            // [B+1]
  const int32_t *prefix_lens;     // [B], or null: no prefixes
  const uint8_t *prefix_mode;     // [B], or null
  const int32_t *block_table;     // [B, bt_stride]
  const void *pool_k[2];          // user, item
  const void *pool_v[2];
  int32_t pool_blocks[2];
  int32_t pool_bs_log2[2];
  int32_t fp8;                    // 1: the pools hold E4M3 codes with these scales
  const float *pool_sk[2];        // fp8: K and V scales [blocks, H_kv] per pool
  const float *pool_sv[2];
  int32_t bt_stride;
  int32_t B, H;
  int32_t H_kv;                   // key/value heads (H for multi-head attention); query
                                  // head h reads key/value head h / (H / H_kv)
  int32_t total_s;
  float scale_log2;               // softmax_scale * log2(e)
  int32_t chunk_len;              // prefix keys per chunk when split (0 = never)
  int32_t prefix_only;            // 1: rows see the prefix only; the kernels write fp32
                                  // partials at part_o / part_lse row q0 + row
  int32_t self_key;               // with prefix_only: each row also sees its own suffix
                                  // token (single-token candidates), and the kernel writes
                                  // the final row to out / lse (bf16 kernels only)
  int32_t max_prefix;             // host bound; longer prefixes are clamped to it (and
                                  // reported by the planner under validation)
  // Work list: the planner's items (an_rows == 0), or, for a batch whose
  // suffixes all have the same length and whose prefixes are not split, the
  // same placement computed from the workgroup index (an_rows row tiles per
  // request and query head, an_groups = B * H_kv groups of an_hg query heads)
  int32_t an_rows, an_groups, an_hg;
  const WorkItem *items;
  const ReqMeta *meta;
  int32_t *err;                   // workspace header error word, or null
  void *out;                      // [total_s, H, D]
  float *lse;                     // [H, total_s] or null
  float *part_o;                  // split partials [part_rows, H, D]
  float *part_lse;                // [part_rows, H]
};

// The launch helpers report the errors of their own launches: an error that
// an earlier runtime call of the caller's thread left behind (and that the
// caller did not collect) is cleared before the launch.
inline void clear_stale_launch_error() { (void)hipGetLastError(); }

// The last HIP error the library saw in this thread (bat_last_hip_error).
extern thread_local hipError_t g_last_hip_error;
inline bool hip_ok(hipError_t e) {
  if (e == hipSuccess) return true;
  g_last_hip_error = e;
  return false;
}
inline hipError_t launch_result() {
  const hipError_t e = hipGetLastError();
  hip_ok(e);
  return e;
}

// Key range of one work item: prefix keys [p_begin, p_end) and, when
// with_suffix, the request's suffix keys.
struct ItemRange {
  int32_t q0, n_s, n_p, mode, p_begin, p_end, n_chunks, part_off;
  bool with_suffix;
  bool partial;  // write an fp32 partial (split chunk, or prefix-only rows)
};

// The work item of workgroup `bid`.  Group g (request g / H_kv, key/value
// head g % H_kv) goes to XCD g % 8 (workgroups are dealt to the XCDs
// round-robin by index) and takes consecutive slots there: its an_hg query
// heads, each with its an_rows row tiles.  This is the planner's placement
// for such a batch, less its longest-first order (all suffixes are equal).
__device__ inline WorkItem work_item(const AttnParams &p, int bid) {
  if (p.an_rows == 0) return p.items[bid];
  const int x = bid % kNumXcd, s = bid / kNumXcd;
  const int T = p.an_hg * p.an_rows;  // items per group
  const int j = s / T, t = s - j * T;
  const int g = x + kNumXcd * j;
  if (g >= p.an_groups) return WorkItem{-1, 0, 0, 0};
  const int r = g / p.H_kv, hk = g - r * p.H_kv;
  return WorkItem{r, hk * p.an_hg + t / p.an_rows, t % p.an_rows, 0};
}

__device__ inline ItemRange item_range(const AttnParams &p, const WorkItem &it) {
  ItemRange x;
  x.q0 = p.cu_s[it.r];
  x.n_s = p.cu_s[it.r + 1] - x.q0;
  // no prefix arrays (prefix-row attention): every request has an empty prefix
  x.n_p = p.prefix_lens ? min(max(p.prefix_lens[it.r], 0), p.max_prefix) : 0;
  x.mode = p.prefix_mode && p.prefix_mode[it.r] ? 1 : 0;
  const ReqMeta m = p.an_rows ? ReqMeta{1, 0} : p.meta[it.r];
  x.n_chunks = m.n_chunks;
  x.part_off = m.part_off;
  if (x.n_chunks <= 1) {
    x.p_begin = 0;
    x.p_end = x.n_p;
    x.with_suffix = true;
  } else {
    x.p_begin = it.chunk * p.chunk_len;
    x.p_end = min(x.n_p, x.p_begin + p.chunk_len);
    x.with_suffix = it.chunk == x.n_chunks - 1;
  }
  x.partial = x.n_chunks > 1;
  if (p.prefix_only) {  // never split: one partial row per suffix row
    x.with_suffix = false;
    x.partial = !p.self_key;
    x.part_off = x.q0;
  }
  return x;
}

// Element offset of prefix token `tok` (logical position in the request's
// prefix) of key/value head h inside its pool, or -1 when the block id is out
// of range.
__device__ inline int64_t prefix_offset(const AttnParams &p, int r, int mode,
                                        int tok, int h, int D) {
  const int lg = p.pool_bs_log2[mode];
  if ((tok >> lg) >= p.bt_stride) return -1;  // prefix longer than its table row
  const int blk = p.block_table[(int64_t)r * p.bt_stride + (tok >> lg)];
  if (blk < 0 || blk >= p.pool_blocks[mode]) return -1;
  return (((int64_t)blk * p.H_kv + h) << lg | (tok & ((1 << lg) - 1))) * D;
}

}  // namespace bat
