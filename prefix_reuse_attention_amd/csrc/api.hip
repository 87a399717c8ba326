// C ABI of libbat: argument validation, workspace layout, kernel dispatch.
// Every launch goes on the caller's stream; nothing here allocates memory.
#include <algorithm>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "common.h"

namespace bat {
thread_local hipError_t g_last_hip_error = hipSuccess;

hipError_t launch_kv_build(const void *k, const void *v, const int32_t *cu, const int32_t *bt,
                           int32_t bt_stride, int32_t B, int32_t H, int32_t D, int32_t total,
                           int elem_bytes, void *pk, void *pv, int32_t num_blocks,
                           int32_t bs_log2, int32_t *err, hipStream_t stream);
hipError_t launch_kv_build_fp8(const void *k, const void *v, const int32_t *cu,
                               const int32_t *bt, int32_t bt_stride, int32_t B, int32_t H,
                               int32_t D, int elem_bytes, void *pk, void *pv, float *sk,
                               float *sv, int32_t num_blocks, int32_t bs_log2, int32_t *err,
                               hipStream_t stream);
hipError_t launch_plan(const int32_t *cu_s, const int32_t *prefix_lens, const PlanBounds &bd,
                       int32_t B, int32_t H, int32_t hg, int32_t bm, int32_t chunk_len,
                       int32_t max_p, int32_t grid, int32_t *g_scratch, ReqMeta *meta,
                       WorkItem *items, int32_t *hdr, hipStream_t stream);
hipError_t launch_attn_bf16(const AttnParams &p, int D, int W, bool flat_gather, int grid,
                            hipStream_t stream);
hipError_t launch_attn_f32(const AttnParams &p, int D, int grid, double scale_log2,
                           hipStream_t stream);
hipError_t launch_merge_split(const AttnParams &p, int D, bool bf16, hipStream_t stream);
hipError_t launch_lse_merge(const float *o_parts, const float *lse_parts, int n_parts, int rows,
                            int H, int D, bool bf16, void *out, float *lse, hipStream_t stream);
hipError_t launch_item_local(const void *q, const void *k, const void *v, int32_t n_items,
                             int32_t T, int32_t H, int32_t D, bool bf16, float scale_log2,
                             void *out, float *lse, const float *o_p, const float *lse_p,
                             const int32_t *cu_s, const int32_t *prefix_lens, int32_t B,
                             int32_t max_prefix, hipStream_t stream);
int bf16_rows_per_item(int W);
int bf16_keys_per_tile(int D, int W, bool fp8);
int f32_rows_per_item();
int f32_keys_per_tile();

// Error words of bat_kv_build under BAT_VALIDATE: each validated call holds
// one of them (per device) from its launch until it has read it back, so
// validated builds on different streams or threads report only their own
// violations.  More than kErrSlots such calls at once on one device wait.
constexpr int kErrSlots = 64;
constexpr int kMaxDevices = 64;
__device__ int32_t g_kv_build_err[kErrSlots];

__global__ void clear_word_kernel(int32_t *w) { *w = 0; }

namespace {

std::mutex g_slot_mu;
std::condition_variable g_slot_cv;
uint64_t g_slot_busy[kMaxDevices];

// An error word of this device's array for one validated call.
class ErrSlot {
 public:
  bat_status acquire() {
    if (!hip_ok(hipGetDevice(&dev_)) || dev_ < 0 || dev_ >= kMaxDevices) return BAT_ERR_HIP;
    int32_t *base = nullptr;
    if (!hip_ok(hipGetSymbolAddress((void **)&base, HIP_SYMBOL(g_kv_build_err))))
      return BAT_ERR_HIP;
    std::unique_lock<std::mutex> lk(g_slot_mu);
    g_slot_cv.wait(lk, [&] { return ~g_slot_busy[dev_] != 0; });
    slot_ = __builtin_ctzll(~g_slot_busy[dev_]);
    g_slot_busy[dev_] |= uint64_t(1) << slot_;
    word = base + slot_;
    return BAT_OK;
  }
  ~ErrSlot() {
    if (slot_ < 0) return;
    {
      std::lock_guard<std::mutex> lk(g_slot_mu);
      g_slot_busy[dev_] &= ~(uint64_t(1) << slot_);
    }
    g_slot_cv.notify_one();
  }
  int32_t *word = nullptr;

 private:
  int dev_ = -1, slot_ = -1;
};

bool validate_enabled() {
  const char *e = std::getenv("BAT_VALIDATE");
  return e && e[0] && std::strcmp(e, "0") != 0;
}

int log2_exact(int x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

bool supported(bat_dtype dt, int D) {
  if (dt == BAT_BF16) return D == 64 || D == 128;
  if (dt == BAT_F32) return D == 32 || D == 64 || D == 128;
  return false;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The decomposition policy: rows per item, keys per tile, prefix chunking.
// A pure function of host-side bounds so that the workspace size and the
// launch agree.
struct Plan {
  int waves = 4;          // bf16 kernel: waves per workgroup (32 rows each)
  bool flat_gather = false;  // bf16 kernel: global instead of buffer loads for per-key gathers
  int bm = 0, bn = 0;
  int chunk_len = 0;      // 0: prefixes are never split
  int max_chunks = 1;
  int64_t grid = 0;       // work-item slots (upper bound, multiple of 8)
  int64_t part_rows = 0;  // split partial rows
  size_t off_items = 0, off_meta = 0, off_scratch = 0, off_part_o = 0, off_part_lse = 0,
         total = 0;
};

// The scales of fp8 pools (user, item): K and V, [blocks, H_kv] each.
struct Fp8Scales {
  const float *k[2], *v[2];
};

// prefix_only: the rows see their prefix only and every row gets an fp32
// partial (candidate-isolated suffixes); prefixes are then never split.
// hg: query heads per key/value head (grouped heads; 1 otherwise).
// per_key: a prefix pool's blocks are smaller than the eight-wave kernel's
// key tile, so its tiles are gathered key by key.
bool make_plan(int32_t B, int32_t H, int32_t D, bat_dtype dt, int32_t total_s, int32_t max_s,
               int32_t max_p, Plan &pl, bool prefix_only = false, int32_t hg = 1,
               bool allow_split = true, bool fp8 = false, bool per_key = false) {
  if (B < 0 || H <= 0 || total_s < 0 || max_s < 0 || max_p < 0) return false;
  if (!supported(dt, D)) return false;
  // bf16: eight waves (256 rows, the ping-pong kernel) share each K/V tile
  // when the suffixes average more than one four-wave item (128 rows), else
  // four (measured at 4096-key prefixes: eight waves even at 96 and 128
  // rows, 17-20 % ahead at 160).
  // At D=64 the ping-pong kernel's 64-key tiles pay when whole pool blocks
  // are copied; per-key gathers run faster in the four-wave kernel's
  // 128-key tiles (measured at D=64: 64-token pages +11 % on eight waves,
  // 4-token item blocks -8 %).
  if (const char *e = std::getenv("BAT_WAVES")) {
    pl.waves = std::atoi(e) == 8 ? 8 : 4;
  } else {
    pl.waves = (B > 0 && (int64_t)total_s > (int64_t)128 * B &&
                !(D == 64 && per_key && !fp8)) ? 8 : 4;
  }
  // fp8 pools: the four-wave kernel at head dim 128 (the eight-wave one
  // copies every tile straight into LDS, with no place to convert codes)
  if (fp8 && D == 128) pl.waves = 4;
  // BAT_GATHER=flat: the per-key gather of small pool blocks always takes
  // the global-load form that pools of 2 GiB or more need
  if (const char *e = std::getenv("BAT_GATHER")) pl.flat_gather = std::strcmp(e, "flat") == 0;
  pl.bm = dt == BAT_BF16 ? bf16_rows_per_item(pl.waves) : f32_rows_per_item();
  pl.bn = dt == BAT_BF16 ? bf16_keys_per_tile(D, pl.waves, fp8) : f32_keys_per_tile();
  // Split a prefix only when the unsplit batch cannot fill the GPU and the
  // prefix is long (2048 keys or more).  A CU holds two four-wave
  // workgroups at once but one eight-wave workgroup, so the GPU is full at
  // about 512 four-wave or 256 eight-wave items on 256 CUs; splitting past
  // that only adds partials and their merge.  The item count is estimated
  // from the host bounds: every request with suffix rows takes at least one
  // row tile.  Each chunk writes an fp32 partial of its rows that the merge
  // reads back: 2048-key chunks keep that traffic well below the chunk's
  // compute (about 1000 flop per partial byte), 512-key ones do not, and are
  // taken only while some CU would otherwise have no item at all.
  const int64_t tiles_per_head =
      std::max<int64_t>((total_s + pl.bm - 1) / pl.bm, std::min<int64_t>(B, total_s));
  const int64_t lower_items = (int64_t)H * tiles_per_head;
  const int64_t target = dt == BAT_BF16 && pl.waves == 8 ? 256 : 512;
  const int64_t min_chunk = lower_items >= 256 ? 2048 : 512;
  pl.chunk_len = 0;
  if (prefix_only || !allow_split) {
    // prefix-only rows: one partial row per suffix row, no split
  } else if (const char *e = std::getenv("BAT_SPLIT_CHUNK")) {
    const int v = std::atoi(e);
    if (v > 0) pl.chunk_len = ((v + pl.bn - 1) / pl.bn) * pl.bn;
  } else if (lower_items > 0 && lower_items < target &&
             max_p >= std::max<int64_t>(2048, 2 * min_chunk)) {
    int64_t c = (target + lower_items - 1) / lower_items;
    if (c > 64) c = 64;
    int64_t len = (max_p + c - 1) / c;
    if (len < min_chunk) len = min_chunk;
    pl.chunk_len = (int)(((len + pl.bn - 1) / pl.bn) * pl.bn);
  }
  pl.max_chunks = (pl.chunk_len > 0 && max_p > pl.chunk_len)
                      ? (max_p + pl.chunk_len - 1) / pl.chunk_len : 1;
  // a group is one (request, key/value head, chunk): hg query heads times
  // up to t_max row tiles, all on one XCD
  if (hg <= 0 || H % hg != 0) return false;
  const int64_t t_max = (max_s + pl.bm - 1) / pl.bm;
  const int64_t n_groups = (int64_t)(H / hg) * B * pl.max_chunks;
  pl.grid = kNumXcd * ((n_groups + kNumXcd - 1) / kNumXcd) * hg * t_max;
  pl.part_rows = prefix_only ? (int64_t)total_s
                             : pl.max_chunks > 1 ? (int64_t)pl.max_chunks * total_s : 0;
  // the planner counts items and split-partial rows in 32 bits
  if (pl.grid > (int64_t)1 << 30 || pl.part_rows >= (int64_t)1 << 31) return false;
  size_t off = align256(kHdrWords * sizeof(int32_t));
  pl.off_items = off;    off = align256(off + sizeof(WorkItem) * (size_t)pl.grid);
  pl.off_meta = off;     off = align256(off + sizeof(ReqMeta) * (size_t)B);
  pl.off_scratch = off;  off = align256(off + 4 * sizeof(int32_t) * (size_t)B);
  pl.off_part_o = off;   off = align256(off + sizeof(float) * (size_t)pl.part_rows * H * D);
  pl.off_part_lse = off; off = align256(off + sizeof(float) * (size_t)pl.part_rows * H);
  pl.total = off;
  return true;
}

// The workspace a call needs whatever its pools hold: the larger of the
// plans with and without per-key gathers (which may change the workgroup
// shape).  Returns 0 if no plan exists.
size_t plan_bound(int32_t B, int32_t H, int32_t D, bat_dtype dt, int32_t total_s, int32_t max_s,
                  int32_t max_p, bool prefix_only = false, int32_t hg = 1,
                  bool allow_split = true, bool fp8 = false) {
  size_t n = 0;
  for (bool per_key : {false, true}) {
    Plan pl;
    if (!make_plan(B, H, D, dt, total_s, max_s, max_p, pl, prefix_only, hg, allow_split, fp8,
                   per_key))
      return 0;
    if (pl.total > n) n = pl.total;
  }
  return n;
}

bat_status pool_desc(const bat_kv_pool *pool, const void *&k, const void *&v, int32_t &blocks,
                     int32_t &lg) {
  if (!pool) {
    k = v = nullptr;
    blocks = 0;
    lg = 0;
    return BAT_OK;
  }
  lg = log2_exact(pool->block_size);
  if (lg < 0 || pool->block_size > 256 || pool->num_blocks < 0) return BAT_ERR_INVALID_ARG;
  if (pool->num_blocks > 0 && (!pool->k || !pool->v)) return BAT_ERR_INVALID_ARG;
  k = pool->k;
  v = pool->v;
  blocks = pool->num_blocks;
  return BAT_OK;
}

}  // namespace
}  // namespace bat

using namespace bat;

extern "C" {

const char *bat_status_string(bat_status s) {
  switch (s) {
    case BAT_OK: return "BAT_OK";
    case BAT_ERR_INVALID_ARG: return "BAT_ERR_INVALID_ARG: null pointer or invalid size";
    case BAT_ERR_UNSUPPORTED: return "BAT_ERR_UNSUPPORTED: no kernel for this dtype/head_dim";
    case BAT_ERR_BLOCK_TABLE: return "BAT_ERR_BLOCK_TABLE: block id or length out of range";
    case BAT_ERR_WORKSPACE: return "BAT_ERR_WORKSPACE: workspace missing or too small";
    case BAT_ERR_HIP: return "BAT_ERR_HIP: HIP runtime or launch error";
  }
  return "unknown bat_status";
}

int32_t bat_version(void) { return 100; }

const char *bat_last_hip_error(void) { return hipGetErrorName(g_last_hip_error); }

bat_status bat_kv_build(const void *k, const void *v, const int32_t *cu_lens,
                        const int32_t *block_table, int32_t bt_stride, int32_t B, int32_t H,
                        int32_t D, int32_t total_tokens, bat_dtype dt, const bat_kv_pool *pool,
                        void *stream) {
  if (!pool || B < 0 || H <= 0 || total_tokens < 0 || bt_stride < 0) return BAT_ERR_INVALID_ARG;
  if (dt != BAT_F32 && dt != BAT_BF16) return BAT_ERR_INVALID_ARG;
  if (!(D == 32 || D == 64 || D == 128)) return BAT_ERR_UNSUPPORTED;
  const int lg = log2_exact(pool->block_size);
  if (lg < 0 || pool->block_size > 256 || pool->num_blocks < 0) return BAT_ERR_INVALID_ARG;
  if (total_tokens == 0) return BAT_OK;
  if (B == 0 || bt_stride == 0) return BAT_ERR_INVALID_ARG;
  if (!k || !v || !cu_lens || !block_table || !pool->k || !pool->v) return BAT_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  const bool val = validate_enabled();
  ErrSlot slot;
  int32_t *err = nullptr;
  if (val) {
    const bat_status s = slot.acquire();
    if (s != BAT_OK) return s;
    err = slot.word;
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, st, err);
  }
  const int eb = dt == BAT_BF16 ? 2 : 4;
  if (!hip_ok(launch_kv_build(k, v, cu_lens, block_table, bt_stride, B, H, D, total_tokens, eb, pool->k,
                      pool->v, pool->num_blocks, lg, err, st)))
    return BAT_ERR_HIP;
  if (val) {
    int32_t h_err = 0;
    if (!hip_ok(hipMemcpyAsync(&h_err, err, sizeof h_err, hipMemcpyDeviceToHost, st)) ||
        !hip_ok(hipStreamSynchronize(st)))
      return BAT_ERR_HIP;
    if (h_err) return BAT_ERR_BLOCK_TABLE;
  }
  return BAT_OK;
}

size_t bat_attn_workspace_size(int32_t B, int32_t H, int32_t D, bat_dtype dt,
                               int32_t total_suffix, int32_t max_suffix_len,
                               int32_t max_prefix_len) {
  return plan_bound(B, H, D, dt, total_suffix, max_suffix_len, max_prefix_len);
}

bat_status bat_kv_build_fp8(const void *k, const void *v, const int32_t *cu_lens,
                            const int32_t *block_table, int32_t bt_stride, int32_t B, int32_t H,
                            int32_t D, int32_t total_tokens, bat_dtype dt,
                            const bat_kv_pool_fp8 *pool, void *stream) {
  if (!pool || B < 0 || H <= 0 || total_tokens < 0 || bt_stride < 0) return BAT_ERR_INVALID_ARG;
  if (dt != BAT_F32 && dt != BAT_BF16) return BAT_ERR_INVALID_ARG;
  if (!(D == 32 || D == 64 || D == 128)) return BAT_ERR_UNSUPPORTED;
  const int lg = log2_exact(pool->block_size);
  if (lg < 0 || pool->block_size > 256 || pool->num_blocks < 0) return BAT_ERR_INVALID_ARG;
  if (total_tokens == 0) return BAT_OK;
  if (B == 0 || bt_stride == 0) return BAT_ERR_INVALID_ARG;
  if ((int64_t)B * bt_stride > 0x7fffffff || H > 65535) return BAT_ERR_INVALID_ARG;
  if (!k || !v || !cu_lens || !block_table || !pool->k || !pool->v || !pool->k_scale ||
      !pool->v_scale)
    return BAT_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  const bool val = validate_enabled();
  ErrSlot slot;
  int32_t *err = nullptr;
  if (val) {
    const bat_status s = slot.acquire();
    if (s != BAT_OK) return s;
    err = slot.word;
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, st, err);
  }
  if (!hip_ok(launch_kv_build_fp8(k, v, cu_lens, block_table, bt_stride, B, H, D,
                                  dt == BAT_BF16 ? 2 : 4, pool->k, pool->v, pool->k_scale,
                                  pool->v_scale, pool->num_blocks, lg, err, st)))
    return BAT_ERR_HIP;
  if (val) {
    int32_t h_err = 0;
    if (!hip_ok(hipMemcpyAsync(&h_err, err, sizeof h_err, hipMemcpyDeviceToHost, st)) ||
        !hip_ok(hipStreamSynchronize(st)))
      return BAT_ERR_HIP;
    if (h_err) return BAT_ERR_BLOCK_TABLE;
  }
  return BAT_OK;
}

size_t bat_attn_fp8_workspace_size(int32_t B, int32_t H, int32_t D, int32_t total_suffix,
                                   int32_t max_suffix_len, int32_t max_prefix_len) {
  Plan pl;
  if (!make_plan(B, H, D, BAT_BF16, total_suffix, max_suffix_len, max_prefix_len, pl, false, 1,
                 true, true))
    return 0;
  return pl.total;
}

size_t bat_attn_prefill_workspace_size(int32_t B, int32_t H, int32_t D, int32_t total_suffix,
                                       int32_t max_prefix_len) {
  // the largest workspace over both dtypes, with max_suffix_len at its
  // largest possible value (one request holding every suffix row)
  size_t n = 0;
  for (bat_dtype dt : {BAT_F32, BAT_BF16}) {
    if (!supported(dt, D)) continue;
    const size_t t = plan_bound(B, H, D, dt, total_suffix, total_suffix, max_prefix_len);
    if (t == 0) return 0;
    if (t > n) n = t;
  }
  return n;
}

}  // extern "C"

namespace bat {
namespace {

// The attention call behind bat_attn_prefill and bat_attn_prefix_rows: rows
// cu[r] .. cu[r+1] of q attend to request r's prefix (none when prefix_lens
// is null) and to the same rows of k/v.  Arguments are checked by the callers.
bat_status attn_rows(const void *q, const void *k, const void *v, const int32_t *cu_suffix_lens,
                     const int32_t *prefix_lens, const uint8_t *prefix_mode,
                     const int32_t *block_table, int32_t bt_stride, const bat_kv_pool *user_pool,
                     const bat_kv_pool *item_pool, int32_t B, int32_t H, int32_t D, bat_dtype dt,
                     float softmax_scale, int32_t total_suffix, int32_t max_suffix_len,
                     int32_t max_prefix_len, void *out, float *lse, void *workspace,
                     size_t workspace_bytes, void *stream, bool prefix_only = false,
                     const float **part_o = nullptr, const float **part_lse = nullptr,
                     int32_t H_kv = 0, bool *self_key = nullptr, bool allow_split = true,
                     const Fp8Scales *f8 = nullptr) {
  if (max_prefix_len > 0 && (!block_table || bt_stride == 0)) return BAT_ERR_INVALID_ARG;
  AttnParams p{};
  for (int i = 0; i < 2; ++i) {
    const bat_status s = pool_desc(i == 0 ? user_pool : item_pool, p.pool_k[i], p.pool_v[i],
                                   p.pool_blocks[i], p.pool_bs_log2[i]);
    if (s != BAT_OK) return s;
  }
  if (max_prefix_len > 0 && p.pool_blocks[0] == 0 && p.pool_blocks[1] == 0)
    return BAT_ERR_INVALID_ARG;
  const int32_t hg = H_kv > 0 ? H / H_kv : 1;
  // a pool whose blocks are smaller than the eight-wave kernel's key tile
  // is gathered key by key
  const int pp_keys = bf16_keys_per_tile(D, 8, false);
  bool per_key = false;
  for (int i = 0; i < 2; ++i)
    per_key |= p.pool_blocks[i] > 0 && (1 << p.pool_bs_log2[i]) < pp_keys;
  Plan pl;
  if (!make_plan(B, H, D, dt, total_suffix, max_suffix_len, max_prefix_len, pl, prefix_only, hg,
                 allow_split, f8 != nullptr, per_key))
    return BAT_ERR_INVALID_ARG;
  if (!workspace) return BAT_ERR_WORKSPACE;
  // the call asks for what its size function reports (the bound over both
  // gather forms), not only what this plan uses
  if (workspace_bytes < plan_bound(B, H, D, dt, total_suffix, max_suffix_len, max_prefix_len,
                                   prefix_only, hg, allow_split, f8 != nullptr))
    return BAT_ERR_WORKSPACE;

  uint8_t *ws = (uint8_t *)workspace;
  if (f8) {
    p.fp8 = 1;
    for (int i = 0; i < 2; ++i) {
      p.pool_sk[i] = f8->k[i];
      p.pool_sv[i] = f8->v[i];
    }
  }
  p.prefix_only = prefix_only ? 1 : 0;
  // prefix-only rows of single-token candidates: the bf16 kernels fold each
  // row's own key into its result and write the final rows themselves
  if (self_key) {
    *self_key = prefix_only && dt == BAT_BF16;
    p.self_key = *self_key ? 1 : 0;
  }
  if (part_o) *part_o = (const float *)(ws + pl.off_part_o);
  if (part_lse) *part_lse = (const float *)(ws + pl.off_part_lse);
  int32_t *hdr = (int32_t *)ws;
  p.q = q;
  p.k = k;
  p.v = v;
  p.cu_s = cu_suffix_lens;
  p.prefix_lens = prefix_lens;
  p.prefix_mode = prefix_mode;
  p.block_table = block_table;
  p.bt_stride = bt_stride;
  p.B = B;
  p.H = H;
  p.H_kv = H_kv > 0 ? H_kv : H;
  p.total_s = total_suffix;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  p.chunk_len = pl.chunk_len;
  p.max_prefix = max_prefix_len;
  p.items = (const WorkItem *)(ws + pl.off_items);
  p.meta = (const ReqMeta *)(ws + pl.off_meta);
  const bool val = validate_enabled();
  p.err = val ? hdr + kHdrError : nullptr;
  p.out = out;
  p.lse = lse;
  p.part_o = (float *)(ws + pl.off_part_o);
  p.part_lse = (float *)(ws + pl.off_part_lse);

  hipStream_t st = (hipStream_t)stream;
  // A batch whose suffixes all have max_suffix_len rows (the bound is tight
  // and sums to total_suffix) and whose prefixes are never split needs no
  // planner launch: the kernels compute the same placement from their
  // workgroup index.  Under validation the planner always runs (it checks
  // the lengths).
  const int64_t t_rows = ((int64_t)max_suffix_len + pl.bm - 1) / pl.bm;
  if (!val && pl.max_chunks == 1 && (int64_t)B * max_suffix_len == total_suffix) {
    p.an_rows = (int32_t)t_rows;
    p.an_groups = B * p.H_kv;
    p.an_hg = hg;
  } else {
    PlanBounds bd{max_suffix_len, total_suffix, prefix_mode, bt_stride, p.pool_bs_log2[0],
                  p.pool_bs_log2[1]};
    if (!hip_ok(launch_plan(cu_suffix_lens, prefix_lens, bd, B, H, hg, pl.bm, pl.chunk_len,
                    max_prefix_len, (int32_t)pl.grid, (int32_t *)(ws + pl.off_scratch),
                    (ReqMeta *)(ws + pl.off_meta), (WorkItem *)(ws + pl.off_items), hdr,
                    st)))
      return BAT_ERR_HIP;
  }
  const hipError_t e = dt == BAT_BF16 ? launch_attn_bf16(p, D, pl.waves, pl.flat_gather, (int)pl.grid, st)
                                      : launch_attn_f32(p, D, (int)pl.grid,
                                                        (double)softmax_scale * 1.4426950408889634074,
                                                        st);
  if (!hip_ok(e)) return BAT_ERR_HIP;
  if (!prefix_only && pl.max_chunks > 1 && !hip_ok(launch_merge_split(p, D, dt == BAT_BF16, st)))
    return BAT_ERR_HIP;
  if (val) {
    int32_t h_err = 0;
    if (!hip_ok(hipMemcpyAsync(&h_err, hdr + kHdrError, sizeof h_err, hipMemcpyDeviceToHost, st)) ||
        !hip_ok(hipStreamSynchronize(st)))
      return BAT_ERR_HIP;
    if (h_err) return BAT_ERR_BLOCK_TABLE;
  }
  return BAT_OK;
}

}  // namespace
}  // namespace bat

extern "C" {

bat_status bat_attn_prefill(const void *q, const void *k, const void *v,
                            const int32_t *cu_suffix_lens, const int32_t *prefix_lens,
                            const uint8_t *prefix_mode, const int32_t *block_table,
                            int32_t bt_stride, const bat_kv_pool *user_pool,
                            const bat_kv_pool *item_pool, int32_t B, int32_t H, int32_t D,
                            bat_dtype dt, float softmax_scale, int32_t total_suffix,
                            int32_t max_suffix_len, int32_t max_prefix_len, void *out,
                            float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  if (dt != BAT_F32 && dt != BAT_BF16) return BAT_ERR_INVALID_ARG;
  if (B < 0 || H <= 0 || total_suffix < 0 || max_suffix_len < 0 || max_prefix_len < 0 ||
      bt_stride < 0)
    return BAT_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == __builtin_inff()) return BAT_ERR_INVALID_ARG;
  if (!supported(dt, D)) return BAT_ERR_UNSUPPORTED;
  if (total_suffix == 0) return BAT_OK;  // nothing to write
  if (B == 0 || max_suffix_len == 0) return BAT_ERR_INVALID_ARG;
  if (!q || !k || !v || !cu_suffix_lens || !prefix_lens || !prefix_mode || !out)
    return BAT_ERR_INVALID_ARG;
  return attn_rows(q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table, bt_stride,
                   user_pool, item_pool, B, H, D, dt, softmax_scale, total_suffix, max_suffix_len,
                   max_prefix_len, out, lse, workspace, workspace_bytes, stream);
}

bat_status bat_attn_prefill_fp8(const void *q, const void *k, const void *v,
                                const int32_t *cu_suffix_lens, const int32_t *prefix_lens,
                                const uint8_t *prefix_mode, const int32_t *block_table,
                                int32_t bt_stride, const bat_kv_pool_fp8 *user_pool,
                                const bat_kv_pool_fp8 *item_pool, int32_t B, int32_t H,
                                int32_t D, float softmax_scale, int32_t total_suffix,
                                int32_t max_suffix_len, int32_t max_prefix_len, void *out,
                                float *lse, void *workspace, size_t workspace_bytes,
                                void *stream) {
  if (B < 0 || H <= 0 || total_suffix < 0 || max_suffix_len < 0 || max_prefix_len < 0 ||
      bt_stride < 0)
    return BAT_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == __builtin_inff()) return BAT_ERR_INVALID_ARG;
  if (!supported(BAT_BF16, D)) return BAT_ERR_UNSUPPORTED;
  if (total_suffix == 0) return BAT_OK;  // nothing to write
  if (B == 0 || max_suffix_len == 0) return BAT_ERR_INVALID_ARG;
  if (!q || !k || !v || !cu_suffix_lens || !prefix_lens || !prefix_mode || !out)
    return BAT_ERR_INVALID_ARG;
  // the code pools travel as plain pool descriptions, their scales beside them
  bat_kv_pool up{}, ip{};
  Fp8Scales sc{};
  const bat_kv_pool_fp8 *src[2] = {user_pool, item_pool};
  bat_kv_pool *dst[2] = {&up, &ip};
  for (int i = 0; i < 2; ++i) {
    if (!src[i]) continue;
    if (src[i]->num_blocks > 0 && (!src[i]->k_scale || !src[i]->v_scale))
      return BAT_ERR_INVALID_ARG;
    *dst[i] = bat_kv_pool{src[i]->k, src[i]->v, src[i]->num_blocks, src[i]->block_size};
    sc.k[i] = src[i]->k_scale;
    sc.v[i] = src[i]->v_scale;
  }
  return attn_rows(q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table, bt_stride,
                   user_pool ? &up : nullptr, item_pool ? &ip : nullptr, B, H, D, BAT_BF16,
                   softmax_scale, total_suffix, max_suffix_len, max_prefix_len, out, lse,
                   workspace, workspace_bytes, stream, false, nullptr, nullptr, 0, nullptr, true,
                   &sc);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Scratch of bat_attn_prefill_noalloc: a file-scope device array (one copy
// per GPU, held until the process ends) in place of the caller's workspace.
// Host code never passes the array's name to a kernel or a copy: its device
// address on each GPU comes from hipGetSymbolAddress, taken once per device
// on the first call there, with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace bat {
namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

bat_status scratch_of_current_device(void **ptr) {
  int dev = -1;
  if (!hip_ok(hipGetDevice(&dev)) || dev < 0 || dev >= kMaxDevices) return BAT_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (!hip_ok(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) || !p) return BAT_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BAT_OK;
}
}  // namespace
}  // namespace bat

extern "C" {

size_t bat_attn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

bat_status bat_attn_prefill_noalloc(const void *q, const void *k, const void *v,
                                    const int32_t *cu_suffix_lens, const int32_t *prefix_lens,
                                    const uint8_t *prefix_mode, const int32_t *block_table,
                                    int32_t bt_stride, const bat_kv_pool *user_pool,
                                    const bat_kv_pool *item_pool, int32_t B, int32_t H,
                                    int32_t D, bat_dtype dt, float softmax_scale,
                                    int32_t total_suffix, int32_t max_suffix_len,
                                    int32_t max_prefix_len, void *out, float *lse,
                                    void *stream) {
  if (dt != BAT_F32 && dt != BAT_BF16) return BAT_ERR_INVALID_ARG;
  if (B < 0 || H <= 0 || total_suffix < 0 || max_suffix_len < 0 || max_prefix_len < 0 ||
      bt_stride < 0)
    return BAT_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == __builtin_inff()) return BAT_ERR_INVALID_ARG;
  if (!supported(dt, D)) return BAT_ERR_UNSUPPORTED;
  if (total_suffix == 0) return BAT_OK;  // nothing to write
  if (B == 0 || max_suffix_len == 0) return BAT_ERR_INVALID_ARG;
  if (!q || !k || !v || !cu_suffix_lens || !prefix_lens || !prefix_mode || !out)
    return BAT_ERR_INVALID_ARG;
  // the plan bat_attn_prefill would take; when its split partials do not
  // fit the scratch, the same call unsplit (the rows are the same up to
  // rounding); beyond that, the batch is too large for this entry point
  bool allow_split = true;
  size_t need = plan_bound(B, H, D, dt, total_suffix, max_suffix_len, max_prefix_len);
  if (need == 0) return BAT_ERR_INVALID_ARG;
  if (need > kNoAllocScratchBytes) {
    allow_split = false;
    need = plan_bound(B, H, D, dt, total_suffix, max_suffix_len, max_prefix_len, false, 1, false);
    if (need == 0 || need > kNoAllocScratchBytes) return BAT_ERR_WORKSPACE;
  }
  void *ws = nullptr;
  const bat_status s = scratch_of_current_device(&ws);
  if (s != BAT_OK) return s;
  return attn_rows(q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table, bt_stride,
                   user_pool, item_pool, B, H, D, dt, softmax_scale, total_suffix, max_suffix_len,
                   max_prefix_len, out, lse, ws, kNoAllocScratchBytes, stream, false, nullptr,
                   nullptr, 0, nullptr, allow_split);
}

bat_status bat_attn_prefix_rows(const void *q, const void *k, const void *v,
                                const int32_t *cu_prefix_lens, int32_t B, int32_t H, int32_t D,
                                bat_dtype dt, float softmax_scale, int32_t total_prefix,
                                int32_t max_prefix_len, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream) {
  if (dt != BAT_F32 && dt != BAT_BF16) return BAT_ERR_INVALID_ARG;
  if (B < 0 || H <= 0 || total_prefix < 0 || max_prefix_len < 0) return BAT_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == __builtin_inff()) return BAT_ERR_INVALID_ARG;
  if (!supported(dt, D)) return BAT_ERR_UNSUPPORTED;
  if (total_prefix == 0) return BAT_OK;  // nothing to write
  if (B == 0 || max_prefix_len == 0) return BAT_ERR_INVALID_ARG;
  if (!q || !k || !v || !cu_prefix_lens || !out) return BAT_ERR_INVALID_ARG;
  // a prefix row sees its request's prefix only: the prefix is the row
  // group itself, with no cached keys before it
  return attn_rows(q, k, v, cu_prefix_lens, nullptr, nullptr, nullptr, 0, nullptr, nullptr, B,
                   H, D, dt, softmax_scale, total_prefix, max_prefix_len, 0, out, lse, workspace,
                   workspace_bytes, stream);
}

bat_status bat_attn_item_local(const void *q, const void *k, const void *v, int32_t n_items,
                               int32_t tokens_per_item, int32_t H, int32_t D, bat_dtype dt,
                               float softmax_scale, void *out, float *lse, void *stream) {
  if (dt != BAT_F32 && dt != BAT_BF16) return BAT_ERR_INVALID_ARG;
  if (n_items < 0 || H <= 0) return BAT_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == __builtin_inff()) return BAT_ERR_INVALID_ARG;
  const int T = tokens_per_item;
  if (!(T == 1 || T == 2 || T == 4 || T == 8)) return BAT_ERR_UNSUPPORTED;
  if (!supported(dt, D)) return BAT_ERR_UNSUPPORTED;
  if ((int64_t)n_items * T > 0x7fffffff || (int64_t)n_items * H > 0x7fff0000)
    return BAT_ERR_INVALID_ARG;
  if (n_items == 0) return BAT_OK;
  if (!q || !k || !v || !out) return BAT_ERR_INVALID_ARG;
  const float scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  if (!hip_ok(launch_item_local(q, k, v, n_items, T, H, D, dt == BAT_BF16, scale_log2, out, lse, nullptr,
                        nullptr, nullptr, nullptr, 0, 0, (hipStream_t)stream)))
    return BAT_ERR_HIP;
  return BAT_OK;
}

size_t bat_attn_gqa_workspace_size(int32_t B, int32_t H, int32_t H_kv, int32_t D, bat_dtype dt,
                                   int32_t total_suffix, int32_t max_suffix_len,
                                   int32_t max_prefix_len) {
  if (H_kv <= 0 || H % H_kv != 0) return 0;
  return plan_bound(B, H, D, dt, total_suffix, max_suffix_len, max_prefix_len, false, H / H_kv);
}

bat_status bat_attn_prefill_gqa(const void *q, const void *k, const void *v,
                                const int32_t *cu_suffix_lens, const int32_t *prefix_lens,
                                const uint8_t *prefix_mode, const int32_t *block_table,
                                int32_t bt_stride, const bat_kv_pool *user_pool,
                                const bat_kv_pool *item_pool, int32_t B, int32_t H,
                                int32_t H_kv, int32_t D, bat_dtype dt, float softmax_scale,
                                int32_t total_suffix, int32_t max_suffix_len,
                                int32_t max_prefix_len, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream) {
  if (dt != BAT_F32 && dt != BAT_BF16) return BAT_ERR_INVALID_ARG;
  if (B < 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || total_suffix < 0 ||
      max_suffix_len < 0 || max_prefix_len < 0 || bt_stride < 0)
    return BAT_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == __builtin_inff()) return BAT_ERR_INVALID_ARG;
  if (!supported(dt, D)) return BAT_ERR_UNSUPPORTED;
  if (total_suffix == 0) return BAT_OK;  // nothing to write
  if (B == 0 || max_suffix_len == 0) return BAT_ERR_INVALID_ARG;
  if (!q || !k || !v || !cu_suffix_lens || !prefix_lens || !prefix_mode || !out)
    return BAT_ERR_INVALID_ARG;
  return attn_rows(q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table, bt_stride,
                   user_pool, item_pool, B, H, D, dt, softmax_scale, total_suffix, max_suffix_len,
                   max_prefix_len, out, lse, workspace, workspace_bytes, stream, false, nullptr,
                   nullptr, H_kv);
}

size_t bat_attn_isolated_workspace_size(int32_t B, int32_t H, int32_t D, bat_dtype dt,
                                        int32_t total_suffix, int32_t max_suffix_len,
                                        int32_t max_prefix_len) {
  return plan_bound(B, H, D, dt, total_suffix, max_suffix_len, max_prefix_len, true);
}

bat_status bat_attn_prefill_isolated(const void *q, const void *k, const void *v,
                                     const int32_t *cu_suffix_lens, const int32_t *prefix_lens,
                                     const uint8_t *prefix_mode, const int32_t *block_table,
                                     int32_t bt_stride, const bat_kv_pool *user_pool,
                                     const bat_kv_pool *item_pool, int32_t B, int32_t H,
                                     int32_t D, bat_dtype dt, float softmax_scale,
                                     int32_t tokens_per_candidate, int32_t total_suffix,
                                     int32_t max_suffix_len, int32_t max_prefix_len, void *out,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     void *stream) {
  if (dt != BAT_F32 && dt != BAT_BF16) return BAT_ERR_INVALID_ARG;
  if (B < 0 || H <= 0 || total_suffix < 0 || max_suffix_len < 0 || max_prefix_len < 0 ||
      bt_stride < 0)
    return BAT_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == __builtin_inff()) return BAT_ERR_INVALID_ARG;
  const int T = tokens_per_candidate;
  if (!(T == 1 || T == 2 || T == 4 || T == 8)) return BAT_ERR_UNSUPPORTED;
  if (!supported(dt, D)) return BAT_ERR_UNSUPPORTED;
  if (total_suffix % T != 0 || (int64_t)(total_suffix / T) * H > 0x7fff0000)
    return BAT_ERR_INVALID_ARG;
  if (total_suffix == 0) return BAT_OK;  // nothing to write
  if (B == 0 || max_suffix_len == 0) return BAT_ERR_INVALID_ARG;
  if (!q || !k || !v || !cu_suffix_lens || !prefix_lens || !prefix_mode || !out)
    return BAT_ERR_INVALID_ARG;
  const float *o_p = nullptr, *lse_p = nullptr;
  if (max_prefix_len > 0) {
    // the prefix part of every row, as fp32 partials in the workspace; for
    // single-token bf16 candidates, the whole row at once
    bool fused = false;
    const bat_status s = attn_rows(q, k, v, cu_suffix_lens, prefix_lens, prefix_mode,
                                   block_table, bt_stride, user_pool, item_pool, B, H, D, dt,
                                   softmax_scale, total_suffix, max_suffix_len, max_prefix_len,
                                   out, lse, workspace, workspace_bytes, stream, true, &o_p,
                                   &lse_p, 0, T == 1 ? &fused : nullptr);
    if (s != BAT_OK) return s;
    if (fused) return BAT_OK;
  }
  // each candidate over its own tokens, merged with its row's prefix part
  const float scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  if (!hip_ok(launch_item_local(q, k, v, total_suffix / T, T, H, D, dt == BAT_BF16, scale_log2, out, lse,
                        o_p, lse_p, cu_suffix_lens, prefix_lens, B, max_prefix_len,
                        (hipStream_t)stream)))
    return BAT_ERR_HIP;
  return BAT_OK;
}

bat_status bat_lse_merge(const float *o_parts, const float *lse_parts, int32_t n_parts,
                         int32_t rows, int32_t H, int32_t D, bat_dtype dt, void *out,
                         float *lse, void *stream) {
  if (dt != BAT_F32 && dt != BAT_BF16) return BAT_ERR_INVALID_ARG;
  if (n_parts <= 0 || rows < 0 || H <= 0 || D <= 0 || (D % 4) != 0) return BAT_ERR_INVALID_ARG;
  if (rows == 0) return BAT_OK;
  if (!o_parts || !lse_parts || !out) return BAT_ERR_INVALID_ARG;
  if (!hip_ok(launch_lse_merge(o_parts, lse_parts, n_parts, rows, H, D, dt == BAT_BF16, out, lse,
                       (hipStream_t)stream)))
    return BAT_ERR_HIP;
  return BAT_OK;
}

}  // extern "C"
