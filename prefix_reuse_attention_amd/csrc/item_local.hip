// Attention inside each cached item of an item pool (the per-item
// block-diagonal prefix rows).
//
// On the Bat page, a request whose prefix is a set of popular items reuses
// those items' key/value blocks from a shared pool (sections "This paper's
// idea" and "Why it works"); an item's cached K/V can only be reused in any
// combination of items if the item's own tokens never saw the others, so the
// prefix rows of an item prefix attend within their own item.  Item i owns
// tokens i*T .. i*T+T-1 of the packed [n_items*T, H, D] inputs; each of its
// rows sees exactly those T keys (no positions, no causal mask):
//     S_ab = scale * <q_a, k_b>,  lse_a = ln sum_b exp(S_ab),
//     out_a = sum_b exp(S_ab - lse_a) v_b          (a, b within the item).
//
// A group of G = D / (elements per 16 bytes) lanes serves one (item, head):
// each lane loads its 16-byte slice of the item's T query, key and value
// rows (coalesced: a group reads whole rows), forms the T*T partial dot
// products of its slice, and the group sums them with lane shuffles.  Every
// lane then holds the item's T*T scores, takes the softmax in fp32 and writes
// its slice of the T output rows.  T*T and G are small, so the kernel is
// bound by the 3*T reads and T writes of D elements per (item, head).
//
// The same kernel finishes candidate-isolated suffix rows (MERGE): there the
// "items" are a request's suffix candidates of T tokens, each row sees its
// request's prefix plus its own candidate, and the prefix part arrives as an
// fp32 partial (output normalised over the prefix and its log-sum-exp) from
// the attention kernels run over the prefix only.  The two partials over
// disjoint keys combine exactly: lse = ln(e^lse_p + e^lse_c),
// out = e^(lse_p - lse) out_p + e^(lse_c - lse) out_c.  A request with no
// prefix has no partial; its rows keep the candidate part alone.
#include "common.h"

namespace bat {

// 16 bytes of a bf16 or fp32 row as floats.
template <bool BF16>
struct Slice {
  static constexpr int N = BF16 ? 8 : 4;
  u32x4 w;
  __device__ __forceinline__ float at(int e) const {
    if constexpr (BF16) {
      const uint32_t x = w[e >> 1];
      return __builtin_bit_cast(float, (e & 1) ? (x & 0xffff0000u) : (x << 16));
    } else {
      // through a scalar: a bit_cast of the element expression itself would
      // read the vector's first element
      const uint32_t x = w[e];
      return __builtin_bit_cast(float, x);
    }
  }
};

// The prefix partial of candidate-isolated rows (MERGE only).
struct PrefixPartial {
  const float *o;              // [rows, H, D] fp32, normalised over the prefix
  const float *lse;            // [rows, H] natural log
  const int32_t *cu_s;         // [B+1] rows of each request
  const int32_t *prefix_lens;  // [B]
  int32_t B, max_prefix;
};

template <int D, int T, bool BF16, bool MERGE>
__global__ __launch_bounds__(256) void item_local_kernel(const void *__restrict__ q,
                                                         const void *__restrict__ k,
                                                         const void *__restrict__ v,
                                                         int32_t n_items, int32_t H,
                                                         float scale_log2, void *__restrict__ out,
                                                         float *__restrict__ lse,
                                                         PrefixPartial pp) {
  using S = Slice<BF16>;
  constexpr int EB = BF16 ? 2 : 4;  // bytes per element
  constexpr int G = D / S::N;       // lanes per (item, head)
  constexpr int GPW = kWave / G;    // groups per wave
  const int lane = threadIdx.x & (kWave - 1);
  // (item, head) pairs number below 2^31 (checked by the caller)
  const int grp = (blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave)) * GPW + lane / G;
  // a group is whole lanes of one wave: either all of its lanes leave here
  // or none, so the shuffles below stay inside live groups
  if (grp >= n_items * H) return;
  const int c = lane % G;
  const int item = grp / H, head = grp - item * H;
  const int64_t row0 = (int64_t)item * T;

  S qs[T], ks[T], vs[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t off = (((row0 + t) * H + head) * D + (int64_t)c * S::N) * EB;
    qs[t].w = *(const u32x4 *)((const uint8_t *)q + off);
    ks[t].w = *(const u32x4 *)((const uint8_t *)k + off);
    vs[t].w = *(const u32x4 *)((const uint8_t *)v + off);
  }

  // this lane's share of every dot product, then the group's sum
  float s[T][T];
#pragma unroll
  for (int a = 0; a < T; ++a)
#pragma unroll
    for (int b = 0; b < T; ++b) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < S::N; ++e) acc = __builtin_fmaf(qs[a].at(e), ks[b].at(e), acc);
      s[a][b] = acc;
    }
#pragma unroll
  for (int m = 1; m < G; m <<= 1)
#pragma unroll
    for (int a = 0; a < T; ++a)
#pragma unroll
      for (int b = 0; b < T; ++b) s[a][b] += __shfl_xor(s[a][b], m, G);

  // MERGE: whether this candidate's request has a prefix partial (the
  // candidates of a request start at multiples of T, so one lookup serves all
  // T rows)
  bool has_prefix = false;
  if constexpr (MERGE) {
    int lo = 0, hi = pp.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pp.cu_s[mid] <= row0) lo = mid; else hi = mid - 1;
    }
    const int n_p = pp.prefix_lens ? min(max(pp.prefix_lens[lo], 0), pp.max_prefix) : 0;
    has_prefix = n_p > 0;
  }

  // softmax per row in the log2 domain, then this lane's slice of the output
  const int64_t total = (int64_t)n_items * T;
#pragma unroll
  for (int a = 0; a < T; ++a) {
    float mx = s[a][0];
#pragma unroll
    for (int b = 1; b < T; ++b) mx = fmaxf(mx, s[a][b]);
    const float m2 = mx * scale_log2;
    float p[T], l = 0.f;
#pragma unroll
    for (int b = 0; b < T; ++b) {
      p[b] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[a][b], scale_log2, -m2));
      l += p[b];
    }
    const float inv = 1.0f / l;
    float o[S::N];
#pragma unroll
    for (int e = 0; e < S::N; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int b = 0; b < T; ++b) acc = __builtin_fmaf(p[b], vs[b].at(e), acc);
      o[e] = acc * inv;
    }
    float lse2 = m2 + __log2f(l);  // this row's log-sum-exp, log2 domain
    if constexpr (MERGE) {
      if (has_prefix) {
        const int64_t pr = (row0 + a) * H + head;
        const float lp = pp.lse[pr] * 1.44269504088896340736f;
        const float mx = fmaxf(lp, lse2);
        const float wp = __builtin_amdgcn_exp2f(lp - mx), wc = __builtin_amdgcn_exp2f(lse2 - mx);
        const float iw = 1.0f / (wp + wc);
        const f32x4 *po = (const f32x4 *)(pp.o + pr * D + (int64_t)c * S::N);
#pragma unroll
        for (int e4 = 0; e4 < S::N / 4; ++e4) {
          const f32x4 x = po[e4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[4 * e4 + i] = (wp * x[i] + wc * o[4 * e4 + i]) * iw;
        }
        lse2 = mx + __log2f(wp + wc);
      }
    }
    const int64_t off = (((row0 + a) * H + head) * D + (int64_t)c * S::N) * EB;
    if constexpr (BF16) {
      typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
      typedef float f32x8 __attribute__((ext_vector_type(8)));
      const f32x8 f = {o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]};
      const bf16x8_t h = __builtin_convertvector(f, bf16x8_t);  // round to nearest even
      *(u32x4 *)((uint8_t *)out + off) = __builtin_bit_cast(u32x4, h);
    } else {
      const f32x4 f = {o[0], o[1], o[2], o[3]};
      *(f32x4 *)((uint8_t *)out + off) = f;
    }
    if (lse && c == 0) lse[(int64_t)head * total + row0 + a] = lse2 * 0.69314718055994530942f;
  }
}

template <int D, int T, bool BF16>
hipError_t launch_item_local_t(const void *q, const void *k, const void *v, int32_t n_items,
                               int32_t H, float scale_log2, void *out, float *lse,
                               const PrefixPartial *pp, hipStream_t stream) {
  clear_stale_launch_error();
  constexpr int G = D / (BF16 ? 8 : 4);
  constexpr int groups_per_block = 4 * (kWave / G);  // four waves
  const int64_t groups = (int64_t)n_items * H;
  if (groups > 0x7fffffff - groups_per_block) return hipErrorInvalidValue;
  const int64_t blocks = (groups + groups_per_block - 1) / groups_per_block;
  if (pp)
    hipLaunchKernelGGL((item_local_kernel<D, T, BF16, true>), dim3((unsigned)blocks), dim3(256),
                       0, stream, q, k, v, n_items, H, scale_log2, out, lse, *pp);
  else
    hipLaunchKernelGGL((item_local_kernel<D, T, BF16, false>), dim3((unsigned)blocks), dim3(256),
                       0, stream, q, k, v, n_items, H, scale_log2, out, lse, PrefixPartial{});
  return launch_result();
}

template <int D, bool BF16>
hipError_t launch_item_local_d(const void *q, const void *k, const void *v, int32_t n_items,
                               int32_t T, int32_t H, float scale_log2, void *out, float *lse,
                               const PrefixPartial *pp, hipStream_t stream) {
  clear_stale_launch_error();
  switch (T) {
    case 1: return launch_item_local_t<D, 1, BF16>(q, k, v, n_items, H, scale_log2, out, lse, pp, stream);
    case 2: return launch_item_local_t<D, 2, BF16>(q, k, v, n_items, H, scale_log2, out, lse, pp, stream);
    case 4: return launch_item_local_t<D, 4, BF16>(q, k, v, n_items, H, scale_log2, out, lse, pp, stream);
    case 8: return launch_item_local_t<D, 8, BF16>(q, k, v, n_items, H, scale_log2, out, lse, pp, stream);
  }
  return hipErrorInvalidValue;
}

// Tokens per item T in {1, 2, 4, 8}; (dtype, D) as the attention kernels.
// With a prefix partial (o_p non-null) the items are suffix candidates and
// the result is merged with it.
hipError_t launch_item_local(const void *q, const void *k, const void *v, int32_t n_items,
                             int32_t T, int32_t H, int32_t D, bool bf16, float scale_log2,
                             void *out, float *lse, const float *o_p, const float *lse_p,
                             const int32_t *cu_s, const int32_t *prefix_lens, int32_t B,
                             int32_t max_prefix, hipStream_t stream) {
  clear_stale_launch_error();
  const PrefixPartial part{o_p, lse_p, cu_s, prefix_lens, B, max_prefix};
  const PrefixPartial *pp = o_p ? &part : nullptr;
  if (bf16) {
    if (D == 64) return launch_item_local_d<64, true>(q, k, v, n_items, T, H, scale_log2, out, lse, pp, stream);
    if (D == 128) return launch_item_local_d<128, true>(q, k, v, n_items, T, H, scale_log2, out, lse, pp, stream);
  } else {
    if (D == 32) return launch_item_local_d<32, false>(q, k, v, n_items, T, H, scale_log2, out, lse, pp, stream);
    if (D == 64) return launch_item_local_d<64, false>(q, k, v, n_items, T, H, scale_log2, out, lse, pp, stream);
    if (D == 128) return launch_item_local_d<128, false>(q, k, v, n_items, T, H, scale_log2, out, lse, pp, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace bat
