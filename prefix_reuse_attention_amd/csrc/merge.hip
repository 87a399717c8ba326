// Log-sum-exp merge of attention partials over disjoint key sets.
//
// Partials o_i normalised over their own keys with log-sum-exp lse_i combine
// exactly: lse = ln sum_i exp(lse_i), o = sum_i exp(lse_i - lse) o_i.  This is
// how a prefix split across workgroups (or devices) is recombined with the
// rest of the row.  HBM-bound: each partial is read once, O written once.
#include "common.h"

namespace bat {

__device__ __forceinline__ void store4(void *out, int64_t off, f32x4 v, bool bf16) {
  if (bf16) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 h = __builtin_convertvector(v, bf16x4);
    *(u32x2 *)((uint16_t *)out + off) = __builtin_bit_cast(u32x2, h);
  } else {
    *(f32x4 *)((float *)out + off) = v;
  }
}

// One thread per (partial row, head, 4 dims); rows of split requests only.
__global__ __launch_bounds__(256) void merge_split_kernel(AttnParams p, int D, int bf16) {
  const int dq = D / 4;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)p.total_s * p.H * dq;
  if (g >= n) return;
  const int c4 = (int)(g % dq);
  const int head = (int)((g / dq) % p.H);
  const int row = (int)(g / ((int64_t)dq * p.H));
  int lo = 0, hi = p.B - 1;  // request owning this suffix row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu_s[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const ReqMeta m = p.meta[lo];
  if (m.n_chunks <= 1) return;
  const int n_s = p.cu_s[lo + 1] - p.cu_s[lo];
  const int i = row - p.cu_s[lo];
  float mx = -__builtin_inff();
  for (int c = 0; c < m.n_chunks; ++c)
    mx = fmaxf(mx, p.part_lse[((int64_t)m.part_off + (int64_t)c * n_s + i) * p.H + head]);
  float sum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < m.n_chunks; ++c) {
    const int64_t pr = (int64_t)m.part_off + (int64_t)c * n_s + i;
    const float w = expf(p.part_lse[pr * p.H + head] - mx);
    sum += w;
    const f32x4 v = *(const f32x4 *)(p.part_o + (pr * p.H + head) * D + 4 * c4);
    acc += w * v;
  }
  const float inv = 1.0f / sum;
  store4(p.out, ((int64_t)row * p.H + head) * D + 4 * c4, acc * inv, bf16 != 0);
  if (p.lse && c4 == 0) p.lse[(int64_t)head * p.total_s + row] = mx + logf(sum);
}

// Standalone merge: o_parts [n_parts, rows, H, D], lse_parts [n_parts, H, rows].
__global__ __launch_bounds__(256) void lse_merge_kernel(const float *__restrict__ o_parts,
                                                        const float *__restrict__ lse_parts,
                                                        int n_parts, int rows, int H, int D,
                                                        int bf16, void *out, float *lse) {
  const int dq = D / 4;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)rows * H * dq;
  if (g >= n) return;
  const int c4 = (int)(g % dq);
  const int head = (int)((g / dq) % H);
  const int row = (int)(g / ((int64_t)dq * H));
  const int64_t lstride = (int64_t)H * rows;
  const int64_t ostride = (int64_t)rows * H * D;
  float mx = -__builtin_inff();
  for (int c = 0; c < n_parts; ++c)
    mx = fmaxf(mx, lse_parts[c * lstride + (int64_t)head * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  if (mx != -__builtin_inff()) {
    for (int c = 0; c < n_parts; ++c) {
      const float l = lse_parts[c * lstride + (int64_t)head * rows + row];
      if (l == -__builtin_inff()) continue;  // empty part
      const float w = expf(l - mx);
      sum += w;
      acc += w * *(const f32x4 *)(o_parts + c * ostride + ((int64_t)row * H + head) * D + 4 * c4);
    }
    acc *= 1.0f / sum;
  }
  store4(out, ((int64_t)row * H + head) * D + 4 * c4, acc, bf16 != 0);
  if (lse && c4 == 0)
    lse[(int64_t)head * rows + row] = mx == -__builtin_inff() ? mx : mx + logf(sum);
}

hipError_t launch_merge_split(const AttnParams &p, int D, bool bf16, hipStream_t stream) {
  clear_stale_launch_error();
  const int64_t n = (int64_t)p.total_s * p.H * (D / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_split_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     p, D, bf16 ? 1 : 0);
  return launch_result();
}

hipError_t launch_lse_merge(const float *o_parts, const float *lse_parts, int n_parts, int rows,
                            int H, int D, bool bf16, void *out, float *lse, hipStream_t stream) {
  clear_stale_launch_error();
  const int64_t n = (int64_t)rows * H * (D / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     o_parts, lse_parts, n_parts, rows, H, D, bf16 ? 1 : 0, out, lse);
  return launch_result();
}

}  // namespace bat
