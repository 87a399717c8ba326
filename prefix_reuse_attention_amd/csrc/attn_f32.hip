// Prefill attention, float32 in / float32 out.  The scores and the running
// sums are taken in float64: a product of two fp32 values is exact there, so
// each score carries one rounding, and the row sum and the output accumulator
// over thousands of keys do not drift (summed in fp32 they miss a 1e-5
// max-abs bar at about 1500 keys).  The exponentials take an fp32 argument,
// s*scale*log2(e) - m formed in fp64, which is small for the terms that
// matter, and run in fp32.
//
// Same semantics and work items as the bf16 kernel (Bat page, "This paper's
// idea": cached prefix, fresh suffix that sees the prefix and itself).  This
// path serves fp32 models and the fp32 parity configuration; it is plain
// VALU code: four lanes share one query row (each holds a quarter of q and
// of the output), keys are staged through LDS in tiles of 32.
#include "common.h"

namespace bat {

constexpr int kF32Rows = 64;   // query rows per item
constexpr int kF32Keys = 32;   // keys per LDS tile
constexpr int kF32Tpr = 4;     // lanes per query row

// cs: softmax_scale * log2(e) in fp64.
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnParams p, double cs) {
  constexpr int DQ = D / kF32Tpr;          // dims held per lane
  constexpr int KROW = D + 4;              // LDS pitch (floats)
  __shared__ __attribute__((aligned(16))) float Ks[kF32Keys * KROW];
  __shared__ __attribute__((aligned(16))) float Vs[kF32Keys * KROW];

  const WorkItem it = work_item(p, blockIdx.x);
  if (it.r < 0 || it.r >= p.B || it.h < 0 || it.h >= p.H) return;
  const ItemRange x = item_range(p, it);
  const int head = it.h;
  const int kv_head = head / (p.H / p.H_kv);
  const int tid = threadIdx.x;
  const int rloc = tid / kF32Tpr, part = tid % kF32Tpr;
  const int row = it.m_tile * kF32Rows + rloc;
  const bool row_ok = row < x.n_s && x.q0 >= 0 && x.q0 + row < p.total_s;

  double q[DQ], o[DQ];
  {
    const float *qp = (const float *)p.q + ((int64_t)(x.q0 + row) * p.H + head) * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; ++d) {
      q[d] = row_ok ? (double)qp[d] : 0.0;
      o[d] = 0.0;
    }
  }
  // m_run: the running max in the log2 domain, held as an fp32 value (any
  // shift works as long as the sums and the lse use the same one)
  float m_run = -__builtin_inff();
  double l_run = 0.0;

  const int n_pkeys = x.p_end - x.p_begin;
  const int n_tiles_p = (n_pkeys + kF32Keys - 1) / kF32Keys;
  const int n_tiles = n_tiles_p + (x.with_suffix ? (x.n_s + kF32Keys - 1) / kF32Keys : 0);
  // prefix-only rows of a request with no prefix: no keys, nothing to write
  // (the merge that follows reads that partial as empty)
  if (n_tiles == 0) return;
  constexpr int V4_PER_ROW = D / 4;

  for (int t = 0; t < n_tiles; ++t) {
    const bool pre = t < n_tiles_p;
    const int base = pre ? x.p_begin + t * kF32Keys : (t - n_tiles_p) * kF32Keys;
    const int valid = pre ? min(kF32Keys, x.p_end - base) : min(kF32Keys, x.n_s - base);
    __syncthreads();  // previous tile fully consumed
    for (int e = tid; e < kF32Keys * V4_PER_ROW; e += 256) {
      const int j = e / V4_PER_ROW, c4 = e % V4_PER_ROW;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (j < valid && (pre || (x.q0 >= 0 && x.q0 + base + j < p.total_s))) {
        int64_t off;
        const float *kb, *vb;
        if (pre) {
          off = prefix_offset(p, it.r, x.mode, base + j, kv_head, D);
          if (off < 0 && p.err) atomicOr(p.err, kErrBlockId);
          kb = (const float *)p.pool_k[x.mode];
          vb = (const float *)p.pool_v[x.mode];
        } else {
          off = ((int64_t)(x.q0 + base + j) * p.H_kv + kv_head) * D;
          kb = (const float *)p.k;
          vb = (const float *)p.v;
        }
        if (off >= 0) {
          kv = *(const f32x4 *)(kb + off + 4 * c4);
          vv = *(const f32x4 *)(vb + off + 4 * c4);
        }
      }
      *(f32x4 *)(Ks + j * KROW + 4 * c4) = kv;
      *(f32x4 *)(Vs + j * KROW + 4 * c4) = vv;
    }
    __syncthreads();
    // scores of this tile (every lane of a row group ends with all of them)
    double s[kF32Keys];
    double mx = -__builtin_inf();
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      double acc = 0.0;
#pragma unroll
      for (int d = 0; d < DQ; ++d)
        acc = __builtin_fma(q[d], (double)Ks[j * KROW + part * DQ + d], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      s[j] = j < valid ? acc : -__builtin_inf();
      mx = __builtin_fmax(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, (float)(mx * cs));
    // the same alpha scales the sum and the accumulator, so its own
    // rounding cancels in their ratio
    const double alpha = (double)exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < DQ; ++d) o[d] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      const double e = (double)exp2f((float)(s[j] * cs - (double)m_run));
      l_run += e;
#pragma unroll
      for (int d = 0; d < DQ; ++d) o[d] = __builtin_fma(e, (double)Vs[j * KROW + part * DQ + d], o[d]);
    }
  }

  if (!row_ok) return;
  const double inv = 1.0 / l_run;
  const float lse_nat = (float)(((double)m_run + log2(l_run)) * 0.69314718055994530942);
  if (!x.partial) {
    float *op = (float *)p.out + ((int64_t)(x.q0 + row) * p.H + head) * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; ++d) op[d] = (float)(o[d] * inv);
    if (p.lse && part == 0) p.lse[(int64_t)head * p.total_s + x.q0 + row] = lse_nat;
  } else {
    const int64_t pr = (int64_t)x.part_off + (int64_t)it.chunk * x.n_s + row;
    float *po = p.part_o + (pr * p.H + head) * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; ++d) po[d] = (float)(o[d] * inv);
    if (part == 0) p.part_lse[pr * p.H + head] = lse_nat;
  }
}

int f32_rows_per_item() { return kF32Rows; }
int f32_keys_per_tile() { return kF32Keys; }

hipError_t launch_attn_f32(const AttnParams &p, int D, int grid, double scale_log2,
                           hipStream_t stream) {
  clear_stale_launch_error();
  if (grid <= 0) return hipSuccess;
  if (D == 32)
    hipLaunchKernelGGL(attn_f32_kernel<32>, dim3(grid), dim3(256), 0, stream, p, scale_log2);
  else if (D == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(256), 0, stream, p, scale_log2);
  else if (D == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(grid), dim3(256), 0, stream, p, scale_log2);
  else
    return hipErrorInvalidValue;
  return launch_result();
}

}  // namespace bat
