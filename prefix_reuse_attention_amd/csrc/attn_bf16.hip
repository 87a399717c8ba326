// Prefill attention of the suffix rows over a paged, cached prefix plus the
// suffix itself, bf16 in / fp32 accumulate, on CDNA4 MFMA.
//
// The method (Bat page, "This paper's idea"): either the user history or a
// set of cached items is the prefix whose K/V is reused; the suffix tokens
// are fresh and see the prefix and each other, with no positions and no
// causal mask.  Per work item (request r, head h, a tile of 128 suffix rows,
// a prefix chunk) one workgroup of four waves streams key tiles: first the
// prefix tiles gathered through the block table, then the request's own
// suffix tiles, with an online softmax.  Crossing from the prefix tiles to
// the suffix tiles is the log-sum-exp merge of the prefix and suffix
// partials, done in registers.
//
// Data flow of one key tile (BN keys):
//   HBM/L2 --16B loads--> VGPRs --ds_write--> LDS (K row-major, V transposed)
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, A = K from LDS, B = Q in VGPRs
//   online softmax  on the S^T accumulator: each lane owns one query row
//   O^T += V^T P^T  v_mfma_f32_32x32x16_bf16, A = V^T from LDS, B = P in VGPRs
// Computing the transposed products makes the query row the lane index of
// both accumulators, so P goes from the S^T accumulator straight into the
// PV operand and the per-row rescale is a per-lane multiply.
#include "common.h"

namespace bat {

template <int D>
struct Bf16Cfg {
  static constexpr int BN = (D == 128) ? 64 : 128;  // keys per tile
  static constexpr int WAVES = 4;
  static constexpr int ROWS = 32;                   // query rows per wave
  static constexpr int BM = WAVES * ROWS;           // query rows per item
  static constexpr int K_STRIDE = D + 8;            // LDS row pitch (elements)
  static constexpr int V_STRIDE = BN + 8;
  static constexpr int K_ELEMS = BN * K_STRIDE;
  static constexpr int V_ELEMS = D * V_STRIDE;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int KG = BN / 4;                 // loader: groups of 4 keys
  static constexpr int DC = D / 8;                  // loader: 16-byte d chunks
  static constexpr int NB = BN / 32;                // 32-key MFMA blocks per tile
  static constexpr int ND = D / 32;                 // 32-wide d blocks of O
  static constexpr int KK = D / 16;                 // k-steps of QK^T
  static_assert(KG * DC == 256, "one 4x8 sub-tile per thread");
};

// Within each 32-key block the K tile is stored in LDS with its rows
// permuted, so that accumulator element i of lane-half hf of S^T holds key
// 16*(i/8) + 8*hf + i%8: eight consecutive keys per half-chunk, which is
// exactly the B-operand layout of the PV MFMA (and lets each lane read V^T
// with one 16-byte access).  pinv maps a key to its LDS row.
__device__ __forceinline__ int k_lds_row(int key) {
  const int k = key & 31;
  const int a = k >> 4, b = (k >> 3) & 1, c = (k >> 2) & 1, t = k & 3;
  return (key & ~31) | (8 * (2 * a + c) + 4 * b + t);
}

struct Bf16Tile {
  u32x4 k[4], v[4];
};

template <int D>
__device__ __forceinline__ void bf16_load_tile(const AttnParams &p, const ItemRange &x,
                                               int r, int head, int tile, int n_tiles_p,
                                               int m, int c, Bf16Tile &T) {
  using C = Bf16Cfg<D>;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if (tile < n_tiles_p) {
    const int key0 = x.p_begin + tile * C::BN + 4 * m;
    const uint16_t *pk = (const uint16_t *)p.pool_k[x.mode];
    const uint16_t *pv = (const uint16_t *)p.pool_v[x.mode];
    if (p.pool_bs_log2[x.mode] >= 2) {
      // the 4 keys share one block (tiles start at multiples of 4)
      int64_t off = key0 < x.p_end ? prefix_offset(p, r, x.mode, key0, head, D) : -1;
      if (key0 < x.p_end && off < 0 && p.err) atomicOr(p.err, kErrBlockId);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = off >= 0 && key0 + i < x.p_end;
        T.k[i] = ok ? *(const u32x4 *)(pk + off + i * D + 8 * c) : zero;
        T.v[i] = ok ? *(const u32x4 *)(pv + off + i * D + 8 * c) : zero;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t off = key0 + i < x.p_end ? prefix_offset(p, r, x.mode, key0 + i, head, D) : -1;
        if (key0 + i < x.p_end && off < 0 && p.err) atomicOr(p.err, kErrBlockId);
        T.k[i] = off >= 0 ? *(const u32x4 *)(pk + off + 8 * c) : zero;
        T.v[i] = off >= 0 ? *(const u32x4 *)(pv + off + 8 * c) : zero;
      }
    }
  } else {
    const int s0 = (tile - n_tiles_p) * C::BN + 4 * m;
    const uint16_t *ks = (const uint16_t *)p.k;
    const uint16_t *vs = (const uint16_t *)p.v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = s0 + i < x.n_s && x.q0 >= 0 && x.q0 + s0 + i < p.total_s;
      const int64_t off = ((int64_t)(x.q0 + s0 + i) * p.H + head) * D + 8 * c;
      T.k[i] = ok ? *(const u32x4 *)(ks + off) : zero;
      T.v[i] = ok ? *(const u32x4 *)(vs + off) : zero;
    }
  }
}

template <int D>
__device__ __forceinline__ void bf16_store_tile(uint16_t *stage, int m, int c, const Bf16Tile &T) {
  using C = Bf16Cfg<D>;
  uint16_t *Ks = stage;
  uint16_t *Vt = stage + C::K_ELEMS;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *(u32x4 *)(Ks + k_lds_row(4 * m + i) * C::K_STRIDE + 8 * c) = T.k[i];
  // transpose the 4 keys x 8 dims sub-tile: V^T[8c + d][4m .. 4m+3]
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t a0 = T.v[0][w], a1 = T.v[1][w], a2 = T.v[2][w], a3 = T.v[3][w];
    u32x2 lo, hi;
    lo[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);  // d = 2w:   keys 0,1
    lo[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);  //           keys 2,3
    hi[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);  // d = 2w+1: keys 0,1
    hi[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
    *(u32x2 *)(Vt + (8 * c + 2 * w) * C::V_STRIDE + 4 * m) = lo;
    *(u32x2 *)(Vt + (8 * c + 2 * w + 1) * C::V_STRIDE + 4 * m) = hi;
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnParams p) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::STAGE];

  const WorkItem it = p.items[blockIdx.x];
  if (it.r < 0 || it.r >= p.B || it.h < 0 || it.h >= p.H) return;
  const ItemRange x = item_range(p, it);
  const int head = it.h;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int lm = tid % C::KG, lc = tid / C::KG;  // loader sub-tile

  // Q fragments (B operand of S^T = K Q^T): lane holds row `col`,
  // dims 16*kk + 8*hf .. +7
  const int row = it.m_tile * C::BM + wave * C::ROWS + col;
  const bool row_ok = row < x.n_s && x.q0 >= 0 && x.q0 + row < p.total_s;
  bf16x8 qf[C::KK];
  {
    const uint16_t *q = (const uint16_t *)p.q + ((int64_t)(x.q0 + row) * p.H + head) * D;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row_ok) w = *(const u32x4 *)(q + 16 * kk + 8 * hf);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int n_pkeys = x.p_end - x.p_begin;
  const int n_tiles_p = (n_pkeys + C::BN - 1) / C::BN;
  const int n_tiles = n_tiles_p + (x.with_suffix ? (x.n_s + C::BN - 1) / C::BN : 0);

  f32x16 o[C::ND];
#pragma unroll
  for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[nd][i] = 0.f;
  float m_run = -__builtin_inff();  // running max, log2 domain (scaled)
  float l_run = 0.f;                // this lane-half's share of the row sum
  const float cs = p.scale_log2;
  constexpr float kTau = 8.0f;      // rescale only when the max grows by > 2^8

  Bf16Tile T;
  if (n_tiles > 0) bf16_load_tile<D>(p, x, it.r, head, 0, n_tiles_p, lm, lc, T);

  for (int t = 0; t < n_tiles; ++t) {
    uint16_t *stage = lds + (t & 1) * C::STAGE;
    bf16_store_tile<D>(stage, lm, lc, T);
    __syncthreads();
    if (t + 1 < n_tiles) bf16_load_tile<D>(p, x, it.r, head, t + 1, n_tiles_p, lm, lc, T);

    const uint16_t *Ks = stage;
    const uint16_t *Vt = stage + C::K_ELEMS;
    // ---- S^T = K Q^T
    f32x16 s[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[nb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        const bf16x8 a = *(const bf16x8 *)(Ks + (32 * nb + col) * C::K_STRIDE + 16 * kk + 8 * hf);
        s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[nb], 0, 0, 0);
      }
    }
    // ---- mask keys past the end of a partial tile
    const int valid = (t < n_tiles_p) ? min(C::BN, n_pkeys - t * C::BN)
                                      : min(C::BN, x.n_s - (t - n_tiles_p) * C::BN);
    if (valid < C::BN) {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * nb + 16 * (i >> 3) + 8 * hf + (i & 7);
          if (key >= valid) s[nb][i] = -__builtin_inff();
        }
    }
    // ---- online softmax (row = this lane's column of S^T)
    float mx = -__builtin_inff();
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[nb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * cs;
    if (__any(mt > m_run + kTau)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[nd][i] *= alpha;
      m_run = m_new;
    }
    float lsum = 0.f;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][i], cs, -m_run));
        s[nb][i] = e;
        lsum += e;
      }
    l_run += lsum;
    // ---- O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int kc = 0; kc < 2 * C::NB; ++kc) {
      const f32x16 &sb = s[kc >> 1];
      const int e0 = 8 * (kc & 1);
      u32x4 pw;
      pw[0] = pack_bf16x2(sb[e0 + 0], sb[e0 + 1]);
      pw[1] = pack_bf16x2(sb[e0 + 2], sb[e0 + 3]);
      pw[2] = pack_bf16x2(sb[e0 + 4], sb[e0 + 5]);
      pw[3] = pack_bf16x2(sb[e0 + 6], sb[e0 + 7]);
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int nd = 0; nd < C::ND; ++nd) {
        const bf16x8 a = *(const bf16x8 *)(Vt + (32 * nd + col) * C::V_STRIDE + 16 * kc + 8 * hf);
        o[nd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[nd], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: normalise, write O (and lse) or the split partial
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  const float lse_nat = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  if (!row_ok) return;
  if (x.n_chunks <= 1) {
    uint16_t *out = (uint16_t *)p.out + ((int64_t)(x.q0 + row) * p.H + head) * D;
#pragma unroll
    for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w[0] = pack_bf16x2(o[nd][4 * j + 0] * inv, o[nd][4 * j + 1] * inv);
        w[1] = pack_bf16x2(o[nd][4 * j + 2] * inv, o[nd][4 * j + 3] * inv);
        *(u32x2 *)(out + 32 * nd + 8 * j + 4 * hf) = w;
      }
    if (p.lse && hf == 0) p.lse[(int64_t)head * p.total_s + x.q0 + row] = lse_nat;
  } else {
    const int64_t pr = (int64_t)x.part_off + (int64_t)it.chunk * x.n_s + row;
    float *po = p.part_o + (pr * p.H + head) * D;
#pragma unroll
    for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 w = {o[nd][4 * j] * inv, o[nd][4 * j + 1] * inv, o[nd][4 * j + 2] * inv,
                   o[nd][4 * j + 3] * inv};
        *(f32x4 *)(po + 32 * nd + 8 * j + 4 * hf) = w;
      }
    if (hf == 0) p.part_lse[pr * p.H + head] = lse_nat;
  }
}

int bf16_rows_per_item(int D) { return D == 128 ? Bf16Cfg<128>::BM : Bf16Cfg<64>::BM; }
int bf16_keys_per_tile(int D) { return D == 128 ? Bf16Cfg<128>::BN : Bf16Cfg<64>::BN; }

hipError_t launch_attn_bf16(const AttnParams &p, int D, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
  else if (D == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bat
