// Prefill attention of the suffix rows over a paged, cached prefix plus the
// suffix itself, bf16 in / fp32 accumulate, on CDNA4 MFMA.
//
// The method (Bat page, "This paper's idea"): either the user history or a
// set of cached items is the prefix whose K/V is reused; the suffix tokens
// are fresh and see the prefix and each other, with no positions and no
// causal mask.  Per work item (request r, head h, a tile of 32*W suffix
// rows, a prefix chunk) one workgroup of W waves (W = 8 for long suffixes,
// else 4) streams key tiles: first the prefix tiles gathered through the
// block table, then the request's own suffix tiles, with an online softmax.
// Crossing from the prefix tiles to the suffix tiles is the log-sum-exp
// merge of the prefix and suffix partials, done in registers.
//
// Two kernels: attn_bf16_kernel (four waves), where every wave runs S^T,
// softmax and PV of each tile in turn, and attn_bf16_pp_kernel (eight
// waves, both head dims), where two groups of four waves alternate between
// the MFMA work and the softmax so that each SIMD always holds one wave of
// each kind.
//
// Data flow of one key tile (BN keys: 16 KB of K and 16 KB of V, 8 + 8 KB
// in the eight-wave kernel at head dim 64):
//   HBM/L2 --buffer_load_dwordx4 ... lds--> LDS, row-major, 16-byte
//            chunks XOR-swizzled per row (no VGPR staging, no LDS store
//            instructions); two LDS stages, the next tile's copy in flight
//            while the current one is consumed, one barrier per tile
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, A = K rows (ds_read_b128),
//                   B = Q held in VGPRs for the whole item
//   online softmax  per 32-key block on the S^T accumulator; each lane owns
//                   one query row, the two lane halves meet through
//                   v_permlane32_swap
//   O^T += V^T P^T  v_mfma_f32_32x32x16_bf16, A = V^T read from the
//                   row-major V tile by ds_read_b64_tr_b16 (the LDS
//                   transpose read), B = P straight from the S^T registers
// Computing the transposed products makes the query row the lane index of
// both accumulators, so P never leaves registers and the per-row rescale
// is a per-lane multiply.
#include "common.h"

#include <utility>

namespace bat {

// 16 zero bytes: the copy source of keys past the end of a tile in the
// global-load gather, so that every lane issues its load and masked keys
// hold zeros.
__device__ __attribute__((aligned(16))) uint32_t g_zero16[4];

// Pools smaller than this are gathered with buffer loads and 32-bit
// offsets; an offset of kPastPool lies past any such pool's end, and with
// the 16 bytes of one load added it still does not wrap.
constexpr int64_t kBufferPoolLimit = 0x7FFFFFF0;
constexpr int kPastPool = 0x7FFFFFF0;

// Workgroup shape: W waves of 32 query rows share every K/V tile.
template <int W>
struct WgCfg {
  static constexpr int WAVES = W;
  static constexpr int THREADS = 64 * W;
  static constexpr int ROWS = 32;                   // query rows per wave
  static constexpr int BM = W * ROWS;               // query rows per item
};

// Keys per tile of the four-wave kernel: a 16 KB tile of K (and of V) at
// either head dim.  The ping-pong kernel takes 64-key tiles at both.
constexpr int bf16_default_bn(int D) { return D == 128 ? 64 : 128; }
constexpr int kPpBN = 64;

// Tile geometry: head dim and keys per tile.
template <int D, int BN_ = bf16_default_bn(D)>
struct Bf16Cfg {
  static constexpr int BN = BN_;                    // keys per tile
  static constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  static constexpr int RB = D * 2;                  // bytes per K/V row
  static constexpr int RPI = 64 / CPR;              // rows per wave copy instruction
  static constexpr int TILE = BN * RB;              // bytes of one K (or V) tile
  static constexpr int PIECES = TILE / 1024;        // one-kilobyte copy pieces per tile
  static constexpr int NB = BN / 32;                // 32-key MFMA blocks per tile
  static constexpr int ND = D / 32;                 // 32-wide d blocks of O
  static constexpr int KK = D / 16;                 // k-steps of QK^T
  static_assert(TILE % 1024 == 0 && BN % 32 == 0, "whole pieces, whole MFMA blocks");
};

// Chunk swizzle of K/V row r: chunk c of the row is stored at c ^ swz(r).
// With 64 LDS banks it makes three access patterns conflict-free: the
// S^T operand read (16 consecutive lanes, 16 distinct rows, one chunk),
// the transpose read (4 consecutive rows x 4 chunks per 32 lanes) and the
// copy itself (contiguous 1 KB per instruction).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// The K operand lane m of a 32-key block reads key row pi(m), so that
// accumulator element i of lane-half hf of S^T holds key
// 16*(i/8) + 8*hf + i%8: eight consecutive keys per half-chunk, which is the
// B-operand layout the PV MFMA wants (and the order the transpose read of V
// produces).
__device__ __forceinline__ int k_row_of_lane(int m) {
  const int j = m >> 3, h = (m >> 2) & 1, t = m & 3;
  return 16 * (j >> 1) + 8 * h + 4 * (j & 1) + t;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// Candidate-isolated rows of single-token candidates: the row sees its
// request's prefix and its own token.  The prefix part arrives as the
// kernel's running state (unnormalised o with row sum l_tot over 2^(s - m)
// in the log2 domain); the own key is one more score, merged exactly:
//     s = scale * <q, k_self>,  lse = log2(2^(m + log2 l_tot) + 2^s),
//     out = (o + 2^(s - m) v_self) / (l_tot + 2^(s - m))  (in safe form).
// The lane pair (lane, lane ^ 32) of a row holds the output elements
// 32*nd + 8*j + 4*hf + e; each lane reads the same elements of q, k_self and
// v_self (8-byte pieces), the pair sums the dot product with one shuffle.
// l_tot == 0 (no prefix keys) leaves the own token alone.
template <int D>
__device__ __forceinline__ void write_with_self_key(const AttnParams &p, int64_t qrow, int head,
                                                    int kv_head, int hf,
                                                    const f32x16 (&o)[D / 32], float m_run,
                                                    float l_tot) {
  constexpr int ND = D / 32;
  const uint16_t *qp = (const uint16_t *)p.q + (qrow * p.H + head) * D + 4 * hf;
  const uint16_t *kp = (const uint16_t *)p.k + (qrow * p.H_kv + kv_head) * D + 4 * hf;
  const uint16_t *vp = (const uint16_t *)p.v + (qrow * p.H_kv + kv_head) * D + 4 * hf;
  u32x2 vw[ND][4];
  float dot = 0.f;
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = 32 * nd + 8 * j;
      const u32x2 qw = *(const u32x2 *)(qp + off);
      const u32x2 kw = *(const u32x2 *)(kp + off);
      vw[nd][j] = *(const u32x2 *)(vp + off);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t a = qw[w], b = kw[w];
        dot = __builtin_fmaf(__builtin_bit_cast(float, a << 16),
                             __builtin_bit_cast(float, b << 16), dot);
        dot = __builtin_fmaf(__builtin_bit_cast(float, a & 0xffff0000u),
                             __builtin_bit_cast(float, b & 0xffff0000u), dot);
      }
    }
  dot += __shfl_xor(dot, 32);
  const float s2 = dot * p.scale_log2;
  const bool have = l_tot > 0.f;
  const float lp = have ? m_run + __log2f(l_tot) : s2;
  const float mx = fmaxf(lp, s2);
  const float wp = have ? __builtin_amdgcn_exp2f(lp - mx) : 0.f;
  const float wc = __builtin_amdgcn_exp2f(s2 - mx);
  const float iw = 1.0f / (wp + wc);
  const float a = have ? wp * iw / l_tot : 0.f, b = wc * iw;
  uint16_t *out = (uint16_t *)p.out + (qrow * p.H + head) * D + 4 * hf;
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[4];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t x = vw[nd][j][w];
        v[2 * w] = __builtin_bit_cast(float, x << 16);
        v[2 * w + 1] = __builtin_bit_cast(float, x & 0xffff0000u);
      }
      u32x2 w;
      w[0] = pack_bf16x2(a * o[nd][4 * j + 0] + b * v[0], a * o[nd][4 * j + 1] + b * v[1]);
      w[1] = pack_bf16x2(a * o[nd][4 * j + 2] + b * v[2], a * o[nd][4 * j + 3] + b * v[3]);
      *(u32x2 *)(out + 32 * nd + 8 * j) = w;
    }
  if (p.lse && hf == 0)
    p.lse[(int64_t)head * p.total_s + qrow] = (mx + __log2f(wp + wc)) * 0.69314718055994530942f;
}


__device__ __forceinline__ float row_max_both_halves(float v) {
  // v_permlane32_swap(v, v) leaves {own, other half} in its two results
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                                  __builtin_bit_cast(uint32_t, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Per-lane byte offsets of the MFMA operand reads inside one LDS stage.  The
// chunk swizzle of a row depends only on the row's low bits, which the
// 32-key block index and the 16-key chunk index do not change, so each read
// is a lane constant plus an immediate (block * 32 rows, chunk * 16 rows).
template <int D>
struct LdsOffsets {
  using C = Bf16Cfg<D>;
  int k[C::KK];      // S^T operand: key row pi(col) of block 0, d chunk 2kk+hf
  int v[C::ND][2];   // transpose read of keys 8hf + 4e4 + 0..3, d block nd
  __device__ __forceinline__ void init(int lane) {
    const int col = lane & 31, hf = lane >> 5, g = lane >> 4, i16 = lane & 15;
    const int krow = k_row_of_lane(col);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
      k[kk] = krow * C::RB + (((2 * kk + hf) ^ swz<D>(krow)) << 4);
    const int kq = i16 >> 2, q = i16 & 3;
#pragma unroll
    for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
      for (int e4 = 0; e4 < 2; ++e4) {
        const int key = 8 * hf + 4 * e4 + kq;
        const int d = 32 * nd + 16 * (g & 1) + 4 * q;
        v[nd][e4] = key * C::RB + (((d >> 3) ^ swz<D>(key)) << 4) + (q & 1) * 8;
      }
  }
};

// Everything one workgroup needs to copy the tiles of its item.
//
// Each wave issues CPW 16-byte-per-lane copies of K and CPW of V per tile;
// copy j of wave w fills LDS bytes [(CPW*w+j)*1024, +1024) of the stage, i.e.
// tile row r = RPI*(CPW*w+j) + lane/CPR, stored chunk lane%CPR, which holds
// the row's global chunk (lane%CPR) ^ swz(r).
//
// When a pool block holds at least one tile (block_size >= BN), a tile is
// one contiguous run inside one block (or of the packed suffix), so the
// copy is a buffer load: a per-tile base in SGPRs, lane-constant offsets,
// and the descriptor's size cutting off rows past the end (they read as
// zero).  Smaller blocks (item pools) gather per lane: a buffer load over
// the whole pool with one 32-bit offset per lane (keys past the end get an
// offset past the descriptor's size and read as zero), or, for a pool of
// 2 GiB or more (FLAT), a global load per lane.  The buffer form keeps the
// LDS-read wait counts exact: a global (FLAT-encoded) copy into LDS counts
// on the LDS counter too, so while one can be in flight every LDS read has
// to be waited for in full.  A block id out of range is remembered in
// `bad` and reported once, after the loop.
template <int D, int W, bool FLAT, int BN_ = bf16_default_bn(D)>
struct TileCopy {
  using C = Bf16Cfg<D, BN_>;
  // copy instructions per wave per tile: each of the W copying waves takes
  // PIECES / W of the tile's one-kilobyte pieces of K and of V
  static constexpr int CPW = C::PIECES / W;
  static_assert(CPW >= 1 && CPW * W == C::PIECES, "pieces per copying wave");
  const uint8_t *pool_k, *pool_v, *ks, *vs;  // prefix pool / suffix K,V bases
  const int32_t *bt_row;                     // this request's block-table row
  int lg, blocks, bt_stride, H, head, q0, n_s, p_begin, p_end, n_tiles_p, n_tiles;
  bool whole_blocks;                         // block_size >= BN
  int64_t block_bytes, head_bytes;           // H*bs*RB, head*bs*RB
  int32_t pool_records;                      // bytes of the prefix pool (< 2 GiB unless FLAT)
  // Per-item table of whole-tile copies: for tile u (a prefix tile of a
  // pool whose blocks hold whole tiles, or a suffix tile) the K source
  // address, byte count and row stride; its V source is the K address plus
  // dv_p (prefix) or dv_s (suffix).  Filled once per item by all threads,
  // it replaces the per-tile block-id load and address arithmetic that
  // every wave would otherwise repeat.  Items of more tiles, and per-key
  // gather tiles, plan each tile as it comes.
  static constexpr int kTabTiles = 512;
  u32x4 *tab;
  bool use_tab;
  int64_t dv_p, dv_s;
  int wave, lane;
  int row[CPW], cb[CPW];                     // tile row and stored-chunk source byte
  bool bad = false;                          // a block id out of range was seen

  // LDS byte offset of this wave's first piece in a stage
  uint32_t wofs;
  // keeps wofs from being folded into per-piece constants that are then
  // held (or spilled) across the tile loop: called once per tile
  __device__ __forceinline__ void anchor() { asm volatile("" : "+s"(wofs)); }

  __device__ __forceinline__ void init_lanes() {
    wofs = CPW * wave * 1024;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      row[j] = C::RPI * (CPW * wave + j) + lane / C::CPR;
      cb[j] = ((lane % C::CPR) ^ swz<D>(row[j])) << 4;
    }
  }

  // block ids of prefix tile `tile` (-1 = none): one per tile for whole
  // blocks, else one per row this lane copies
  __device__ __forceinline__ void load_ids(int tile, int (&ids)[CPW]) const {
    if (use_tab && whole_blocks) return;  // the table holds the block ids
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int key = p_begin + tile * C::BN + (whole_blocks ? 0 : row[j]);
      const int slot = key >> lg;
      const bool ok = tile < n_tiles_p && key < p_end && slot < bt_stride &&
                      (j == 0 || !whole_blocks);
      ids[j] = ok ? bt_row[slot] : -1;
    }
  }

  // Where the 2*CPW copy instructions of one tile read from: a buffer
  // descriptor per tensor and a byte offset per lane (FLAT gathers: an
  // address per lane).  Planning is separate from issuing so that the
  // instructions can be spread over the MFMAs of the previous tile: issued
  // together by all waves they queue at the texture unit and stall every
  // wave's in-order issue.  A tile past the last plans zero-size copies.
  struct Plan {
    __amdgpu_buffer_rsrc_t rk, rv;
    int voff[CPW];
    const uint8_t *ksrc[FLAT ? CPW : 1], *vsrc[FLAT ? CPW : 1];
    bool flat_gather;
  };

  // Fill the table (thread tid of nthreads); the caller waits for the LDS
  // stores and meets the other waves at a barrier before the first plan.
  __device__ __forceinline__ void fill_tab(int tid, int nthreads) {
    for (int u = tid; u < n_tiles; u += nthreads) {
      const uint8_t *addr = pool_k;
      int records = 0, stride = C::RB;
      if (u < n_tiles_p) {
        if (whole_blocks) {
          const int key0 = p_begin + u * C::BN;
          const int slot = key0 >> lg;
          const int blk = slot < bt_stride ? bt_row[slot] : -1;
          const bool inb = blk >= 0 && blk < blocks;
          bad |= !inb;
          if (inb) {
            addr = pool_k + (int64_t)blk * block_bytes + head_bytes +
                   (int64_t)(key0 & ((1 << lg) - 1)) * C::RB;
            records = min(C::BN, p_end - key0) * C::RB;
          }
        }
      } else {
        const int s0 = (u - n_tiles_p) * C::BN;
        addr = ks + ((int64_t)(q0 + s0) * H + head) * C::RB;
        stride = H * C::RB;
        const int nv = min(C::BN, n_s - s0);
        records = nv > 0 ? (nv - 1) * stride + C::RB : 0;
      }
      const uint64_t a = (uint64_t)addr;
      tab[u] = u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)records, (uint32_t)stride};
    }
  }

  __device__ __forceinline__ Plan plan(int tile, const int (&ids)[CPW]) {
    constexpr int kFlags = 0x00020000;  // raw buffer, 32-bit dword format
    Plan pl;
    pl.flat_gather = false;
    if (use_tab && (tile >= n_tiles_p || whole_blocks)) {
      // whole-tile copy from the table (a tile past the last copies nothing)
      const u32x4 e = tile < n_tiles ? tab[tile] : u32x4{0u, 0u, 0u, 0u};
      const uint64_t a = ((uint64_t)__builtin_amdgcn_readfirstlane(e[1]) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane(e[0]);
      const int records = __builtin_amdgcn_readfirstlane(e[2]);
      const int stride = __builtin_amdgcn_readfirstlane(e[3]);
      const uint8_t *kb = (const uint8_t *)a;
      const uint8_t *vb = kb + (tile < n_tiles_p ? dv_p : dv_s);
      pl.rk = __builtin_amdgcn_make_buffer_rsrc((void *)kb, (short)0, records, kFlags);
      pl.rv = __builtin_amdgcn_make_buffer_rsrc((void *)vb, (short)0, records, kFlags);
#pragma unroll
      for (int j = 0; j < CPW; ++j) pl.voff[j] = row[j] * stride + cb[j];
      return pl;
    }
    if (tile < n_tiles_p && !whole_blocks) {
      pl.flat_gather = FLAT;
      pl.rk = __builtin_amdgcn_make_buffer_rsrc((void *)pool_k, (short)0,
                                                FLAT ? 0 : pool_records, kFlags);
      pl.rv = __builtin_amdgcn_make_buffer_rsrc((void *)pool_v, (short)0,
                                                FLAT ? 0 : pool_records, kFlags);
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        const int key = p_begin + tile * C::BN + row[j];
        const int blk = ids[j];
        const bool inb = blk >= 0 && blk < blocks;
        bad |= key < p_end && !inb;
        const bool use = key < p_end && inb;
        const int64_t off =
            ((((int64_t)blk * H + head) << lg) | (key & ((1 << lg) - 1))) * C::RB + cb[j];
        pl.voff[j] = use ? (int)off : kPastPool;
        if constexpr (FLAT) {
          pl.ksrc[j] = use ? pool_k + off : (const uint8_t *)g_zero16;
          pl.vsrc[j] = use ? pool_v + off : (const uint8_t *)g_zero16;
        }
      }
      return pl;
    }
    const uint8_t *kb, *vb;
    int records, stride;
    if (tile < n_tiles_p) {
      const int key0 = p_begin + tile * C::BN;
      const int blk = __builtin_amdgcn_readfirstlane(ids[0]);
      const bool inb = blk >= 0 && blk < blocks;
      bad |= !inb;
      const int64_t off = inb ? (int64_t)blk * block_bytes + head_bytes +
                                    (int64_t)(key0 & ((1 << lg) - 1)) * C::RB
                              : 0;
      kb = pool_k + off;
      vb = pool_v + off;
      records = inb ? min(C::BN, p_end - key0) * C::RB : 0;
      stride = C::RB;
    } else {
      const int s0 = max(tile - n_tiles_p, 0) * C::BN;
      const int64_t off = ((int64_t)(q0 + s0) * H + head) * C::RB;
      kb = ks + off;
      vb = vs + off;
      const int nv = tile < n_tiles ? min(C::BN, n_s - s0) : 0;
      stride = H * C::RB;
      records = nv > 0 ? (nv - 1) * stride + C::RB : 0;
    }
    pl.rk = __builtin_amdgcn_make_buffer_rsrc((void *)kb, (short)0, records, kFlags);
    pl.rv = __builtin_amdgcn_make_buffer_rsrc((void *)vb, (short)0, records, kFlags);
#pragma unroll
    for (int j = 0; j < CPW; ++j) pl.voff[j] = row[j] * stride + cb[j];
    return pl;
  }

  // The table entry of tile `tile` (zeros past the last tile); read a step
  // ahead of plan_tab so that its LDS latency is hidden.
  __device__ __forceinline__ u32x4 tab_entry(int tile) const {
    return tile < n_tiles ? tab[tile] : u32x4{0u, 0u, 0u, 0u};
  }
  // The plan of a whole-tile copy from its table entry (items whose tiles
  // all come from the table: use_tab and whole_blocks).
  __device__ __forceinline__ Plan plan_tab(int tile, const u32x4 &e) const {
    constexpr int kFlags = 0x00020000;  // raw buffer, 32-bit dword format
    Plan pl;
    pl.flat_gather = false;
    const uint64_t a = ((uint64_t)__builtin_amdgcn_readfirstlane(e[1]) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane(e[0]);
    const int records = __builtin_amdgcn_readfirstlane(e[2]);
    const int stride = __builtin_amdgcn_readfirstlane(e[3]);
    const uint8_t *kb = (const uint8_t *)a;
    const uint8_t *vb = kb + (tile < n_tiles_p ? dv_p : dv_s);
    pl.rk = __builtin_amdgcn_make_buffer_rsrc((void *)kb, (short)0, records, kFlags);
    pl.rv = __builtin_amdgcn_make_buffer_rsrc((void *)vb, (short)0, records, kFlags);
#pragma unroll
    for (int j = 0; j < CPW; ++j) pl.voff[j] = row[j] * stride + cb[j];
    return pl;
  }

  // Copy instruction j of 2*CPW (K pieces first, then V) into the stage at
  // kl / vl.
  __device__ __forceinline__ void fire(const Plan &pl, int j, uint8_t *kl, uint8_t *vl) const {
    const bool is_v = j >= CPW;
    const int q = is_v ? j - CPW : j;
    uint8_t *dst = (is_v ? vl : kl) + wofs + q * 1024;
    if (FLAT && pl.flat_gather)
      __builtin_amdgcn_global_load_lds(is_v ? pl.vsrc[FLAT ? q : 0] : pl.ksrc[FLAT ? q : 0], dst,
                                       16, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_v ? pl.rv : pl.rk, dst, 16, pl.voff[q], 0, 0, 0);
  }

  // Issue the whole copy of tile `tile` into one stage at once.
  __device__ __forceinline__ void issue(int tile, const int (&ids)[CPW], uint8_t *kl,
                                        uint8_t *vl) {
    const Plan pl = plan(tile, ids);
#pragma unroll
    for (int j = 0; j < 2 * CPW; ++j) fire(pl, j, kl, vl);
  }
};

struct SoftmaxState {
  float m_run = -__builtin_inff();  // running max, log2 domain (scaled)
  float l_run = 0.f;                // this lane-half's share of the row sum
};

__device__ __forceinline__ float max16(const f32x16 &v) {
  // max3 tree: 8 instructions for 16 values
  const float a = fmaxf(fmaxf(v[0], v[1]), v[2]), b = fmaxf(fmaxf(v[3], v[4]), v[5]);
  const float c = fmaxf(fmaxf(v[6], v[7]), v[8]), d = fmaxf(fmaxf(v[9], v[10]), v[11]);
  const float e = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(fmaxf(a, b), fmaxf(c, d)), fmaxf(e, v[15]));
}

// One key tile: S^T, then per 32-key block the online softmax and
// O^T += V^T P^T.  hook(i) runs after S^T MFMA i.  Every LDS operand is read two MFMAs ahead of its use
// (hard scheduling barriers keep the compiler from moving the reads back
// next to their MFMAs, where each would wait out the full LDS latency),
// and the first two V operands of a block are read before its softmax so
// that they arrive during the exponentials.
template <int D, typename Hook>
__device__ __forceinline__ void compute_tile(const uint8_t *kl, const uint8_t *vl,
                                             const bf16x8 (&qf)[Bf16Cfg<D>::KK],
                                             f32x16 (&o)[Bf16Cfg<D>::ND], SoftmaxState &sm,
                                             float cs, int valid, int lane,
                                             const LdsOffsets<D> &lo, Hook &&hook) {
  using C = Bf16Cfg<D>;
  constexpr float kTau = 8.0f;  // rescale only when the max grows by > 2^8
  constexpr int NS = C::NB * C::KK;  // MFMAs of S^T
  constexpr int NV = 2 * C::ND;      // PV MFMAs per 32-key block
  const int hf = lane >> 5;

  // ---- S^T: MFMA i accumulates block i % NB, k-step i / NB, so that
  // consecutive MFMAs are independent
  auto kread = [&](int i) __attribute__((always_inline)) {
    return *(const bf16x8 *)(kl + lo.k[i / C::NB] + (i % C::NB) * 32 * C::RB);
  };
  f32x16 s[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[nb][i] = 0.f;
  bf16x8 a[3];
  a[0] = kread(0);
  a[1] = kread(1);
  // MFMA runs at raised wave priority: while this wave issues MFMAs, the
  // other wave on the SIMD fills the gaps with its vector work
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (i + 2 < NS) a[(i + 2) % 3] = kread(i + 2);
    s[i % C::NB] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % 3], qf[i / C::NB], s[i % C::NB], 0, 0, 0);
    hook(i);  // the caller's copy instructions, spread over the S^T MFMAs
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);

  // PV operand j of block nb: 16-key chunk 2nb + j / ND, d block j % ND,
  // two transpose reads (group lane 4k+q loads V[key0 + k][d0 + 4q .. +3]
  // and lane i of the group receives V[key0 + 0..3][d0 + i])
  auto vread = [&](int nb, int j) __attribute__((always_inline)) {
    const int kc = 2 * nb + j / C::ND, nd = j % C::ND;
    const v4i16 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(vl + lo.v[nd][0] + kc * 16 * C::RB));
    const v4i16 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(vl + lo.v[nd][1] + kc * 16 * C::RB));
    const v8i16 av = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
    return __builtin_bit_cast(bf16x8, av);
  };

  // ---- one row maximum for the whole tile (keys past a partial tile's
  // end are -inf first), and the lazy rescale it may call for
  bf16x8 b[3];
  b[0] = vread(0, 0);
  b[1] = vread(0, 1);
  __builtin_amdgcn_sched_barrier(0);
  if (valid < C::BN) {
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * nb + 16 * (i >> 3) + 8 * hf + (i & 7);
        if (key >= valid) s[nb][i] = -__builtin_inff();
      }
  }
  float mloc = max16(s[0]);
#pragma unroll
  for (int nb = 1; nb < C::NB; ++nb) mloc = fmaxf(mloc, max16(s[nb]));
  const float mt = row_max_both_halves(mloc) * cs;
  if (__any(mt > sm.m_run + kTau)) {
    const float m_new = fmaxf(sm.m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(sm.m_run - m_new);
    sm.l_run *= alpha;
#pragma unroll
    for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[nd][i] *= alpha;
    sm.m_run = m_new;
  }
  const float nm = -sm.m_run;

  // probabilities p = 2^(s*cs - m) of block nb, elements i, i+1 (this
  // lane-half's share of the row sum goes to la / lb), packed to bf16 in
  // the PV B operand words
  u32x4 pw[C::NB][2];
  float la = 0.f, lb = 0.f;
  auto probs2 = [&](int nb, int i) __attribute__((always_inline)) {
    float x0 = s[nb][i], x1 = s[nb][i + 1];
    asm volatile("" : "+v"(x0), "+v"(x1));
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x0, cs, nm));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x1, cs, nm));
    const bool first = nb == 0 && i == 0;  // the sums start at this pair
    la = first ? p0 : la + p0;
    lb = first ? p1 : lb + p1;
    uint32_t w = pack_bf16x2(p0, p1);
    asm volatile("" : "+v"(w), "+v"(la), "+v"(lb));
    pw[nb][i >> 3][(i & 7) >> 1] = w;
  };
#pragma unroll
  for (int i = 0; i < 16; i += 2) probs2(0, i);
  __builtin_amdgcn_sched_barrier(0);

  // ---- O^T += V^T P^T block by block; the MFMAs of block nb carry the
  // exponentials of block nb+1 between them
  constexpr int PPS = 16 / NV;  // probabilities of the next block per PV MFMA
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    const bf16x8 pb0 = __builtin_bit_cast(bf16x8, pw[nb][0]);
    const bf16x8 pb1 = __builtin_bit_cast(bf16x8, pw[nb][1]);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      // operand reads run two MFMAs ahead, across block boundaries; the
      // three operand registers rotate on the tile-wide MFMA index g
      const int g = nb * NV + j, jn = j + 2;
      if (jn < NV)
        b[(g + 2) % 3] = vread(nb, jn);
      else if (nb + 1 < C::NB)
        b[(g + 2) % 3] = vread(nb + 1, jn - NV);
      o[j % C::ND] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[g % 3], j < C::ND ? pb0 : pb1,
                                                             o[j % C::ND], 0, 0, 0);
      if (nb + 1 < C::NB) {
#pragma unroll
        for (int q = 0; q < PPS; q += 2) probs2(nb + 1, PPS * j + q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  sm.l_run += la + lb;
}

// Wait for this wave's outstanding tile copies (vmcnt = 0), then barrier:
// after it every wave's copies of the next tile have landed in LDS.
__device__ __forceinline__ void copies_landed_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt unchanged
  __syncthreads();
}

// Prefix tiles read from an fp8 pool (E4M3 codes, one power-of-two scale per
// block and head).  Each thread owns NP 16-byte pieces (16 codes of one key
// row) of K and of V: during the compute of tile t it loads the pieces of
// tile t+1 into registers with their blocks' scales (the block ids were
// loaded during tile t-1), and after that compute it converts them -- code
// value * scale, exact in bfloat16 -- into the next LDS stage in the stage's
// swizzled layout.  The kernel's compute is then the bfloat16 one.
template <int D, int W>
struct Fp8Prefix {
  using C = Bf16Cfg<D>;
  static constexpr int THREADS = 64 * W;
  static constexpr int CPR8 = D / 16;         // 16-byte pieces of codes per key row
  static constexpr int NP = C::BN * CPR8 / THREADS;
  static_assert(NP >= 1 && NP * THREADS == C::BN * CPR8, "pieces per thread");
  static_assert(D == 128 || D == 64, "the piece mapping below covers these head dims");
  const uint8_t *pk, *pv;                     // code pools
  const float *sk, *sv;                       // scales [blocks, H_kv]
  const int32_t *bt_row;
  int lg, blocks, bt_stride, H, head, p_begin, p_end;
  int row[NP], c;
  int blk[NP];                                // block of each piece's row, next tile
  u32x4 dk[NP], dv[NP];
  float fk[NP], fv[NP];
  bool bad = false;

  // Which piece a thread converts.  LDS takes a 64-lane 16-byte store eight
  // lanes at a time, 128 bytes a cycle, so eight consecutive lanes have to
  // store to eight different 16-byte slots of a 128-byte bank line.  Piece c
  // of row r is stored as chunks 2c and 2c+1, at (2c) ^ swz(r) and
  // (2c+1) ^ swz(r): four pieces of one row take four slots of one parity,
  // that of bit 0 of the swizzle, (r >> 2) & 1.  So each eight lanes take
  // four pieces of row r and the same four of row r+4 (D=128: lanes 0-3 and
  // 8-11 of sixteen hold row r, 4-7 and 12-15 row r+4; D=64, a row being four
  // pieces: rows b, b+4, b+1, b+5 in four-lane runs, so that sixteen lanes
  // also cover a 256-byte line once).  Each run of four lanes reads 64
  // contiguous bytes of codes.
  __device__ __forceinline__ void init(int tid) {
    const int k = tid >> 4, l = tid & 15;
    int r0;
    if constexpr (D == 128) {
      r0 = (k & 3) + 8 * (k >> 2) + 4 * ((l >> 2) & 1);
      c = 4 * (l >> 3) + (l & 3);
    } else {
      r0 = 2 * (k & 1) + 8 * (k >> 1) + ((0x5140 >> (4 * (l >> 2))) & 0xF);
      c = l & 3;
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) row[j] = r0 + (THREADS / CPR8) * j;
  }
  __device__ __forceinline__ void load_ids(int tile) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int key = p_begin + tile * C::BN + row[j];
      const int slot = key >> lg;
      blk[j] = (key < p_end && slot < bt_stride) ? bt_row[slot] : -1;
    }
  }
  __device__ __forceinline__ void load(int tile) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int key = p_begin + tile * C::BN + row[j];
      const bool inb = blk[j] >= 0 && blk[j] < blocks;
      bad |= key < p_end && !inb;
      dk[j] = dv[j] = u32x4{0u, 0u, 0u, 0u};
      fk[j] = fv[j] = 0.f;
      if (key < p_end && inb) {
        const int64_t bh = (int64_t)blk[j] * H + head;
        const int64_t off = ((bh << lg) | (key & ((1 << lg) - 1))) * D + c * 16;
        dk[j] = *(const u32x4 *)(pk + off);
        dv[j] = *(const u32x4 *)(pv + off);
        fk[j] = sk[bh];
        fv[j] = sv[bh];
      }
    }
  }
  // 16 codes -> 16 bfloat16 values (two 16-byte chunks)
  __device__ __forceinline__ static void convert(const u32x4 &d, float s, u32x4 &lo, u32x4 &hi) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[w], s, false);
      const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[w], s, true);
      u32x4 &dst = w < 2 ? lo : hi;
      dst[2 * (w & 1)] = __builtin_bit_cast(uint32_t, a);
      dst[2 * (w & 1) + 1] = __builtin_bit_cast(uint32_t, b);
    }
  }
  __device__ __forceinline__ void store(uint8_t *kl, uint8_t *vl) const {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int sw = swz<D>(row[j]);
      const int o0 = row[j] * C::RB + (((2 * c) ^ sw) << 4);
      const int o1 = row[j] * C::RB + (((2 * c + 1) ^ sw) << 4);
      u32x4 lo, hi;
      convert(dk[j], fk[j], lo, hi);
      *(u32x4 *)(kl + o0) = lo;
      *(u32x4 *)(kl + o1) = hi;
      convert(dv[j], fv[j], lo, hi);
      *(u32x4 *)(vl + o0) = lo;
      *(u32x4 *)(vl + o1) = hi;
    }
  }
};

template <int D, int W, bool FLAT, bool FP8>
__global__ __launch_bounds__(64 * W, 2) void attn_bf16_kernel(AttnParams p) {
  using C = Bf16Cfg<D>;
  using G = WgCfg<W>;
  // two LDS stages, K and V each a separate object, so that the compiler can
  // tell the copy into one stage from the reads of the other and inserts no
  // wait for the in-flight copy inside the compute
  __shared__ __attribute__((aligned(1024))) uint8_t st0k[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t st0v[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1k[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1v[C::TILE];

  const WorkItem it = work_item(p, blockIdx.x);
  if (it.r < 0 || it.r >= p.B || it.h < 0 || it.h >= p.H) return;
  const ItemRange x = item_range(p, it);
  const int head = it.h;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;

  // Q fragments (B operand of S^T = K Q^T): lane holds row `col`,
  // dims 16*kk + 8*hf .. +7
  const int row = it.m_tile * G::BM + wave * G::ROWS + col;
  const bool row_ok = row < x.n_s && x.q0 >= 0 && x.q0 + row < p.total_s;
  bf16x8 qf[C::KK];

  TileCopy<D, W, FLAT> cp;
  cp.pool_k = (const uint8_t *)p.pool_k[x.mode];  // (fp8 pools: prefix tiles go through f8)
  cp.pool_v = (const uint8_t *)p.pool_v[x.mode];
  cp.ks = (const uint8_t *)p.k;
  cp.vs = (const uint8_t *)p.v;
  cp.bt_row = p.block_table + (int64_t)it.r * p.bt_stride;
  cp.lg = p.pool_bs_log2[x.mode];
  cp.blocks = p.pool_blocks[x.mode];
  cp.bt_stride = p.bt_stride;
  cp.H = p.H_kv;                       // the copies read key/value heads
  cp.head = head / (p.H / p.H_kv);
  cp.q0 = x.q0;
  // suffix rows that lie past total_s (inconsistent lengths) are never read
  cp.n_s = (x.q0 >= 0) ? min(x.n_s, p.total_s - x.q0) : 0;
  cp.p_begin = x.p_begin;
  cp.p_end = x.p_end;
  const int n_pkeys = x.p_end - x.p_begin;
  cp.n_tiles_p = n_pkeys > 0 ? (n_pkeys + C::BN - 1) / C::BN : 0;
  cp.wave = wave;
  cp.lane = lane;
  cp.whole_blocks = (1 << cp.lg) >= C::BN;
  cp.block_bytes = (int64_t)p.H_kv * ((int64_t)C::RB << cp.lg);
  cp.head_bytes = (int64_t)cp.head * ((int64_t)C::RB << cp.lg);
  cp.pool_records = (int32_t)min((int64_t)cp.blocks * cp.block_bytes, kBufferPoolLimit);
  cp.init_lanes();
  const int n_tiles = cp.n_tiles_p + (x.with_suffix ? (x.n_s + C::BN - 1) / C::BN : 0);
  // prefix-only rows of a request with no prefix: no keys, nothing to write
  // (the merge that follows reads that partial as empty); with the row's own
  // key folded in, the row is that key alone
  if (n_tiles == 0) {
    if (p.self_key && row_ok) {
      f32x16 z[C::ND];
#pragma unroll
      for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
        for (int i = 0; i < 16; ++i) z[nd][i] = 0.f;
      write_with_self_key<D>(p, x.q0 + row, head, cp.head, hf, z, 0.f, 0.f);
    }
    return;
  }
  cp.n_tiles = n_tiles;
  __shared__ u32x4 s_tab[TileCopy<D, W, FLAT>::kTabTiles];
  cp.tab = s_tab;
  const bool use_tab = n_tiles <= TileCopy<D, W, FLAT>::kTabTiles;
  cp.use_tab = false;  // tile 0 is planned from the block table (below)
  cp.dv_p = cp.pool_v - cp.pool_k;
  cp.dv_s = cp.vs - cp.ks;
  LdsOffsets<D> lo;
  lo.init(lane);

  f32x16 o[C::ND];
#pragma unroll
  for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[nd][i] = 0.f;
  SoftmaxState sm;
  const float cs = p.scale_log2;
  auto valid_keys = [&](int t) {
    return t < cp.n_tiles_p ? min(C::BN, n_pkeys - t * C::BN)
                            : min(C::BN, x.n_s - (t - cp.n_tiles_p) * C::BN);
  };

  // Every copy writes its whole stage (lanes past the end of the data write
  // zeros), so the stages need no clearing.  The Q loads go out between the
  // block-id load of tile 0 and its copy, so that the latencies overlap, and
  // tile 0 is planned from the block table itself, so that its copy is in
  // flight while the copy table is filled.
  int ids[TileCopy<D, W, FLAT>::CPW];  // (fp8 pools: never read, suffix tiles plan without them)
  // fp8 pool: the prefix tiles come through f8 (register-staged, converted
  // to bfloat16 into the stage); suffix tiles are copied as usual
  Fp8Prefix<D, W> f8;
  if constexpr (FP8) {
    f8.pk = (const uint8_t *)p.pool_k[x.mode];
    f8.pv = (const uint8_t *)p.pool_v[x.mode];
    f8.sk = p.pool_sk[x.mode];
    f8.sv = p.pool_sv[x.mode];
    f8.bt_row = cp.bt_row;
    f8.lg = cp.lg;
    f8.blocks = cp.blocks;
    f8.bt_stride = p.bt_stride;
    f8.H = p.H_kv;
    f8.head = cp.head;
    f8.p_begin = x.p_begin;
    f8.p_end = x.p_end;
    f8.init(tid);
    f8.load_ids(0);
  } else {
    cp.load_ids(0, ids);
  }
  {
    const uint16_t *q = (const uint16_t *)p.q + ((int64_t)(x.q0 + row) * p.H + head) * D;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row_ok) w = *(const u32x4 *)(q + 16 * kk + 8 * hf);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
  if (FP8 && cp.n_tiles_p > 0) {
    f8.load(0);
    f8.load_ids(1);
    f8.store(st0k, st0v);
  } else {
    cp.issue(0, ids, st0k, st0v);
  }
  cp.use_tab = use_tab;
  if constexpr (!FP8) cp.load_ids(1, ids);
  if (use_tab) {
    cp.fill_tab(tid, G::THREADS);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's entries stored
  }
  copies_landed_barrier();  // tile 0 in LDS, Q in registers, every table entry visible

  // Tile t is consumed from one stage while the copy of tile t+1 into the
  // other goes out one instruction every SPACING S^T MFMAs (a tile past the
  // last copies nothing).
  constexpr int SPACING = (C::NB * C::KK) / (2 * TileCopy<D, W, FLAT>::CPW);
  auto tile_step = [&](int t, uint8_t *kc, uint8_t *vc, uint8_t *kn, uint8_t *vn)
      __attribute__((always_inline)) {
    if (FP8 && t + 1 < cp.n_tiles_p) {
      // the next tile is an fp8 prefix tile: its codes load during this
      // tile's compute and are converted into the other stage after it
      f8.load(t + 1);
      f8.load_ids(t + 2);
      compute_tile<D>(kc, vc, qf, o, sm, cs, valid_keys(t), lane, lo, [](int) {});
      f8.store(kn, vn);
    } else {
      const auto pl = cp.plan(t + 1, ids);
      if constexpr (!FP8) cp.load_ids(t + 2, ids);
      compute_tile<D>(kc, vc, qf, o, sm, cs, valid_keys(t), lane, lo, [&](int i) {
        if (i % SPACING == 0) cp.fire(pl, i / SPACING, kn, vn);
      });
    }
    copies_landed_barrier();  // tile t+1 landed everywhere; this stage free
  };
  for (int t = 0; t < n_tiles; t += 2) {
    tile_step(t, st0k, st0v, st1k, st1v);
    if (t + 1 >= n_tiles) break;
    tile_step(t + 1, st1k, st1v, st0k, st0v);
  }

  // ---- epilogue: report bad block ids, normalise, write O (and lse) or the split partial
  bool bad = cp.bad;
  if constexpr (FP8) bad |= f8.bad;
  if (p.err && __any(bad) && lane == 0) atomicOr(p.err, kErrBlockId);
  const float l_tot = sm.l_run + __shfl_xor(sm.l_run, 32);
  const float inv = 1.0f / l_tot;
  const float lse_nat = (sm.m_run + log2f(l_tot)) * 0.69314718055994530942f;
  if (!row_ok) return;
  if (p.self_key) {
    write_with_self_key<D>(p, x.q0 + row, head, cp.head, hf, o, sm.m_run, l_tot);
    return;
  }
  if (!x.partial) {
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

template <typename F, int... J>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
// f(integral_constant<int, j>) for j = 0 .. N-1, each a separate compile-time instance
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// Ping-pong (D = 128, W = 8).  Waves w and w+4 share a SIMD; waves 0-3 form
// group A and waves 4-7 group B.  Every tile step has two phases with a workgroup
// barrier between them, and in each phase one group issues MFMAs while the
// other runs its softmax, so that each SIMD holds one wave of each kind and
// the vector work of one passes under the MFMAs of the other:
//   step t, phase 1:  A: O += V(t-1)^T P(t-1)^T, then S(t)^T = K(t) Q^T
//                     B: softmax of S(t-1); copies of K(t+1) and V(t)
//   step t, phase 2:  A: softmax of S(t)
//                     B: O += V(t-1)^T P(t-1)^T, then S(t)^T = K(t) Q^T
// K(t) and V(t) sit in stage t % 2.  The copy of K(t+1) replaces K(t-1) and
// that of V(t) replaces V(t-2), both last read in step t-1; they land before
// the barrier that ends step t.  Group B issues every copy, spread over its
// softmax.  Tiles are 64 keys at both head dims: at D=64 a 64-key tile
// keeps the score, probability and output registers of a wave small enough
// for two waves per SIMD, and its softmax phase (twice the exponentials per
// MFMA of D=128) still runs under the other group's MFMAs for most of it.
template <int D, bool FLAT>
__global__ __launch_bounds__(512, 2) void attn_bf16_pp_kernel(AttnParams p) {
  using C = Bf16Cfg<D, kPpBN>;
  using TC = TileCopy<D, 4, FLAT, kPpBN>;  // group B's four waves copy every tile
  constexpr int CPW = TC::CPW;
  constexpr int NS = C::NB * C::KK;
  constexpr int NV = 2 * C::ND;
  constexpr int NPV = C::NB * NV;
  constexpr float kTauSum = 256.0f;  // largest kept share of a block's row sum
  constexpr int BM = 256;

  __shared__ __attribute__((aligned(1024))) uint8_t k0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t k1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v1[C::TILE];
  __shared__ u32x4 s_tab[TC::kTabTiles];

  const WorkItem it = work_item(p, blockIdx.x);
  if (it.r < 0 || it.r >= p.B || it.h < 0 || it.h >= p.H) return;
  // The first block id of an item that starts at its request's first key
  // is entry 0 of the request's block-table row: loaded here, beside the
  // request's lengths, instead of after them.
  const bool first_chunk = it.chunk == 0 && p.block_table != nullptr && p.bt_stride > 0;
  const int32_t blk0 = first_chunk ? p.block_table[(int64_t)it.r * p.bt_stride] : -1;
  const ItemRange x = item_range(p, it);
  const int head = it.h;
  const int tid = threadIdx.x;
  // the wave index as a scalar, so that the compiler sees branches on the
  // group as uniform
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  const bool grp_a = wave < 4;

  // The rows of this item.  A request of n_s rows has ceil(n_s / 256) row
  // tiles (as planned), and its 32-row blocks are dealt over them evenly
  // (counts differing by at most one), not 256 rows at a time with the rest
  // left to the last tile.  Inside a tile of a multi-tile request the
  // blocks alternate between the groups (waves 0, 4, 1, 5, ...), so that
  // every tile keeps live waves in both groups.  The tiles of a request
  // then take about equally long per step and read the same prefix tiles at
  // about the same time, through L2; a short tile on group A alone ran
  // ahead of its full partners, which then fetched the prefix from memory
  // again once its lead passed what L2 holds.  A single-tile request has no
  // partner and keeps the plain order (a short one stays on group A, where
  // its steps cost less).
  int blk_first = 0, blk_count = 8, blk_rows = wave;
  {
    const int n_tiles_r = (x.n_s + BM - 1) / BM;
    if (n_tiles_r > 1) {
      const int nblk = (x.n_s + 31) >> 5;
      const int q = nblk / n_tiles_r, rem = nblk - q * n_tiles_r;
      blk_first = it.m_tile * q + min(it.m_tile, rem);
      blk_count = q + (it.m_tile < rem ? 1 : 0);
      blk_rows = (wave & 3) * 2 + (wave >> 2);
    }
  }
  const bool in_tile = blk_rows < blk_count;
  const int row = (blk_first + blk_rows) * 32 + col;
  // A wave whose 32 rows all lie outside the item (past the suffix's end, or
  // in a block the tile does not hold) computes nothing: it skips its
  // operand reads, MFMAs and softmax, and keeps only its part in the
  // barriers and, in group B, in the copies.
  const bool live = __builtin_amdgcn_readfirstlane(
                        (int)(in_tile && (blk_first + blk_rows) * 32 < x.n_s)) != 0;
  const bool row_ok = in_tile && row < x.n_s && x.q0 >= 0 && x.q0 + row < p.total_s;
  bf16x8 qf[C::KK];

  TC cp;
  cp.pool_k = (const uint8_t *)p.pool_k[x.mode];
  cp.pool_v = (const uint8_t *)p.pool_v[x.mode];
  cp.ks = (const uint8_t *)p.k;
  cp.vs = (const uint8_t *)p.v;
  cp.bt_row = p.block_table + (int64_t)it.r * p.bt_stride;
  cp.lg = p.pool_bs_log2[x.mode];
  cp.blocks = p.pool_blocks[x.mode];
  cp.bt_stride = p.bt_stride;
  cp.H = p.H_kv;                       // the copies read key/value heads
  cp.head = head / (p.H / p.H_kv);
  cp.q0 = x.q0;
  cp.n_s = (x.q0 >= 0) ? min(x.n_s, p.total_s - x.q0) : 0;
  cp.p_begin = x.p_begin;
  cp.p_end = x.p_end;
  const int n_pkeys = x.p_end - x.p_begin;
  cp.n_tiles_p = n_pkeys > 0 ? (n_pkeys + C::BN - 1) / C::BN : 0;
  cp.wave = wave & 3;
  cp.lane = lane;
  cp.whole_blocks = (1 << cp.lg) >= C::BN;
  cp.block_bytes = (int64_t)p.H_kv * ((int64_t)C::RB << cp.lg);
  cp.head_bytes = (int64_t)cp.head * ((int64_t)C::RB << cp.lg);
  cp.pool_records = (int32_t)min((int64_t)cp.blocks * cp.block_bytes, kBufferPoolLimit);
  cp.init_lanes();
  const int n_tiles = cp.n_tiles_p + (x.with_suffix ? (x.n_s + C::BN - 1) / C::BN : 0);
  // prefix-only rows of a request with no prefix: no keys, nothing to write
  // (the merge that follows reads that partial as empty); with the row's own
  // key folded in, the row is that key alone
  if (n_tiles == 0) {
    if (p.self_key && row_ok) {
      f32x16 z[C::ND];
#pragma unroll
      for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
        for (int i = 0; i < 16; ++i) z[nd][i] = 0.f;
      write_with_self_key<D>(p, x.q0 + row, head, cp.head, hf, z, 0.f, 0.f);
    }
    return;
  }
  cp.n_tiles = n_tiles;
  cp.tab = s_tab;
  cp.use_tab = n_tiles <= TC::kTabTiles;
  cp.dv_p = cp.pool_v - cp.pool_k;
  cp.dv_s = cp.vs - cp.ks;
  LdsOffsets<D> lo;
  lo.init(lane);

  f32x16 o[C::ND];
#pragma unroll
  for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[nd][i] = 0.f;
  // running max (log2 domain): finite before the first key, so that the
  // first tile's probabilities overflow to +inf and take the rescale path
  // (-inf would make masked keys NaN); la: this lane-half's row-sum share
  float m_run = -1e30f, la = 0.f;
  f32x16 s[C::NB];
  u32x4 pw[C::NB][2];
  const float cs = p.scale_log2;
  auto valid_keys = [&](int t) __attribute__((always_inline)) {
    return t < cp.n_tiles_p ? min(C::BN, n_pkeys - t * C::BN)
                            : min(C::BN, x.n_s - (t - cp.n_tiles_p) * C::BN);
  };

  auto kread = [&](const uint8_t *kl, int i) __attribute__((always_inline)) {
    return *(const bf16x8 *)(kl + lo.k[i / C::NB] + (i % C::NB) * 32 * C::RB);
  };
  auto vread = [&](const uint8_t *vl, int i) __attribute__((always_inline)) {
    const int nb = i / NV, j = i % NV;
    const int kc = 2 * nb + j / C::ND, nd = j % C::ND;
    const v4i16 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(vl + lo.v[nd][0] + kc * 16 * C::RB));
    const v4i16 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(vl + lo.v[nd][1] + kc * 16 * C::RB));
    const v8i16 av = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
    return __builtin_bit_cast(bf16x8, av);
  };

  // The MFMA phase: O += V(t-1)^T P(t-1)^T (when PV), then S(t)^T, operand
  // reads two MFMAs ahead through three rotating registers.
  auto gemm = [&](const uint8_t *kt, const uint8_t *vp, auto pv_c) __attribute__((always_inline)) {
    if (!live) return;
    constexpr bool PV = decltype(pv_c)::value;
    constexpr int N0 = PV ? NPV : 0, N = N0 + NS;
    auto op = [&](int j) __attribute__((always_inline)) {
      return j < N0 ? vread(vp, j) : kread(kt, j - N0);
    };
    bf16x8 r[3];
    r[0] = op(0);
    r[1] = op(1);
    const f32x16 zero = {};
    static_for<N>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j + 2 < N) r[(j + 2) % 3] = op(j + 2);
      if constexpr (j < N0) {
        constexpr int nb = j / NV, jj = j % NV;
        o[jj % C::ND] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            r[j % 3], __builtin_bit_cast(bf16x8, pw[nb][jj / C::ND]), o[jj % C::ND], 0, 0, 0);
      } else {
        constexpr int i = j - N0;
        s[i % C::NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            r[j % 3], qf[i / C::NB], i < C::NB ? zero : s[i % C::NB], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // The softmax phase for tile t.  The probabilities are taken against the
  // running max m_run with no row maximum on the common path: a 32-key
  // block is kept when no lane's share of its row sum exceeds 2^8, which
  // bounds every probability by 2^8 (the lazy-rescale bound).  Otherwise
  // (rarely after an item's first tile) the tile's row maximum is taken, O
  // and l are rescaled and the tile's probabilities recomputed.  An item's
  // first tile, where the running max is not yet a row value, takes the row
  // maximum first and computes its probabilities once.
  // hook(k) runs after pair k (group B issues its copies there).
  auto softmax = [&](int t, auto &&hook) __attribute__((always_inline)) {
    if (!live) {  // only the copies the hook issues
#pragma unroll
      for (int k = 0; k < 8 * C::NB; ++k) hook(k);
      return;
    }
    const int valid = valid_keys(t);
    if (valid < C::BN) {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * nb + 16 * (i >> 3) + 8 * hf + (i & 7);
          if (key >= valid) s[nb][i] = -__builtin_inff();
        }
    }
    float bl[C::NB];
    auto probs = [&](float nm, bool with_hook) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        float sa, sb;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int i = 2 * q;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][i], cs, nm));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][i + 1], cs, nm));
          sa = q ? sa + p0 : p0;
          sb = q ? sb + p1 : p1;
          pw[nb][i >> 3][(i & 7) >> 1] = pack_bf16x2(p0, p1);
          if (with_hook) hook(8 * nb + q);
        }
        bl[nb] = sa + sb;
      }
    };
    auto tile_max = [&]() __attribute__((always_inline)) {
      float mloc = max16(s[0]);
#pragma unroll
      for (int nb = 1; nb < C::NB; ++nb) mloc = fmaxf(mloc, max16(s[nb]));
      return row_max_both_halves(mloc) * cs;
    };
    // first tile: o and the row sum are still zero, so only the running max
    // moves; every probability is then at most 1 and the check below passes
    if (t == 0) m_run = fmaxf(m_run, tile_max());
    probs(-m_run, true);
    bool over = false;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) over |= !(bl[nb] <= kTauSum);
    if (__any(over)) {
      const float m_new = fmaxf(m_run, tile_max());
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      la *= alpha;
#pragma unroll
      for (int nd = 0; nd < C::ND; ++nd)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[nd][i] *= alpha;
      m_run = m_new;
      probs(-m_run, false);
    }
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) la += bl[nb];
  };
  auto mid_barrier = []() __attribute__((always_inline)) {
    // no memory fence: group B's copies stay in flight across it
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: Q, the copy of K(0) (group B), the copy table, barrier.
  // K(0) is planned from the block table itself, so that its copy is in
  // flight while the table is filled: one memory round trip before the
  // first tile instead of two.
  int ids[CPW];
  typename TC::Plan pl_v;  // the plan of the tile whose V goes out next
  {
    const uint16_t *q = (const uint16_t *)p.q + ((int64_t)(x.q0 + row) * p.H + head) * D;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row_ok) w = *(const u32x4 *)(q + 16 * kk + 8 * hf);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
  if (!grp_a) {
    const bool tab = cp.use_tab;
    cp.use_tab = false;
    if (cp.whole_blocks && first_chunk) {
      // tile 0 of whole blocks reads one block id, the one loaded above
#pragma unroll
      for (int j = 0; j < CPW; ++j) ids[j] = j == 0 && cp.n_tiles_p > 0 ? blk0 : -1;
    } else {
      cp.load_ids(0, ids);
    }
    pl_v = cp.plan(0, ids);
#pragma unroll
    for (int j = 0; j < CPW; ++j) cp.fire(pl_v, j, k0, v0);
    cp.use_tab = tab;
    cp.load_ids(1, ids);
  }
  if (cp.use_tab) {
    cp.fill_tab(tid, 512);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's entries stored
  }
  copies_landed_barrier();  // K(0) and Q landed, every table entry visible

  auto pv_only = [&](const uint8_t *vl) __attribute__((always_inline)) {
    if (!live) return;
    bf16x8 r[3];
    r[0] = vread(vl, 0);
    r[1] = vread(vl, 1);
    static_for<NPV>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j + 2 < NPV) r[(j + 2) % 3] = vread(vl, j + 2);
      constexpr int nb = j / NV, jj = j % NV;
      o[jj % C::ND] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          r[j % 3], __builtin_bit_cast(bf16x8, pw[nb][jj / C::ND]), o[jj % C::ND], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Each group runs its own copy of the whole tile loop (a separate
  // instance, so that neither carries the other's registers).
  auto run = [&](auto role_c, auto tab_c) __attribute__((always_inline)) {
    constexpr bool A = decltype(role_c)::value;
    // group B on an item whose tiles all come from the table plans from the
    // table alone (fewer live scalars than the general plan)
    constexpr bool TAB = decltype(tab_c)::value;
    u32x4 e_next = {0u, 0u, 0u, 0u};
    if constexpr (!A && TAB) e_next = cp.tab_entry(2);
    auto plan_next = [&](int tile) __attribute__((always_inline)) {
      if constexpr (TAB) {
        const auto pl = cp.plan_tab(tile, e_next);
        e_next = cp.tab_entry(tile + 1);
        return pl;
      } else {
        const auto pl = cp.plan(tile, ids);
        cp.load_ids(tile + 1, ids);
        return pl;
      }
    };
    // step 0: no PV yet
    if constexpr (A) {
      gemm(k0, v1, std::integral_constant<bool, false>{});
      mid_barrier();
      softmax(0, [](int) {});
    } else {
      {
        const auto pk = TAB ? cp.plan_tab(1, cp.tab_entry(1)) : cp.plan(1, ids);
        if constexpr (!TAB) cp.load_ids(2, ids);
#pragma unroll
        for (int j = 0; j < 2 * CPW; ++j) cp.fire(j < CPW ? pk : pl_v, j, k1, v0);
        pl_v = pk;
      }
      mid_barrier();
      gemm(k0, v1, std::integral_constant<bool, false>{});
    }
    copies_landed_barrier();

    // steps 1 .. n-1: kt = K(t), vp = V(t-1), kc / vc = copy targets of
    // K(t+1) / V(t)
    auto step = [&](int t, const uint8_t *kt, const uint8_t *vp, uint8_t *kc, uint8_t *vc)
        __attribute__((always_inline)) {
      if constexpr (A) {
        gemm(kt, vp, std::integral_constant<bool, true>{});
        mid_barrier();
        softmax(t, [](int) {});
      } else {
        cp.anchor();
        const auto pk = plan_next(t + 1);
        constexpr int EVERY = (8 * C::NB) / (2 * CPW);
        softmax(t - 1, [&](int k) __attribute__((always_inline)) {
          if (k % EVERY == EVERY - 1) {
            const int j = k / EVERY;
            __builtin_amdgcn_sched_barrier(0);
            cp.fire(j < CPW ? pk : pl_v, j, kc, vc);
            __builtin_amdgcn_sched_barrier(0);
          }
        });
        pl_v = pk;
        mid_barrier();
        gemm(kt, vp, std::integral_constant<bool, true>{});
      }
      copies_landed_barrier();
    };
    int t = 1;
    for (; t + 1 < n_tiles; t += 2) {
      step(t, k1, v0, k0, v1);
      step(t + 1, k0, v1, k1, v0);
    }
    if (t < n_tiles) step(t, k1, v0, k0, v1);

    // tail: the last tile's PV (group A), its softmax then PV (group B)
    const int tl = n_tiles - 1;
    if constexpr (A) {
      if (tl & 1) pv_only(v1); else pv_only(v0);
      mid_barrier();
    } else {
      softmax(tl, [](int) {});
      mid_barrier();
      if (tl & 1) pv_only(v1); else pv_only(v0);
    }
  };
  if (grp_a)
    run(std::integral_constant<bool, true>{}, std::integral_constant<bool, false>{});
  else if (cp.use_tab && cp.whole_blocks)
    run(std::integral_constant<bool, false>{}, std::integral_constant<bool, true>{});
  else
    run(std::integral_constant<bool, false>{}, std::integral_constant<bool, false>{});

  // ---- epilogue: report bad block ids, normalise, write O (and lse) or the split partial
  if (p.err && __any(cp.bad) && lane == 0) atomicOr(p.err, kErrBlockId);
  const float l_tot = la + __shfl_xor(la, 32);
  const float inv = 1.0f / l_tot;
  const float lse_nat = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  if (!row_ok) return;
  if (p.self_key) {
    write_with_self_key<D>(p, x.q0 + row, head, cp.head, hf, o, m_run, l_tot);
    return;
  }
  if (!x.partial) {
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

// Explicit instantiations of every kernel launched below (two kernel
// templates that share device helpers otherwise lose one set of host stubs).
template __global__ void attn_bf16_kernel<128, 4, false, false>(AttnParams);
template __global__ void attn_bf16_kernel<128, 4, true, false>(AttnParams);
template __global__ void attn_bf16_kernel<64, 4, false, false>(AttnParams);
template __global__ void attn_bf16_kernel<64, 4, true, false>(AttnParams);
template __global__ void attn_bf16_kernel<128, 4, false, true>(AttnParams);
template __global__ void attn_bf16_kernel<64, 4, false, true>(AttnParams);
template __global__ void attn_bf16_kernel<64, 8, false, true>(AttnParams);
template __global__ void attn_bf16_pp_kernel<128, false>(AttnParams);
template __global__ void attn_bf16_pp_kernel<128, true>(AttnParams);
template __global__ void attn_bf16_pp_kernel<64, false>(AttnParams);
template __global__ void attn_bf16_pp_kernel<64, true>(AttnParams);

int bf16_rows_per_item(int W) { return W == 8 ? WgCfg<8>::BM : WgCfg<4>::BM; }
// keys per tile of the kernel a plan launches: the ping-pong kernel for
// eight waves (fp8 pools excepted), else the four-wave (or fp8) kernel
int bf16_keys_per_tile(int D, int W, bool fp8) {
  if (W == 8 && !fp8) return kPpBN;
  return D == 128 ? Bf16Cfg<128>::BN : Bf16Cfg<64>::BN;
}

template <int D, int W>
static void launch_one(const AttnParams &p, bool flat, int grid, hipStream_t stream) {
  if (p.fp8)  // fp8 pools are read by plain loads (no per-pool address limit)
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, false, true>), dim3(grid), dim3(64 * W), 0,
                       stream, p);
  else if (flat)
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, true, false>), dim3(grid), dim3(64 * W), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, false, false>), dim3(grid), dim3(64 * W), 0,
                       stream, p);
}

template <int D>
static void launch_pp(const AttnParams &p, bool flat, int grid, hipStream_t stream) {
  if (flat)
    hipLaunchKernelGGL((attn_bf16_pp_kernel<D, true>), dim3(grid), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_bf16_pp_kernel<D, false>), dim3(grid), dim3(512), 0, stream, p);
}

hipError_t launch_attn_bf16(const AttnParams &p, int D, int W, bool flat_gather, int grid,
                            hipStream_t stream) {
  clear_stale_launch_error();
  if (grid <= 0) return hipSuccess;
  // Only per-key gathers (pool blocks smaller than a key tile) address the
  // whole pool from one descriptor with 32-bit offsets; whole-block tiles
  // take a 64-bit base per tile, so a pool of any size copies them by buffer
  // loads.  The global-load gather form is needed only for a per-key pool of
  // 2 GiB or more.
  bool flat = flat_gather;
  const int bn = bf16_keys_per_tile(D, W, p.fp8 != 0);
  for (int m = 0; m < 2; ++m)
    flat |= (1 << p.pool_bs_log2[m]) < bn &&
            (int64_t)p.pool_blocks[m] * p.H_kv * ((int64_t)2 * D << p.pool_bs_log2[m]) >
                kBufferPoolLimit;
  if (p.fp8 && D == 128 && W != 4) return hipErrorInvalidValue;  // fp8: four waves at D=128
  if (D == 128 && W == 8)
    launch_pp<128>(p, flat, grid, stream);
  else if (D == 128 && W == 4)
    launch_one<128, 4>(p, flat, grid, stream);
  else if (D == 64 && W == 8 && p.fp8)  // fp8 pools: the eight-wave kernel with the fp8 path
    hipLaunchKernelGGL((attn_bf16_kernel<64, 8, false, true>), dim3(grid), dim3(512), 0, stream,
                       p);
  else if (D == 64 && W == 8)
    launch_pp<64>(p, flat, grid, stream);
  else if (D == 64 && W == 4)
    launch_one<64, 4>(p, flat, grid, stream);
  else
    return hipErrorInvalidValue;
  return launch_result();
}

}  // namespace bat
