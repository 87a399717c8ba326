// Prefix KV build into an fp8 pool: each (block, head) of a prefix's keys
// (and, separately, values) is stored as OCP FP8 E4M3 codes with one
// power-of-two scale 2^e, e the smallest integer with amax <= 448 * 2^e (amax:
// the block's largest magnitude; e = 0 for an all-zero block).  A value x is
// stored as the E4M3 code nearest to x / 2^e, ties to the even code, sign
// kept; it reads back as code value * 2^e, which bfloat16 holds exactly.
//
// The pool holds half the bytes of a bfloat16 pool, so twice the prefixes
// fit (the Bat page, "What it costs (trade-offs and scope)", counts cache
// memory against item caches).  HBM-bound like the bfloat16 build: each
// input byte is read once (a second pass over the block for the codes hits
// L2), each code written once.
#include "common.h"

namespace bat {

// E4M3 code of y, |y| <= 448: nearest value, ties to the even code.  Below
// 2^-6 the codes are multiples of 2^-9 (code = y * 2^9 rounded); above, the
// exponent field is floor(log2 |y|) + 7 and the three mantissa bits the
// fraction rounded to eighths, a carry into the exponent field being the next
// code.  Products by powers of two are exact; rintf rounds half to even.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 31) << 7;
  const float a = fabsf(y);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = (uint32_t)rintf(a * 512.0f);
  } else {
    const int ex = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
    mag = (uint32_t)((ex + 7) * 8) + (uint32_t)rintf(ldexpf(a, 3 - ex)) - 8u;
  }
  return sign | mag;
}

// The scale exponent of a block: the smallest e with amax <= 448 * 2^e.
// With amax = f * 2^x, f in [1, 2): e = x - 8 when f <= 1.75 (448 = 1.75 * 2^8),
// else x - 7.
__device__ __forceinline__ int fp8_scale_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int bias = 0;
  if (amax < 1e-30f) {  // subnormal or near it: scale up first (exact)
    amax = ldexpf(amax, 64);
    bias = 64;
  }
  const uint32_t b = __float_as_uint(amax);
  const int x = (int)((b >> 23) & 0xFF) - 127;
  return x - 8 + ((b & 0x7FFFFF) > 0x600000u ? 1 : 0) - bias;
}

template <int ELEM>
__device__ __forceinline__ void load8(const uint8_t *p, float (&x)[8]) {
  if constexpr (ELEM == 2) {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 c = *reinterpret_cast<const f32x4 *>(p + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = c[i];
    }
  }
}

// One workgroup per (request r, block j of its tokens, head h): amax over
// the block's tokens, the scale, then the codes, for K and then for V.
// Groups of 8 consecutive elements of a token row are the unit of work.
template <int ELEM>
__global__ __launch_bounds__(256) void kv_build_fp8_kernel(
    const uint8_t *__restrict__ k, const uint8_t *__restrict__ v,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ bt, int32_t bt_stride, int32_t B,
    int32_t H, int32_t D, uint8_t *__restrict__ pk, uint8_t *__restrict__ pv,
    float *__restrict__ sk, float *__restrict__ sv, int32_t num_blocks, int32_t bs_log2,
    int32_t *err) {
  __shared__ float s_max[4];
  const int rj = blockIdx.x, h = blockIdx.y;
  const int r = rj / bt_stride, j = rj - r * bt_stride;
  if (r >= B) return;
  const int n = cu[r + 1] - cu[r];
  if (j == 0 && err && threadIdx.x == 0 && (n < 0 || n > (bt_stride << bs_log2)))
    atomicOr(err, kErrLength);  // tokens the table row cannot hold are not written
  const int t0 = j << bs_log2;
  if (t0 >= n) return;
  const int nt = min(n - t0, 1 << bs_log2);
  const int blk = bt[rj];
  if (blk < 0 || blk >= num_blocks) {
    if (err && threadIdx.x == 0) atomicOr(err, kErrBlockId);
    return;
  }
  const int gpr = D / 8;  // groups per token row
  const int groups = nt * gpr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int64_t in_row0 = (int64_t)cu[r] + t0;
  const int64_t out_base = (((int64_t)blk * H + h) << bs_log2) * D;
  for (int which = 0; which < 2; ++which) {
    const uint8_t *src = which ? v : k;
    uint8_t *dst = which ? pv : pk;
    float amax = 0.f;
    for (int g = threadIdx.x; g < groups; g += blockDim.x) {
      const int row = g / gpr, c = g - row * gpr;
      float x[8];
      load8<ELEM>(src + (((in_row0 + row) * H + h) * D + c * 8) * ELEM, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (lane == 0) s_max[wave] = amax;
    __syncthreads();
    amax = s_max[0];
    for (int w = 1; w < nwaves; ++w) amax = fmaxf(amax, s_max[w]);
    const int e = fp8_scale_exponent(amax);
    for (int g = threadIdx.x; g < groups; g += blockDim.x) {
      const int row = g / gpr, c = g - row * gpr;
      float x[8];
      load8<ELEM>(src + (((in_row0 + row) * H + h) * D + c * 8) * ELEM, x);
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0 |= e4m3_code(ldexpf(x[i], -e)) << (8 * i);
        w1 |= e4m3_code(ldexpf(x[4 + i], -e)) << (8 * i);
      }
      *reinterpret_cast<u32x2 *>(dst + out_base + (int64_t)row * D + c * 8) = u32x2{w0, w1};
    }
    if (threadIdx.x == 0) (which ? sv : sk)[(int64_t)blk * H + h] = ldexpf(1.0f, e);
    __syncthreads();  // s_max is reused for V
  }
}

hipError_t launch_kv_build_fp8(const void *k, const void *v, const int32_t *cu,
                               const int32_t *bt, int32_t bt_stride, int32_t B, int32_t H,
                               int32_t D, int elem_bytes, void *pk, void *pv, float *sk,
                               float *sv, int32_t num_blocks, int32_t bs_log2, int32_t *err,
                               hipStream_t stream) {
  clear_stale_launch_error();
  const int groups = (D / 8) << bs_log2;  // per (block, head)
  const int threads = groups >= 256 ? 256 : groups >= 128 ? 128 : 64;
  const dim3 grid((unsigned)B * (unsigned)bt_stride, (unsigned)H);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(kv_build_fp8_kernel<2>, grid, dim3(threads), 0, stream,
                       (const uint8_t *)k, (const uint8_t *)v, cu, bt, bt_stride, B, H, D,
                       (uint8_t *)pk, (uint8_t *)pv, sk, sv, num_blocks, bs_log2, err);
  else
    hipLaunchKernelGGL(kv_build_fp8_kernel<4>, grid, dim3(threads), 0, stream,
                       (const uint8_t *)k, (const uint8_t *)v, cu, bt, bt_stride, B, H, D,
                       (uint8_t *)pk, (uint8_t *)pv, sk, sv, num_blocks, bs_log2, err);
  return launch_result();
}

}  // namespace bat
