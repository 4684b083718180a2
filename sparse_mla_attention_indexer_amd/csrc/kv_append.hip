// kv_append.hip — new tokens into the caches on gfx950: each token's latent row is quantised into
// its 656-byte FP8 row, and its indexer key is copied into the key cache. This is the step before
// the indexer and the attention of every decode or prefill-chunk step.
//
// Row layout (the pages size the FP8 latent row at 656 bytes, FlashMLA's fp8_ds_mla format:
// "Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "Why the numbers work"): the 512 value
// dims as OCP E4M3 codes, four little-endian fp32 scales (one per 128 value dims), the 64 rope dims
// as bf16. Block scale = fp32(amax / 448), 1 for an all-zero block; a value's code is the exact
// quotient value / scale rounded to nearest-even on the E4M3 grid and saturated at 448.
#include "smla_internal.h"

namespace smla {

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int LAT_DIMS = 576;  // 512 value dims + 64 rope dims, bf16
constexpr int ROW_BYTES = MLA_ROW_BYTES;

// E4M3 code of the quotient x: round to nearest-even on the code grid, worked on the binary64
// bits. Normal codes keep the top 3 of the 52 fraction bits (exponents -6..8); below 2^-6 the
// grid is the multiples of 2^-9. Anything at or above 448 takes the largest finite code.
__device__ __forceinline__ uint32_t e4m3_rne(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(b >> 63) << 7;
  const uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  const double a = __longlong_as_double((long long)mag);
  if (a >= 448.0) return sign | 0x7Eu;
  const int exp = (int)(mag >> 52) - 1023;
  if (exp < -6) return sign | (uint32_t)rint(a * 512.0);  // 0..8 (8 is the code of 2^-6)
  const uint64_t frac = mag & 0xFFFFFFFFFFFFFull;
  uint32_t code = ((uint32_t)(exp + 7) << 3) | (uint32_t)(frac >> 49);
  const uint64_t rest = frac & ((1ull << 49) - 1), halfway = 1ull << 48;
  if (rest > halfway || (rest == halfway && (code & 1u))) ++code;  // a carry moves the exponent
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// E4M3 code of v / s (s > 0) given r = RN(1 / s): the fp32 estimate x = |v| r is within 2^-22
// (relative) of the quotient, so rounding x gives the quotient's code unless x lies within a few
// of its last 20 bits of a rounding midpoint; there (rarely, and at every exact tie) the
// decision is taken again from the binary64 quotient. Above 448 the code saturates.
__device__ __forceinline__ uint32_t e4m3_code(float v, float r, double ds) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  const float x = a * r;
  uint32_t code;
  bool near;
  if (!(x < 448.f)) {
    code = 0x7Eu;
    near = false;
  } else if (x < 0.015625f) {  // below 2^-6: multiples of 2^-9
    const float t = x * 512.f;
    near = fabsf(t - floorf(t) - 0.5f) < 1.0f / 65536.f;
    code = (uint32_t)rintf(t);
  } else {
    const uint32_t b = __float_as_uint(x);
    const uint32_t rest = b & 0xFFFFFu;  // the 20 mantissa bits below the code's 3
    code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
    near = rest - (0x80000u - 16u) < 32u;
    if (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) ++code;
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  if (near) code = e4m3_rne((double)a / ds);
  return sign | code;
}

// One wave per token: lane l converts value dims [8 l, 8 l + 8), block l / 16; lanes 0..7 move
// the rope dims, and the first D_I / 16 lanes the indexer key.
__global__ __launch_bounds__(256) void kv_append_kernel(int64_t n, const uint16_t* __restrict__ latent,
                                                        const int64_t* __restrict__ rows,
                                                        unsigned char* __restrict__ kv,
                                                        const int8_t* __restrict__ k_new, int D_I,
                                                        int8_t* __restrict__ k_idx) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const uint16_t* src = latent + r * LAT_DIMS;
  const int64_t row = rows[r];
  unsigned char* dst = kv + row * ROW_BYTES;

  const v4u x = *reinterpret_cast<const v4u*>(src + 8 * lane);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(x[i] << 16);
    v[2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));  // the lane's block
  const float scale = amax > 0.f ? (float)((double)amax / 448.0) : 1.0f;
  const double ds = (double)scale;
  const float rcp = 1.0f / scale;  // correctly rounded
  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= e4m3_code(v[i], rcp, ds) << (8 * i);
    hi |= e4m3_code(v[4 + i], rcp, ds) << (8 * i);
  }
  *reinterpret_cast<v2u*>(dst + 8 * lane) = v2u{lo, hi};
  if ((lane & 15) == 0) *reinterpret_cast<float*>(dst + 512 + 4 * (lane >> 4)) = scale;
  if (lane < 8)
    *reinterpret_cast<v4u*>(dst + 528 + 16 * lane) = *reinterpret_cast<const v4u*>(src + 512 + 8 * lane);
  if (k_new && 16 * lane < D_I)
    *reinterpret_cast<v4u*>(k_idx + row * D_I + 16 * lane) =
        *reinterpret_cast<const v4u*>(k_new + r * D_I + 16 * lane);
}

}  // namespace

hipError_t launch_kv_append(int64_t n, const void* latent, const int64_t* rows, void* kv,
                            const int8_t* k_new, int32_t D_I, int8_t* k_idx, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, n,
                     static_cast<const uint16_t*>(latent), rows, static_cast<unsigned char*>(kv),
                     k_new, D_I, k_idx);
  return hipGetLastError();
}

}  // namespace smla
