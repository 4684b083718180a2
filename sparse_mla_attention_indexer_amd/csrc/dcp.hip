// dcp.hip — the merges of decode context parallelism, on one GPU.
//
// The pages shard the latent KV cache round robin, every n-th token to one GPU, so each GPU
// scores and attends only its own rows, and then merge what the shards computed: the per-shard
// top-k lists into the global top-k, and the per-shard attention partials by log-sum-exp
// ("Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "DCP"). With shard l holding the
// tokens l, l + n, l + 2n, ..., a shard's local row j is global row j n + l. The merge is exact:
// a member of the global top-k has fewer than k rows above it anywhere, so it is in its own
// shard's top-k too.
//
//  - the top-k merge lives with the other selection kernels (topk.hip: topk_merge_kernel);
//  - local_indices_kernel: each shard's part of a global selection, as ascending local indices,
//    compacted to the front (the attention kernel skips trailing padding tiles).
//  - lse_merge_kernel: per (token, head), weights exp(lse_i - max) over the parts, bf16 in and out.
//  - the top-k merge can also write every shard's local list itself (topk_merge_kernel); the
//    local-indices kernel here serves selections from anywhere else.
#include "smla_internal.h"

namespace smla {

namespace {


// Every shard's part of a global selection: shard s (blockIdx.y) gets the entries g with
// g mod n == s, as g div n, in order, then -1. One 256-thread workgroup per (token, shard); each
// thread takes a contiguous chunk.
__global__ __launch_bounds__(256) void local_indices_kernel(int total_q, int top_k,
                                                            const int32_t* __restrict__ idx,
                                                            int n_shards,
                                                            int32_t* __restrict__ local_idx) {
  __shared__ int wsum[4];
  const int64_t t = blockIdx.x;
  const int shard = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = (top_k + 255) / 256;
  const int j0 = min(tid * chunk, top_k), j1 = min(j0 + chunk, top_k);
  const int32_t* row = idx + t * top_k;
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += row[j] >= 0 && row[j] % n_shards == shard;
  // exclusive prefix of the counts: a shuffle scan in each wave, then the four wave totals
  int x = cnt;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int pos = x - cnt, total = 0;
  for (int w = 0; w < 4; ++w) {
    pos += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  int32_t* out = local_idx + ((int64_t)shard * total_q + t) * top_k;
  for (int j = j0; j < j1; ++j) {
    const int32_t g = row[j];
    if (g >= 0 && g % n_shards == shard) out[pos++] = g / n_shards;
  }
  for (int j = total + tid; j < top_k; j += 256) out[j] = -1;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  typedef __bf16 bf;
  return __builtin_bit_cast(uint16_t, (bf)f);
}

// One wave per (token, head), four per workgroup. Lane i < n_parts holds part i's lse; the max,
// the weights exp(lse_i - max) and their sum come from wave reductions, and lane x then covers
// dims 8x .. 8x + 7 (then 512 further on), reading every part's eight bf16 values in one 16-byte
// load when rows are 16-byte aligned.
constexpr int LM_WAVES = 4;
__global__ __launch_bounds__(64 * LM_WAVES) void lse_merge_kernel(int total_q, int H, int D_v,
                                                                  int n_parts,
                                                                  const uint16_t* __restrict__ outs,
                                                                  const float* __restrict__ lses,
                                                                  uint16_t* __restrict__ out,
                                                                  float* __restrict__ lse_out) {
  const int64_t th = (int64_t)blockIdx.x * LM_WAVES + (threadIdx.x >> 6);  // token * H + head
  const int64_t plane_o = (int64_t)total_q * H * D_v, plane_l = (int64_t)total_q * H;
  if (th >= plane_l) return;  // whole waves
  const int lane = threadIdx.x & 63;
  const float li = lane < n_parts ? lses[lane * plane_l + th] : -INFINITY;
  float m = li;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float wi = li == -INFINITY ? 0.f : __expf(li - m);
  float z = wi;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  const float inv = z > 0.f ? 1.f / z : 0.f;
  const bool vec = (D_v & 7) == 0 && ((uintptr_t)outs & 15) == 0 && ((uintptr_t)out & 15) == 0;
  for (int d0 = 8 * lane; d0 < D_v; d0 += 512) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < n_parts; i0 += 8) {  // up to eight parts' loads in flight
      uint4 v[8];
      float w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k;
        w[k] = i < n_parts ? __shfl(wi, i) : 0.f;
        if (vec && w[k] != 0.f)
          v[k] = *reinterpret_cast<const uint4*>(outs + i * plane_o + th * D_v + d0);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (w[k] == 0.f) continue;  // an empty part (or none)
        if (vec) {
          const uint32_t u[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += w[k] * __uint_as_float(u[e] << 16);
            acc[2 * e + 1] += w[k] * __uint_as_float(u[e] & 0xFFFF0000u);
          }
        } else {
          const uint16_t* src = outs + (i0 + k) * plane_o + th * D_v + d0;
          for (int e = 0; e < 8 && d0 + e < D_v; ++e) acc[e] += w[k] * bf16_to_f32(src[e]);
        }
      }
    }
    if (vec) {
      uint32_t u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        u[e] = (uint32_t)f32_to_bf16(acc[2 * e] * inv) | ((uint32_t)f32_to_bf16(acc[2 * e + 1] * inv) << 16);
      *reinterpret_cast<uint4*>(out + th * D_v + d0) = make_uint4(u[0], u[1], u[2], u[3]);
    } else {
      for (int e = 0; e < 8 && d0 + e < D_v; ++e) out[th * D_v + d0 + e] = f32_to_bf16(acc[e] * inv);
    }
  }
  if (lse_out && lane == 0) lse_out[th] = z > 0.f ? m + __logf(z) : -INFINITY;
}

}  // namespace

hipError_t launch_local_indices(int32_t total_q, int32_t top_k, const int32_t* idx, int32_t n_shards,
                                int32_t* local_idx, hipStream_t s) {
  hipLaunchKernelGGL(local_indices_kernel, dim3((unsigned)total_q, (unsigned)n_shards), dim3(256), 0, s,
                     total_q, top_k, idx, n_shards, local_idx);
  return hipGetLastError();
}

hipError_t launch_lse_merge(int32_t total_q, int32_t H, int32_t D_v, int32_t n_parts,
                            const void* outs, const float* lses, void* out, float* lse,
                            hipStream_t s) {
  const int64_t waves = (int64_t)total_q * H;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((waves + LM_WAVES - 1) / LM_WAVES)),
                     dim3(64 * LM_WAVES), 0, s,
                     total_q, H, D_v, n_parts, static_cast<const uint16_t*>(outs), lses,
                     static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace smla
