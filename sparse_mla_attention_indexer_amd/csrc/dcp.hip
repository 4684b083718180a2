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
//  - topk_merge_kernel: one workgroup per query token; the union of the shards' lists as unique
//    64-bit keys (score << 32 | ~global index) in LDS, an MSD radix select over 8-bit digits for
//    the k-th largest key, then the selected (global index, score) pairs sorted by index
//    (bitonic, in LDS).
//  - local_indices_kernel: a shard's part of a global selection, as ascending local indices,
//    compacted to the front (the attention kernel skips trailing padding tiles).
//  - lse_merge_kernel: per (token, head), weights exp(lse_i - max) over the parts, bf16 in and out.
#include "smla_internal.h"

namespace smla {

namespace {


constexpr int NT_M = 256;

__global__ __launch_bounds__(NT_M) void topk_merge_kernel(int n_lists, int k_in,
                                                          const int32_t* __restrict__ idx_lists,
                                                          const int32_t* __restrict__ score_lists,
                                                          int64_t list_stride, int top_k,
                                                          int32_t* __restrict__ idx_out,
                                                          int32_t* __restrict__ score_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);                      // [MERGE_MAX_CAND]
  uint64_t* sel = keys + MERGE_MAX_CAND;  // [TOPK_MAX_K] (global index << 32 | score), pow2
  __shared__ int hist[256];
  __shared__ int nkeys, nsel, digit, need_s;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) nkeys = 0, nsel = 0;
  __syncthreads();

  // the union: every valid entry of every list, as (score, global index) keys
  const int ncand = n_lists * k_in;
  for (int c = tid; c < ncand; c += NT_M) {
    const int l = c / k_in, j = c - l * k_in;
    const int64_t off = l * list_stride + t * k_in + j;
    const int32_t local = idx_lists[off];
    if (local >= 0) {
      const uint32_t g = (uint32_t)local * (uint32_t)n_lists + (uint32_t)l;
      const int slot = atomicAdd(&nkeys, 1);
      keys[slot] = ((uint64_t)(uint32_t)score_lists[off] << 32) | (uint64_t)(0xFFFFFFFFu - g);
    }
  }
  __syncthreads();
  const int n = nkeys;

  // the cut: the min(top_k, n)-th largest key, digit by digit from the top
  uint64_t prefix = 0, mask = 0;
  const int take = min(top_k, n);
  if (take < n) {
    int need = take;
    for (int shift = 56; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += NT_M)
        if ((keys[i] & mask) == prefix) atomicAdd(&hist[(keys[i] >> shift) & 255], 1);
      __syncthreads();
      if (tid == 0) {
        int above = 0, d = 255;
        for (; d > 0; --d) {
          if (above + hist[d] >= need) break;
          above += hist[d];
        }
        digit = d;
        need_s = need - above;
      }
      __syncthreads();
      prefix |= (uint64_t)digit << shift;
      mask |= (uint64_t)255 << shift;
      need = need_s;
      __syncthreads();
    }
  }
  // selected: every key at or above the cut (keys are unique: exactly `take` of them)
  for (int i = tid; i < n; i += NT_M) {
    if (take == n || keys[i] >= prefix) {
      const int slot = atomicAdd(&nsel, 1);
      if (slot < TOPK_MAX_K)  // duplicate indices in the lists (invalid input) cannot overrun
        sel[slot] = ((uint64_t)(0xFFFFFFFFu - (uint32_t)keys[i]) << 32) | (keys[i] >> 32);
    }
  }
  __syncthreads();
  // ascending global index: bitonic sort of the selected pairs, padded with all-ones
  int m = 1;
  while (m < take) m <<= 1;
  for (int i = take + tid; i < m; i += NT_M) sel[i] = ~0ull;
  __syncthreads();
  for (int size = 2; size <= m; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < m / 2; i += NT_M) {
        const int lo = 2 * i - (i & (stride - 1));  // first element of the i-th pair
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = sel[lo], b = sel[hi];
        if ((a > b) == up) {
          sel[lo] = b;
          sel[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  int32_t* oi = idx_out + t * top_k;
  int32_t* os = score_out ? score_out + t * top_k : nullptr;
  for (int j = tid; j < top_k; j += NT_M) {
    oi[j] = j < take ? (int32_t)(sel[j] >> 32) : -1;
    if (os) os[j] = j < take ? (int32_t)(uint32_t)sel[j] : -1;
  }
}

// Shard `shard` of n_shards: the entries g of a global selection with g mod n == shard, as
// g div n, in order, then -1. One 256-thread workgroup per token; each thread a contiguous chunk.
__global__ __launch_bounds__(256) void local_indices_kernel(int top_k, const int32_t* __restrict__ idx,
                                                            int n_shards, int shard,
                                                            int32_t* __restrict__ local_idx) {
  __shared__ int pre[257];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int chunk = (top_k + 255) / 256;
  const int j0 = min(tid * chunk, top_k), j1 = min(j0 + chunk, top_k);
  const int32_t* row = idx + t * top_k;
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += row[j] >= 0 && row[j] % n_shards == shard;
  pre[tid + 1] = cnt;
  if (tid == 0) pre[0] = 0;
  __syncthreads();
  if (tid == 0)
    for (int i = 1; i <= 256; ++i) pre[i] += pre[i - 1];
  __syncthreads();
  int32_t* out = local_idx + t * top_k;
  int pos = pre[tid];
  for (int j = j0; j < j1; ++j) {
    const int32_t g = row[j];
    if (g >= 0 && g % n_shards == shard) out[pos++] = g / n_shards;
  }
  for (int j = pre[256] + tid; j < top_k; j += 256) out[j] = -1;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  typedef __bf16 bf;
  return __builtin_bit_cast(uint16_t, (bf)f);
}

// One 64-thread block per (token, head); thread x covers dims x, x + 64, ...
__global__ __launch_bounds__(64) void lse_merge_kernel(int total_q, int H, int D_v, int n_parts,
                                                       const uint16_t* __restrict__ outs,
                                                       const float* __restrict__ lses,
                                                       uint16_t* __restrict__ out,
                                                       float* __restrict__ lse_out) {
  const int64_t th = blockIdx.x;  // token * H + head
  const int64_t plane_o = (int64_t)total_q * H * D_v, plane_l = (int64_t)total_q * H;
  float m = -INFINITY;
  for (int i = 0; i < n_parts; ++i) m = fmaxf(m, lses[i * plane_l + th]);
  float z = 0.f;
  for (int i = 0; i < n_parts; ++i) {
    const float li = lses[i * plane_l + th];
    z += li == -INFINITY ? 0.f : __expf(li - m);
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  for (int d = threadIdx.x; d < D_v; d += 64) {
    float acc = 0.f;
    for (int i = 0; i < n_parts; ++i) {
      const float li = lses[i * plane_l + th];
      if (li == -INFINITY) continue;
      acc += __expf(li - m) * bf16_to_f32(outs[i * plane_o + th * D_v + d]);
    }
    out[th * D_v + d] = f32_to_bf16(acc * inv);
  }
  if (lse_out && threadIdx.x == 0) lse_out[th] = z > 0.f ? m + __logf(z) : -INFINITY;
}

}  // namespace

size_t topk_merge_lds_bytes() {
  return sizeof(uint64_t) * (MERGE_MAX_CAND + TOPK_MAX_K);
}

hipError_t launch_topk_merge(int32_t total_q, int32_t n_lists, int32_t k_in, const int32_t* idx_lists,
                             const int32_t* score_lists, int64_t list_stride, int32_t top_k,
                             int32_t* idx, int32_t* score, hipStream_t s) {
  const size_t lds = topk_merge_lds_bytes();
  static const bool lds_set = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_merge_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return true;
  }();
  (void)lds_set;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)total_q), dim3(NT_M), lds, s, n_lists, k_in,
                     idx_lists, score_lists, list_stride, top_k, idx, score);
  return hipGetLastError();
}

hipError_t launch_local_indices(int32_t total_q, int32_t top_k, const int32_t* idx, int32_t n_shards,
                                int32_t shard, int32_t* local_idx, hipStream_t s) {
  hipLaunchKernelGGL(local_indices_kernel, dim3((unsigned)total_q), dim3(256), 0, s, top_k, idx,
                     n_shards, shard, local_idx);
  return hipGetLastError();
}

hipError_t launch_lse_merge(int32_t total_q, int32_t H, int32_t D_v, int32_t n_parts,
                            const void* outs, const float* lses, void* out, float* lse,
                            hipStream_t s) {
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((int64_t)total_q * H)), dim3(64), 0, s,
                     total_q, H, D_v, n_parts, static_cast<const uint16_t*>(outs), lses,
                     static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace smla
