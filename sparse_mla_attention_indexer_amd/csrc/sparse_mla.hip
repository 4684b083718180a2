// sparse_mla.hip — sparse Multi-head Latent Attention in MQA form on gfx950.
//
// Every head of a query token attends over the same top-k latent rows; one gathered row serves
// all 64 heads, which is what lifts the intensity from ~26 to ~191 FLOP per byte on the pages
// ("Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", sections "PCP: split tokens, not heads" and
// "Why the numbers work": QK over 576 dims, PV over 512, BF16 queries and outputs, 656-byte FP8
// rows). Partial results over disjoint row sets merge by log-sum-exp (section "DCP").
//
// FP8 kernel (64 heads, 576/512 dims, 656-byte rows), one workgroup of 4 waves per (token,
// split), 64-row tiles:
//  1. all 256 threads gather the tile's rows (each wave instruction reads 512 contiguous bytes
//     of one row), dequantise e4m3 * block scale to bf16 and store the tile twice in LDS:
//     row-major K[row][576] for QK^T and transposed V^T[512][row] for PV (16-byte chunks
//     XOR-swizzled so both the writes and the MFMA operand reads are bank-conflict free);
//  2. wave (g, r) holds Q of heads [32g, 32g+32) in registers and computes S^T for rows
//     [32r, 32r+32) on v_mfma_f32_32x32x16_bf16 with the rows as M and the heads as N, so each
//     lane owns one head's logits;
//  3. the two waves of a head group share the tile maximum through LDS and keep one running
//     maximum per head; O is rescaled only when the maximum grows by more than 2^8 (so P stays
//     <= 256 and a bf16 P loses nothing);
//  4. P goes to LDS and wave (g, r) accumulates O^T for dims [256r, 256r+256) of its 32 heads as
//     V^T * P^T over all 64 rows (the same lane-owns-a-head layout as S^T).
// Decode splits a token's rows across workgroups and merges the partials by log-sum-exp.
#include "smla_internal.h"

namespace smla {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

namespace {

constexpr int NT = 256;
constexpr int TILE = MLA_TILE;           // 64 rows
constexpr int KCH = MLA_DQK / 8;         // 72 16-byte chunks per K row
constexpr int K_BYTES = TILE * MLA_DQK * 2;     // 73728
constexpr int VT_BYTES = MLA_DV * TILE * 2;     // 65536
constexpr int P_BYTES = MLA_H * TILE * 2;       // 8192
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_LOG2 = 8.0f;

struct __align__(16) MlaSmem {
  unsigned char k[K_BYTES];   // K[row][chunk ^ (row & 7)] (16-byte chunks of 8 bf16)
  unsigned char vt[VT_BYTES]; // V^T[dim][chunk ^ ((dim + dim/8) & 7)] (chunks of 8 rows)
  unsigned char p[P_BYTES];   // P[head][chunk ^ (head & 7)] (chunks of 8 rows)
  float scale[TILE][4];
  int rowidx[TILE];
  float tmax[2][2][32];
  float lsum[2][2][32];
};

__device__ __forceinline__ int k_off(int row, int chunk) { return (row * KCH + (chunk ^ (row & 7))) * 16; }
__device__ __forceinline__ int vt_off(int dim, int chunk) {
  return (dim * (TILE / 8) + (chunk ^ ((dim + (dim >> 3)) & 7))) * 16;
}
__device__ __forceinline__ int p_off(int head, int chunk) {
  return (head * (TILE / 8) + (chunk ^ (head & 7))) * 16;
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  v2f x = {a, b};
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  v2bf y = __builtin_convertvector(x, v2bf);
  return __builtin_bit_cast(unsigned, y);
}

// Gather + dequantise one tile into LDS. Rows whose index is < 0 are stored as zeros.
__device__ void load_tile(MlaSmem& sm, const unsigned char* __restrict__ kv_req,
                          const int32_t* __restrict__ idx_row, int r0, int r1, int pos) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  if (tid < TILE) {
    const int j = r0 + tid;
    int ix = j < r1 ? idx_row[j] : -1;
    if (ix > pos) ix = -1;  // rows past the token's position are never read
    sm.rowidx[tid] = ix;
    float4 sc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ix >= 0) sc = *reinterpret_cast<const float4*>(kv_req + (int64_t)ix * MLA_ROW_BYTES + 512);
    sm.scale[tid][0] = sc.x;
    sm.scale[tid][1] = sc.y;
    sm.scale[tid][2] = sc.z;
    sm.scale[tid][3] = sc.w;
  }
  __syncthreads();
  // rope dims 512..575 (bf16 as stored): thread -> row 16*wave + lane/4, 32 bytes
  {
    const int row = 16 * wave + (lane >> 2), part = lane & 3;
    const int ix = sm.rowidx[row];
    v4u a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (ix >= 0) {
      const v4u* src = reinterpret_cast<const v4u*>(kv_req + (int64_t)ix * MLA_ROW_BYTES + 528 + 32 * part);
      a = src[0];
      b = src[1];
    }
    *reinterpret_cast<v4u*>(sm.k + k_off(row, 64 + 2 * part)) = a;
    *reinterpret_cast<v4u*>(sm.k + k_off(row, 64 + 2 * part + 1)) = b;
  }
  // value dims 0..511: lane -> dims [8*lane, 8*lane + 8); wave -> two blocks of 8 rows
  const int c = lane;
  const int blk = c >> 4;  // 128-dim scale block
#pragma unroll 1
  for (int rb = 0; rb < 2; ++rb) {
    const int rbase = 16 * wave + 8 * rb;
    v2u raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ix = sm.rowidx[rbase + i];
      raw[i] = ix >= 0 ? *reinterpret_cast<const v2u*>(kv_req + (int64_t)ix * MLA_ROW_BYTES + 8 * c)
                       : v2u{0u, 0u};
    }
    const int rchunk = rbase >> 3;
    // four dims at a time (one dword of codes per row) keeps the live set small
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float f[8][4];  // [row][dim]
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float s = sm.scale[rbase + i][blk];
        const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[i][h], false);
        const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[i][h], true);
        f[i][0] = lo[0] * s;
        f[i][1] = lo[1] * s;
        f[i][2] = hi[0] * s;
        f[i][3] = hi[1] * s;
        v2u o = {pack_bf16(f[i][0], f[i][1]), pack_bf16(f[i][2], f[i][3])};
        *reinterpret_cast<v2u*>(sm.k + k_off(rbase + i, c) + 8 * h) = o;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        v4u o = {pack_bf16(f[0][d], f[1][d]), pack_bf16(f[2][d], f[3][d]), pack_bf16(f[4][d], f[5][d]),
                 pack_bf16(f[6][d], f[7][d])};
        *reinterpret_cast<v4u*>(sm.vt + vt_off(8 * c + 4 * h + d, rchunk)) = o;
      }
    }
  }
  __syncthreads();
}

// One (token, split): rows idx_row[r_begin, r_end) of the token's request.
// Writes either the final bf16 output (+ lse) or an fp32 partial (+ lse) for the combine.
__global__ __launch_bounds__(NT, 1) void mla_fp8_kernel(const Tok* __restrict__ toks,
                                                        const __bf16* __restrict__ q,
                                                        const unsigned char* __restrict__ kv,
                                                        const int32_t* __restrict__ idx,
                                                        int top_k, int rows_per_split,
                                                        float sm_scale, __bf16* __restrict__ out,
                                                        float* __restrict__ lse_out,
                                                        float* __restrict__ part_o,
                                                        float* __restrict__ part_lse) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  MlaSmem& sm = *reinterpret_cast<MlaSmem*>(smem_raw);
  const int64_t t = blockIdx.x;
  const int split = blockIdx.y;
  const int nsplit = gridDim.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hg = wave >> 1, rr = wave & 1;
  const int col = lane & 31, half = lane >> 5;
  const int head = 32 * hg + col;

  const Tok tk = toks[t];
  const unsigned char* kv_req = kv + tk.row_start * MLA_ROW_BYTES;
  const int32_t* idx_row = idx + t * top_k;
  const int r_begin = split * rows_per_split;
  const int r_end = min(top_k, r_begin + rows_per_split);

  // Q^T fragments: head `head`, dims [8*half + 16*ks, +8)
  v8bf qf[MLA_DQK / 16];
  {
    const __bf16* qh = q + (t * MLA_H + head) * MLA_DQK + 8 * half;
#pragma unroll
    for (int ks = 0; ks < MLA_DQK / 16; ++ks) qf[ks] = *reinterpret_cast<const v8bf*>(qh + 16 * ks);
  }
  v16f o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = v16f{};
  // Per-lane LDS bases. The XOR swizzles only touch the low three chunk bits, so every
  // operand read is one of a few bases plus a compile-time offset.
  const unsigned char* kbase[4];  // K row 32*rr + col, chunks half + 2u (+ 8 per 64 dims)
  {
    const int row = 32 * rr + col;
#pragma unroll
    for (int u = 0; u < 4; ++u) kbase[u] = sm.k + k_off(row, half + 2 * u);
  }
  const unsigned char* vbase[4][2];  // V^T dims 256*rr + 32*m + col, m = 0 or 1; chunk half + 2ks
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int m = 0; m < 2; ++m) vbase[ks][m] = sm.vt + vt_off(256 * rr + 32 * m + col, half + 2 * ks);
  const unsigned char* pbase[4];  // P of `head`, chunk half + 2ks
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) pbase[ks] = sm.p + p_off(head, half + 2 * ks);
  float m_run = -INFINITY;  // running max of this lane's head, log2 units
  float l_run = 0.f;        // this lane's share of the softmax denominator
  const float c = sm_scale * LOG2E;

#pragma unroll 1
  for (int r0 = r_begin; r0 < r_end; r0 += TILE) {
    load_tile(sm, kv_req, idx_row, r0, r_end, tk.pos);
    bool any_valid = false;
    {
      const int ix = sm.rowidx[lane];
      any_valid = __any(ix >= 0);
    }
    if (!any_valid) {
      __syncthreads();
      continue;
    }
    // S^T for rows [32*rr, 32*rr + 32) of the tile x heads [32*hg, +32)
    v16f s = v16f{};
#pragma unroll
    for (int kc = 0; kc < MLA_DQK / 64; ++kc) {
      v8bf a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = *reinterpret_cast<const v8bf*>(kbase[u] + 128 * kc);
#pragma unroll
      for (int u = 0; u < 4; ++u) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], qf[4 * kc + u], s, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane holds head `head`, rows 32*rr + 8*(i/4) + 4*half + i%4
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * rr + 8 * (i >> 2) + 4 * half + (i & 3);
      const float v = sm.rowidx[row] >= 0 ? s[i] * c : -INFINITY;
      s[i] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (half == 0) sm.tmax[hg][rr][col] = tmax;
    __syncthreads();
    tmax = fmaxf(tmax, sm.tmax[hg][rr ^ 1][col]);
    // both waves of a head group see the same maxima and take the same decision
    const float m_new = fmaxf(m_run, tmax);
    if (__any(m_new > m_run + RESCALE_LOG2)) {
      const float alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    // P = exp2(s - m_run) -> LDS as bf16, rows in groups of 4
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float p4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p4[i] = exp2f(s[4 * g4 + i] - m_run);
        l_run += p4[i];
      }
      const int row0 = 32 * rr + 8 * g4 + 4 * half;  // first of 4 consecutive rows
      v2u pk = {pack_bf16(p4[0], p4[1]), pack_bf16(p4[2], p4[3])};
      *reinterpret_cast<v2u*>(sm.p + p_off(head, row0 >> 3) + 8 * ((row0 >> 2) & 1)) = pk;
    }
    __syncthreads();
    // O^T[dims 256*rr + 32*mt + m][head] += V^T[dim][rows] * P^T[rows][head]
#pragma unroll
    for (int ks = 0; ks < TILE / 16; ++ks) {
      const v8bf b = *reinterpret_cast<const v8bf*>(pbase[ks]);
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
        v8bf a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int mt = 4 * mh + u;  // dims 256*rr + 32*mt + col; swizzle depends on mt & 1
          a[u] = *reinterpret_cast<const v8bf*>(vbase[ks][mt & 1] + (mt >> 1) * (64 * TILE * 2));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[4 * mh + u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b, o[4 * mh + u], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  }

  // denominator of each head: both lane halves and both row halves
  l_run += __shfl_xor(l_run, 32);
  if (half == 0) sm.lsum[hg][rr][col] = l_run;
  __syncthreads();
  const float l_tot = l_run + sm.lsum[hg][rr ^ 1][col];
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float lse = empty ? -INFINITY : (m_run + log2f(l_tot)) * (1.0f / LOG2E);

  if (part_o == nullptr) {
    __bf16* orow = out + (t * MLA_H + head) * MLA_DV;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dim = 256 * rr + 32 * mt + 8 * g4 + 4 * half;
        v2u pk = {pack_bf16(o[mt][4 * g4] * inv, o[mt][4 * g4 + 1] * inv),
                  pack_bf16(o[mt][4 * g4 + 2] * inv, o[mt][4 * g4 + 3] * inv)};
        *reinterpret_cast<v2u*>(orow + dim) = pk;
      }
    if (lse_out && rr == 0 && half == 0) lse_out[t * MLA_H + head] = lse;
  } else {
    float* prow = part_o + ((t * nsplit + split) * MLA_H + head) * MLA_DV;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dim = 256 * rr + 32 * mt + 8 * g4 + 4 * half;
        float4 v = make_float4(o[mt][4 * g4] * inv, o[mt][4 * g4 + 1] * inv, o[mt][4 * g4 + 2] * inv,
                               o[mt][4 * g4 + 3] * inv);
        *reinterpret_cast<float4*>(prow + dim) = v;
      }
    if (rr == 0 && half == 0) part_lse[(t * nsplit + split) * MLA_H + head] = lse;
  }
}

// Merge split partials by log-sum-exp: one 128-thread block per (token, head), 4 dims/thread.
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          int nsplit, __bf16* __restrict__ out,
                                                          float* __restrict__ lse_out) {
  const int64_t th = blockIdx.x;  // t * H + h
  const int64_t t = th / MLA_H;
  const int h = (int)(th % MLA_H);
  float m = -INFINITY;
  for (int j = 0; j < nsplit; ++j) m = fmaxf(m, part_lse[(t * nsplit + j) * MLA_H + h]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  const int d = 4 * threadIdx.x;
  if (m != -INFINITY) {
    for (int j = 0; j < nsplit; ++j) {
      const float lj = part_lse[(t * nsplit + j) * MLA_H + h];
      if (lj == -INFINITY) continue;
      const float wj = __expf(lj - m);
      wsum += wj;
      const float4 v = *reinterpret_cast<const float4*>(part_o + ((t * nsplit + j) * MLA_H + h) * MLA_DV + d);
      acc[0] += wj * v.x;
      acc[1] += wj * v.y;
      acc[2] += wj * v.z;
      acc[3] += wj * v.w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  v2u pk = {pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<v2u*>(out + th * MLA_DV + d) = pk;
  if (lse_out && threadIdx.x == 0) lse_out[th] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

// Generic bf16-row kernel for small head counts (H <= 16, D_qk <= 256): one 256-thread block
// per token; fp32 logits of all selected rows in LDS, exact softmax, then PV.
constexpr int GEN_MAX_H = 16;
constexpr int GEN_MAX_D = 256;

__global__ __launch_bounds__(256) void mla_generic_kernel(const Tok* __restrict__ toks,
                                                          const __bf16* __restrict__ q,
                                                          const __bf16* __restrict__ kv, int H,
                                                          int D_qk, int D_v,
                                                          const int32_t* __restrict__ idx,
                                                          int top_k, float sm_scale,
                                                          __bf16* __restrict__ out,
                                                          float* __restrict__ lse_out) {
  extern __shared__ float gsm[];
  float* qs = gsm;                       // [H][D_qk]
  float* lg = qs + GEN_MAX_H * GEN_MAX_D; // [H][top_k]
  __shared__ int ridx[TOPK_MAX_K];
  __shared__ float hmax[GEN_MAX_H], hsum[GEN_MAX_H];
  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const __bf16* kv_req = kv + tk.row_start * D_qk;
  for (int i = threadIdx.x; i < H * D_qk; i += blockDim.x) qs[i] = (float)q[t * H * D_qk + i];
  for (int i = threadIdx.x; i < top_k; i += blockDim.x) {
    const int ix = idx[t * top_k + i];
    ridx[i] = ix <= tk.pos ? ix : -1;  // rows past the token's position are never read
  }
  __syncthreads();
  for (int e = threadIdx.x; e < H * top_k; e += blockDim.x) {
    const int h = e / top_k, i = e % top_k;
    const int ix = ridx[i];
    float v = -INFINITY;
    if (ix >= 0) {
      const __bf16* row = kv_req + (int64_t)ix * D_qk;
      float acc = 0.f;
      for (int d = 0; d < D_qk; ++d) acc += qs[h * D_qk + d] * (float)row[d];
      v = acc * sm_scale;
    }
    lg[h * top_k + i] = v;
  }
  __syncthreads();
  // per-head max and sum: one wave per head (4 waves, loop)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int h = wave; h < H; h += 4) {
    float m = -INFINITY;
    for (int i = lane; i < top_k; i += 64) m = fmaxf(m, lg[h * top_k + i]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float s = 0.f;
    if (m != -INFINITY)
      for (int i = lane; i < top_k; i += 64) s += __expf(lg[h * top_k + i] - m);
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) {
      hmax[h] = m;
      hsum[h] = s;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < H * D_v; e += blockDim.x) {
    const int h = e / D_v, d = e % D_v;
    const float m = hmax[h], s = hsum[h];
    float acc = 0.f;
    if (s > 0.f)
      for (int i = 0; i < top_k; ++i) {
        const int ix = ridx[i];
        if (ix < 0) continue;
        acc += __expf(lg[h * top_k + i] - m) * (float)kv_req[(int64_t)ix * D_qk + d];
      }
    out[(t * H + h) * D_v + d] = (__bf16)(s > 0.f ? acc / s : 0.f);
  }
  if (lse_out)
    for (int h = threadIdx.x; h < H; h += blockDim.x)
      lse_out[t * H + h] = hsum[h] > 0.f ? hmax[h] + __logf(hsum[h]) : -INFINITY;
}

}  // namespace

int mla_decode_splits(const smla_batch& b, int32_t top_k) {
  const int tiles = (top_k + TILE - 1) / TILE;
  int s = (256 + b.total_q - 1) / b.total_q;  // aim at one workgroup per CU
  if (s > tiles) s = tiles;
  if (s < 1) s = 1;
  return s;
}

size_t mla_workspace_bytes(const smla_batch& b, int32_t H, int32_t D_v, int32_t top_k, int decode) {
  if (!decode) return 0;
  const int s = mla_decode_splits(b, top_k);
  if (s <= 1) return 0;
  const size_t n = (size_t)b.total_q * s * H;
  return align_up(n * D_v * sizeof(float), 256) + align_up(n * sizeof(float), 256);
}

hipError_t launch_mla_fp8(const smla_batch& b, const void* q, const void* kv, const int32_t* idx,
                          int32_t top_k, float sm_scale, void* out, float* lse, void* ws,
                          int decode, hipStream_t s) {
  TableView tv = table_view(b.table, b.batch, b.total_q);
  const int nsplit = decode ? mla_decode_splits(b, top_k) : 1;
  const int tiles = (top_k + TILE - 1) / TILE;
  const int rows_per_split = ((tiles + nsplit - 1) / nsplit) * TILE;
  const size_t lds = sizeof(MlaSmem);
  static const bool lds_set = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&mla_fp8_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return true;
  }();
  (void)lds_set;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (nsplit > 1) {
    part_o = static_cast<float*>(ws);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                        align_up((size_t)b.total_q * nsplit * MLA_H * MLA_DV * sizeof(float), 256));
  }
  mark_stage(STAGE_MLA, false, s);
  hipLaunchKernelGGL(mla_fp8_kernel, dim3(b.total_q, nsplit), dim3(NT), lds, s, tv.tok,
                     static_cast<const __bf16*>(q), static_cast<const unsigned char*>(kv), idx, top_k,
                     rows_per_split, sm_scale, static_cast<__bf16*>(out), lse, part_o, part_lse);
  mark_stage(STAGE_MLA, true, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  mark_stage(STAGE_COMBINE, false, s);
  hipLaunchKernelGGL(mla_combine_kernel, dim3(b.total_q * MLA_H), dim3(128), 0, s, part_o, part_lse,
                     nsplit, static_cast<__bf16*>(out), lse);
  mark_stage(STAGE_COMBINE, true, s);
  return hipGetLastError();
}

hipError_t launch_mla_generic(const smla_batch& b, const void* q, const void* kv, int32_t H,
                              int32_t D_qk, int32_t D_v, const int32_t* idx, int32_t top_k,
                              float sm_scale, void* out, float* lse, hipStream_t s) {
  TableView tv = table_view(b.table, b.batch, b.total_q);
  const size_t lds = sizeof(float) * (GEN_MAX_H * GEN_MAX_D + (size_t)GEN_MAX_H * top_k);
  static const bool lds_set = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&mla_generic_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(sizeof(float) * (GEN_MAX_H * GEN_MAX_D + GEN_MAX_H * TOPK_MAX_K)));
    return true;
  }();
  (void)lds_set;
  hipLaunchKernelGGL(mla_generic_kernel, dim3(b.total_q), dim3(256), lds, s, tv.tok,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(kv), H, D_qk, D_v, idx,
                     top_k, sm_scale, static_cast<__bf16*>(out), lse);
  return hipGetLastError();
}

}  // namespace smla
