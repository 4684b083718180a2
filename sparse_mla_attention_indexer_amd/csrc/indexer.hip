// indexer.hip — lightning-indexer scores on gfx950.
//
// score(t, s) = sum_h w_h * ReLU(q_I[t,h] . k_I[s]) for every earlier token s <= p(t): the
// indexer that scores every earlier token so sparse MLA can keep the best 2,048 ("Serving
// GLM-5.3 ... PCP, DCP, Hybrid HiSparse", sections "Why DP8 and TP8 fall short" and "PCP:
// split tokens, not heads"; the formula is the workload definition of the tiny causal prefill).
//
// 64 heads x 128 dims: a dense int8 contraction per (query, key) pair, run on
// v_mfma_i32_32x32x32_i8 with the heads of one query token as the M dimension (two 32-row
// tiles) and 32 keys as N. Keys go straight from HBM into B-operand registers: the contraction
// order over the 128 dims is permuted so every lane reads 64 contiguous bytes of its key (lane
// half h covers dims [64h, 64h+64)), and the query fragments use the same permutation. The
// ReLU * w head reduction runs in the accumulator registers, then across the two lane halves.
//
// FP8 keys (the pages' deployed key: 128 E4M3 values and one fp32 scale per token, 132 bytes;
// section "Why the numbers work") take the same kernels with v_mfma_f32_32x32x64_f8f6f4 (two
// 64-dim k-steps instead of four 32-dim ones, the same bytes per lane), fp32 accumulators, fp32
// per-token head weights and the key's scale applied to the head sum (a positive factor passes
// through the ReLU). The scales of a key tile ride with its keys into LDS.
//
// Work is planned on the host (smla_batch_build): query tiles of up to 4 tokens are paired
// front with back (tile i with tile n-1-i), the pages' load-balanced chunk pairing applied to
// causal query tiles on one GPU, and each pair's combined key range is cut into equal chunks.
#include <type_traits>

#include "smla_internal.h"

namespace smla {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

namespace {

constexpr int IDX_H = 64;
constexpr int IDX_D = 128;


// Waits until at most N of this wave's vector-memory operations are outstanding (inline
// assembly, so that it keeps its place among the hand-counted memory operations).
template <int N>
__device__ __forceinline__ void idx_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits for all of this wave's loads, visibly to the compiler (it then knows that registers
// loaded earlier are ready and adds no waits of its own after the hand-counted loads start).
__device__ __forceinline__ void idx_wait_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  asm volatile("" ::: "memory");
}

// The weights of a lane's heads (w < 2^10 by the weight contract): lo[r] for head
// 8 (r / 4) + 4 half + r % 4, hi[r] for the same + 32. Kept unpacked so that the multiply-adds
// need no sub-dword operand selection and fuse into v_mad_u32_u24.
struct HeadW {
  uint32_t lo[16], hi[16];
};

// a * b + c with 24-bit operands, one instruction (left to itself the compiler splits it into a
// multiply and a three-input add, which costs more per product)
__device__ __forceinline__ uint32_t mad_u24(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// The score of the lane's key: sum over its 32 heads of ReLU(dot) * w, plus the other lane half's
// (the other 32 heads). ReLU(dot) <= 2^21 and w < 2^10, so 24-bit multiplies are exact and run at
// full rate; four independent partial sums keep the chain of dependent adds from setting the pace.
__device__ __forceinline__ uint32_t relu_weighted_sum(const v16i& acc0, const v16i& acc1,
                                                      const HeadW& w) {
  uint32_t ps[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    ps[r & 3] = mad_u24((uint32_t)max(acc0[r], 0), w.lo[r], ps[r & 3]);
    ps[r & 3] = mad_u24((uint32_t)max(acc1[r], 0), w.hi[r], ps[r & 3]);
  }
  const uint32_t sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  const auto b = __builtin_amdgcn_permlane32_swap(sum, sum, false, false);  // no LDS round trip
  return (uint32_t)b[0] + (uint32_t)b[1];
}

// With the weights folded into the queries: the lane's key score is the plain sum over its 32
// heads of ReLU(dot), plus the other lane half's; one max per value and one three-input add per
// two values.
__device__ __forceinline__ uint32_t relu_sum(const v16i& acc0, const v16i& acc1) {
  uint32_t ps[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < 16; ++r)
    ps[r & 3] = (uint32_t)max(acc0[r], 0) + (uint32_t)max(acc1[r], 0) + ps[r & 3];
  const uint32_t sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  const auto b = __builtin_amdgcn_permlane32_swap(sum, sum, false, false);
  return (uint32_t)b[0] + (uint32_t)b[1];
}

// The weights folded into a lane's query fragments (heads col and 32 + col; wown = their
// weights): w_h ReLU(q_h . k) = ReLU((w_h q_h) . k) exactly when w_h >= 0 and every w_h q_h[d]
// fits int8, and then the epilogue needs no multiplies. Returns whether that holds for the whole
// wave (one query token), and then leaves the folded fragments in qa; otherwise qa is unchanged.
// The check keeps each head's smallest and largest byte; the fold multiplies the bytes two at a
// time in 16-bit halves and keeps each product's low byte (the same for signed and unsigned).
typedef unsigned short fold_u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bool fold_weights(v4i (&qa)[2][4], const int (&wown)[2]) {
  bool ok = true;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    int mx = -128, mn = 127;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = (uint32_t)qa[mt][j][e];
        const int b0 = (int)(x << 24) >> 24, b1 = (int)(x << 16) >> 24;
        const int b2 = (int)(x << 8) >> 24, b3 = (int)x >> 24;
        mx = max(mx, max(max(b0, b1), max(b2, b3)));
        mn = min(mn, min(min(b0, b1), min(b2, b3)));
      }
    const int w = wown[mt];
    ok = ok && w >= 0 && w * mx <= 127 && w * mn >= -128;
  }
  if (!__all(ok)) return false;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const fold_u16x2 w2 = {(unsigned short)wown[mt], (unsigned short)wown[mt]};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = (uint32_t)qa[mt][j][e];
        const fold_u16x2 ev = __builtin_bit_cast(fold_u16x2, x & 0x00FF00FFu) * w2;
        const fold_u16x2 od = __builtin_bit_cast(fold_u16x2, (x >> 8) & 0x00FF00FFu) * w2;
        qa[mt][j][e] = (int)((__builtin_bit_cast(uint32_t, ev) & 0x00FF00FFu) |
                             ((__builtin_bit_cast(uint32_t, od) & 0x00FF00FFu) << 8));
      }
  }
  return true;
}

// FP8 keys: fp32 weights of a lane's heads (same head order as HeadW), per query token.
struct HeadWF {
  float lo[16], hi[16];
};

__device__ __forceinline__ HeadWF load_head_wf(const float* w_tok) {
  const int half = (threadIdx.x & 63) >> 5;
  HeadWF wl;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int h = 8 * (r >> 2) + 4 * half + (r & 3);
    wl.lo[r] = w_tok[h];
    wl.hi[r] = w_tok[32 + h];
  }
  return wl;
}

// ReLU of an fp32 value as one integer max on its bits: every negative value (-0 included) has
// the sign bit set and becomes +0. (A float max would first quiet the operand: two instructions.)
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// FP8 keys: the lane's key score before its scale, sum over the 64 heads of ReLU(dot) * w in fp32
// (four partial sums from +0, so the result is never -0).
__device__ __forceinline__ float relu_weighted_sum_f(const v16f& acc0, const v16f& acc1,
                                                     const HeadWF& w) {
  float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    ps[r & 3] = __builtin_fmaf(relu_bits(acc0[r]), w.lo[r], ps[r & 3]);
    ps[r & 3] = __builtin_fmaf(relu_bits(acc1[r]), w.hi[r], ps[r & 3]);
  }
  const float sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, sum),
                                                  __builtin_bit_cast(unsigned, sum), false, false);
  return __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
}

// One E4M3 x E4M3 step over 64 dims: lane half h supplies the same 32 bytes (dims) of its head
// and of its key, so the contraction pairs equal dims whatever the instruction's k order.
__device__ __forceinline__ v16f mfma_f8(const v4i& a0, const v4i& a1, const v4i& b0, const v4i& b1,
                                        const v16f& c) {
  const v8i a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  const v8i b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
  // format 0 (E4M3) for both operands; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Raw buffer descriptor (stride 0) over `bytes` bytes at `base`: stores at offsets >= bytes are
// dropped by the hardware, yet count as memory operations like any other.
typedef int idx_v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ idx_v4s idx_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  idx_v4s r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// One 4-byte buffer store as inline assembly: the compiler can neither merge, drop nor move it
// across the other hand-counted operations.
__device__ __forceinline__ void idx_store32(const idx_v4s& rs, uint32_t off, uint32_t v) {
  asm volatile("buffer_store_dword %0, %1, %2, 0 offen" ::"v"(v), "v"(off), "s"(rs) : "memory");
}

// Barrier that waits for this wave's LDS operations only (key loads of later groups keep flying).
__device__ __forceinline__ void idx_lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One load-to-LDS instruction (inline assembly, so that the compiler neither counts it nor
// drains it before LDS writes): lane l's 16 bytes at g land at lds + 16 l. M0 is restored.
__device__ __forceinline__ void idx_lds_load16(const void* g, void* lds) {
  const unsigned a = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(a)
      : "memory");
}

// As idx_lds_load16 with 4 bytes per lane (lane l's dword lands at lds + 4 l).
__device__ __forceinline__ void idx_lds_load4(const void* g, void* lds) {
  const unsigned a = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(a)
      : "memory");
}

// ---- single-token query tiles: each wave streams its own key tiles through LDS ----------------
// One wave: query token t against key tiles s = s_begin, s_begin + step, ... < s_end, s <= p.
// Key tiles reach LDS by the load-to-LDS path in whole 128-byte lines (eight lanes per key, one
// 1 KB instruction per eight keys), KR tiles ahead in a ring of the wave's own; the slot of
// piece P (16 bytes) of key c is 8 c + (P ^ ((c >> 1) & 7)), which keeps the B-operand reads
// (32 keys, one piece) free of bank conflicts. The products of tile i+1 are issued before the
// epilogue of tile i. `lh` (LDS, optional) receives the histogram code of every score.
// F8: a fifth load per tile brings the tile's 32 key scales into `scl` (one slot per ring tile).
constexpr int KR = 4;  // key tiles per wave in flight or in use

template <bool F8>
__device__ __forceinline__ void indexer_wave(const Tok& tk, int64_t t, int s_begin, int s_end,
                                             int step, const int8_t* __restrict__ q_idx,
                                             const int8_t* __restrict__ k_idx,
                                             const float* __restrict__ k_scale,
                                             const HeadW& wl, const int32_t* __restrict__ w_i,
                                             const float* __restrict__ w_f,
                                             int32_t* __restrict__ out_row,
                                             int* lh, v4i (*ring)[256], float (*scl)[64]) {
  using Acc = std::conditional_t<F8, v16f, v16i>;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int p = tk.pos;
  const int last = s_end - 1 < p ? s_end - 1 : p;  // last key this wave may score
  if (s_begin > last) return;
  // A fragments: head 32*mt + col, dims [64*half + 16*j, +16)
  v4i qa[2][4];
  const int8_t* qbase = q_idx + t * (IDX_H * IDX_D);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qa[mt][j] = *reinterpret_cast<const v4i*>(qbase + (32 * mt + col) * IDX_D + 64 * half + 16 * j);
  HeadWF wf;
  int wown[2] = {0, 0};
  if constexpr (F8) wf = load_head_wf(w_f + t * IDX_H);
  else wown[0] = w_i[col], wown[1] = w_i[32 + col];
  idx_wait_loads();  // the fragments are in before any key load goes out
  bool fold = false;
  if constexpr (!F8) fold = fold_weights(qa, wown);

  // Scores go out through a buffer resource whose range ends at key `last`: the hardware drops
  // the stores of keys past it, of the upper lane half and of the placeholder stores below, so
  // every step issues exactly one store and the waits below can count this wave's memory
  // operations exactly.
  const idx_v4s out_rs = idx_rsrc(out_row, (last + 1) * 4);
  const int8_t* kbase = k_idx + tk.row_start * IDX_D;
  const float* sbase = F8 ? k_scale + tk.row_start : nullptr;
  const int ntile = (last - s_begin) / step + 1;
  const int dkey = lane >> 3, dpc = lane & 7;  // load lanes: key 8d + dkey, slot piece dpc
  auto dma = [&](int i) {  // tile i (past the end: clamped keys, never scored)
    const int s = s_begin + i * step;
    v4i* dst = ring[i % KR];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int c = 8 * d + dkey;
      const int key = min(s + c, last);
      idx_lds_load16(kbase + (int64_t)key * IDX_D + 16 * (dpc ^ ((c >> 1) & 7)), dst + 64 * d);
    }
    if constexpr (F8) idx_lds_load4(sbase + min(s + (lane & 31), last), scl[i % KR]);
  };
  auto placeholder_store = [&]() { idx_store32(out_rs, 0x7FFFFFF0u, 0u); };
  auto products = [&](int i, Acc& acc0, Acc& acc1) {
    const v4i* kt = ring[i % KR];
    v4i kb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kb[j] = kt[8 * col + ((4 * half + j) ^ ((col >> 1) & 7))];
    // all four operand reads go out before the first matrix instruction (left alone, the compiler
    // may hold one back and stall the matrix sequence on its own LDS round trip)
    __builtin_amdgcn_sched_barrier(0);
    acc0 = Acc{};
    acc1 = Acc{};
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        acc0 = mfma_f8(qa[0][j], qa[0][j + 1], kb[j], kb[j + 1], acc0);
        acc1 = mfma_f8(qa[1][j], qa[1][j + 1], kb[j], kb[j + 1], acc1);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[0][j], kb[j], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[1][j], kb[j], acc1, 0, 0, 0);
      }
    }
  };
  // lane holds key `col`, heads 32*mt + 8*(r/4) + 4*half + r%4
  auto epilogue = [&](auto foldc, const Acc& acc0, const Acc& acc1, int i) {
    uint32_t sum;
    if constexpr (F8)
      sum = __builtin_bit_cast(uint32_t, relu_weighted_sum_f(acc0, acc1, wf) * scl[i % KR][col]);
    else if constexpr (decltype(foldc)::value)
      sum = relu_sum(acc0, acc1);
    else
      sum = relu_weighted_sum(acc0, acc1, wl);
    const int key = s_begin + i * step + col;
    idx_store32(out_rs, half ? 0x7FFFFFF0u : (uint32_t)key * 4u, sum);
    if (lh && half == 0 && key <= last) atomicAdd(&lh[F8 ? topk_fbin(sum) : topk_bin(sum)], 1);
  };

  // Prologue: tiles 0 .. KR-2 with a placeholder store after each, as if earlier steps had run;
  // then step i: load tile i+KR-1, wait for tile i+1 (after its loads: one store, then tile
  // i+2's loads and a store, ..., tile i+KR-1's loads = 5 (KR-2) operations; 6 (KR-2) with the
  // scale loads), products of tile i+1, epilogue of tile i.
  static_assert(KR == 4, "wait counts below assume four tiles");
  constexpr int OPS = F8 ? 6 : 5;  // memory operations per tile and step
  dma(0);
  placeholder_store();
  dma(1);
  placeholder_store();
  dma(2);
  placeholder_store();
  idx_wait_vmcnt<2 * OPS + 1>();  // tile 0: after it, a store, tile 1, a store, tile 2, a store
  // the loop is compiled once per epilogue (folded weights or not: uniform per wave)
  auto run = [&](auto foldc) {
    Acc a0[2], a1[2];
    products(0, a0[0], a1[0]);
#pragma unroll 1
    for (int i = 0; i < ntile; i += 2) {
      dma(i + 3);
      idx_wait_vmcnt<2 * OPS>();
      if (i + 1 < ntile) products(i + 1, a0[1], a1[1]);
      epilogue(foldc, a0[0], a1[0], i);
      if (i + 1 >= ntile) break;
      dma(i + 4);
      idx_wait_vmcnt<2 * OPS>();
      if (i + 2 < ntile) products(i + 2, a0[0], a1[0]);
      epilogue(foldc, a0[1], a1[1], i + 1);
    }
  };
  if (fold) run(std::true_type{});
  else run(std::false_type{});
  idx_wait_vmcnt<0>();  // no key load may still be writing this wave's ring when it returns
}

// ---- batches with query tiles of several tokens: key tiles shared through LDS -----------------
// The tokens of one query tile see (almost) the same keys, so the workgroup loads each 32-key
// tile once, straight into LDS (load-to-LDS, no registers), and every wave reads its B operands
// from there. Key tiles go through a ring of two groups of four: the loads of group g+1 are
// issued right after the barrier that opens group g (every wave has then finished group g-1,
// whose slots they take). The ring and histograms fit 48 KB, so three workgroups share a CU and
// hide each other's latencies. The LDS histograms count in 16 bits, two bins per word (a
// workgroup scores at most 1.25 KEY_CHUNK keys per token and segment, so a count stays below
// 2^16).
constexpr int SG = 4;      // key tiles per group
constexpr int SRING = 2;   // groups in the ring

// Segment of nq (1..4) tokens against keys [s0, s1) (one token: one wave works; such tiles only
// end a request). `ring`: SRING * SG tiles of 256 16-byte slots; slot 32 * piece + key holds
// bytes [16 piece, 16 piece + 16) of the tile's key `key`, so a wave's operand read (32 keys, one
// piece) is 512 consecutive bytes.
// F8: each wave's key load also brings its tile's 32 key scales into `scl`.
template <bool F8>
__device__ __forceinline__ void indexer_shared_seg(const Seg& sg, const Tok* __restrict__ toks,
                                                   const int8_t* __restrict__ q_idx,
                                                   const int8_t* __restrict__ k_idx,
                                                   const float* __restrict__ k_scale,
                                                   const HeadW& wl, const int32_t* __restrict__ w_i,
                                                   const float* __restrict__ w_f,
                                                   int32_t* __restrict__ scores, int64_t stride,
                                                   bool hist_on, int hist_min_n,
                                                   unsigned (*lhist)[TOPK_BINS / 2],
                                                   v4i (*ring)[256], float (*scl)[64]) {
  using Acc = std::conditional_t<F8, v16f, v16i>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  // waves per token: 2 for two tokens (they take alternate key tiles), else 1
  const int qpw = sg.nq == 2 ? 2 : 1;
  const int qi = wave / qpw, par = wave % qpw;
  const bool active = qi < sg.nq;
  const int64_t t = sg.q0 + (active ? qi : 0);
  const Tok tk = toks[t];
  const Tok tl = toks[sg.q0 + sg.nq - 1];  // the tile's last token sees the most keys
  const int kmax = min(sg.s1 - 1, tl.pos);   // last key any token of the tile may score
  const int last = min(sg.s1 - 1, tk.pos);   // last key of this wave's token
  const int ntile = (kmax - sg.s0) / 32 + 1;
  const int ngroup = (ntile + SG - 1) / SG;

  v4i qa[2][4];
  const int8_t* qbase = q_idx + t * (IDX_H * IDX_D);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qa[mt][j] = *reinterpret_cast<const v4i*>(qbase + (32 * mt + col) * IDX_D + 64 * half + 16 * j);
  HeadWF wf;
  int wown[2] = {0, 0};
  if constexpr (F8) wf = load_head_wf(w_f + t * IDX_H);
  else wown[0] = w_i[col], wown[1] = w_i[32 + col];
  idx_wait_loads();  // the fragments are in before any key load goes out
  bool fold = false;
  if constexpr (!F8) fold = fold_weights(qa, wown);

  // key loads: wave w loads tile SG*g + w of group g; instruction d covers slots 64d .. 64d+63
  const int8_t* kbase = k_idx + tk.row_start * IDX_D + 16 * (2 * 0 + half);
  const float* sbase = F8 ? k_scale + tk.row_start : nullptr;
  auto load_group = [&](int g) {
    const int k = SG * g + wave;
    const int key = min(sg.s0 + 32 * k + col, kmax);  // clamped: never past the visible rows
    const int8_t* src = kbase + (int64_t)key * IDX_D;
    v4i* dst = ring[(g % SRING) * SG + wave];
#pragma unroll
    for (int d = 0; d < 4; ++d) idx_lds_load16(src + 32 * d, dst + 64 * d);
    if constexpr (F8) idx_lds_load4(sbase + key, scl[(g % SRING) * SG + wave]);
  };
  load_group(0);

  int32_t* out_row = scores + (stride ? t * stride : tk.cand_off);
  const __amdgpu_buffer_rsrc_t out_rs =
      __builtin_amdgcn_make_buffer_rsrc(out_row, 0, active ? (last + 1) * 4 : 0, 0x00020000);
  unsigned* lh = active && hist_on && tk.pos + 1 > hist_min_n ? lhist[qi] : nullptr;

  auto epilogue = [&](auto foldc, const Acc& acc0, const Acc& acc1, int k) {
    uint32_t sum;
    if constexpr (F8)
      sum = __builtin_bit_cast(uint32_t, relu_weighted_sum_f(acc0, acc1, wf) *
                                             scl[((k / SG) % SRING) * SG + k % SG][col]);
    else if constexpr (decltype(foldc)::value)
      sum = relu_sum(acc0, acc1);
    else
      sum = relu_weighted_sum(acc0, acc1, wl);
    const int key = sg.s0 + 32 * k + col;
    __builtin_amdgcn_raw_buffer_store_b32(sum, out_rs, half ? 0x7FFFFFF0 : key * 4, 0, 0);
    if (lh && half == 0 && key <= last) {
      const int b = F8 ? topk_fbin(sum) : topk_bin(sum);
      atomicAdd(&lh[b >> 1], 1u << (16 * (b & 1)));
    }
  };
  auto products = [&](int g, int i, Acc& acc0, Acc& acc1) {
    const v4i* kt = ring[(g % SRING) * SG + i];
    v4i kb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kb[j] = kt[32 * (4 * half + j) + col];
    __builtin_amdgcn_sched_barrier(0);  // all four operand reads before the first product
    acc0 = Acc{};
    acc1 = Acc{};
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        acc0 = mfma_f8(qa[0][j], qa[0][j + 1], kb[j], kb[j + 1], acc0);
        acc1 = mfma_f8(qa[1][j], qa[1][j + 1], kb[j], kb[j + 1], acc1);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[0][j], kb[j], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[1][j], kb[j], acc1, 0, 0, 0);
      }
    }
  };
  auto group_tiles = [&](auto foldc, auto ntw, int g, int first, int stride) {
    constexpr int NTW = decltype(ntw)::value;
    Acc a0[2], a1[2];
    products(g, first, a0[0], a1[0]);
#pragma unroll
    for (int u = 1; u < NTW; ++u) {
      products(g, first + stride * u, a0[u & 1], a1[u & 1]);
      epilogue(foldc, a0[(u - 1) & 1], a1[(u - 1) & 1], SG * g + first + stride * (u - 1));
    }
    epilogue(foldc, a0[(NTW - 1) & 1], a1[(NTW - 1) & 1], SG * g + first + stride * (NTW - 1));
  };
  // the group loop, compiled once per epilogue (folded weights or not: uniform per wave, and the
  // two loops need different registers live)
  auto run = [&](auto foldc) {
#pragma unroll 1
    for (int g = 0; g < ngroup; ++g) {
      // this wave's loads of group g have landed, then everyone's; group g+1 goes into the slots
      // of group g-1, which every wave has finished
      idx_wait_vmcnt<0>();
      idx_lds_barrier();
      if (g + 1 < ngroup) load_group(g + 1);
      if (active) {
        // software pipelined over the wave's tiles of the group: the products of tile u+1 are
        // issued before the ReLU/weight epilogue of tile u, so the matrix cores and the vector
        // ALUs work at the same time (tiles past the segment compute on clamped keys; their
        // stores fall outside the buffer range and are dropped)
        if (qpw == 1) group_tiles(foldc, std::integral_constant<int, SG>{}, g, 0, 1);
        else group_tiles(foldc, std::integral_constant<int, SG / 2>{}, g, par, 2);
      }
    }
  };
  if (fold) run(std::true_type{});
  else run(std::false_type{});
  idx_wait_vmcnt<0>();
}

// One work item (up to two segments: a front and a back query tile) per workgroup. MULTI: the
// batch has query tiles of several tokens (shared key tiles, three workgroups per CU); otherwise
// every tile is one token (decode: each wave streams its own key tiles, two workgroups per CU).
// F8: FP8 keys (q and k as E4M3 codes, k_scale per key, fp32 weights per query token, scores as
// fp32 bit patterns); otherwise int8 keys and int32 weights shared by every token.
template <bool MULTI, bool F8>
__global__ __launch_bounds__(256, MULTI ? 3 : 2) void indexer_mfma_kernel(
    const Item* __restrict__ items, const Tok* __restrict__ toks, const int8_t* __restrict__ q_idx,
    const int8_t* __restrict__ k_idx, const float* __restrict__ k_scale, const void* __restrict__ w,
    int32_t* __restrict__ scores, int64_t stride, int* __restrict__ hist, int hist_min_n) {
  // LDS: the key ring, then the histograms (QT packed ones, or one of int counters), then (F8)
  // one slot of 64 key scales per ring tile
  constexpr int TILE_INTS = 256 * 4;
  constexpr int RING_TILES = MULTI ? SRING * SG : 4 * KR;
  constexpr int HIST_INTS = MULTI ? QT * TOPK_BINS / 2 : TOPK_BINS;
  constexpr int LDS_INTS = RING_TILES * TILE_INTS + HIST_INTS + (F8 ? RING_TILES * 64 : 0);
  __shared__ __attribute__((aligned(16))) int smem[LDS_INTS];
  v4i (*const ring)[256] = reinterpret_cast<v4i (*)[256]>(smem);
  int* const lhist_base = smem + RING_TILES * TILE_INTS;
  float (*const scl)[64] = reinterpret_cast<float (*)[64]>(lhist_base + HIST_INTS);
  const float* const w_f = static_cast<const float*>(w);
  const Item it = items[blockIdx.x];
  // wave-uniform (a scalar): everything derived from it (the query, its score row) stays in
  // scalar registers, as buffer resources must
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  // the weights of this lane's heads (w < 2^10 by the weight contract; F8: per token, loaded
  // with the token's query)
  HeadW wl;
  const int32_t* const w_i = F8 ? nullptr : static_cast<const int32_t*>(w);
  if constexpr (!F8) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = 8 * (r >> 2) + 4 * half + (r & 3);
      wl.lo[r] = (uint32_t)w_i[h];
      wl.hi[r] = (uint32_t)w_i[32 + h];
    }
  }

#pragma unroll 1
  for (int sgi = 0; sgi < 2; ++sgi) {
    const Seg sg = sgi == 0 ? it.a : it.b;
    if (sg.nq <= 0) continue;  // uniform over the workgroup
    // rows whose top-k reads the indexer's histogram get it (the last token of the tile has the
    // longest row)
    const bool hist_on = hist != nullptr && toks[sg.q0 + sg.nq - 1].pos + 1 > hist_min_n;
    constexpr int HIST_WORDS = MULTI ? TOPK_BINS / 2 : TOPK_BINS;  // per token
    if (hist_on) {
      for (int i = threadIdx.x; i < sg.nq * HIST_WORDS; i += 256) lhist_base[i] = 0;
      __syncthreads();
    }
    if constexpr (MULTI) {
      indexer_shared_seg<F8>(sg, toks, q_idx, k_idx, k_scale, wl, w_i, w_f, scores, stride, hist_on,
                             hist_min_n, reinterpret_cast<unsigned (*)[TOPK_BINS / 2]>(lhist_base), ring,
                             scl);
    } else {
      // one token: the 4 waves split its key tiles, each through its own part of the ring
      const int64_t t = sg.q0;
      const Tok tk = toks[t];
      int32_t* out_row = scores + (stride ? t * stride : tk.cand_off);
      int* lh = hist_on ? lhist_base : nullptr;
      indexer_wave<F8>(tk, t, sg.s0 + 32 * wave, sg.s1, 128, q_idx, k_idx, k_scale, wl, w_i, w_f,
                       out_row, lh, ring + KR * wave, scl + KR * wave);
    }
    __syncthreads();  // the ring (and the histograms) are reused by the next segment
    if (hist_on) {
      for (int q = 0; q < sg.nq; ++q) {
        const int64_t t = sg.q0 + q;
        if (toks[t].pos + 1 <= hist_min_n) continue;
        int* g = hist + t * TOPK_BINS;
        const int* lq = lhist_base + q * HIST_WORDS;
        for (int i = threadIdx.x; i < HIST_WORDS; i += 256) {
          const unsigned c = (unsigned)lq[i];
          if (MULTI) {
            if (c & 0xFFFFu) atomicAdd(&g[topk_hist_slot(2 * i)], (int)(c & 0xFFFFu));
            if (c >> 16) atomicAdd(&g[topk_hist_slot(2 * i + 1)], (int)(c >> 16));
          } else if (c) {
            atomicAdd(&g[topk_hist_slot(i)], (int)c);
          }
        }
      }
      __syncthreads();
    }
  }
}

// Generic small-shape indexer: one thread per (query, key); H_I <= 16, D_I % 4 == 0, <= 256.
__global__ __launch_bounds__(256) void indexer_generic_kernel(const Tok* __restrict__ toks,
                                                              const int8_t* __restrict__ q_idx,
                                                              const int8_t* __restrict__ k_idx,
                                                              const int32_t* __restrict__ w,
                                                              int H_I, int D_I,
                                                              int32_t* __restrict__ scores,
                                                              int64_t stride, int* __restrict__ hist,
                                                              int hist_min_n) {
  __shared__ int qs[16 * 64];
  __shared__ int ws[16];
  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const int nw = D_I / 4;
  const int* qsrc = reinterpret_cast<const int*>(q_idx + t * H_I * D_I);
  for (int i = threadIdx.x; i < H_I * nw; i += blockDim.x) qs[i] = qsrc[i];
  if (threadIdx.x < H_I) ws[threadIdx.x] = w[threadIdx.x];
  __syncthreads();
  const int64_t s = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
  if (s > tk.pos) return;
  const int* kr = reinterpret_cast<const int*>(k_idx + (tk.row_start + s) * D_I);
  uint32_t score = 0;
  for (int h = 0; h < H_I; ++h) {
    int dot = 0;
    for (int i = 0; i < nw; ++i) dot = __builtin_amdgcn_sdot4(qs[h * nw + i], kr[i], dot, false);
    score += (uint32_t)max(dot, 0) * (uint32_t)ws[h];
  }
  int32_t* out_row = scores + (stride ? t * stride : tk.cand_off);
  out_row[s] = (int32_t)score;
  if (hist && tk.pos + 1 > hist_min_n) atomicAdd(&hist[t * TOPK_BINS + topk_hist_slot(topk_bin(score))], 1);
}

}  // namespace

hipError_t launch_indexer_mfma(const smla_batch& b, const int8_t* q_idx, const int8_t* k_idx,
                               const int32_t* w, int32_t* scores, int compact, int* hist,
                               hipStream_t s) {
  if (b.n_items <= 0) return hipSuccess;
  TableView tv = table_view(b.table, b.batch, b.total_q);
  const int64_t stride = compact ? 0 : b.max_kv;
  if (b.max_q <= 1)
    hipLaunchKernelGGL((indexer_mfma_kernel<false, false>), dim3(b.n_items), dim3(256), 0, s,
                       tv.item, tv.tok, q_idx, k_idx, nullptr, w, scores, stride, hist,
                       topk_hist_min_n(b.total_q));
  else
    hipLaunchKernelGGL((indexer_mfma_kernel<true, false>), dim3(b.n_items), dim3(256), 0, s,
                       tv.item, tv.tok, q_idx, k_idx, nullptr, w, scores, stride, hist,
                       topk_hist_min_n(b.total_q));
  return hipGetLastError();
}

hipError_t launch_indexer_fp8(const smla_batch& b, const uint8_t* q, const uint8_t* k,
                              const float* k_scale, const float* w, int32_t* scores, int compact,
                              int* hist, hipStream_t s) {
  if (b.n_items <= 0) return hipSuccess;
  TableView tv = table_view(b.table, b.batch, b.total_q);
  const int64_t stride = compact ? 0 : b.max_kv;
  const int8_t* qi = reinterpret_cast<const int8_t*>(q);
  const int8_t* ki = reinterpret_cast<const int8_t*>(k);
  if (b.max_q <= 1)
    hipLaunchKernelGGL((indexer_mfma_kernel<false, true>), dim3(b.n_items), dim3(256), 0, s,
                       tv.item, tv.tok, qi, ki, k_scale, w, scores, stride, hist,
                       topk_hist_min_n(b.total_q));
  else
    hipLaunchKernelGGL((indexer_mfma_kernel<true, true>), dim3(b.n_items), dim3(256), 0, s,
                       tv.item, tv.tok, qi, ki, k_scale, w, scores, stride, hist,
                       topk_hist_min_n(b.total_q));
  return hipGetLastError();
}

hipError_t launch_indexer_generic(const smla_batch& b, const int8_t* q_idx, const int8_t* k_idx,
                                  const int32_t* w, int32_t H_I, int32_t D_I, int32_t* scores,
                                  int compact, int* hist, hipStream_t s) {
  TableView tv = table_view(b.table, b.batch, b.total_q);
  const int64_t stride = compact ? 0 : b.max_kv;
  dim3 grid((unsigned)b.total_q, (unsigned)((b.max_kv + 255) / 256));
  hipLaunchKernelGGL(indexer_generic_kernel, grid, dim3(256), 0, s, tv.tok, q_idx, k_idx, w, H_I,
                     D_I, scores, stride, hist,
                       topk_hist_min_n(b.total_q));
  return hipGetLastError();
}

}  // namespace smla
