// sparse_mla.hip — sparse Multi-head Latent Attention in MQA form on gfx950.
//
// Every head of a query token attends over the same top-k latent rows; one gathered row serves
// all 64 heads, which is what lifts the intensity from ~26 to ~191 FLOP per byte on the pages
// ("Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", sections "PCP: split tokens, not heads" and
// "Why the numbers work": QK over 576 dims, PV over 512, BF16 queries and outputs, 656-byte FP8
// rows). Partial results over disjoint row sets merge by log-sum-exp (section "DCP").
//
// FP8 kernel (64 heads, 576/512 dims, 656-byte rows): one workgroup of 4 waves (one per SIMD,
// 512 registers each) per (token, split), 32-row tiles. Every wave works on all stages, software
// pipelined so that the matrix cores, the vector ALUs and the memory paths overlap:
//  1. the rows of tile t+3 are moved from HBM straight into a ring of raw tiles in LDS by the
//     load-to-LDS path (no registers involved), three tiles ahead of the one being computed;
//  2. while tile t is multiplied, tile t+1 is dequantised from its raw copy into the other half
//     of a double-buffered row-major K[row][576] fp16 tile: v_cvt_scalef32_pk_f16_fp8
//     applies the power-of-two part of the block scale exactly and one packed fp16 multiply
//     applies the rest; the bf16 rope dims are widened to fp16;
//  3. wave (g, h) holds Q (fp16) of heads [32g, 32g+32) over dims [288h, 288h+288) and computes
//     that half of S^T = K Q^T on v_mfma_f32_32x32x16_f16 (rows as M, heads as N, so each lane
//     owns one head); the two waves of a head group add their halves through LDS;
//  4. one running maximum per head; O is rescaled only when the maximum grows by more than 2^8
//     (so P <= 256 and an fp16 P keeps 11 significant bits);
//  5. P stays in registers: its accumulator layout is reused as the B operand of
//     O^T = V^T P^T (the contraction runs over rows in the order the accumulator holds them);
//     V^T comes straight from the row-major tile through transposing LDS reads
//     (ds_read_b64_tr_b16). Wave (g, h) accumulates O^T for dims [256h, 256h+256) of its 32
//     heads.
// The K tile's 16-byte chunks are XOR-swizzled by row so that the operand reads, the
// transposing reads and the dequantiser's writes all spread over the 64 LDS banks. Rows without
// an index (padding) read the request's first row and are masked out of the softmax, so the
// latent cache must hold finite values.
// Decode splits a token's rows across workgroups and merges the fp16 partials by log-sum-exp.
#include "smla_internal.h"

namespace smla {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

namespace {

constexpr int NT = 256;                    // 4 waves, one per SIMD
constexpr int TILE = 32;                   // rows per tile
constexpr int KCH = MLA_DQK / 8;           // 72 16-byte chunks per K row
constexpr int K_BYTES = TILE * MLA_DQK * 2;  // 36864 per buffer
constexpr int RB16 = 16 * KCH * 16;        // bytes between rows r and r + 16 (same swizzle)
constexpr int ROW_CH = MLA_ROW_BYTES / 16;   // 41 16-byte chunks per stored row
constexpr int RAW_CHUNKS = TILE * ROW_CH;    // 1312 per tile
constexpr int RAW_INSTR = (RAW_CHUNKS + 63) / 64;  // 21 wave instructions per tile
constexpr int RAW_SLOT = RAW_INSTR * 1024;   // 21504 bytes (the last instruction's tail is padding)
constexpr int NRAW = 3;                    // raw tiles in flight
constexpr float LOG2E = 1.4426950408889634f;
// Softmax reference (log2 units): P = 2^(logit - ref) with ref fixed for the whole split, so the
// output accumulators are only ever touched by the matrix cores. The first tile with a valid
// row sets ref = its maximum + REF_MARGIN; a later logit more than REF_HEADROOM above ref would
// push an fp16 P towards its range limit, and then the split is recomputed with ref = the true
// maximum, which the first pass has tracked.
constexpr float REF_MARGIN = 4.0f;
constexpr float REF_HEADROOM = 15.0f;

struct __align__(16) MlaSmem {
  unsigned char k[2][K_BYTES];        // K[row][chunk ^ swz(row)], two tiles
  unsigned char raw[NRAW][RAW_SLOT];  // gathered rows as stored (656 bytes each, back to back)
  float sx[4][4][64][4];              // per wave: its half of S^T, [i/4][lane][i%4]
  int idx[TOPK_MAX_K];                // the split's row indices (-1: skip)
};
static_assert(sizeof(MlaSmem) <= 160 * 1024 - 16, "LDS budget");

// Row swizzle of 16-byte chunks (a bijection on the low three chunk bits, from row bits 0..3).
// With 72 chunks per row, rows alternate between the two halves of the 64 banks; the swizzle
// spreads (a) 32 rows at one chunk, (b) 4 aligned rows x 4 aligned chunks and (c) the
// dequantiser's writes over all 16 bank groups, so every access is conflict free.
__device__ __forceinline__ int swz(int row) {
  return (((row >> 1) & 1) << 2) | (((row >> 2) ^ row) & 1) | (((row >> 3) & 1) << 1);
}
__device__ __forceinline__ int k_off(int row, int chunk) { return (row * KCH + (chunk ^ swz(row))) * 16; }

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  v2f x = {a, b};
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  v2bf y = __builtin_convertvector(x, v2bf);
  return __builtin_bit_cast(unsigned, y);
}

__device__ __forceinline__ unsigned pack_f16(float a, float b) {
  v2f x = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(x, v2h));
}

// Two bf16 (one dword) -> two fp16 (one dword), exact within the fp16 range.
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned x) {
  return pack_f16(__builtin_bit_cast(float, x << 16), __builtin_bit_cast(float, x & 0xFFFF0000u));
}

__device__ __forceinline__ float swap_halves_max(float v) {
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (unsigned)b[0]), __builtin_bit_cast(float, (unsigned)b[1]));
}
__device__ __forceinline__ float swap_halves_sum(float v) {
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false, false);
  return __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
}

// Barrier for LDS hand-offs inside the tile loop: waits for this wave's LDS operations only,
// so the gathers of later tiles keep flying (a full __syncthreads would wait for them too). The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Waits until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Gather instructions per tile: instruction q goes to wave q % 4, so wave 0 issues six and the
// others five. Waits until this wave's gathers of all but the last `later` tiles it issued have
// landed (`later` at most 2).
__device__ __forceinline__ void wait_tiles_but(int later, int wave) {
  if (wave == 0) {
    if (later >= 2) wait_vmcnt<12>(); else if (later == 1) wait_vmcnt<6>(); else wait_vmcnt<0>();
  } else {
    if (later >= 2) wait_vmcnt<10>(); else if (later == 1) wait_vmcnt<5>(); else wait_vmcnt<0>();
  }
}

// One load-to-LDS instruction: lane l's 16 bytes at g land at lds + 16 l (lds wave-uniform).
// Written as inline assembly so that the compiler does not track it: the tile loop waits for
// these loads itself (wait_tiles_but), instead of the compiler draining every one of them before
// each LDS write it cannot prove disjoint. M0 (the LDS base operand) is saved and restored.
__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
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

// Gathers one tile (rows sidx[0..TILE)) into a raw slot: chunk c of the tile is the 16 bytes at
// offset 16 (c % 41) of row c / 41, placed at slot + 16 c. Wave w issues instructions w + 4j
// (j < 5) and wave 0 also instruction 20, so every wave issues a fixed number (waits count
// them). Lanes past the tile's last chunk and rows without an index read the request's first
// row. A lane's chunk positions are the same for every tile: `base[j]` is the request's first
// row plus the chunk's offset inside its row, `roff[j]` the byte offset of its row's index in
// the tile's index list.
struct GatherPlan {
  const unsigned char* base[6];
  int roff[6];
};

__device__ __forceinline__ GatherPlan gather_plan(int wave, const unsigned char* kv_req) {
  const int lane = threadIdx.x & 63;
  GatherPlan gp;
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int qq = j < 5 ? wave + 4 * j : 20;
    const int c = 64 * qq + lane;
    const int row = c < RAW_CHUNKS ? c / ROW_CH : 0;
    gp.roff[j] = 4 * row;
    gp.base[j] = kv_req + 16 * (c - ROW_CH * (c / ROW_CH));
  }
  return gp;
}

// The row indices of a lane's chunks (LDS reads) and the loads that use them, separately so that
// the reads can go out well before the loads.
__device__ __forceinline__ void gather_rows(const int* sidx, const GatherPlan& gp, int (&ix)[6]) {
#pragma unroll
  for (int j = 0; j < 6; ++j)
    ix[j] = *reinterpret_cast<const int*>(reinterpret_cast<const char*>(sidx) + gp.roff[j]);
}

__device__ __forceinline__ void gather_issue(unsigned char* slot, const int (&ix)[6],
                                             const GatherPlan& gp, int wave) {
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    if (j == 5 && wave != 0) break;  // wave-uniform
    const int qq = j < 5 ? wave + 4 * j : 20;
    lds_load16(gp.base[j] + (uint64_t)(uint32_t)max(ix[j], 0) * MLA_ROW_BYTES, slot + 1024 * qq);
  }
}

__device__ __forceinline__ void tile_gather(unsigned char* slot, const int* sidx,
                                            const GatherPlan& gp, int wave) {
  int ix[6];
  gather_rows(sidx, gp, ix);
  gather_issue(slot, ix, gp, wave);
}

// Dequantises a raw tile into the fp16 K tile. Thread (r, m) = (tid / 8, tid % 8) takes 64 e4m3
// codes of row r (dims 128 i + 16 m .. +16, i < 4) and 8 bf16 rope dims (512 + 8 m .. +8). The
// scale s = 2^e * mant (1 <= mant < 2): the conversion applies 2^e exactly and a packed multiply
// fp16(mant); the rope dims are widened. Rows without an index hold the request's first row,
// which the softmax masks out.
// The pieces are separate so that the tile loop can place them between the matrix instructions
// of the previous tile: load() reads the thread's raw bytes, block(i) converts and stores dims
// 128 i + 16 m .. +16, rope() the rope dims.
struct Dequant {
  v4u code[4];
  v4u scale;
  v4u rope;
  __device__ __forceinline__ void load(const unsigned char* slot, int r, int m) {
    const unsigned char* row = slot + r * MLA_ROW_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) code[i] = *reinterpret_cast<const v4u*>(row + 128 * i + 16 * m);
    scale = *reinterpret_cast<const v4u*>(row + 512);
    rope = *reinterpret_cast<const v4u*>(row + 528 + 16 * m);
  }
  __device__ __forceinline__ void block(unsigned char* kb, int r, int m, int i) const {
    // the conversion reads only the exponent of its scale operand
    const float sc = __builtin_bit_cast(float, scale[i] & 0x7F800000u);
    const float mt = __builtin_bit_cast(float, (scale[i] & 0x807FFFFFu) | 0x3F800000u);
    const v2h mm = {(_Float16)mt, (_Float16)mt};
    unsigned pk[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const v2h lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(code[i][h], sc, false) * mm;
      const v2h hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(code[i][h], sc, true) * mm;
      pk[2 * h] = __builtin_bit_cast(unsigned, lo);
      pk[2 * h + 1] = __builtin_bit_cast(unsigned, hi);
    }
    *reinterpret_cast<v4u*>(kb + k_off(r, 16 * i + 2 * m)) = v4u{pk[0], pk[1], pk[2], pk[3]};
    *reinterpret_cast<v4u*>(kb + k_off(r, 16 * i + 2 * m + 1)) = v4u{pk[4], pk[5], pk[6], pk[7]};
  }
  __device__ __forceinline__ void rope_store(unsigned char* kb, int r, int m) const {
    *reinterpret_cast<v4u*>(kb + k_off(r, 64 + m)) =
        v4u{bf16x2_to_f16x2(rope[0]), bf16x2_to_f16x2(rope[1]), bf16x2_to_f16x2(rope[2]), bf16x2_to_f16x2(rope[3])};
  }
};

__device__ __forceinline__ void tile_dequant(const unsigned char* slot, unsigned char* kb, int r, int m) {
  Dequant dq;
  dq.load(slot, r, m);
#pragma unroll
  for (int i = 0; i < 4; ++i) dq.block(kb, r, m, i);
  dq.rope_store(kb, r, m);
}

// One (token, split): the split's share of the tiles of the token's index list, up to its last
// valid entry.
// Writes either the final bf16 output (+ lse) or an fp16 partial (+ lse) for the combine.
__global__ __launch_bounds__(NT, 1) void mla_fp8_kernel(const Tok* __restrict__ toks,
                                                        const __bf16* __restrict__ q,
                                                        const unsigned char* __restrict__ kv,
                                                        const int32_t* __restrict__ idx,
                                                        int top_k,
                                                        float sm_scale, __bf16* __restrict__ out,
                                                        float* __restrict__ lse_out,
                                                        _Float16* __restrict__ part_o,
                                                        float* __restrict__ part_lse) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  MlaSmem& sm = *reinterpret_cast<MlaSmem*>(smem_raw);
  const int64_t t = blockIdx.x;
  const int split = blockIdx.y;
  const int nsplit = gridDim.y;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  const int32_t* idx_row = idx + t * top_k;

  // The split's indices. First guess, right for a list whose last entry is valid: the splits share
  // all of the list's tiles. The last entry is loaded with them to check.
  __shared__ int last_all, last_valid;
  if (tid == 0) last_all = -1, last_valid = -1;
  constexpr int PER = TOPK_MAX_K / NT;
  const int tiles_k = (top_k + TILE - 1) / TILE;
  int per_split = (tiles_k + nsplit - 1) / nsplit;
  int r_begin = min(split * per_split, tiles_k) * TILE;
  int r_end = min(top_k, (split + 1) * per_split * TILE);
  int ixs[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int j = u * NT + tid;
    ixs[u] = r_begin + j < r_end ? idx_row[r_begin + j] : -1;
  }
  const int32_t last_entry = idx_row[top_k - 1];
  // this lane's Q^T fragments go out with the indices: head `head`, dims
  // [288*kh + 16*ks + 8*half, +8), bf16 as loaded (widened to fp16 below)
  const int hg = wave >> 1, kh = wave & 1;
  const int col = lane & 31, half = lane >> 5;
  const int head = 32 * hg + col;
  v4u qraw[18];
  {
    const __bf16* qh = q + (t * MLA_H + head) * MLA_DQK + 288 * kh + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qraw[ks] = *reinterpret_cast<const v4u*>(qh + 16 * ks);
  }
  const Tok tk = toks[t];
  __syncthreads();
  {
    int lv = -1;
    if (last_entry >= 0 && last_entry <= tk.pos) {  // uniform
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int j = u * NT + tid;
        const int ix = ixs[u] > tk.pos ? -1 : ixs[u];
        sm.idx[j] = ix;
        if (ix >= 0) lv = j;
      }
    } else {
      // Padding at the end (a short context, a shard's part of a selection): the splits share
      // the tiles up to the last valid entry instead, so the valid rows spread over all of them.
      int la = -1;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int j = u * NT + tid;
        ixs[u] = j < top_k ? idx_row[j] : -1;
        if (ixs[u] > tk.pos) ixs[u] = -1;
        if (ixs[u] >= 0) la = j;
      }
      if (la >= 0) atomicMax(&last_all, la);
      __syncthreads();
      const int tiles_all = (last_all + TILE) / TILE;
      per_split = (tiles_all + nsplit - 1) / nsplit;
      r_begin = min(split * per_split, tiles_all) * TILE;
      r_end = max(r_begin, min((split + 1) * per_split * TILE, last_all + 1));
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int j = u * NT + tid;
        if (j >= r_begin && j < r_end) {  // entry j goes to slot j - r_begin
          sm.idx[j - r_begin] = ixs[u];
          if (ixs[u] >= 0) lv = j - r_begin;
        }
        if (j >= r_end - r_begin) sm.idx[j] = -1;  // the slots no entry lands in
      }
    }
    if (lv >= 0) atomicMax(&last_valid, lv);
  }
  __syncthreads();
  const int ntiles = (last_valid + TILE) / TILE;  // trailing invalid tiles are skipped

  v8h qf[18];
#pragma unroll
  for (int ks = 0; ks < 18; ++ks)
    qf[ks] = __builtin_bit_cast(v8h, v4u{bf16x2_to_f16x2(qraw[ks][0]), bf16x2_to_f16x2(qraw[ks][1]),
                                         bf16x2_to_f16x2(qraw[ks][2]), bf16x2_to_f16x2(qraw[ks][3])});
  // per-lane LDS offsets: S operand (K row `col`, chunk 36*kh + 2u + half (+ 8m)), and the
  // transposing V reads (16-lane group g: dims +16*(g&1); 4 rows from 4*(g>>1) + lane%16 / 4).
  // The transposing V reads of (ks, second half, mt = 2m + par) sit at
  // voff[hi][par] + RB16 * ks + 128 m: rows 16 apart share their swizzle, and the chunk of dim
  // vdim + 32mt is (vdim >> 3) + 4par + 8m, whose bit 3 and up the swizzle leaves alone.
  int koff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) koff[u] = k_off(col, 36 * kh + 2 * u + half);
  const int grp = lane >> 4, gl = lane & 15;
  const int vrow = 4 * (grp >> 1) + (gl >> 2);
  const int vdim = 256 * kh + 16 * (grp & 1) + 4 * (gl & 3);
  int voff[2][2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int par = 0; par < 2; ++par)
      voff[hi][par] = k_off(8 * hi + vrow, (vdim >> 3) + 4 * par) + 2 * (vdim & 7);

  // the Q fragments are in registers before any gather goes out (the compiler does not count the
  // gathers, so a later wait of its own for Q would drain them)
  wait_vmcnt<0>();
  // dequantiser's share: tile row tid / 8, pieces m = tid % 8
  const int pr = tid >> 3, pm = tid & 7;
  const GatherPlan gp = gather_plan(wave, kv + tk.row_start * MLA_ROW_BYTES);
  const float c = sm_scale * LOG2E;
  float ref = -INFINITY;     // softmax reference of this lane's head (log2 units)
  float seen = -INFINITY;    // largest scaled logit of this lane's head so far
  __shared__ int redo;
  v16f o[8];
  float l_run;  // this lane's share of the softmax denominator

#pragma unroll 1
  for (int pass = 0;; ++pass) {
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = v16f{};
  l_run = 0.f;
  bool over = false;  // a logit above ref + REF_HEADROOM
  for (int j = 0; j < NRAW && j < ntiles; ++j) tile_gather(sm.raw[j], sm.idx + j * TILE, gp, wave);
  if (ntiles > 0) {
    wait_tiles_but(min(ntiles, NRAW) - 1, wave);
    lds_barrier();  // every wave's part of tile 0 has landed
    tile_dequant(sm.raw[0], sm.k[0], pr, pm);
    if (ntiles > 1) wait_tiles_but(min(ntiles, NRAW) - 2, wave);
  }
  if (tid == 0) redo = 0;
  lds_barrier();  // tile 0 is in K[0], tile 1 in raw slot 1

  // Entering iteration `it`: K[it & 1] holds tile it, raw slot (it+1) % 3 holds tile it+1
  // (landed and visible), tile it+2 is in flight, slot it % 3 is free.
#pragma unroll 1
  for (int it = 0; it < ntiles; ++it) {
    const unsigned char* kb = sm.k[it & 1];
    // half of S^T over this wave's dims (one accumulation chain: a dependent 32x32x16 MFMA
    // issues at full rate). The matrix instructions run on their own while the wave issues the
    // work placed between them: the gather of tile it+3 and the fp16 copy of tile it+1 (the
    // latter unconditional: after the last tile it converts a stale slot into the idle buffer,
    // which nothing reads). Scheduling barriers keep the compiler from regrouping the pieces.
    v16f s = v16f{};
    {
      unsigned char* kn = sm.k[(it + 1) & 1];
      const bool gather = it + NRAW < ntiles;
      int ix[6];
      if (gather) gather_rows(sm.idx + (it + NRAW) * TILE, gp, ix);
      Dequant dq;
      // operand reads eight k-steps ahead of their MFMA (LDS latency under load exceeds the
      // time of a few MFMAs)
      v8h a[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) a[ks] = *reinterpret_cast<const v8h*>(kb + koff[ks & 3] + 128 * (ks >> 2));
      dq.load(sm.raw[(it + 1) % NRAW], pr, pm);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks & 7], qf[ks], s, 0, 0, 0);
        if (ks + 8 < 18)
          a[ks & 7] = *reinterpret_cast<const v8h*>(kb + koff[ks & 3] + 128 * ((ks + 8) >> 2));
        if (ks == 1 && gather) gather_issue(sm.raw[it % NRAW], ix, gp, wave);
        if (ks == 4 || ks == 7 || ks == 10 || ks == 13) dq.block(kn, pr, pm, (ks - 4) / 3);
        if (ks == 15) dq.rope_store(kn, pr, pm);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<float4*>(&sm.sx[wave][g4][lane][0]) =
          make_float4(s[4 * g4], s[4 * g4 + 1], s[4 * g4 + 2], s[4 * g4 + 3]);
    lds_barrier();
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 o4 = *reinterpret_cast<const float4*>(&sm.sx[wave ^ 1][g4][lane][0]);
      s[4 * g4] += o4.x;
      s[4 * g4 + 1] += o4.y;
      s[4 * g4 + 2] += o4.z;
      s[4 * g4 + 3] += o4.w;
    }
    // lane holds head `head`, rows 8*(i/4) + 4*half + i%4 of the tile; raw logits stay unscaled
    // (c > 0 keeps their order) and c enters the exponent below
    const uint64_t valid = __ballot(sm.idx[it * TILE + col] >= 0);  // bit r: row r is valid
    if ((uint32_t)valid != 0xFFFFFFFFu) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * half + (i & 3);
        if (!((valid >> row) & 1)) s[i] = -INFINITY;
      }
    }
    float tmax = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) tmax = __builtin_fmaxf(tmax, s[i]);
    tmax = swap_halves_max(tmax) * c;
    // both waves of a head group hold identical logits and take the same decisions
    seen = __builtin_fmaxf(seen, tmax);
    ref = ref == -INFINITY && tmax != -INFINITY ? tmax + REF_MARGIN : ref;
    over |= tmax > ref + REF_HEADROOM;
    // P in registers, packed as the B operand of the two 16-row k-steps (no valid row so far:
    // every logit is -inf and P must come out 0, not NaN)
    const float m_use = ref == -INFINITY ? 0.f : ref;
    v8h pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float p8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p8[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * ks + j], c, -m_use));  // underflow to 0 is harmless
        l_run += p8[j];
      }
      v4u pk = {pack_f16(p8[0], p8[1]), pack_f16(p8[2], p8[3]), pack_f16(p8[4], p8[5]),
                pack_f16(p8[6], p8[7])};
      pb[ks] = __builtin_bit_cast(v8h, pk);
    }
    // O^T[dims 256*kh + 32*mt + m][head] += V^T[dim][rows] P^T[rows][head]
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int par = mt & 1, mm = mt >> 1;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(kb + voff[0][par] + RB16 * ks + 128 * mm));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(kb + voff[1][par] + RB16 * ks + 128 * mm));
        const v8h a = __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[ks], o[mt], 0, 0, 0);
      }
    }
    // tile it+2 must have landed before the next iteration dequantises it; only tile it+3 (issued
    // at the top of this iteration) may still be in flight
    if (it + 2 < ntiles) wait_tiles_but(it + 3 < ntiles ? 1 : 0, wave);
    lds_barrier();
  }
  wait_vmcnt<0>();  // no gather may still be writing this workgroup's LDS
  if (__any(over)) redo = 1;  // any wave: every wave redoes the split
  __syncthreads();
  if (!redo || pass == 1) break;
  ref = seen;  // the second pass cannot exceed it
  __syncthreads();
  }

  // denominator of each head: both lane halves, both waves of the head group hold the same
  l_run = swap_halves_sum(l_run);
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
  const float lse = empty ? -INFINITY : (ref + log2f(l_run)) * (1.0f / LOG2E);

  // The output goes out through LDS (the K buffers, idle once the tile loop is done) so that every
  // global store writes whole lines: head h's 512 16-bit values sit at h * 1024 with 16-byte
  // chunk c at 16 (c ^ (h & 63)), and a wave stores one head's row (1 KB) per instruction.
  const bool split_out = part_o != nullptr;
  unsigned char* stage = &sm.k[0][0];
  static_assert(sizeof(sm.k) >= MLA_H * MLA_DV * 2, "output staging");
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float v0 = o[mt][4 * g4] * inv, v1 = o[mt][4 * g4 + 1] * inv;
      const float v2 = o[mt][4 * g4 + 2] * inv, v3 = o[mt][4 * g4 + 3] * inv;
      const v2u pk = split_out ? v2u{pack_f16(v0, v1), pack_f16(v2, v3)}
                               : v2u{pack_bf16(v0, v1), pack_bf16(v2, v3)};
      const int chunk = 32 * kh + 4 * mt + g4;  // dims 256 kh + 32 mt + 8 g4 .. +8
      *reinterpret_cast<v2u*>(stage + head * 1024 + 16 * (chunk ^ (head & 63)) + 8 * half) = pk;
    }
  __syncthreads();
  unsigned char* dst = split_out ? reinterpret_cast<unsigned char*>(part_o + (t * nsplit + split) * MLA_H * MLA_DV)
                                 : reinterpret_cast<unsigned char*>(out + t * MLA_H * MLA_DV);
#pragma unroll 4
  for (int hh = wave; hh < MLA_H; hh += NT / 64)
    *reinterpret_cast<v4u*>(dst + hh * 1024 + 16 * lane) =
        *reinterpret_cast<const v4u*>(stage + hh * 1024 + 16 * (lane ^ (hh & 63)));
  if (kh == 0 && half == 0) {
    if (split_out) part_lse[(t * nsplit + split) * MLA_H + head] = lse;
    else if (lse_out) lse_out[t * MLA_H + head] = lse;
  }
}

// Merge split partials by log-sum-exp: one 128-thread block per (token, head), 4 dims per
// thread. The first eight splits' partials go out together with their lse values, so a merge of
// up to eight splits costs one memory round trip. Block b takes token b % n_tok: workgroups are
// dealt to the XCDs round robin, so with n_tok a multiple of 8 a token's merge runs on the XCD
// whose L2 holds the partials its splits just wrote (the attention grid puts every split of
// token t on XCD t % 8 too).

__global__ __launch_bounds__(128) void mla_combine_kernel(const _Float16* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          int nsplit, int n_tok,
                                                          __bf16* __restrict__ out,
                                                          float* __restrict__ lse_out) {
  const int64_t t = blockIdx.x % n_tok;
  const int h = (int)(blockIdx.x / n_tok);
  const int64_t th = t * MLA_H + h;
  const float* pl = part_lse + t * nsplit * MLA_H + h;
  const _Float16* po = part_o + (t * nsplit * MLA_H + h) * MLA_DV + 4 * threadIdx.x;
  v4h v[8];
  float lj[8];
  auto load8 = [&](int j0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + u, nsplit - 1);
      v[u] = *reinterpret_cast<const v4h*>(po + (int64_t)j * MLA_H * MLA_DV);
      lj[u] = j0 + u < nsplit ? pl[j * MLA_H] : -INFINITY;
    }
  };
  load8(0);
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < 8; ++u) m = fmaxf(m, lj[u]);
  for (int j = 8; j < nsplit; ++j) m = fmaxf(m, pl[j * MLA_H]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int j0 = 0; j0 < nsplit; j0 += 8) {
      if (j0 > 0) load8(j0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wj = lj[u] != -INFINITY ? __expf(lj[u] - m) : 0.f;
        wsum += wj;
        acc[0] += wj * (float)v[u][0];
        acc[1] += wj * (float)v[u][1];
        acc[2] += wj * (float)v[u][2];
        acc[3] += wj * (float)v[u][3];
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  v2u pk = {pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<v2u*>(out + th * MLA_DV + 4 * threadIdx.x) = pk;
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
  return align_up(n * D_v * sizeof(_Float16), 256) + align_up(n * sizeof(float), 256);
}

hipError_t launch_mla_fp8(const smla_batch& b, const void* q, const void* kv, const int32_t* idx,
                          int32_t top_k, float sm_scale, void* out, float* lse, void* ws,
                          int decode, hipStream_t s) {
  TableView tv = table_view(b.table, b.batch, b.total_q);
  const int nsplit = decode ? mla_decode_splits(b, top_k) : 1;
  const size_t lds = sizeof(MlaSmem);
  static const bool lds_set = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&mla_fp8_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return true;
  }();
  (void)lds_set;
  _Float16* part_o = nullptr;
  float* part_lse = nullptr;
  if (nsplit > 1) {
    part_o = static_cast<_Float16*>(ws);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                        align_up((size_t)b.total_q * nsplit * MLA_H * MLA_DV * sizeof(_Float16), 256));
  }
  mark_stage(STAGE_MLA, false, s);
  hipLaunchKernelGGL(mla_fp8_kernel, dim3(b.total_q, nsplit), dim3(NT), lds, s, tv.tok,
                     static_cast<const __bf16*>(q), static_cast<const unsigned char*>(kv), idx, top_k,
                     sm_scale, static_cast<__bf16*>(out), lse, part_o, part_lse);
  mark_stage(STAGE_MLA, true, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  mark_stage(STAGE_COMBINE, false, s);
  hipLaunchKernelGGL(mla_combine_kernel, dim3(b.total_q * MLA_H), dim3(128), 0, s, part_o, part_lse,
                     nsplit, b.total_q, static_cast<__bf16*>(out), lse);
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
