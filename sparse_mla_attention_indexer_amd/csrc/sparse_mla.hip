// sparse_mla.hip — sparse Multi-head Latent Attention in MQA form on gfx950.
//
// Every head of a query token attends over the same top-k latent rows; one gathered row serves
// all 64 heads, which is what lifts the intensity from ~26 to ~191 FLOP per byte on the pages
// ("Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", sections "PCP: split tokens, not heads" and
// "Why the numbers work": QK over 576 dims, PV over 512, BF16 queries and outputs, 656-byte FP8
// rows). Partial results over disjoint row sets merge by log-sum-exp (section "DCP").
//
// FP8 kernel (64 heads, 576/512 dims, 656-byte rows): one workgroup of 8 waves (two per SIMD)
// per (token, split), over 32-row tiles, in two teams of four waves (wave b of each team on
// SIMD b; b is also the FP8 block of value dims 128b..128b+127 the wave owns):
//  - gather (QK team): the rows of a tile move from HBM straight into LDS by the load-to-LDS
//    path, two tiles ahead, as stored (row r at 656 r): each load instruction covers 1 KB of
//    consecutive row bytes, and since a row is an odd number (41) of 16-byte chunks, one chunk of
//    16 consecutive rows falls on 16 distinct bank groups, so every operand read below is free of
//    bank conflicts;
//  - QK (QK wave b): all 32 rows of a tile times all 64 heads over block b's 128 E4M3 codes,
//    converted exactly to bf16 without their scale (v_cvt_scalef32_pk_bf16_fp8, scale 1), on
//    v_mfma_f32_16x16x32_bf16 with rows as M and heads as N (four head tiles share each converted
//    fragment). The block's fp32 scale then multiplies the code part of each row's partial logit,
//    and a 16-deep k-step (v_mfma_f32_16x16x16_bf16) adds 16 of the 64 bf16 rope dims:
//    partial_b = s_b[row] * (q_b . code_b) + q_rope_b . rope_b. The wave reads and converts a
//    tile's K fragments in the phase before its products, and writes block b's column of the
//    tile's u table: u_b = s_b / 2^E_b, the scale relative to a power of two fixed per split (the
//    first tile's largest scale of the block), zero for rows without an index;
//  - reduce (PV wave b): head tile b over all 32 rows, so a head's softmax state never leaves
//    its wave: the four block partials summed, P = 2^(logit * c - ref) in fp32, then
//    P'_b' = P u_b'[row] for each block b' as the product of P and u rounded to fp16, in fp16;
//  - PV (PV wave b): O^T for block b's 128 dims of all 64 heads over the 32 rows on
//    v_mfma_f32_16x16x32_f16: V^T comes from the raw codes through transposing 8-bit LDS reads
//    (ds_read_b64_tr_b8) and the exact conversion to fp16, P'_b^T from LDS, so
//    O_b = 2^E_b sum_r P_r u_b[r] code_r / sum_r P_r.
// The K and V operands are therefore exact (an E4M3 code is a bf16 and an fp16 value, and q is
// bf16 as given) and the scales are applied in fp32 (logits) or as fp16 numbers (P'). P' is
// fp16 while every row's u stays within [2^-10, 2^3] (or is 0); the QK waves check that for each
// tile, and a split whose rows fall outside is recomputed with P' = P * s in fp32, rounded to bf16
// (full range, 8 bits).
// Rows without an index (padding) are masked: their logits become -inf, their P' is zero and
// their V codes are zeroed before the products, so a padding row's bytes (which may be NaN)
// never reach an output.
// The reduction of tile t and the products of tile t-1 share one phase between barriers, so the
// matrix cores and the vector ALUs overlap across the two waves of each SIMD. In each phase the
// wave that issues the matrix instructions runs at a raised wave priority (s_setprio), so that
// its products and the conversions feeding them are not queued behind the other wave's vector
// work.
// Decode splits a token's rows across workgroups and merges bf16 partials by log-sum-exp.
#include <mutex>
#include <type_traits>

#include "smla_internal.h"

namespace smla {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

namespace {

constexpr int NT = 512;                       // 8 waves, two per SIMD
constexpr int TILE = 32;                      // rows per tile
constexpr int RB = MLA_ROW_BYTES;             // 656 bytes = 41 chunks of 16
constexpr int ROW_CH = RB / 16;               // 41
constexpr int SCALE_OFF = 512;                // the four fp32 block scales in a row
constexpr int ROPE_OFF = 528;                 // the 64 bf16 rope dims in a row
constexpr int TILE_CH = TILE * ROW_CH;        // 1312 chunks of rows per tile
// The rows' relative scales u_b of a tile: fp16 [block][row] (fp16 P'), fp32 [row][block] (bf16)
constexpr int U_OFF = TILE * RB;              // 20992
constexpr int RAW_INSTR = 21;                 // load instructions per tile (64 chunks each)
constexpr int RAW_SLOT = RAW_INSTR * 1024;    // 21504 bytes: the rows, then the u table
constexpr int NRAW = 4;                       // tile slots: two computed on, two in flight
constexpr int Q_BYTES = MLA_H * MLA_DQK * 2;  // one token's Q, staged from the last tile slot on
constexpr float LOG2E = 1.4426950408889634f;
// Softmax reference (log2 units): P = 2^(logit - ref) with ref fixed for the whole split, so the
// output accumulators are only ever touched by the matrix cores. The first tile with a valid row
// sets ref = its maximum + REF_MARGIN; a later logit more than REF_HEADROOM above ref would let P
// (and the fp32 sums built on it) grow without bound, and then the split is recomputed with
// ref = the true maximum, which the first pass has tracked.
// With P <= 2^REF_HEADROOM and u < 2^U_MAX_LOG2, P' stays below 2^14 (fp16 max is 65504).
constexpr float REF_MARGIN = 4.0f;
constexpr float REF_HEADROOM = 11.0f;
constexpr float U_MAX = 8.0f;          // 2^3
constexpr float U_MIN = 0.0009765625f;  // 2^-10: the dominant row's P' (P >= 2^-4) stays normal

struct __align__(16) MlaSmem {
  unsigned char raw[NRAW][RAW_SLOT];  // tiles as gathered (row r at 656 r), then their u tables
  v4f part[2][4][4][64];              // [row half][head tile][block][lane]: partial logits
  v4u pp[4][4][4][16];                // [block][head tile][row group][head]: 8 rows of P'
  unsigned char qtail[Q_BYTES - RAW_SLOT - 32768 - 16384];  // Q's last bytes (see below)
  int idx[TOPK_MAX_K];                // the split's row indices (-1: skip)
  float xmax[2][MLA_H];               // per row half: logit maxima of each head
  float xsum[2][MLA_H];               // per row half: softmax denominators of each head
  int eb[4];                          // E_b of the split (fp16 P'), 0 in the bf16 fallback
};
static_assert(sizeof(MlaSmem) <= 160 * 1024 - 64, "LDS budget");
static_assert(MLA_H * MLA_DV * 2 <= sizeof(MlaSmem::raw), "output staging");
// The token's Q is staged in raw[3], part, pp and qtail, one contiguous range that the first
// three tiles' slots (and the index list) do not touch, so those tiles can be gathered while the
// Q copy is still in flight.
static_assert(Q_BYTES % 4096 == 0, "Q staging: four waves of 1 KB instructions");
static_assert(offsetof(MlaSmem, part) == offsetof(MlaSmem, raw) + NRAW * RAW_SLOT &&
                  offsetof(MlaSmem, pp) == offsetof(MlaSmem, part) + sizeof(MlaSmem::part) &&
                  offsetof(MlaSmem, qtail) == offsetof(MlaSmem, pp) + sizeof(MlaSmem::pp) &&
                  offsetof(MlaSmem, qtail) + sizeof(MlaSmem::qtail) ==
                      offsetof(MlaSmem, raw) + (NRAW - 1) * RAW_SLOT + Q_BYTES,
              "Q staging range");

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  v2f x = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(x, v2bf));
}

// Eight E4M3 codes (two dwords, code i in byte i) -> eight bf16 values, exactly.
__device__ __forceinline__ v8bf e4m3x8_to_bf16(unsigned lo, unsigned hi) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight E4M3 codes -> eight fp16 values, exactly (|code| <= 448, smallest 2^-9).
__device__ __forceinline__ v8h e4m3x8_to_f16(unsigned lo, unsigned hi) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ unsigned pack_f16(float a, float b) {
  v2f x = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(x, v2h));
}

// 0xFF in byte i for each set bit i of the four low bits of x.
__device__ __forceinline__ unsigned byte_mask4(unsigned x) {
  return (((x & 15u) * 0x00204081u) & 0x01010101u) * 0xFFu;
}

// Barrier for LDS hand-offs inside the tile loop: waits for this wave's LDS operations only,
// so the gathers of later tiles keep flying (a full __syncthreads would wait for them too). The
// empty asm statements keep the compiler from moving memory accesses across it.
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

// Gather instructions per tile (the QK team issues them all): wave b issues instructions b + 4 j,
// j < 6, of the tile's 21, so wave 0 issues six and waves 1..3 five. Waits until this wave's
// gathers of all but the last `later` tiles it issued have landed (`later` at most 3).
__device__ __forceinline__ void wait_tiles_but(int later, int wave) {
  if (wave == 0) {
    if (later >= 3) wait_vmcnt<18>(); else if (later == 2) wait_vmcnt<12>();
    else if (later == 1) wait_vmcnt<6>(); else wait_vmcnt<0>();
  } else {
    if (later >= 3) wait_vmcnt<15>(); else if (later == 2) wait_vmcnt<10>();
    else if (later == 1) wait_vmcnt<5>(); else wait_vmcnt<0>();
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

// One (token, split): the split's share of the tiles of the token's index list, up to its last
// valid entry. Writes either the final bf16 output (+ lse) or a bf16 partial (+ lse) for the
// combine.
//
// Two teams of four waves, one wave of each on every SIMD, work on consecutive tiles at the same
// time, so that one team's matrix instructions run while the other's vector instructions do:
//  - the QK team (waves 0..3, wave b = FP8 block b) computes the partial logits of tile t,
//    holds them in registers across the middle barrier and then stores them; it also issues
//    every gather, and wave b writes block b's column of each tile's u table;
//  - the PV team (waves 4..7, wave b) reduces head tile b of tile t - 1 (all 32 rows, so the
//    softmax state of heads 16b..16b+15 stays inside the wave), writes P', and after the middle
//    barrier accumulates O for block b's 128 dims of all 64 heads.
// Per iteration: [QK(t) | reduce(t-1)] barrier [store partials(t), K and u column of tile t+1 |
// PV(t-1)] barrier.
__global__ __launch_bounds__(NT, 1) void mla_fp8_kernel(const Tok* __restrict__ toks,
                                                        const __bf16* __restrict__ q,
                                                        const unsigned char* __restrict__ kv,
                                                        const int32_t* __restrict__ idx,
                                                        int top_k,
                                                        float sm_scale, __bf16* __restrict__ out,
                                                        float* __restrict__ lse_out,
                                                        __bf16* __restrict__ part_o,
                                                        float* __restrict__ part_lse) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  MlaSmem& sm = *reinterpret_cast<MlaSmem*>(smem_raw);
  const int64_t t_tok = blockIdx.x;
  const int split = blockIdx.y;
  const int nsplit = gridDim.y;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool qk_team = wave < 4;
  const int b = wave & 3;
  const int G = lane >> 4, l16 = lane & 15;

  const int32_t* idx_row = idx + t_tok * top_k;

  // The split's indices. First guess, right for a list whose last entry is valid: the splits share
  // all of the list's tiles. The last entry is loaded with them to check.
  __shared__ int last_all, last_valid, logit_over, scale_over;
  if (tid == 0) last_all = -1, last_valid = -1, logit_over = 0, scale_over = 0;
  if (tid < 4) sm.eb[tid] = 0;
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
  const Tok tk = toks[t_tok];
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
  // The QK team copies the token's Q (64 heads x 576 bf16 values, 73,728 bytes) by the
  // load-to-LDS path, once its index-list loads have been used: the compiler's waits for those
  // would otherwise wait for the copy too. Head h's 72 sixteen-byte pieces sit at
  // qs + 1,152 h, piece p at slot p ^ (h & 7), so that the 16 heads a fragment read touches
  // fall on different banks.
  unsigned char* const qs = &sm.raw[NRAW - 1][0];
  if (qk_team) {
    const unsigned char* qsrc = reinterpret_cast<const unsigned char*>(q + t_tok * (int64_t)(MLA_H * MLA_DQK));
#pragma unroll
    for (int j = 0; j < Q_BYTES / 4096; ++j) {
      const int pc = 64 * (b + 4 * j) + lane;  // the LDS piece this lane fills
      const int h = pc / 72, sl = pc - 72 * h;
      lds_load16(qsrc + 16 * (72 * h + (sl ^ (h & 7))), qs + 1024 * (b + 4 * j));
    }
  }
  lds_barrier();  // the index list and last_valid are visible; the Q copy may still fly
  const int ntiles = (last_valid + TILE) / TILE;  // trailing invalid tiles are skipped

  // Gather plan (QK team): instruction gq = b + 4 j (j < 6, gq <= 20) loads the tile's chunks
  // 64 gq .. 64 gq + 63 (chunk ci = 16 bytes at offset 16 (ci % 41) of row ci / 41); instruction
  // 20's upper half would pass the last row, where the u table sits, and loads nothing.
  const unsigned char* kv_req = kv + tk.row_start * MLA_ROW_BYTES;
  int grow[6], goff[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int ci = min(64 * (b + 4 * j) + lane, TILE_CH - 1);
    grow[j] = ci / ROW_CH;
    goff[j] = 16 * (ci - ROW_CH * grow[j]);
  }
  // the row indices of a tile's gather, read ahead of it (a load's asm statement orders the LDS
  // reads after it behind it, so they must not sit between the loads)
  auto gather_ix = [&](int tile, int (&ix)[6]) {
    const int* ti = sm.idx + tile * TILE;
#pragma unroll
    for (int j = 0; j < 6; ++j) ix[j] = ti[grow[j]];
  };
  auto gather_go = [&](int tile, const int (&ix)[6]) {
    unsigned char* dst = sm.raw[tile % NRAW];
#pragma unroll
    for (int j = 0; j < 5; ++j)
      lds_load16(kv_req + (uint64_t)(uint32_t)max(ix[j], 0) * RB + goff[j], dst + 1024 * (b + 4 * j));
    if (b == 0 && lane < 32)
      lds_load16(kv_req + (uint64_t)(uint32_t)max(ix[5], 0) * RB + goff[5], dst + 1024 * 20);
  };
  auto gather = [&](int tile) {
    int ix[6];
    gather_ix(tile, ix);
    gather_go(tile, ix);
  };
  // valid-row masks of the split's tiles (bit r: row r has an index), lane i holding tile i's
  // (at most 64 tiles): the same in every wave, read with a lane read instead of LDS
  uint32_t vmr = 0;
#pragma unroll 4
  for (int tl = 0; tl < ntiles; ++tl) {
    const uint32_t m = (uint32_t)__ballot(sm.idx[tl * TILE + (lane & 31)] >= 0);
    if (lane == tl) vmr = m;
  }
  auto tile_valid = [&](int tile) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_readlane((int)vmr, tile);
  };

  const float c = sm_scale * LOG2E;
  bool f16 = true;         // P' and V in fp16 (else the bf16 fallback)
  bool u_out = false;      // QK team: a row's u of its block outside [U_MIN, U_MAX)

  // Each team runs its own pass loop (so that Q and O never share registers); both issue the same
  // barriers in the same order. A second pass runs when a logit left the reference window
  // (ref = the true maximum then, P <= 1), and with P' in bf16 when some row's scale left the
  // fp16 window.
  const bool split_out = part_o != nullptr;
  unsigned char* stage = &sm.raw[0][0];
  if (qk_team) {
    // the first three tiles go out now, beside the Q copy (their slots hold no part of Q)
    const int early = min(ntiles, NRAW - 1);
    for (int u = 0; u < early; ++u) gather(u);
    wait_tiles_but(early, b);  // this wave's part of the Q copy has landed
    lds_barrier();             // every QK wave's part has
    // The QK team's Q fragments, read from the copy in LDS: head tile ht, head 16 ht + l16; code
    // k-step ks: dims 128 b + 64 (ks >> 1) + 16 G + 8 (ks & 1) .. +8 (the order in which the K
    // fragments hold them); rope: dims 512 + 16 b + 4 G .. +4 (a 16-deep k-step covers the
    // block's share of the 64 rope dims). Reading Q from LDS (not from global memory) also keeps
    // the compiler from adding waits of its own for Q inside the tile loop, where the
    // vector-memory counter counts the gathers too.
    v8bf qc[4][4];
    v4s qr[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const int h = 16 * ht + l16;
      const unsigned char* qh = qs + 1152 * h;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int pc = 16 * b + 8 * (ks >> 1) + 2 * G + (ks & 1);
        qc[ht][ks] = *reinterpret_cast<const v8bf*>(qh + 16 * (pc ^ (h & 7)));
      }
      const int pr = 64 + 2 * b + (G >> 1);
      qr[ht] = *reinterpret_cast<const v4s*>(qh + 16 * (pr ^ (h & 7)) + 8 * (G & 1));
    }
    lds_barrier();  // every QK wave holds its Q before the gathers reuse its range
  // ---- QK team: one pass over the split's tiles. Phase 1 of iteration t issues only the
    // products of tile t (its K fragments were read and converted in the phase before); phase 2
    // stores the partials, then reads and converts tile t + 1 and writes its block's column of
    // tile t + 1's u table, so the conversions run beside the PV team's products.
    auto qk_pass = [&](auto f16_tag, bool first_pass) {
      constexpr bool F16 = decltype(f16_tag)::value;
      bool have_e = false;
      int e_b = 0;  // E_b of this wave's block
      int gix[6];   // row indices of the next tile to gather
      u_out = false;
      v8bf kc[2][4];     // tile's K codes as bf16: [row half][k-step]
      v4s kr[2];         // tile's rope dims: [row half]
      float sb[2][4];    // tile's block-b scales: [row half][i], rows 16 h + 4 G + i
      auto load_k = [&](int tile) {
        const unsigned char* rt = sm.raw[tile % NRAW];
        v4u k0[2], k1[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const unsigned char* rr = rt + RB * (16 * h + l16);
          k0[h] = *reinterpret_cast<const v4u*>(rr + 16 * (8 * b + G));
          k1[h] = *reinterpret_cast<const v4u*>(rr + 16 * (8 * b + 4 + G));
          kr[h] = *reinterpret_cast<const v4s*>(rr + ROPE_OFF + 32 * b + 8 * G);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sb[h][i] = *reinterpret_cast<const float*>(rt + RB * (16 * h + 4 * G + i) + SCALE_OFF + 4 * b);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const v4u& kk = ks < 2 ? k0[h] : k1[h];
            kc[h][ks] = e4m3x8_to_bf16(kk[2 * (ks & 1)], kk[2 * (ks & 1) + 1]);
          }
      };
      // u_b[r] = s_b[r] / 2^E_b for a tile's rows (lane: row lane & 31), 0 for rows without an
      // index; E_b is fixed by the first tile with a valid row (the exponent of its largest scale
      // of block b), 0 in the bf16 fallback. Wave b writes block b's column.
      auto u_col = [&](int tile) {
        unsigned char* rt = sm.raw[tile % NRAW];
        const int r = lane & 31;
        const float sc = *reinterpret_cast<const float*>(rt + RB * r + SCALE_OFF + 4 * b);
        const uint32_t vm = tile_valid(tile);
        const bool valid = (vm >> r) & 1u;
        if (F16 && !have_e && vm != 0) {  // uniform in the wave
          float m = valid ? sc : 0.f;
#pragma unroll
          for (int sh = 1; sh < 32; sh <<= 1) m = fmaxf(m, __shfl_xor(m, sh));
          e_b = m > 0.f && m <= 3.402823466e38f ? __builtin_amdgcn_frexp_expf(m) : 0;
          have_e = true;
        }
        const float uu = valid ? (F16 ? __builtin_amdgcn_ldexpf(sc, -e_b) : sc) : 0.f;
        u_out |= F16 && !((uu >= U_MIN && uu < U_MAX) || uu == 0.f);
        if (lane < 32) {
          if (F16)  // u < 2^3 or 0, and >= 2^-10: an fp16 normal number
            *reinterpret_cast<_Float16*>(rt + U_OFF + 2 * (32 * b + r)) = (_Float16)uu;
          else
            *reinterpret_cast<float*>(rt + U_OFF + 16 * r + 4 * b) = uu;
        }
      };
      const int first = min(ntiles, NRAW);
      for (int u = first_pass ? early : 0; u < first; ++u) gather(u);  // tiles 0..2 went out early
      if (ntiles > 0) wait_tiles_but(first - 1, b);
      lds_barrier();  // every wave's part of tile 0 has landed
      if (ntiles > 0) {
        load_k(0);
        u_col(0);
      }
      if (ntiles > 4) gather_ix(4, gix);
#pragma unroll 1
      for (int t = 0; t <= ntiles; ++t) {
        v4f acc[2][4];
        if (t < ntiles) {
          if (t >= 2 && t + 2 < ntiles) gather_go(t + 2, gix);  // its slot held tile t - 2, done with
          // the products go out at a raised priority: the PV wave on the same SIMD issues the
          // reduction's vector instructions meanwhile, and a product waiting behind them idles the
          // matrix core
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) acc[h][ht] = v4f{};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
              for (int ht = 0; ht < 4; ++ht)
                acc[h][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[h][ks], qc[ht][ks], acc[h][ht], 0, 0, 0);
          }
          // the block scale multiplies the code part; the rope part then accumulates on top
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[h][ht][i] *= sb[h][i];
              acc[h][ht] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr[h], qr[ht], acc[h][ht], 0, 0, 0);
            }
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_setprio(0);
          // tile t + 1 must have landed before phase 2 reads it; later tiles may still be in flight
          if (t + 1 < ntiles) {
            const int last_issued = min(ntiles - 1, max(NRAW - 1, t + 2));
            wait_tiles_but(last_issued - (t + 1), b);
          }
        }
        lds_barrier();  // the PV team has read the partials of tile t - 1; tile t + 1 has landed
        if (t < ntiles) {
          // lane: head 16 ht + l16, rows 16 h + 4 G + i
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) sm.part[h][ht][b][lane] = acc[h][ht];
          if (t + 1 < ntiles) {
            load_k(t + 1);
            u_col(t + 1);
          }
          if (t >= 2 && t + 3 < ntiles) gather_ix(t + 3, gix);  // gathered in the next phase 1
        }
        lds_barrier();
      }
      wait_vmcnt<0>();  // no gather may still be writing this workgroup's LDS
      if (lane == 0) sm.eb[b] = F16 ? e_b : 0;
    };

#pragma unroll 1
    for (int pass = 0;; ++pass) {
      if (f16) qk_pass(std::true_type{}, pass == 0);
      else qk_pass(std::false_type{}, pass == 0);
      if (__any(u_out)) scale_over = 1;
      __syncthreads();
      if (!(logit_over || scale_over) || pass == 1) break;
      f16 = !scale_over;
      __syncthreads();
    }
    __syncthreads();  // the PV team's output is staged
  } else {
    float ref = -INFINITY;   // softmax reference of head 16 b + l16 (log2 units)
    float seen = -INFINITY;  // largest logit (before the scale c) of that head in this lane's rows
    float lsum = 0.f;        // this lane's share of the head's softmax denominator
    v4f o[8][4];             // O^T [dim tile][head tile] for dims 128 b + 16 dt + 4 G + i
    bool over = false;       // a logit above ref + REF_HEADROOM
    lds_barrier();           // pairs with the QK team's barrier once Q has landed
    lds_barrier();           // pairs with the QK team's barrier after its Q reads
  // ---- PV team: one pass over the split's tiles, one tile behind the QK team
    auto pv_pass = [&](auto f16_tag, bool have_ref) {
      constexpr bool F16 = decltype(f16_tag)::value;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[i][j] = v4f{};
      lsum = 0.f;
      lds_barrier();  // tile 0 has landed
      const int voff = RB * (8 * G + (l16 >> 1)) + 16 * (8 * b) + 8 * (l16 & 1);
      v2i fv[8];          // V fragments of tile u, read at the end of phase 1
      uint32_t vm_u = 0;  // valid rows of tile u
#pragma unroll 1
      for (int t = 0; t <= ntiles; ++t) {
        const int u = t - 1;
        if (t >= 1) {
          // reduction of tile u, head tile b (lane: head 16 b + l16), rows 16 h + 4 G + i
          const unsigned char* rt = sm.raw[u % NRAW];
          // every LDS read of the reduction goes out first
          v4f ps[2][4];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b2 = 0; b2 < 4; ++b2) ps[h][b2] = sm.part[h][b][b2][lane];
          // u of the lane's rows 16 h + 4 G .. +3: fp16 per block (fp16 P'), fp32 per row (bf16)
          v2u uh[2][4];
          v4f uv[2][4];
          if constexpr (F16) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int b2 = 0; b2 < 4; ++b2)
                uh[h][b2] = *reinterpret_cast<const v2u*>(rt + U_OFF + 2 * (32 * b2 + 16 * h + 4 * G));
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                uv[h][i] = *reinterpret_cast<const v4f*>(rt + U_OFF + 16 * (16 * h + 4 * G + i));
          }
          vm_u = tile_valid(u);
          const uint32_t vm = vm_u;
          float y[2][4];  // logits before the scale c (c > 0); -inf for rows without an index
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const v4f sum = ps[h][0] + ps[h][1] + ps[h][2] + ps[h][3];
            if (vm == 0xFFFFFFFFu) {  // uniform
#pragma unroll
              for (int i = 0; i < 4; ++i) y[h][i] = sum[i];
            } else {
              const unsigned vb = (vm >> (16 * h + 4 * G)) & 15u;
#pragma unroll
              for (int i = 0; i < 4; ++i) y[h][i] = (vb >> i) & 1 ? sum[i] : -INFINITY;
            }
          }
          if (!have_ref && vm != 0) {  // uniform: the first tile with a valid row sets ref
            float m = fmaxf(fmaxf(fmaxf(y[0][0], y[0][1]), fmaxf(y[0][2], y[0][3])),
                            fmaxf(fmaxf(y[1][0], y[1][1]), fmaxf(y[1][2], y[1][3])));
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            ref = m * c + REF_MARGIN;
            have_ref = true;
          }
          const float m_use = ref == -INFINITY ? 0.f : ref;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              seen = fmaxf(seen, y[h][i]);  // a logit above m_use + REF_HEADROOM asks for a second pass
              // P = 2^(y c - ref): -inf -> 0; underflow to 0 is harmless
              pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(y[h][i], c, -m_use));
              lsum += pr[i];
            }
            // P'_b2 = P u_b2[row]; u is 0 for a row without an index, whose P is 0 too. fp16: P
            // (<= 2^11) and u (in [2^-10, 2^3]) are fp16 numbers, multiplied in pairs of rows
            if constexpr (F16) {
              const v2h p01 = __builtin_bit_cast(v2h, pack_f16(pr[0], pr[1]));
              const v2h p23 = __builtin_bit_cast(v2h, pack_f16(pr[2], pr[3]));
#pragma unroll
              for (int b2 = 0; b2 < 4; ++b2) {
                const unsigned u01 = uh[h][b2].x, u23 = uh[h][b2].y;
                const v2h w01 = p01 * __builtin_bit_cast(v2h, u01);
                const v2h w23 = p23 * __builtin_bit_cast(v2h, u23);
                unsigned* dst = reinterpret_cast<unsigned*>(&sm.pp[b2][b][2 * h + (G >> 1)][l16]) + 2 * (G & 1);
                *reinterpret_cast<v2u*>(dst) = v2u{__builtin_bit_cast(unsigned, w01), __builtin_bit_cast(unsigned, w23)};
              }
            } else {
#pragma unroll
              for (int b2 = 0; b2 < 4; ++b2) {
                float w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = pr[i] * uv[h][i][b2];
                unsigned* dst = reinterpret_cast<unsigned*>(&sm.pp[b2][b][2 * h + (G >> 1)][l16]) + 2 * (G & 1);
                *reinterpret_cast<v2u*>(dst) = v2u{pack_bf16(w[0], w[1]), pack_bf16(w[2], w[3])};
              }
            }
          }
          // the V fragments of tile u go out now, to land during the barrier
          const unsigned char* rv = sm.raw[u % NRAW];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            fv[dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i*)(rv + voff + 16 * dt));
        }
        lds_barrier();  // P' of tile u visible; the partials of tile u read
        if (t >= 1) {
          // PV of tile u: dims 128 b + 16 dt + 4 G + i of every head. The wave's priority is raised
          // until its products are issued: the QK wave on the same SIMD (older, so preferred at
          // equal priority) converts K meanwhile, and its vector instructions would otherwise
          // delay the conversions and products here. (Raised for the products alone, the phase is
          // 2% longer: the conversions before them are on its critical path too.)
          __builtin_amdgcn_s_setprio(2);
          const unsigned vb = (vm_u >> (8 * G)) & 0xFFu;
          const unsigned mlo = byte_mask4(vb), mhi = byte_mask4(vb >> 4);
          v4u pb[4];
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) pb[ht] = sm.pp[b][ht][G][l16];
          // every V fragment is converted while P' is in flight; then the products go out back to
          // back (converting between them would leave the matrix core idle)
          using VT = std::conditional_t<F16, v8h, v8bf>;
          VT va[8];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const v2i f = fv[dt];
            if constexpr (F16) va[dt] = e4m3x8_to_f16((unsigned)f[0] & mlo, (unsigned)f[1] & mhi);
            else va[dt] = e4m3x8_to_bf16((unsigned)f[0] & mlo, (unsigned)f[1] & mhi);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
              if constexpr (F16)
                o[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[dt], __builtin_bit_cast(v8h, pb[ht]), o[dt][ht], 0, 0, 0);
              else
                o[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], __builtin_bit_cast(v8bf, pb[ht]), o[dt][ht], 0, 0, 0);
            }
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_setprio(0);
        }
        lds_barrier();
      }
    };


#pragma unroll 1
    for (int pass = 0;; ++pass) {
      if (f16) pv_pass(std::true_type{}, pass > 0);
      else pv_pass(std::false_type{}, pass > 0);
      // denominators and maxima of each head: all 32 rows of a tile are in this wave
      lsum += __shfl_xor(lsum, 16);
      lsum += __shfl_xor(lsum, 32);
      float sn = fmaxf(seen, __shfl_xor(seen, 16));
      sn = fmaxf(sn, __shfl_xor(sn, 32));
      sn *= c;  // the largest scaled logit
      if (G == 0) {
        sm.xsum[0][16 * b + l16] = lsum;
        sm.xmax[0][16 * b + l16] = sn;
      }
      over = seen * c > (ref == -INFINITY ? 0.f : ref) + REF_HEADROOM;
      if (__any(over)) logit_over = 1;  // any wave: every wave redoes the split
      __syncthreads();
      if (!(logit_over || scale_over) || pass == 1) break;
      ref = sn;
      f16 = !scale_over;
      __syncthreads();
    }
    // The output goes out through LDS (the raw slots, idle once the tile loop is done) so that
    // every global store writes whole lines: head h's 512 16-bit values sit at h * 1024 with
    // 16-byte chunk c at 16 (c ^ (h & 63)), and a wave stores one head's row (1 KB) per
    // instruction.
    const int e_out = sm.eb[b];  // O_b = 2^E_b sum_r P_r u_b[r] code_r / sum_r P_r
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const int h = 16 * ht + l16;
      const float l = sm.xsum[0][h];
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int chunk = 16 * b + 2 * dt + (G >> 1);  // dims 128 b + 16 dt + 8 (G >> 1)
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_ldexpf(o[dt][ht][i] * inv, e_out);
        *reinterpret_cast<v2u*>(stage + h * 1024 + 16 * (chunk ^ (h & 63)) + 8 * (G & 1)) =
            v2u{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
    }
    if (G == 0) {
      const int h = 16 * b + l16;
      const float l = sm.xsum[0][h];
      const float m_use = ref == -INFINITY ? 0.f : ref;  // the reference P was formed against
      const float lse = l > 0.f ? (m_use + __log2f(l)) * (1.0f / LOG2E) : -INFINITY;
      if (split_out) part_lse[(t_tok * nsplit + split) * MLA_H + h] = lse;
      else if (lse_out) lse_out[t_tok * MLA_H + h] = lse;
    }
    __syncthreads();
  }
  unsigned char* dst = split_out ? reinterpret_cast<unsigned char*>(part_o + (t_tok * nsplit + split) * MLA_H * MLA_DV)
                                 : reinterpret_cast<unsigned char*>(out + t_tok * MLA_H * MLA_DV);
#pragma unroll 4
  for (int hh = wave; hh < MLA_H; hh += NT / 64)
    *reinterpret_cast<v4u*>(dst + hh * 1024 + 16 * lane) =
        *reinterpret_cast<const v4u*>(stage + hh * 1024 + 16 * (lane ^ (hh & 63)));
}

// Merge split partials by log-sum-exp: one 128-thread block per (token, head), 4 dims per
// thread. The first eight splits' partials go out together with their lse values, so a merge of
// up to eight splits costs one memory round trip. Block b takes token b % n_tok: workgroups are
// dealt to the XCDs round robin, so with n_tok a multiple of 8 a token's merge runs on the XCD
// whose L2 holds the partials its splits just wrote (the attention grid puts every split of
// token t on XCD t % 8 too).
__global__ __launch_bounds__(128) void mla_combine_kernel(const __bf16* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          int nsplit, int n_tok,
                                                          __bf16* __restrict__ out,
                                                          float* __restrict__ lse_out) {
  const int64_t t = blockIdx.x % n_tok;
  const int h = (int)(blockIdx.x / n_tok);
  const int64_t th = t * MLA_H + h;
  const float* pl = part_lse + t * nsplit * MLA_H + h;
  const __bf16* po = part_o + (t * nsplit * MLA_H + h) * MLA_DV + 4 * threadIdx.x;
  v4bf v[8];
  float lj[8];
  auto load8 = [&](int j0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + u, nsplit - 1);
      v[u] = *reinterpret_cast<const v4bf*>(po + (int64_t)j * MLA_H * MLA_DV);
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
        if (lj[u] == -INFINITY) continue;  // a split that saw no row: its partial is not read
        const float wj = __expf(lj[u] - m);
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

// Scratch for callers that cannot allocate (smla_sparse_mla_decode_noalloc): the decode split
// partials of up to MLA_SCRATCH_SPLITS (token, split) pairs, laid out as a workspace of that size
// (bf16 partial outputs, then fp32 lse). The split rule below never needs more than 510 pairs.
// Each GPU that runs the library holds one copy for the life of the process; the host reaches
// it only through the address hipGetSymbolAddress returns for the current device.
constexpr int MLA_SCRATCH_SPLITS = 512;
constexpr size_t MLA_SCRATCH_BYTES =
    (size_t)MLA_SCRATCH_SPLITS * MLA_H * MLA_DV * 2 + (size_t)MLA_SCRATCH_SPLITS * MLA_H * 4;
static __device__ __align__(256) unsigned char scratch[MLA_SCRATCH_BYTES];

size_t mla_scratch_bytes() { return MLA_SCRATCH_BYTES; }

hipError_t mla_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

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
  return align_up(n * D_v * sizeof(__bf16), 256) + align_up(n * sizeof(float), 256);
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
  __bf16* part_o = nullptr;
  float* part_lse = nullptr;
  if (nsplit > 1) {
    part_o = static_cast<__bf16*>(ws);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                        align_up((size_t)b.total_q * nsplit * MLA_H * MLA_DV * sizeof(__bf16), 256));
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
