// topk.hip — exact per-query top-k over int32 indexer scores on gfx950.
//
// The indexer keeps, for every query token, the 2,048 earlier tokens with the largest scores
// ("Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "Why DP8 and TP8 fall short"); ties
// go to the lower token index, and every s <= p is kept when p + 1 <= k.
//
// Selection order is the total order of the unique 64-bit key (score << 32) | ~s, so the top-k
// set is unique. A select finds it without sorting:
//  1. a 2048-bin histogram of a monotone, floating-point-like code of the score (5-bit exponent,
//     6 bits below the leading one) locates the bin b* that holds the k-th largest key;
//     everything in higher bins is selected;
//  2. inside b* an MSD radix select over 8-bit digits of the 64-bit key finds the exact cut.
// Rows of up to 32,768 candidates are selected by one 512-thread workgroup with the scores held
// in registers and the histogram built in LDS (two rows per CU).
// Longer rows use the histogram the indexer kernel accumulated while scoring: in batches with
// many query tokens, rows of up to 73,728 candidates are held in one workgroup's registers;
// otherwise (and for longer rows) rows are cut into 4,096-candidate segments handled by three
// kernels (count, resolve, emit). Selected indices always come out in ascending order, each
// written at its rank.
#include "smla_internal.h"

namespace smla {

namespace {

// Histogram code of a score: integer scores (int8 keys) or the bit patterns of non-negative fp32
// scores (FP8 keys); both codes are monotone in the 32-bit pattern.
template <bool FB>
__device__ __forceinline__ int score_bin(uint32_t s) { return FB ? topk_fbin(s) : topk_bin(s); }
template <bool FB>
__device__ __forceinline__ uint64_t bin_lo(int b) { return FB ? topk_fbin_lo(b) : topk_bin_lo(b); }

__device__ __forceinline__ uint64_t sel_key(int32_t score, int64_t s) {
  return ((uint64_t)(uint32_t)score << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)s);
}

// Inclusive scan over the block (NT threads, multiple of 64); `red` holds NT/64 + 1 ints and
// red[NT/64] holds the block total on return. Every wave reads all wave totals and reduces the
// ones before it itself (a butterfly over the first NT/64 lanes), so no thread walks them.
template <int NT>
__device__ int block_incl_scan(int v, int* red) {
  constexpr int NW = NT / 64;
  static_assert((NW & (NW - 1)) == 0 && NW <= 64, "a power-of-two number of waves");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) red[wv] = v;
  __syncthreads();
  const int s = lane < NW ? red[lane] : 0;
  int before = lane < wv ? s : 0, all = s;
#pragma unroll
  for (int o = 1; o < NW; o <<= 1) {
    before += __shfl_xor(before, o);
    all += __shfl_xor(all, o);
  }
  v += __shfl(before, 0);
  if (threadIdx.x == 0) red[NW] = all;
  __syncthreads();  // red[NW] visible; red is free for the next scan
  return v;
}

// Over hist[0..NB): the bin b holding the k-th largest element counting from the top, and the
// number of elements in bins above it. Results land in out[0] (bin) and out[1] (count above).
// Requires sum(hist) >= k >= 1.
template <int NT>
__device__ void find_cut(const int* hist, int NB, int k, int* red, int* out) {
  if (threadIdx.x == 0) {  // in range even if sum(hist) < k were ever violated
    out[0] = 0;
    out[1] = 0;
  }
  const int per = NB >= NT ? NB / NT : 1;
  const int lo = threadIdx.x * per;
  int local = 0;
  if (lo < NB)
    for (int i = 0; i < per; ++i) local += hist[lo + i];
  const int incl = block_incl_scan<NT>(local, red);
  const int total = red[NT / 64];
  const int above = total - incl;  // elements in bins past my range
  if (lo < NB && above < k && above + local >= k) {
    int c = above;
    for (int b = lo + per - 1; b >= lo; --b) {
      if (c + hist[b] >= k) {
        out[0] = b;
        out[1] = c;
        break;
      }
      c += hist[b];
    }
  }
  __syncthreads();
}

// MSD radix select over 8-bit digits of 64-bit keys produced by `key_of(i)` for i in [0, n)
// restricted to `member(i)`: finds (prefix, mask) such that exactly `need` members satisfy
// (key & mask) >= prefix... i.e. the members with (key & mask) > prefix plus those equal to it.
template <int NT, typename KeyOf, typename Member>
__device__ void radix_cut(int n, int need, KeyOf key_of, Member member, int* hist2, int* red,
                          int* cut, uint64_t* pm) {
  uint64_t prefix = 0, mask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) hist2[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      if (!member(i)) continue;
      const uint64_t key = key_of(i);
      if ((key & mask) != prefix) continue;
      atomicAdd(&hist2[(int)((key >> shift) & 255u)], 1);
    }
    __syncthreads();
    find_cut<NT>(hist2, 256, need, red, cut);
    const int dg = cut[0];
    const int gt = cut[1];
    const int eq = hist2[dg];
    need -= gt;
    prefix |= (uint64_t)dg << shift;
    mask |= (uint64_t)255u << shift;
    __syncthreads();
    if (eq == need) break;
  }
  if (threadIdx.x == 0) {
    pm[0] = prefix;
    pm[1] = mask;
  }
  __syncthreads();
}

// Single-wave MSD radix select over n unique 64-bit keys in LDS, key i read by key_at(i) (call
// from one whole wave):
// returns (prefix, mask) such that exactly `need` keys satisfy (key & mask) >= prefix. The
// digits above the highest bit where the keys differ are skipped, so a bin of near-equal scores
// resolves in one or two passes. `h` is a 256-int LDS scratch owned by this wave.
template <typename KeyAt>
__device__ void wave_radix_cut(KeyAt key_at, int n, int need, int* h, uint64_t* prefix_out,
                               uint64_t* mask_out) {
  const int lane = threadIdx.x & 63;
  uint64_t a = ~0ull, o = 0ull;
  for (int i = lane; i < n; i += 64) {
    const uint64_t key = key_at(i);
    a &= key;
    o |= key;
  }
  for (int d = 32; d > 0; d >>= 1) {
    a &= __shfl_xor(a, d);
    o |= __shfl_xor(o, d);
  }
  uint64_t prefix = 0, mask = 0;
  if (n != need && (a ^ o) != 0) {
    const int hb = 63 - __builtin_clzll(a ^ o);
    int shift = (hb / 8) * 8;
    mask = shift + 8 >= 64 ? 0ull : ~((1ull << (shift + 8)) - 1);
    prefix = a & mask;  // common bits above the first differing digit
    for (; shift >= 0; shift -= 8) {
      // a digit every key shares splits nothing (the high bits of the index half of the keys,
      // for a start): take it from `a` without a pass
      if ((((a ^ o) >> shift) & 255u) == 0) {
        prefix |= a & (255ull << shift);
        mask |= 255ull << shift;
        continue;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) h[4 * lane + j] = 0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      for (int i = lane; i < n; i += 64) {
        const uint64_t key = key_at(i);
        if ((key & mask) == prefix) atomicAdd(&h[(int)((key >> shift) & 255u)], 1);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // lane l owns digits [4l, 4l + 4); count of digits above each lane's range
      const int c0 = h[4 * lane], c1 = h[4 * lane + 1], c2 = h[4 * lane + 2], c3 = h[4 * lane + 3];
      const int local = c0 + c1 + c2 + c3;
      int incl = local;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d);
        if (lane >= d) incl += u;
      }
      const int total = __shfl(incl, 63);
      const int above = total - incl;
      int dg = -1, gt = 0, eq = 0;
      if (above < need && above + local >= need) {
        int cc = above;
        const int cs[4] = {c0, c1, c2, c3};
        for (int j = 3; j >= 0; --j) {
          if (cc + cs[j] >= need) {
            dg = 4 * lane + j;
            gt = cc;
            eq = cs[j];
            break;
          }
          cc += cs[j];
        }
      }
      const uint64_t who = __ballot(dg >= 0);
      const int src = who ? __builtin_ctzll(who) : 0;
      dg = __shfl(dg, src);
      gt = __shfl(gt, src);
      eq = __shfl(eq, src);
      need -= gt;
      prefix |= (uint64_t)dg << shift;
      mask |= (uint64_t)255u << shift;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (eq == need) break;
    }
  }
  *prefix_out = prefix;
  *mask_out = mask;
}

constexpr int NT_A = 1024;                          // the DCP merge's workgroup
constexpr int MERGE_PER = MERGE_MAX_CAND / NT_A;    // candidates per thread, in registers
constexpr int MERGE_WORDS = MERGE_MAX_CAND / 32;    // selection bitmap words

// MSD radix select as radix_cut, over the PER keys each thread holds in registers; element u
// takes part iff member(u).
template <int NT, int PER, typename Member>
__device__ void radix_cut_regs(const uint64_t (&key)[PER], Member member, int need, int* hist2,
                               int* red, int* cut, uint64_t* pm) {
  uint64_t prefix = 0, mask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) hist2[i] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (member(u) && (key[u] & mask) == prefix)
        atomicAdd(&hist2[(int)((key[u] >> shift) & 255u)], 1);
    __syncthreads();
    find_cut<NT>(hist2, 256, need, red, cut);
    const int dg = cut[0];
    const int gt = cut[1];
    const int eq = hist2[dg];
    need -= gt;
    prefix |= (uint64_t)dg << shift;
    mask |= (uint64_t)255u << shift;
    __syncthreads();
    if (eq == need) break;
  }
  if (threadIdx.x == 0) {
    pm[0] = prefix;
    pm[1] = mask;
  }
  __syncthreads();
}

// ---- DCP top-k merge: the union of per-shard lists, one 1024-thread workgroup per token ----
// Shard l of n_lists holds the tokens l, l + n_lists, ...; list entry (local j, score) is global
// index g = j n_lists + l. Candidate c = l k_in + (position in list l); thread tid holds the
// candidates u NT_A + tid in registers, with their keys and score codes (AL: k_in is a multiple
// of NT_A, so each u lies in one list for the whole workgroup). The cut is found as for a row: a
// histogram of score codes locates the bin of the take-th key, an exact radix select inside that
// bin finds the key itself. The selection is kept as a bitmap over c, and F(c), the number of
// selected candidates before c, is a popcount away. Per-candidate steps are written without
// branches (invalid entries go to a spare histogram bin and spare LDS slots), since the
// workgroup's time is the instructions its 16 waves issue on one CU.
// Output order: for g = j n + l, ascending g is ascending (j, l). When every list holds its
// valid entries in ascending order followed only by padding (what the indexer's top-k returns),
// the selected entries, numbered F(c), are list after list and ascending inside each list. The
// entry numbered r of list l then has output position (r - F(l k_in)) plus, for each other list
// l', the number of l''s selected entries with local index below j (l' > l) or at most j (l' <
// l), no sort: the local indices are cut into NBK buckets of width W, a table holds every list's
// count of selected entries below each bucket (a histogram and one block scan), and an entry
// reads that count for its own bucket and then compares only the few entries of that bucket.
// r - F(l k_in) is also its position in its shard's local list. Each thread ranks the entries
// numbered tid and tid + 1024.
// Otherwise the selected (index, score) pairs are sorted by index (bitonic), and each shard's
// local list is cut out of the sorted selection by one block scan per shard.
template <bool FB, bool AL>
__global__ __launch_bounds__(NT_A) void topk_merge_kernel(int n_lists, int k_in,
                                                          const int32_t* __restrict__ idx_lists,
                                                          const int32_t* __restrict__ score_lists,
                                                          int64_t list_stride, int top_k,
                                                          int32_t* __restrict__ idx_out,
                                                          int32_t* __restrict__ score_out,
                                                          int32_t* __restrict__ local_out,
                                                          int64_t local_stride) {
  extern __shared__ __align__(16) unsigned char smem_m[];
  uint64_t* work = reinterpret_cast<uint64_t*>(smem_m);  // [TOPK_MAX_K + 1], the last a spare
  uint64_t* sel = work + TOPK_MAX_K + 1;  // [TOPK_MAX_K + 1] numbered entries (score, j); spare
  int32_t* lidx = reinterpret_cast<int32_t*>(sel + TOPK_MAX_K + 1);  // [MERGE_MAX_CAND] local j
  int* hist = reinterpret_cast<int*>(lidx + MERGE_MAX_CAND);         // [TOPK_BINS + 1]; spare
  uint32_t* bits = reinterpret_cast<uint32_t*>(hist + TOPK_BINS + 1);  // [MERGE_WORDS]
  int* wpre = reinterpret_cast<int*>(bits + MERGE_WORDS);              // [MERGE_WORDS + 1]
  __shared__ int hist2[256];
  __shared__ int red[NT_A / 64 + 1];
  __shared__ int cut[2];
  __shared__ uint64_t pm[2];
  __shared__ int nval[MERGE_FAST_LISTS], lbase[MERGE_FAST_LISTS + 1];
  __shared__ uint8_t sel_list[TOPK_MAX_K + 1];  // list of each numbered entry; spare
  __shared__ int nvalid, unsorted;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncand = n_lists * k_in;
  const bool fast_ok = n_lists <= MERGE_FAST_LISTS;
  if (tid == 0) nvalid = 0, unsorted = fast_ok ? 0 : 1;
  if (tid < MERGE_FAST_LISTS) nval[tid] = 0;
  for (int i = tid; i <= TOPK_BINS; i += NT_A) hist[i] = 0;
  // list of candidate c: floor((c + 0.5) / k_in) in fp32 is exact here, since the quotient's
  // distance to an integer (>= 0.5 / k_in) exceeds its rounding error ((c + 0.5) 2^-23 / k_in)
  // for every c < 2^22
  const float inv_k = 1.0f / (float)k_in;
  auto list_of = [&](int c) { return (int)(((float)c + 0.5f) * inv_k); };
  int lu[MERGE_PER];  // AL: list of slot u, the same for every thread
  if (AL) {
    const int per_list = k_in / NT_A;
    int l = 0, left = per_list;
#pragma unroll
    for (int u = 0; u < MERGE_PER; ++u) {
      lu[u] = l;
      if (--left == 0) left = per_list, ++l;
    }
  }
  auto list_u = [&](int u, int c) { return AL ? lu[u] : list_of(c); };
  int32_t li[MERGE_PER];
  uint64_t key[MERGE_PER];  // 0: no candidate (valid keys have ~index >= 2^31)
  int bin[MERGE_PER];       // score code; TOPK_BINS (the spare bin) for no candidate
  {
    int32_t sv[MERGE_PER];
#pragma unroll
    for (int u = 0; u < MERGE_PER; ++u) {  // every load in flight before any is used
      const int c = u * NT_A + tid;
      const int l = list_u(u, c);
      const int64_t off = l * list_stride + t * k_in + (c - l * k_in);
      li[u] = c < ncand ? idx_lists[off] : -1;
      sv[u] = c < ncand ? score_lists[off] : 0;
    }
    __syncthreads();  // hist and the counters are cleared
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < MERGE_PER; ++u) {
      const int c = u * NT_A + tid;
      if (c < ncand) lidx[c] = li[u];
      const bool v = li[u] >= 0;
      key[u] = v ? sel_key(sv[u], (int64_t)li[u] * n_lists + list_u(u, c)) : 0ull;
      bin[u] = v ? score_bin<FB>((uint32_t)sv[u]) : TOPK_BINS;
      atomicAdd(&hist[bin[u]], 1);
      cnt += __popcll(__ballot(v));
    }
    if (lane == 0 && cnt) atomicAdd(&nvalid, cnt);
  }
  __syncthreads();
  // the fast order needs every list ascending, then padding; nval[l] = its valid entries
  if (fast_ok) {
    int32_t nb[MERGE_PER];
#pragma unroll
    for (int u = 0; u < MERGE_PER; ++u) {  // the next entries first, all reads in flight
      const int c = u * NT_A + tid;
      nb[u] = c + 1 < ncand ? lidx[c + 1] : -1;
    }
    bool bad = false;
#pragma unroll
    for (int u = 0; u < MERGE_PER; ++u) {
      const int c = u * NT_A + tid;
      const int l = list_u(u, c), j = c - l * k_in;
      const int32_t a = li[u], b = j + 1 < k_in ? nb[u] : -1;
      bad |= c < ncand && !(b < 0 || (a >= 0 && a < b));
      if (c < ncand && a >= 0 && b < 0) nval[l] = j + 1;
    }
    if (__ballot(bad) && lane == 0) unsorted = 1;
  }
  const int n = nvalid;
  const int take = min(top_k, n);
  int bstar = -1;  // every valid key selected
  uint64_t prefix = 0, mask = 0;
  if (take < n) {
    find_cut<NT_A>(hist, TOPK_BINS, take, red, cut);
    bstar = cut[0];
    const int need = take - cut[1];
    const int nbin = hist[bstar];
    if (nbin != need) {
      if (nbin <= TOPK_MAX_K) {  // the bin's keys to LDS, then one wave selects inside them
        int mine = 0;
#pragma unroll
        for (int u = 0; u < MERGE_PER; ++u) mine += bin[u] == bstar;
        int pos = block_incl_scan<NT_A>(mine, red) - mine;
#pragma unroll
        for (int u = 0; u < MERGE_PER; ++u) {
          const bool in = bin[u] == bstar;
          work[in ? pos : TOPK_MAX_K] = key[u];
          pos += in;
        }
        __syncthreads();
        if (wave == 0) {
          uint64_t pf, mk;
          wave_radix_cut([&](int i) { return work[i]; }, nbin, need, hist2, &pf, &mk);
          if (lane == 0) {
            pm[0] = pf;
            pm[1] = mk;
          }
        }
        __syncthreads();
      } else {
        radix_cut_regs<NT_A, MERGE_PER>(key, [&](int u) { return bin[u] == bstar; }, need, hist2,
                                        red, cut, pm);
      }
      prefix = pm[0];
      mask = pm[1];
    }
  }
  // the selection as a bitmap over c: each wave's 64 candidates of a u are two aligned words
  uint64_t msk[MERGE_PER];  // the same words, per wave (uniform)
#pragma unroll
  for (int u = 0; u < MERGE_PER; ++u) {
    const bool s = key[u] != 0 &&
                   (bstar < 0 || bin[u] > bstar || (bin[u] == bstar && (key[u] & mask) >= prefix));
    const uint64_t m = __ballot(s);
    msk[u] = m;
    const int w0 = (u * NT_A + wave * 64) >> 5;
    if (lane < 2) bits[w0 + lane] = (uint32_t)(lane ? m >> 32 : m);
  }
  __syncthreads();
  {
    const int pc = tid < MERGE_WORDS ? __popc(bits[tid]) : 0;
    const int incl = block_incl_scan<NT_A>(pc, red);
    if (tid < MERGE_WORDS) wpre[tid] = incl - pc;
    if (tid == MERGE_WORDS - 1) wpre[MERGE_WORDS] = incl;
  }
  __syncthreads();
  // F(c): selected candidates before c (0 <= c <= MERGE_MAX_CAND)
  auto F = [&](int c) {
    const int w = c >> 5, r = c & 31;
    return r ? wpre[w] + __popc(bits[w] & ((1u << r) - 1u)) : wpre[w];
  };
  auto selected = [&](int c) { return (bits[c >> 5] >> (c & 31)) & 1u; };
  int32_t* oi = idx_out + t * top_k;
  int32_t* os = score_out ? score_out + t * top_k : nullptr;
  const int32_t pad = FB ? (int32_t)0xBF800000u : -1;
  if (!unsorted) {
    if (tid <= n_lists) lbase[tid] = F(tid * k_in);
    const uint64_t below = (1ull << lane) - 1ull;
    int wp[MERGE_PER];
#pragma unroll
    for (int u = 0; u < MERGE_PER; ++u) wp[u] = wpre[(u * NT_A + wave * 64) >> 5];
#pragma unroll
    for (int u = 0; u < MERGE_PER; ++u) {  // number the selected entries: sel[F(c)]
      const int r = wp[u] + __popcll(msk[u] & below);
      const int dst = ((msk[u] >> lane) & 1ull) && r < TOPK_MAX_K ? r : TOPK_MAX_K;
      sel[dst] = (key[u] & 0xFFFFFFFF00000000ull) | (uint32_t)li[u];
      sel_list[dst] = (uint8_t)list_u(u, u * NT_A + tid);
    }
    __syncthreads();
    // the local indices of the numbered entries, alone, for the searches (reuses `lidx`)
    int32_t* selj = lidx;
    for (int r = tid; r < take; r += NT_A) selj[r] = (int32_t)(uint32_t)sel[r];
    // bucket table over the local indices: cum[l (NBK + 1) + b] = list l's selected entries in
    // buckets below b (then the whole list at b = NBK); it sits in `lidx` past the first
    // TOPK_MAX_K words
    const int NBK = TOPK_MAX_K / n_lists;  // n_lists (NBK + 1) <= TOPK_MAX_K + MERGE_FAST_LISTS
    int* cum = lidx + TOPK_MAX_K;
    const int ncum = n_lists * (NBK + 1);
    for (int i = tid; i < ncum; i += NT_A) cum[i] = 0;
    int jmax = -1;
    for (int r = tid; r < take; r += NT_A) jmax = max(jmax, (int)(uint32_t)sel[r]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) jmax = max(jmax, __shfl_xor(jmax, o));
    if (lane == 0) hist2[wave] = jmax;
    __syncthreads();
    jmax = -1;
    for (int w = 0; w < NT_A / 64; ++w) jmax = max(jmax, hist2[w]);
    const int W = jmax / NBK + 1;  // buckets of W local indices cover [0, jmax]
    bool on[2];
    int le[2], own[2], rank[2], bk[2];
    int32_t je[2];
    uint64_t ent[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {  // entries tid and tid + 1024 (take <= 2048)
      const int r = tid + e * NT_A;
      on[e] = r < take;
      ent[e] = on[e] ? sel[r] : 0ull;
      le[e] = on[e] ? sel_list[r] : 0;
      je[e] = (int32_t)(uint32_t)ent[e];
      bk[e] = je[e] / W;
      own[e] = on[e] ? r - lbase[le[e]] : 0;
      rank[e] = own[e];
      if (on[e]) atomicAdd(&cum[le[e] * (NBK + 1) + bk[e]], 1);
    }
    __syncthreads();
    {  // exclusive prefix over the whole table (three words per thread); minus the list's start
      int v[3], loc = 0;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int i = 3 * tid + k;
        v[k] = i < ncum ? cum[i] : 0;
        loc += v[k];
      }
      int pre = block_incl_scan<NT_A>(loc, red) - loc;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int i = 3 * tid + k;
        if (i < ncum) cum[i] = pre - lbase[i / (NBK + 1)];
        pre += v[k];
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (!on[e]) continue;
      for (int l2 = 0; l2 < n_lists; ++l2) {
        if (l2 == le[e]) continue;
        const int32_t tg = l2 < le[e] ? je[e] + 1 : je[e];
        const int* c2 = cum + l2 * (NBK + 1) + bk[e];
        const int32_t* s2 = selj + lbase[l2];
        int cnt = c2[0];
        for (int x = c2[0]; x < c2[1]; ++x) cnt += s2[x] < tg;
        rank[e] += cnt;
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (!on[e]) continue;
      if (rank[e] < TOPK_MAX_K)
        work[rank[e]] = ((uint64_t)(uint32_t)(je[e] * n_lists + le[e]) << 32) | (ent[e] >> 32);
      if (local_out) local_out[le[e] * local_stride + t * top_k + own[e]] = je[e];
    }
    __syncthreads();
    if (local_out)
      for (int l = 0; l < n_lists; ++l) {
        int32_t* lo = local_out + l * local_stride + t * top_k;
        for (int r = lbase[l + 1] - lbase[l] + tid; r < top_k; r += NT_A) lo[r] = -1;
      }
  } else {
    int mine = 0;
#pragma unroll
    for (int u = 0; u < MERGE_PER; ++u) mine += u * NT_A + tid < ncand && selected(u * NT_A + tid);
    int pos = block_incl_scan<NT_A>(mine, red) - mine;
#pragma unroll
    for (int u = 0; u < MERGE_PER; ++u)
      if (u * NT_A + tid < ncand && selected(u * NT_A + tid) && pos < TOPK_MAX_K)
        work[pos++] = ((uint64_t)(0xFFFFFFFFu - (uint32_t)key[u]) << 32) | (key[u] >> 32);
    // ascending global index: bitonic sort of the selected (index, score) pairs
    int m = 1;
    while (m < take) m <<= 1;
    __syncthreads();
    for (int i = take + tid; i < m; i += NT_A) work[i] = ~0ull;
    __syncthreads();
    for (int size = 2; size <= m; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < m / 2; i += NT_A) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const uint64_t a = work[lo], b = work[hi];
          if ((a > b) == up) {
            work[lo] = b;
            work[hi] = a;
          }
        }
        __syncthreads();
      }
    }
    if (local_out) {  // each shard's entries of the sorted selection, in order (thread: 2 ranks)
      const int r0 = 2 * tid;
      for (int l = 0; l < n_lists; ++l) {
        const uint32_t g0 = r0 < take ? (uint32_t)(work[r0] >> 32) : 0u;
        const uint32_t g1 = r0 + 1 < take ? (uint32_t)(work[r0 + 1] >> 32) : 0u;
        const bool s0 = r0 < take && g0 % (uint32_t)n_lists == (uint32_t)l;
        const bool s1 = r0 + 1 < take && g1 % (uint32_t)n_lists == (uint32_t)l;
        const int mc = (int)s0 + (int)s1;
        const int incl = block_incl_scan<NT_A>(mc, red);
        const int total = red[NT_A / 64];
        int32_t* lo = local_out + l * local_stride + t * top_k;
        int p = incl - mc;
        if (s0) lo[p++] = (int32_t)(g0 / (uint32_t)n_lists);
        if (s1) lo[p] = (int32_t)(g1 / (uint32_t)n_lists);
        for (int r = total + tid; r < top_k; r += NT_A) lo[r] = -1;
        __syncthreads();  // red is reused by the next shard's scan
      }
    }
  }
  for (int j = tid; j < top_k; j += NT_A) {
    oi[j] = j < take ? (int32_t)(work[j] >> 32) : -1;
    if (os) os[j] = j < take ? (int32_t)(uint32_t)work[j] : pad;
  }
}

// ---- rows of n > TOPK_LDS_MAX: workspace layout ------------------------------------------
__host__ __device__ inline TopkWs topk_ws(void* base, int64_t total_q, int64_t nseg) {
  char* p = static_cast<char*>(base);
  TopkWs w;
  w.hist = reinterpret_cast<int*>(p);
  p += align_up(sizeof(int) * TOPK_BINS * (size_t)total_q, 256);
  w.rec = reinterpret_cast<int*>(p);
  p += align_up(sizeof(int) * TOPK_REC * (size_t)total_q, 256);
  w.seg = reinterpret_cast<int*>(p);
  p += align_up(sizeof(int) * (size_t)nseg * (size_t)total_q, 256);
  w.cand = reinterpret_cast<uint64_t*>(p);
  w.nseg = nseg;
  return w;
}

// ---- register-resident passes shared by the row and segment kernels --------------------------
// A lane holds V scores: element u is at index i0 + 64 u of the row, and it lies inside the row
// (or segment) iff 64 u < rem. Masks are ballots of compares, so the per-element cost is one or
// two vector compares; counting and rank arithmetic are scalar.

__device__ __forceinline__ int lanes_below(uint64_t m) {  // set bits of m below this lane
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Loads v[u] = base[ib + 64 u] for u < V. One buffer resource per group of 16 u (1024 elements)
// keeps every per-load offset in the instruction's 12-bit immediate, so a single address register
// serves all loads; each resource's range is what is left of [0, len) past the group's base, so
// loads past the end return 0 instead of faulting. aux: cache-policy bits.
template <int V>
__device__ __forceinline__ void lane_load(uint32_t (&v)[V], const int32_t* base, int len, int ib,
                                          int aux) {
  const int voff = ib * 4;
#pragma unroll
  for (int g = 0; g < (V + 15) / 16; ++g) {
    const int left = max(0, len - 1024 * g);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(base + 1024 * g), 0, left * 4, 0x00020000);
#pragma unroll
    for (int j = 0; j < 16 && 16 * g + j < V; ++j) {
      if (aux)
        v[16 * g + j] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 256 * j, 0, 1);
      else
        v[16 * g + j] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 256 * j, 0, 0);
    }
  }
}

// The wave's elements at or above thr (wave-uniform): a count per lane on the vector unit, then a
// butterfly over the wave, instead of a ballot and a scalar population count per register.
template <int V>
__device__ __forceinline__ int wave_count_ge(const uint32_t (&v)[V], uint32_t thr) {
  // an opaque copy of the threshold: the compiler would otherwise keep these compares (one
  // register each) alive for the placement pass that repeats them
  uint32_t t = thr;
  asm volatile("" : "+v"(t));
  int c = 0;
#pragma unroll
  for (int u = 0; u < V; ++u) c += v[u] >= t ? 1 : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  return c;
}

// Counts the lane-group's elements above bin b* = [lo, hm1] (returned, wave-uniform) and appends
// the keys of the b* candidates to klo/khi (slots from *nk, at most cap). FULL: no range mask.
template <int V, bool FULL>
__device__ __forceinline__ int pass_gather(const uint32_t (&v)[V], int i0, int rem, uint32_t lo,
                                           uint32_t hm1, uint32_t* klo, uint32_t* khi, int* nk,
                                           int cap) {
  const int lane = threadIdx.x & 63;
  int above = 0;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const uint32_t x = v[u];
    uint64_t ma = __ballot(x > hm1);
    uint64_t mc = __ballot(x >= lo) & ~ma;
    if (!FULL) {
      const uint64_t in = __ballot(64 * u < rem);
      ma &= in;
      mc &= in;
    }
    above += __popcll(ma);
    if (mc) {
      int base = 0;
      if (lane == 0) base = atomicAdd(nk, __popcll(mc));
      base = __builtin_amdgcn_readfirstlane(base);
      if ((mc >> lane) & 1) {
        const int slot = base + lanes_below(mc);
        if (slot < cap) {
          klo[slot] = 0xFFFFFFFFu - (uint32_t)(i0 + 64 * u);
          khi[slot] = x;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one element's masks live at a time (SGPR pressure)
  }
  return above;
}

// Selected iff the key (score, then lower index) is at least the cut key (th, tl); the index
// comparison only matters for elements whose score equals the cut score.
template <bool FULL>
__device__ __forceinline__ uint64_t sel_mask(uint32_t x, int i, int u, int rem, uint32_t th,
                                             uint32_t tl) {
  uint64_t m = __ballot(x > th);
  if (__ballot(x == th)) m |= __ballot((x == th) & (0xFFFFFFFFu - (uint32_t)i >= tl));
  if (!FULL) m &= __ballot(64 * u < rem);
  return m;
}

template <int V, bool FULL>
__device__ __forceinline__ int pass_count(const uint32_t (&v)[V], int i0, int rem, uint32_t th,
                                          uint32_t tl) {
  int c = 0;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    c += __popcll(sel_mask<FULL>(v[u], i0 + 64 * u, u, rem, th, tl));
    __builtin_amdgcn_sched_barrier(0);
  }
  return c;
}

// Writes every selected element's index (and score) at its rank, from `pos` (wave-uniform).
template <int V, bool FULL>
__device__ __forceinline__ void pass_write(const uint32_t (&v)[V], int i0, int rem, uint32_t th,
                                           uint32_t tl, int pos, int top_k, int32_t* oi,
                                           int32_t* os) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int i = i0 + 64 * u;
    const uint64_t m = sel_mask<FULL>(v[u], i, u, rem, th, tl);
    if (m) {
      if ((m >> lane) & 1) {
        const int p = pos + lanes_below(m);
        if (p < top_k) {  // exactly top_k are selected; the guard only bounds the writes
          oi[p] = i;
          if (os) os[p] = (int32_t)v[u];
        }
      }
      pos += __popcll(m);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The cut key inside b*: keys are unique, so the selection is a threshold on the key. When every
// candidate is taken the threshold is the bottom of b*.
__device__ __forceinline__ uint64_t cut_key(uint64_t prefix, uint32_t lo) {
  return max(prefix, (uint64_t)lo << 32);
}

template <bool FB>
__device__ __forceinline__ uint32_t bin_hm1(int b) {  // top score of bin b
  return (uint32_t)min(bin_lo<FB>(b + 1) - 1, (uint64_t)0xFFFFFFFFu);
}

// b* and the count above it from a row's global histogram, 2048 / NT bins per thread in
// registers. Results in out[0] (bin) and out[1] (count above).
template <int NT>
__device__ void hist_cut(const int* __restrict__ gh, int k, int* red, int* out) {
  constexpr int PER = TOPK_BINS / NT;
  static_assert(PER * NT == TOPK_BINS, "bins per thread");
  int h[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) h[j] = gh[topk_hist_slot(threadIdx.x * PER + j)];
  int local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) local += h[j];
  if (threadIdx.x == 0) {
    out[0] = 0;
    out[1] = 0;
  }
  const int incl = block_incl_scan<NT>(local, red);
  const int above = red[NT / 64] - incl;
  if (above < k && above + local >= k) {
    int c = above;
#pragma unroll
    for (int b = PER - 1; b >= 0; --b) {
      if (c + h[b] >= k) {
        out[0] = threadIdx.x * PER + b;
        out[1] = c;
        break;
      }
      c += h[b];
    }
  }
  __syncthreads();
}

// ---- rows of TOPK_LDS_MAX < n <= TOPK_ROW_MAX: one 1024-thread workgroup per row ----------
// For batches with many long rows. Each of the 16 waves owns a contiguous chunk of the row and
// holds it in registers (72 scores per lane). As for the shorter rows, a threshold from a sample
// comes first: one register in eight fills the histogram, the bin of the sample's k_s-th largest
// score bounds the selection from below, two compare-and-ballot passes count and compact the
// candidates in index order, and the exact cut and the ranks are found among them. Without at
// least k candidates that fit the buffer, the row's whole histogram is built in LDS: a pass counts
// the elements above its cut bin b* and gathers the b* candidates, one wave resolves the exact cut,
// the selected candidates are credited to the waves that hold them, and a second pass (reloading
// the chunk, by then in L2) writes every selected index at its rank.
constexpr int NT_R = 1024;
constexpr int NW_R = NT_R / 64;
constexpr int V_R = TOPK_ROW_MAX / NT_R;  // scores per lane
static_assert((64 * V_R) % 512 == 0, "a wave's chunk is a whole number of 512-element blocks");

template <bool FB>
__global__ __launch_bounds__(NT_R) void topk_row_kernel(const Tok* __restrict__ toks,
                                                        const int32_t* __restrict__ scores,
                                                        int top_k, int32_t* __restrict__ idx_out,
                                                        int32_t* __restrict__ score_out) {
  // candidate keys as two planes (low words: ~index, high words: score) so the compiler never
  // pairs a score with an index into a 64-bit register; then the members of the cut bin
  __shared__ uint32_t klo[TOPK_CAND_CAP], khi[TOPK_CAND_CAP];
  __shared__ uint32_t mlo[TOPK_CAND_CAP], mhi[TOPK_CAND_CAP];
  __shared__ int hist[TOPK_BINS];
  __shared__ int hist2[256];
  __shared__ int red[NT_R / 64 + 1];
  __shared__ int cut[2];
  __shared__ uint64_t pm[2];
  __shared__ int nk;
  __shared__ int wsel[NW_R], woff[NW_R], wcnt[NW_R];
  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  if (n <= TOPK_LDS_MAX || n > TOPK_ROW_MAX) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int32_t* row = scores + tk.cand_off;
  const int ib = wv * (64 * V_R) + lane;
  const int rem = n - ib;
  const bool full = n >= (wv + 1) * (64 * V_R);
  int32_t* oi = idx_out + t * top_k;
  int32_t* os = score_out ? score_out + t * top_k : nullptr;
  {
    uint32_t v[V_R];
    lane_load<V_R>(v, row, n, ib, 0);
    for (int i = threadIdx.x; i < TOPK_BINS; i += NT_R) hist[i] = 0;
    if (threadIdx.x == 0) nk = 0;
    __syncthreads();
    // the sample: registers u = 8 j, index i with i mod 512 < 64 (ns of them inside the row; the
    // slots past the row's end read 0 and are taken back out of zero's bin)
    const int ns = 64 * (n / 512) + min(n % 512, 64);
#pragma unroll
    for (int u = 0; u < V_R; u += 8) atomicAdd(&hist[score_bin<FB>(v[u])], 1);
    __syncthreads();
    if (threadIdx.x == 0) hist[score_bin<FB>(0u)] -= NT_R * (V_R / 8) - ns;
    __syncthreads();
    const float kf = (float)top_k * (float)ns / (float)n;
    const int ks = min(ns, (int)ceilf(kf + 4.0f * sqrtf(kf)) + 16);
    find_cut<NT_R>(hist, TOPK_BINS, ks, red, cut);
    const uint32_t thr = (uint32_t)bin_lo<FB>(cut[0]);
    // loads past the row's end read 0: with thr > 0 no such element is a candidate
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < V_R; ++u) {
      cnt += __popcll(__ballot(v[u] >= thr));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (lane == 0) wcnt[wv] = cnt;
    __syncthreads();
    int nc = 0, off = 0;
#pragma unroll
    for (int w = 0; w < NW_R; ++w) {
      off += w < wv ? wcnt[w] : 0;
      nc += wcnt[w];
    }
    if (thr > 0 && nc >= top_k && nc <= TOPK_CAND_CAP) {  // uniform
      const uint64_t below_lane = (1ull << lane) - 1ull;
#pragma unroll
      for (int u = 0; u < V_R; ++u) {
        const uint32_t x = v[u];
        const bool c = x >= thr;
        const uint64_t mc = __ballot(c);
        if (mc) {
          if (c) {
            const int slot = off + __popcll(mc & below_lane);
            klo[slot] = 0xFFFFFFFFu - (uint32_t)(ib + 64 * u);
            khi[slot] = x;
          }
          off += __popcll(mc);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int i = threadIdx.x; i < TOPK_BINS; i += NT_R) hist[i] = 0;
      __syncthreads();
      for (int c = threadIdx.x; c < nc; c += NT_R) atomicAdd(&hist[score_bin<FB>(khi[c])], 1);
      __syncthreads();
      find_cut<NT_R>(hist, TOPK_BINS, top_k, red, cut);
      const int bstar = cut[0];
      const int need = top_k - cut[1];
      const uint32_t lo = (uint32_t)bin_lo<FB>(bstar);
      for (int c = threadIdx.x; c < nc; c += NT_R) {
        const uint32_t x = khi[c];
        if (score_bin<FB>(x) == bstar) {
          const int m = atomicAdd(&nk, 1);
          mlo[m] = klo[c];
          mhi[m] = x;
        }
      }
      __syncthreads();
      if (wv == 0) {
        uint64_t pf, mk;
        wave_radix_cut([&](int i) { return ((uint64_t)mhi[i] << 32) | mlo[i]; }, nk, need, hist2,
                       &pf, &mk);
        if (lane == 0) pm[0] = cut_key(pf, lo);
        (void)mk;
      }
      __syncthreads();
      const uint64_t ck = pm[0];
      const int per = (nc + NT_R - 1) / NT_R;
      const int c0 = min(nc, (int)threadIdx.x * per), c1 = min(nc, c0 + per);
      int sc = 0;
      for (int c = c0; c < c1; ++c) sc += (((uint64_t)khi[c] << 32) | klo[c]) >= ck;
      int pos = block_incl_scan<NT_R>(sc, red) - sc;
      for (int c = c0; c < c1; ++c) {
        const uint32_t x = khi[c], l = klo[c];
        if ((((uint64_t)x << 32) | l) >= ck && pos < top_k) {
          oi[pos] = (int32_t)(0xFFFFFFFFu - l);
          if (os) os[pos] = (int32_t)x;
          ++pos;
        }
      }
      return;
    }
    // the row's whole histogram; the slots past the row's end read 0 and are taken back out of
    // zero's bin, so no per-element range mask is needed
    for (int i = threadIdx.x; i < TOPK_BINS; i += NT_R) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < V_R; ++u) atomicAdd(&hist[score_bin<FB>(v[u])], 1);
    __syncthreads();
    if (threadIdx.x == 0) hist[score_bin<FB>(0u)] -= NT_R * V_R - n;
    __syncthreads();
    find_cut<NT_R>(hist, TOPK_BINS, top_k, red, cut);
  }
  const int bstar = cut[0];
  const int need = top_k - cut[1];
  const uint32_t lo = (uint32_t)bin_lo<FB>(bstar);
  {
    uint32_t v[V_R];
    lane_load<V_R>(v, row, n, ib, 1);  // glc: a distinct load the compiler cannot merge with the first
    const uint32_t hm1 = bin_hm1<FB>(bstar);
    const int above = full ? pass_gather<V_R, true>(v, ib, rem, lo, hm1, klo, khi, &nk, TOPK_CAND_CAP)
                           : pass_gather<V_R, false>(v, ib, rem, lo, hm1, klo, khi, &nk, TOPK_CAND_CAP);
    if (lane == 0) wsel[wv] = above;
  }
  __syncthreads();

  const int ncand = nk;
  if (ncand <= TOPK_CAND_CAP) {
    // pass 2's loads go out before the cut so their latency hides behind it
    uint32_t v[V_R];
    lane_load<V_R>(v, row, n, ib, 1);
    if (wv == 0) {
      uint64_t pf, mk;
      wave_radix_cut([&](int i) { return ((uint64_t)khi[i] << 32) | klo[i]; }, ncand, need, hist2,
                     &pf, &mk);
      if (lane == 0) pm[0] = cut_key(pf, lo);
      (void)mk;
    }
    __syncthreads();
    const uint64_t ck = pm[0];
    // selected candidates per owning wave (the index says which wave holds the score)
    for (int c = threadIdx.x; c < ncand; c += NT_R) {
      const uint64_t key = ((uint64_t)khi[c] << 32) | klo[c];
      if (key >= ck) atomicAdd(&wsel[(int)(0xFFFFFFFFu - klo[c]) / (64 * V_R)], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int acc = 0;
      for (int w = 0; w < NW_R; ++w) {
        woff[w] = acc;
        acc += wsel[w];
      }
    }
    __syncthreads();
    const uint32_t th = (uint32_t)(ck >> 32), tl = (uint32_t)ck;
    const int pos = __builtin_amdgcn_readfirstlane(woff[wv]);
    if (full)
      pass_write<V_R, true>(v, ib, rem, th, tl, pos, top_k, oi, os);
    else
      pass_write<V_R, false>(v, ib, rem, th, tl, pos, top_k, oi, os);
    return;
  }
  // more candidates than LDS holds (heavy ties): cut and emit straight from the score row
  radix_cut<NT_R>(
      n, need, [&](int i) { return sel_key(row[i], i); },
      [&](int i) { return score_bin<FB>((uint32_t)row[i]) == bstar; }, hist2, red, cut, pm);
  const uint64_t ck = cut_key(pm[0], lo);
  const uint32_t th = (uint32_t)(ck >> 32), tl = (uint32_t)ck;
  const int c0 = wv * (64 * V_R);
  const int c1 = min(n, c0 + 64 * V_R);
  int cp = 0;
  for (int i = c0 + lane; i < c1; i += 64) {
    const uint32_t x = (uint32_t)row[i];
    cp += x > th || (x == th && 0xFFFFFFFFu - (uint32_t)i >= tl);
  }
  for (int d = 32; d > 0; d >>= 1) cp += __shfl_xor(cp, d);
  if (lane == 0) wsel[wv] = cp;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < NW_R; ++w) {
      woff[w] = acc;
      acc += wsel[w];
    }
  }
  __syncthreads();
  int pos = woff[wv];
  for (int b0 = c0; b0 < c1; b0 += 64) {
    const int i = b0 + lane;
    const uint32_t x = i < c1 ? (uint32_t)row[i] : 0u;
    const bool f = i < c1 && (x > th || (x == th && 0xFFFFFFFFu - (uint32_t)i >= tl));
    const uint64_t m = __ballot(f);
    if (f) {
      const int p = pos + lanes_below(m);
      if (p < top_k) {
        oi[p] = i;
        if (os) os[p] = (int32_t)x;
      }
    }
    pos += __popcll(m);
  }
}

// ---- rows of top_k < n <= TOPK_LDS_MAX: one 512-thread workgroup per row, in registers -------
// Each of the 8 waves owns a contiguous chunk of 64 V scores of the row (V = 8, 16, 32 or 64, the
// smallest that covers the row), held in registers; the score histogram is built in LDS from
// them; then one pass counts the elements above b* and gathers the b* candidates, each wave into
// its own slice of the candidate buffer (a wave-uniform counter, no atomics); one wave finds the
// exact cut among them, every wave counts its selected candidates, and a second pass over the
// registers writes every selected index at its rank. The writes are branch-free buffer
// stores whose offsets fall outside the output row unless the element is selected. 41 KB of
// LDS, so two rows share a CU and hide each other's latencies.
constexpr int NT_B = 512;
constexpr int NW_B = NT_B / 64;
constexpr int CAND_W = TOPK_CAND_CAP / NW_B;  // candidate slots per wave

template <bool FB, int V>
__device__ __forceinline__ void topk_short_row(const int32_t* __restrict__ row, int n, int top_k,
                                               int32_t* __restrict__ oi, int32_t* __restrict__ os,
                                               int* hist, uint32_t (*whist)[TOPK_BINS / 2],
                                               uint32_t* klo, uint32_t* khi,
                                               int* hist2, int* red, int* cut, uint64_t* pm,
                                               int* wcnt, int* wsel, int* woff) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ib = wv * (64 * V) + lane;
  const int rem = n - ib;  // this lane's element u is in the row iff 64 u < rem
  uint32_t v[V];
  lane_load<V>(v, row, n, ib, 0);
  {  // this wave's histogram: 16-bit counts, two bins per word (a wave holds at most 4,096)
    uint4* wz = reinterpret_cast<uint4*>(whist[wv]);
#pragma unroll
    for (int i = lane; i < TOPK_BINS / 8; i += 64) wz[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int u = 0; u < V; ++u)
    if (64 * u < rem) {
      const int b = score_bin<FB>(v[u]);
      atomicAdd(&whist[wv][b >> 1], 1u << (16 * (b & 1)));
    }
  __syncthreads();
  {  // the row's histogram: thread t sums bins 4t .. 4t + 3 over the waves
    uint32_t s01 = 0, s23 = 0;  // two packed 16-bit sums each (a row holds at most 32,768)
#pragma unroll
    for (int w = 0; w < NW_B; ++w) {
      const uint2 p = reinterpret_cast<const uint2*>(whist[w])[threadIdx.x];
      s01 += p.x;
      s23 += p.y;
    }
    reinterpret_cast<int4*>(hist)[threadIdx.x] =
        make_int4((int)(s01 & 0xFFFFu), (int)(s01 >> 16), (int)(s23 & 0xFFFFu), (int)(s23 >> 16));
  }
  __syncthreads();
  find_cut<NT_B>(hist, TOPK_BINS, top_k, red, cut);
  const int bstar = cut[0];
  const int need = top_k - cut[1];
  const uint32_t lo = (uint32_t)bin_lo<FB>(bstar);
  const uint32_t hm1 = bin_hm1<FB>(bstar);
  // this wave's elements above b*: its histogram's bins past b* (lane: bins 32 lane .. +31)
  int above = 0;
  {
    const uint4* wq = reinterpret_cast<const uint4*>(whist[wv]) + 4 * lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 q = wq[k];
      const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b0 = 32 * lane + 8 * k + 2 * e;
        above += (b0 > bstar ? (int)(wd[e] & 0xFFFFu) : 0) + (b0 + 1 > bstar ? (int)(wd[e] >> 16) : 0);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) above += __shfl_xor(above, o);
  }
  // gather the b* candidates into this wave's slice
  const uint64_t below_lane = (1ull << lane) - 1ull;
  const uint32_t span = hm1 - lo;
  int nc = 0;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const uint32_t x = v[u];
    const bool c = 64 * u < rem && x - lo <= span;
    const uint64_t mc = __ballot(c);
    if (mc) {  // rare: the b* candidates go to this wave's slice, a wave-uniform count ahead
      const int slot = nc + __popcll(mc & below_lane);
      if (c && slot < CAND_W) {
        klo[wv * CAND_W + slot] = 0xFFFFFFFFu - (uint32_t)(ib + 64 * u);
        khi[wv * CAND_W + slot] = x;
      }
      nc += __popcll(mc);
    }
    __builtin_amdgcn_sched_barrier(0);  // one element's masks live at a time (SGPR pressure)
  }
  if (lane == 0) {
    wcnt[wv] = nc;
    wsel[wv] = above;
  }
  __syncthreads();
  int ncand = 0;
  bool overflow = false;
#pragma unroll
  for (int w = 0; w < NW_B; ++w) {
    ncand += wcnt[w];
    overflow |= wcnt[w] > CAND_W;
  }
  uint64_t ck;
  if (!overflow) {
    if (wv == 0) {  // candidate i lives in the slice of the wave whose running count passes i
      uint64_t pf, mk;
      wave_radix_cut(
          [&](int i) {
            int w = 0, base = 0;
#pragma unroll
            for (int k = 0; k < NW_B - 1; ++k) {
              const bool past = i >= base + wcnt[w];
              base += past ? wcnt[w] : 0;
              w += past;
            }
            const int sl = w * CAND_W + (i - base);
            return ((uint64_t)khi[sl] << 32) | klo[sl];
          },
          ncand, need, hist2, &pf, &mk);
      if (lane == 0) pm[0] = cut_key(pf, lo);
      (void)mk;
    }
    __syncthreads();
    ck = pm[0];
    // every wave counts its selected candidates
    int sc = 0;
    for (int c0 = 0; c0 < nc; c0 += 64) {
      const int sl = wv * CAND_W + c0 + lane;
      const bool f = c0 + lane < nc && (((uint64_t)khi[sl] << 32) | klo[sl]) >= ck;
      sc += __popcll(__ballot(f));
    }
    if (lane == 0) wsel[wv] += sc;
  } else {
    // more candidates than a wave's slice holds (heavy ties): the exact cut by radix select over
    // the row, then every wave counts its own selected elements
    radix_cut<NT_B>(
        n, need, [&](int i) { return sel_key(row[i], i); },
        [&](int i) { return score_bin<FB>((uint32_t)row[i]) == bstar; }, hist2, red, cut, pm);
    ck = cut_key(pm[0], lo);
    const uint32_t th = (uint32_t)(ck >> 32), tl = (uint32_t)ck;
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const uint32_t x = v[u];
      const bool f = 64 * u < rem && (x > th || (x == th && 0xFFFFFFFFu - (uint32_t)(ib + 64 * u) >= tl));
      cnt += __popcll(__ballot(f));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (lane == 0) wsel[wv] = cnt;
  }
  __syncthreads();
  int pos = 0;
#pragma unroll
  for (int w = 0; w < NW_B; ++w) pos += w < wv ? wsel[w] : 0;
  // write: each selected element's index (and score) at its rank; other lanes' offsets fall
  // outside the row's range and the hardware drops those stores
  const uint32_t th = (uint32_t)(ck >> 32), tl = (uint32_t)ck;
  const __amdgpu_buffer_rsrc_t rs_i = __builtin_amdgcn_make_buffer_rsrc(oi, 0, top_k * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_s =
      __builtin_amdgcn_make_buffer_rsrc(os ? os : oi, 0, os ? top_k * 4 : 0, 0x00020000);
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const uint32_t x = v[u];
    const int i = ib + 64 * u;
    const bool f = 64 * u < rem && (x > th || (x == th && 0xFFFFFFFFu - (uint32_t)i >= tl));
    const uint64_t m = __ballot(f);
    const int p = pos + __popcll(m & below_lane);
    const int off = f && p < top_k ? 4 * p : 0x7FFFFFF0;
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)i, rs_i, off, 0, 0);
    if (os) __builtin_amdgcn_raw_buffer_store_b32(x, rs_s, off, 0, 0);
    pos += __popcll(m);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Rows of more than 8 NT_B candidates with k <= n / 2 first try a threshold taken from a sample: the
// elements of one register in eight (index i with i mod 512 < 64, about n / 8 of them) fill the
// histogram, and the bin of the sample's k_s-th largest score, k_s = k f + 4 sqrt(k f) + 16 with
// f the sampled fraction, bounds the selection from below. A count per lane finds how many
// elements lie at or above that bin's lowest score, a ballot pass writes them to LDS in index order
// (about 2,700 for k = 2,048), and the exact cut and the ranks are then found among those
// candidates only, so the histogram atomics and the rank pass no longer touch every element.
// Every element outside the candidates scores below every candidate, so the k largest keys are
// among them whenever there are at least k. With fewer than k, or more than the buffer holds
// (heavy ties), the row returns false and the full-row path runs instead; the result is exact
// either way.
template <bool FB, int V>
__device__ __forceinline__ bool topk_short_row_sampled(const int32_t* __restrict__ row, int n,
                                                       int top_k, int32_t* __restrict__ oi,
                                                       int32_t* __restrict__ os, int* hist,
                                                       uint32_t (*whist)[TOPK_BINS / 2],
                                                       uint32_t* klo, uint32_t* khi, int* hist2,
                                                       int* red, int* cut, uint64_t* pm, int* wcnt,
                                                       int* wsel) {
  static_assert(V >= 16 && V % 8 == 0, "a wave's chunk is a multiple of 1,024 elements");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ib = wv * (64 * V) + lane;
  const int rem = n - ib;  // this lane's element u is in the row iff 64 u < rem
  uint32_t v[V];
  lane_load<V>(v, row, n, ib, 0);
  {  // this wave's histogram of its sampled registers (at most 64 V / 8 per wave: 16-bit counts)
    uint4* wz = reinterpret_cast<uint4*>(whist[wv]);
#pragma unroll
    for (int i = lane; i < TOPK_BINS / 8; i += 64) wz[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int u = 0; u < V; u += 8)
    if (64 * u < rem) {
      const int b = score_bin<FB>(v[u]);
      atomicAdd(&whist[wv][b >> 1], 1u << (16 * (b & 1)));
    }
  __syncthreads();
  {  // the sample's histogram: thread t sums bins 4t .. 4t + 3 over the waves
    uint32_t s01 = 0, s23 = 0;
#pragma unroll
    for (int w = 0; w < NW_B; ++w) {
      const uint2 q = reinterpret_cast<const uint2*>(whist[w])[threadIdx.x];
      s01 += q.x;
      s23 += q.y;
    }
    reinterpret_cast<int4*>(hist)[threadIdx.x] =
        make_int4((int)(s01 & 0xFFFFu), (int)(s01 >> 16), (int)(s23 & 0xFFFFu), (int)(s23 >> 16));
  }
  __syncthreads();
  // sampled elements: index i < n with i mod 512 < 64 (a wave's chunk starts at a multiple of
  // 1,024, and register u = 8 j adds 512 j)
  const int ns = 64 * (n / 512) + min(n % 512, 64);
  const float kf = (float)top_k * (float)ns / (float)n;
  const int ks = min(ns, (int)ceilf(kf + 4.0f * sqrtf(kf)) + 16);
  find_cut<NT_B>(hist, TOPK_BINS, ks, red, cut);
  const uint32_t thr = (uint32_t)bin_lo<FB>(cut[0]);
  // count the candidates (score >= thr), then place them in index order: wave w's after those of
  // the waves before it. Loads past the row's end returned 0, so with thr > 0 no element outside
  // the row is ever a candidate and the passes need no range mask (thr == 0: the full-row path).
  const int cnt = wave_count_ge<V>(v, thr);
  if (lane == 0) wcnt[wv] = cnt;
  __syncthreads();
  int nc = 0, off = 0;
#pragma unroll
  for (int w = 0; w < NW_B; ++w) {
    off += w < wv ? wcnt[w] : 0;
    nc += wcnt[w];
  }
  if (thr == 0 || nc < top_k || nc > TOPK_CAND_CAP) {  // uniform: the full-row path takes the row
    __syncthreads();
    return false;
  }
  const uint64_t below_lane = (1ull << lane) - 1ull;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const uint32_t x = v[u];
    const bool c = x >= thr;
    const uint64_t mc = __ballot(c);
    if (mc) {
      if (c) {
        const int slot = off + __popcll(mc & below_lane);
        klo[slot] = 0xFFFFFFFFu - (uint32_t)(ib + 64 * u);
        khi[slot] = x;
      }
      off += __popcll(mc);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // the candidates' histogram, exact this time
  for (int i = threadIdx.x; i < TOPK_BINS; i += NT_B) hist[i] = 0;
  if (threadIdx.x == 0) wsel[0] = 0;
  __syncthreads();
  for (int c = threadIdx.x; c < nc; c += NT_B) atomicAdd(&hist[score_bin<FB>(khi[c])], 1);
  __syncthreads();
  find_cut<NT_B>(hist, TOPK_BINS, top_k, red, cut);
  const int bstar = cut[0];
  const int need = top_k - cut[1];
  const uint32_t lo = (uint32_t)bin_lo<FB>(bstar);
  // b*'s members (keys) into the sample histograms' space, which is free now
  uint32_t* mlo = &whist[0][0];
  uint32_t* mhi = mlo + TOPK_CAND_CAP;
  static_assert(2 * TOPK_CAND_CAP <= NW_B * (TOPK_BINS / 2), "member keys fit the histograms");
  for (int c = threadIdx.x; c < nc; c += NT_B) {
    const uint32_t x = khi[c];
    if (score_bin<FB>(x) == bstar) {
      const int m = atomicAdd(&wsel[0], 1);
      mlo[m] = klo[c];
      mhi[m] = x;
    }
  }
  __syncthreads();
  if (wv == 0) {
    uint64_t pf, mk;
    wave_radix_cut([&](int i) { return ((uint64_t)mhi[i] << 32) | mlo[i]; }, wsel[0], need, hist2,
                   &pf, &mk);
    if (lane == 0) pm[0] = cut_key(pf, lo);
    (void)mk;
  }
  __syncthreads();
  const uint64_t ck = pm[0];
  // ranks: thread t takes a run of consecutive candidates, so a block scan of its count of
  // selected ones gives its first output position
  const int per = (nc + NT_B - 1) / NT_B;
  const int c0 = min(nc, (int)threadIdx.x * per), c1 = min(nc, c0 + per);
  int sc = 0;
  for (int c = c0; c < c1; ++c) sc += (((uint64_t)khi[c] << 32) | klo[c]) >= ck;
  int pos = block_incl_scan<NT_B>(sc, red) - sc;
  for (int c = c0; c < c1; ++c) {
    const uint32_t x = khi[c], l = klo[c];
    if ((((uint64_t)x << 32) | l) >= ck && pos < top_k) {
      oi[pos] = (int32_t)(0xFFFFFFFFu - l);
      if (os) os[pos] = (int32_t)x;
      ++pos;
    }
  }
  return true;
}

template <bool FB>
__global__ __launch_bounds__(NT_B, 4) void topk_short_kernel(const Tok* __restrict__ toks,
                                                          const int32_t* __restrict__ scores,
                                                          int top_k, int32_t* __restrict__ idx_out,
                                                          int32_t* __restrict__ score_out,
                                                          int32_t pad_score) {
  __shared__ __align__(16) int hist[TOPK_BINS];
  __shared__ __align__(16) uint32_t whist[NW_B][TOPK_BINS / 2];  // per-wave packed histograms
  __shared__ uint32_t klo[TOPK_CAND_CAP], khi[TOPK_CAND_CAP];
  __shared__ int hist2[256];
  __shared__ int red[NW_B + 1];
  __shared__ int cut[2];
  __shared__ uint64_t pm[2];
  __shared__ int wcnt[NW_B], wsel[NW_B], woff[NW_B];
  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  if (n > TOPK_LDS_MAX) return;
  int32_t* oi = idx_out + t * top_k;
  int32_t* os = score_out ? score_out + t * top_k : nullptr;
  const int32_t* row = scores + tk.cand_off;
  if (n <= top_k) {  // every row is taken, in order
    for (int j = threadIdx.x; j < top_k; j += NT_B) {
      oi[j] = j < n ? j : -1;
      if (os) os[j] = j < n ? row[j] : pad_score;
    }
    return;
  }
  static_assert(NT_B * 64 == TOPK_LDS_MAX, "8 waves x 64 x 64 scores cover the longest short row");
  // rows of more than 8 NT_B candidates with k at most half the row try the sampled threshold
  // first (for k = 2,048 it admits about 2,700 candidates, which the buffer holds)
  const bool sample = top_k * 2 <= n && n > NT_B * 8;
  if (n <= NT_B * 8)
    topk_short_row<FB, 8>(row, n, top_k, oi, os, hist, whist, klo, khi, hist2, red, cut, pm, wcnt, wsel, woff);
  else if (n <= NT_B * 16) {
    if (!sample || !topk_short_row_sampled<FB, 16>(row, n, top_k, oi, os, hist, whist, klo, khi, hist2, red, cut, pm, wcnt, wsel))
      topk_short_row<FB, 16>(row, n, top_k, oi, os, hist, whist, klo, khi, hist2, red, cut, pm, wcnt, wsel, woff);
  } else if (n <= NT_B * 32) {
    if (!sample || !topk_short_row_sampled<FB, 32>(row, n, top_k, oi, os, hist, whist, klo, khi, hist2, red, cut, pm, wcnt, wsel))
      topk_short_row<FB, 32>(row, n, top_k, oi, os, hist, whist, klo, khi, hist2, red, cut, pm, wcnt, wsel, woff);
  } else {
    if (!sample || !topk_short_row_sampled<FB, 64>(row, n, top_k, oi, os, hist, whist, klo, khi, hist2, red, cut, pm, wcnt, wsel))
      topk_short_row<FB, 64>(row, n, top_k, oi, os, hist, whist, klo, khi, hist2, red, cut, pm, wcnt, wsel, woff);
  }
}

// ---- segmented rows: count / resolve / emit over TOPK_SEG-candidate segments ---------------
// For rows longer than TOPK_ROW_MAX, and for every row longer than TOPK_LDS_MAX when the batch has
// few query tokens (one workgroup per row would leave most of the chip idle). Kernel boundaries
// order the three kernels; no workgroup waits on another.
//  count   (segment x row): b* from the row's histogram; the segment's elements above b* and its
//          b* candidates (gathered in LDS, then appended to the row's candidate buffer with one
//          atomic per workgroup).
//  resolve (row): the exact cut key among the candidates (or, when they overflowed the buffer,
//          by radix select over the row) and each segment's output offset; clears the row's
//          histogram and candidate counter for the next call.
//  emit    (segment x row): counts per wave, then writes each selected index at its rank.
constexpr int NT_S = 256;
constexpr int V_S = TOPK_SEG / NT_S;  // 16 per lane: wave w owns [1024 w, 1024 (w + 1))
static_assert(V_S == 16, "one buffer resource per segment");

template <bool FB>
__global__ __launch_bounds__(NT_S) void topk_seg_count_kernel(const Tok* __restrict__ toks,
                                                              const int32_t* __restrict__ scores,
                                                              int top_k, int seg_min_n,
                                                              TopkWs ws) {
  __shared__ uint32_t klo[TOPK_SEG], khi[TOPK_SEG];
  __shared__ int red[NT_S / 64 + 1];
  __shared__ int cut[2];
  __shared__ int nk, gbase;
  __shared__ int wab[NT_S / 64];
  const int64_t t = blockIdx.y;
  const int g = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  const int s0 = g * TOPK_SEG;
  if (n <= seg_min_n || s0 >= n) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int len = min(n - s0, TOPK_SEG);
  const int ib = wv * (64 * V_S) + lane;
  const int rem = len - ib;
  const bool full = len >= (wv + 1) * (64 * V_S);
  uint32_t v[V_S];
  lane_load<V_S>(v, scores + tk.cand_off + s0, len, ib, 0);
  if (threadIdx.x == 0) nk = 0;
  hist_cut<NT_S>(ws.hist + t * TOPK_BINS, top_k, red, cut);
  const int bstar = cut[0];
  const uint32_t lo = (uint32_t)bin_lo<FB>(bstar), hm1 = bin_hm1<FB>(bstar);
  const int above = full ? pass_gather<V_S, true>(v, s0 + ib, rem, lo, hm1, klo, khi, &nk, TOPK_SEG)
                         : pass_gather<V_S, false>(v, s0 + ib, rem, lo, hm1, klo, khi, &nk, TOPK_SEG);
  if (lane == 0) wab[wv] = above;
  __syncthreads();
  int* rec = ws.rec + t * TOPK_REC;
  if (threadIdx.x == 0) {
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NT_S / 64; ++w) tot += wab[w];
    ws.seg[t * ws.nseg + g] = tot;
    gbase = nk ? atomicAdd(&rec[0], nk) : 0;
    if (g == 0) {
      rec[1] = bstar;
      rec[2] = cut[1];
    }
  }
  __syncthreads();
  const int nl = nk, base = gbase;
  uint64_t* cand = ws.cand + t * TOPK_CAND_CAP;
  for (int i = threadIdx.x; i < nl && base + i < TOPK_CAND_CAP; i += NT_S)
    cand[base + i] = ((uint64_t)khi[i] << 32) | klo[i];
}

template <bool FB>
__global__ __launch_bounds__(NT_R) void topk_seg_resolve_kernel(const Tok* __restrict__ toks,
                                                                const int32_t* __restrict__ scores,
                                                                int top_k, int seg_min_n,
                                                                TopkWs ws) {
  __shared__ uint32_t klo[TOPK_CAND_CAP], khi[TOPK_CAND_CAP];
  __shared__ int segc[TOPK_SEG_MAX];
  __shared__ int hist2[256];
  __shared__ int red[NT_R / 64 + 1];
  __shared__ int cut[2];
  __shared__ uint64_t pm[2];
  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  if (n <= seg_min_n) return;
  const int nseg_t = (n + TOPK_SEG - 1) / TOPK_SEG;
  int* rec = ws.rec + t * TOPK_REC;
  int* segv = ws.seg + t * ws.nseg;
  // every candidate slot goes out together with the row record (slots past the count hold stale
  // keys and are dropped below), so the count costs no round trip of its own
  const uint64_t* cand = ws.cand + t * TOPK_CAND_CAP;
  constexpr int CPT = TOPK_CAND_CAP / NT_R;
  uint64_t kc[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) kc[u] = cand[u * NT_R + threadIdx.x];
  const int sv0 = (int)threadIdx.x < nseg_t ? segv[threadIdx.x] : 0;  // elements above b*
  const int ncand = rec[0];
  const int bstar = rec[1];
  const int need = top_k - rec[2];
  const uint32_t lo = (uint32_t)bin_lo<FB>(bstar);
  if ((int)threadIdx.x < nseg_t) segc[threadIdx.x] = sv0;
  for (int g = threadIdx.x + NT_R; g < nseg_t; g += NT_R) segc[g] = segv[g];
  uint64_t ck;
  if (ncand <= TOPK_CAND_CAP) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int i = u * NT_R + threadIdx.x;
      if (i < ncand) {
        klo[i] = (uint32_t)kc[u];
        khi[i] = (uint32_t)(kc[u] >> 32);
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      uint64_t pf, mk;
      wave_radix_cut([&](int i) { return ((uint64_t)khi[i] << 32) | klo[i]; }, ncand, need, hist2,
                     &pf, &mk);
      if (threadIdx.x == 0) pm[0] = cut_key(pf, lo);
      (void)mk;
    }
    __syncthreads();
    ck = pm[0];
    for (int i = threadIdx.x; i < ncand; i += NT_R) {
      const uint64_t key = ((uint64_t)khi[i] << 32) | klo[i];
      if (key >= ck) atomicAdd(&segc[(int)(0xFFFFFFFFu - klo[i]) / TOPK_SEG], 1);
    }
  } else {
    // more candidates than the buffer holds (heavy ties): cut straight from the score row
    const int32_t* row = scores + tk.cand_off;
    radix_cut<NT_R>(
        n, need, [&](int i) { return sel_key(row[i], i); },
        [&](int i) { return score_bin<FB>((uint32_t)row[i]) == bstar; }, hist2, red, cut, pm);
    ck = cut_key(pm[0], lo);
    for (int i = threadIdx.x; i < n; i += NT_R) {
      const uint32_t x = (uint32_t)row[i];
      if (x >= lo && sel_key((int32_t)x, i) >= ck && score_bin<FB>(x) == bstar)
        atomicAdd(&segc[i / TOPK_SEG], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the per-segment counts -> output offsets (one wave when they fit)
  if (nseg_t <= 64) {
    if (threadIdx.x < 64) {
      const int v = threadIdx.x < nseg_t ? segc[threadIdx.x] : 0;
      int incl = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d);
        if ((int)threadIdx.x >= d) incl += u;
      }
      if ((int)threadIdx.x < nseg_t) segv[threadIdx.x] = incl - v;
    }
  } else {
    int carry = 0;
    for (int c0 = 0; c0 < nseg_t; c0 += NT_R) {
      const int c = c0 + threadIdx.x;
      const int v = c < nseg_t ? segc[c] : 0;
      const int incl = block_incl_scan<NT_R>(v, red);
      const int tot = red[NT_R / 64];
      if (c < nseg_t) segv[c] = carry + incl - v;
      carry += tot;
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    rec[0] = 0;  // the candidate counter starts the next call at zero
    rec[4] = (int)(uint32_t)ck;
    rec[5] = (int)(uint32_t)(ck >> 32);
  }
  int* gh = ws.hist + t * TOPK_BINS;
  for (int i = threadIdx.x; i < TOPK_BINS; i += NT_R) gh[i] = 0;
}

__global__ __launch_bounds__(NT_S) void topk_seg_emit_kernel(const Tok* __restrict__ toks,
                                                             const int32_t* __restrict__ scores,
                                                             int top_k, int seg_min_n, TopkWs ws,
                                                             int32_t* __restrict__ idx_out,
                                                             int32_t* __restrict__ score_out) {
  __shared__ int wc[NT_S / 64];
  const int64_t t = blockIdx.y;
  const int g = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  const int s0 = g * TOPK_SEG;
  if (n <= seg_min_n || s0 >= n) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int len = min(n - s0, TOPK_SEG);
  const int ib = wv * (64 * V_S) + lane;
  const int rem = len - ib;
  const bool full = len >= (wv + 1) * (64 * V_S);
  uint32_t v[V_S];
  lane_load<V_S>(v, scores + tk.cand_off + s0, len, ib, 0);
  const int* rec = ws.rec + t * TOPK_REC;
  const uint32_t tl = (uint32_t)rec[4], th = (uint32_t)rec[5];
  const int off = ws.seg[t * ws.nseg + g];
  const int cnt = full ? pass_count<V_S, true>(v, s0 + ib, rem, th, tl)
                       : pass_count<V_S, false>(v, s0 + ib, rem, th, tl);
  if (lane == 0) wc[wv] = cnt;
  __syncthreads();
  int pos = off;
  for (int w = 0; w < wv; ++w) pos += wc[w];
  pos = __builtin_amdgcn_readfirstlane(pos);
  int32_t* oi = idx_out + t * top_k;
  int32_t* os = score_out ? score_out + t * top_k : nullptr;
  if (full)
    pass_write<V_S, true>(v, s0 + ib, rem, th, tl, pos, top_k, oi, os);
  else
    pass_write<V_S, false>(v, s0 + ib, rem, th, tl, pos, top_k, oi, os);
}

}  // namespace

int64_t topk_nseg(const smla_batch& b) { return (b.max_kv + TOPK_SEG - 1) / TOPK_SEG; }

size_t topk_workspace_bytes(const smla_batch& b, int32_t /*top_k*/) {
  if (b.max_kv <= TOPK_LDS_MAX) return 0;
  const size_t tq = (size_t)b.total_q;
  return align_up(sizeof(int) * TOPK_BINS * tq, 256) + align_up(sizeof(int) * TOPK_REC * tq, 256) +
         align_up(sizeof(int) * (size_t)topk_nseg(b) * tq, 256) +
         align_up(sizeof(uint64_t) * TOPK_CAND_CAP * tq, 256);
}

TopkWs topk_workspace(const smla_batch& b, void* ws) {
  if (b.max_kv <= TOPK_LDS_MAX || !ws) return TopkWs{};
  return topk_ws(ws, b.total_q, topk_nseg(b));
}

namespace {

template <bool FB>
hipError_t launch_topk_t(const smla_batch& b, const int32_t* scores, int32_t top_k, int32_t* idx,
                         int32_t* score, const TopkWs& w, hipStream_t s) {
  TableView tv = table_view(b.table, b.batch, b.total_q);
  const int32_t pad = FB ? (int32_t)0xBF800000u : -1;  // -1.0f or -1
  hipError_t e = hipSuccess;
  if (b.min_cand <= TOPK_LDS_MAX) {
    hipLaunchKernelGGL(topk_short_kernel<FB>, dim3(b.total_q), dim3(NT_B), 0, s, tv.tok, scores,
                       top_k, idx, score, pad);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (b.max_kv <= TOPK_LDS_MAX) return e;
  // few query tokens: every long row goes through the segment kernels, which spread a row over
  // many workgroups; otherwise one workgroup per row up to TOPK_ROW_MAX
  const bool seg_all = b.total_q <= TOPK_SEG_ALL_MAX_Q;
  const int seg_min_n = seg_all ? TOPK_LDS_MAX : TOPK_ROW_MAX;
  if (!seg_all) {
    hipLaunchKernelGGL(topk_row_kernel<FB>, dim3(b.total_q), dim3(NT_R), 0, s, tv.tok, scores, top_k,
                       idx, score);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (b.max_kv <= seg_min_n) return e;
  const unsigned nseg = (unsigned)topk_nseg(b);
  hipLaunchKernelGGL(topk_seg_count_kernel<FB>, dim3(nseg, b.total_q), dim3(NT_S), 0, s, tv.tok,
                     scores, top_k, seg_min_n, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_seg_resolve_kernel<FB>, dim3(b.total_q), dim3(NT_R), 0, s, tv.tok, scores,
                     top_k, seg_min_n, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_seg_emit_kernel, dim3(nseg, b.total_q), dim3(NT_S), 0, s, tv.tok, scores,
                     top_k, seg_min_n, w, idx, score);
  return hipGetLastError();
}

}  // namespace

size_t topk_merge_lds_bytes() {
  return 2 * sizeof(uint64_t) * (TOPK_MAX_K + 1) + sizeof(int32_t) * MERGE_MAX_CAND +
         sizeof(int) * (TOPK_BINS + 1) + sizeof(uint32_t) * MERGE_WORDS + sizeof(int) * (MERGE_WORDS + 1);
}

hipError_t launch_topk_merge(int32_t total_q, int32_t n_lists, int32_t k_in, const int32_t* idx_lists,
                             const int32_t* score_lists, int64_t list_stride, int32_t top_k,
                             int32_t* idx, int32_t* score, int32_t* local_idx, bool fscores,
                             hipStream_t s) {
  const int64_t local_stride = (int64_t)total_q * top_k;
  const size_t lds = topk_merge_lds_bytes();
  static const bool lds_set = [&] {
    for (const void* f : {reinterpret_cast<const void*>(&topk_merge_kernel<false, false>),
                          reinterpret_cast<const void*>(&topk_merge_kernel<false, true>),
                          reinterpret_cast<const void*>(&topk_merge_kernel<true, false>),
                          reinterpret_cast<const void*>(&topk_merge_kernel<true, true>)})
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return true;
  }();
  (void)lds_set;
  const bool al = k_in % NT_A == 0;
  auto kern = fscores ? (al ? &topk_merge_kernel<true, true> : &topk_merge_kernel<true, false>)
                      : (al ? &topk_merge_kernel<false, true> : &topk_merge_kernel<false, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)total_q), dim3(NT_A), lds, s, n_lists, k_in, idx_lists,
                     score_lists, list_stride, top_k, idx, score, local_idx, local_stride);
  return hipGetLastError();
}

hipError_t launch_topk(const smla_batch& b, const int32_t* scores, int32_t top_k, int32_t* idx,
                       int32_t* score, const TopkWs& w, hipStream_t s, bool fscores) {
  return fscores ? launch_topk_t<true>(b, scores, top_k, idx, score, w, s)
                 : launch_topk_t<false>(b, scores, top_k, idx, score, w, s);
}

}  // namespace smla
