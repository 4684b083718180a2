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
// Rows of up to 32,768 candidates are selected by one workgroup with the scores held in LDS.
// Longer rows use the histogram the indexer kernel accumulated while scoring: rows of up to
// 73,728 candidates are held in one workgroup's registers; longer rows are cut into
// 8,192-candidate segments handled by three kernels (count, resolve, emit). Selected indices always come out in
// ascending order, each written at its rank.
#include "smla_internal.h"

namespace smla {

namespace {

__device__ __forceinline__ int score_bin(uint32_t s) { return topk_bin(s); }

__device__ __forceinline__ uint64_t sel_key(int32_t score, int64_t s) {
  return ((uint64_t)(uint32_t)score << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)s);
}

// Inclusive scan over the block (NT threads, multiple of 64); `red` holds NT/64 + 1 ints.
template <int NT>
__device__ int block_incl_scan(int v, int* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) red[wv] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < NT / 64; ++i) {
      int x = red[i];
      red[i] = acc;
      acc += x;
    }
    red[NT / 64] = acc;
  }
  __syncthreads();
  v += red[wv];
  __syncthreads();
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

// Ordered emission: the block's NW waves each own a contiguous chunk of [0, len); a first pass
// counts the selected elements per wave, a second writes each at its rank (ballot prefix), so
// the output keeps ascending index order with conflict-free, consecutive LDS reads.
template <int NT, typename Sel, typename Emit>
__device__ void emit_in_order(int len, int base, Sel sel, Emit emit, int* wcnt) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int chunk = ((len + NW - 1) / NW + 63) & ~63;
  const int c0 = min(len, wv * chunk), c1 = min(len, c0 + chunk);
  int cnt = 0;
  for (int i0 = c0; i0 < c1; i0 += 64) {
    const int i = i0 + lane;
    cnt += __popcll(__ballot(i < c1 && sel(i)));
  }
  if (lane == 0) wcnt[wv] = cnt;
  __syncthreads();
  int pos = base;
  for (int w = 0; w < wv; ++w) pos += wcnt[w];
  for (int i0 = c0; i0 < c1; i0 += 64) {
    const int i = i0 + lane;
    const bool f = i < c1 && sel(i);
    const uint64_t m = __ballot(f);
    if (f) emit(i, pos + __popcll(m & ((1ull << lane) - 1)));
    pos += __popcll(m);
  }
}

// ---- path A: rows of n <= TOPK_LDS_MAX, one 1024-thread workgroup per row ----------------
constexpr int NT_A = 1024;

__global__ __launch_bounds__(NT_A) void topk_lds_kernel(const Tok* __restrict__ toks,
                                                        const int32_t* __restrict__ scores,
                                                        int top_k, int32_t* __restrict__ idx_out,
                                                        int32_t* __restrict__ score_out) {
  extern __shared__ int smem[];
  int* sc = smem;                 // [TOPK_LDS_MAX]
  int* hist = sc + TOPK_LDS_MAX;  // [TOPK_BINS]
  __shared__ int hist2[256];
  __shared__ int red[NT_A / 64 + 1];
  __shared__ int cut[2];
  __shared__ uint64_t pm[2];

  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  if (n > TOPK_LDS_MAX) return;
  int32_t* oi = idx_out + t * top_k;
  int32_t* os = score_out ? score_out + t * top_k : nullptr;
  const int32_t* row = scores + tk.cand_off;
  if (n <= top_k) {
    for (int j = threadIdx.x; j < top_k; j += NT_A) {
      oi[j] = j < n ? j : -1;
      if (os) os[j] = j < n ? row[j] : -1;
    }
    return;
  }
  for (int i = threadIdx.x; i < TOPK_BINS; i += NT_A) hist[i] = 0;
  __syncthreads();
  {
    // every load of the row in flight before any is used
    constexpr int PER = TOPK_LDS_MAX / NT_A;
    int vals[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = j * NT_A + threadIdx.x;
      vals[j] = i < n ? row[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = j * NT_A + threadIdx.x;
      if (i < n) {
        sc[i] = vals[j];
        atomicAdd(&hist[score_bin((uint32_t)vals[j])], 1);
      }
    }
  }
  __syncthreads();
  find_cut<NT_A>(hist, TOPK_BINS, top_k, red, cut);
  const int bstar = cut[0];
  const int above = cut[1];
  const int need = top_k - above;
  __syncthreads();
  uint64_t prefix = 0, mask = 0;
  if (hist[bstar] != need) {
    const int ncand = hist[bstar];
    if (ncand <= TOPK_MAX_K) {
      // gather the b* candidates' keys, then one wave finds the exact cut among them
      __shared__ uint64_t keys[TOPK_MAX_K];
      __shared__ int nk;
      if (threadIdx.x == 0) nk = 0;
      __syncthreads();
      const int lane = threadIdx.x & 63;
      for (int i0 = 0; i0 < n; i0 += NT_A) {
        const int i = i0 + threadIdx.x;
        const bool f = i < n && score_bin((uint32_t)sc[i]) == bstar;
        const uint64_t m = __ballot(f);
        if (m) {
          int base = 0;
          const int leader = __builtin_ctzll(m);
          if (lane == leader) base = atomicAdd(&nk, __popcll(m));
          base = __shfl(base, leader);
          if (f) keys[base + __popcll(m & ((1ull << lane) - 1))] = sel_key(sc[i], i);
        }
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        uint64_t pf, mk;
        wave_radix_cut([&](int i) { return keys[i]; }, ncand, need, hist2, &pf, &mk);
        if (threadIdx.x == 0) {
          pm[0] = pf;
          pm[1] = mk;
        }
      }
      __syncthreads();
    } else {
      radix_cut<NT_A>(
          n, need, [&](int i) { return sel_key(sc[i], i); },
          [&](int i) { return score_bin((uint32_t)sc[i]) == bstar; }, hist2, red, cut, pm);
    }
    prefix = pm[0];
    mask = pm[1];
  }
  // emit in ascending index order
  __shared__ int wcnt[NT_A / 64];
  emit_in_order<NT_A>(
      n, 0,
      [&](int i) {
        const int bn = score_bin((uint32_t)sc[i]);
        return bn > bstar || (bn == bstar && (sel_key(sc[i], i) & mask) >= prefix);
      },
      [&](int i, int pos) {
        if (pos < top_k) {  // exactly top_k are selected; the guard only bounds the writes
          oi[pos] = i;
          if (os) os[pos] = sc[i];
        }
      },
      wcnt);
}

// ---- path B: rows of n > TOPK_LDS_MAX ----------------------------------------------------
constexpr int NT_B = 256;

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

// ---- rows of TOPK_LDS_MAX < n <= TOPK_ROW_MAX: one 1024-thread workgroup per row ----------
// The score histogram comes from the indexer, so b* is known at once. Each of the 16 waves owns a
// contiguous chunk of the row and holds it in registers (72 scores per lane, every load issued
// before any is used); a first pass over the registers counts the elements above b* and gathers
// the b* candidates in LDS, one wave resolves the exact cut among them, and a second pass writes
// every selected index at its rank. No state is shared across workgroups.
constexpr int NT_R = 1024;
constexpr int NW_R = NT_R / 64;
constexpr int V_R = TOPK_ROW_MAX / NT_R;  // scores per lane

// Loads the V_R elements row[ib + 64 u] of this lane. One buffer resource per group of 16 u
// (1024 elements) keeps every per-load offset in the instruction's 12-bit immediate, so a single
// address register serves all V_R loads; each resource's range is what is left of the row past
// the group's base, and loads past the end return 0. aux: cache-policy bits.
__device__ __forceinline__ void row_load(uint32_t (&v)[V_R], const int32_t* row, int n, int ib,
                                         int aux) {
  const int voff = ib * 4;
#pragma unroll
  for (int g = 0; g < (V_R + 15) / 16; ++g) {
    const int left = max(0, n - 1024 * g);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(row + 1024 * g), 0, left * 4, 0x00020000);
#pragma unroll
    for (int j = 0; j < 16 && 16 * g + j < V_R; ++j) {
      if (aux)
        v[16 * g + j] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 256 * j, 0, 1);
      else
        v[16 * g + j] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 256 * j, 0, 0);
    }
  }
}

__device__ __forceinline__ int lanes_below(uint64_t m) {  // set bits of m below this lane
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Row pass 1 over one wave's register-resident chunk: count the elements above bin b* = [lo, hm1]
// (returned, wave-uniform) and append the keys of the b* candidates to klo/khi. The masks are
// ballots of compares, so the per-element work is two vector compares; everything else is scalar.
// FULL: the whole chunk lies inside the row (no range mask).
template <bool FULL>
__device__ __forceinline__ int row_pass1(const uint32_t (&v)[V_R], int ib, int rem, uint32_t lo,
                                         uint32_t hm1, uint32_t* klo, uint32_t* khi, int* nk) {
  const int lane = threadIdx.x & 63;
  int above = 0;
#pragma unroll
  for (int u = 0; u < V_R; ++u) {
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
        if (slot < TOPK_CAND_CAP) {
          klo[slot] = 0xFFFFFFFFu - (uint32_t)(ib + 64 * u);
          khi[slot] = x;
        }
      }
    }
  }
  return above;
}

// Row pass 2: write every element whose key (score, then lower index) is at least the cut key
// (th, tl) at its rank, starting at `pos` (wave-uniform). Index comparisons happen only for
// elements whose score equals the cut score.
template <bool FULL>
__device__ __forceinline__ void row_pass2(const uint32_t (&v)[V_R], int ib, int rem, uint32_t th,
                                          uint32_t tl, int pos, int top_k, int32_t* oi,
                                          int32_t* os) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < V_R; ++u) {
    const uint32_t x = v[u];
    const int i = ib + 64 * u;
    uint64_t m = __ballot(x > th);
    if (__ballot(x == th)) m |= __ballot((x == th) & (0xFFFFFFFFu - (uint32_t)i >= tl));
    if (!FULL) m &= __ballot(64 * u < rem);
    if (m) {
      if ((m >> lane) & 1) {
        const int p = pos + lanes_below(m);
        if (p < top_k) {  // exactly top_k are selected; the guard only bounds the writes
          oi[p] = i;
          if (os) os[p] = (int32_t)x;
        }
      }
      pos += __popcll(m);
    }
  }
}

__global__ __launch_bounds__(NT_R) void topk_row_kernel(const Tok* __restrict__ toks,
                                                        const int32_t* __restrict__ scores,
                                                        int top_k, TopkWs ws,
                                                        int32_t* __restrict__ idx_out,
                                                        int32_t* __restrict__ score_out) {
  __shared__ int hist[TOPK_BINS];
  // candidate keys as two planes (low words: ~index, high words: score) so the compiler never
  // pairs a score with an index into a 64-bit register
  __shared__ uint32_t klo[TOPK_CAND_CAP], khi[TOPK_CAND_CAP];
  __shared__ int hist2[256];
  __shared__ int red[NT_R / 64 + 1];
  __shared__ int cut[2];
  __shared__ uint64_t pm[2];
  __shared__ int nk;
  __shared__ int wsel[NW_R], woff[NW_R];
  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  if (n <= TOPK_LDS_MAX || n > TOPK_ROW_MAX) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int32_t* row = scores + tk.cand_off;
  // Element u of this lane is row[ib + 64 u]: wave w owns [w 64 V_R, (w + 1) 64 V_R). Buffer
  // loads with the row length as the range return 0 past the end instead of faulting; the
  // range mask drops those in the one wave whose chunk crosses the end. Each pass issues all
  // V_R loads before using any.
  const int ib = wv * (64 * V_R) + lane;
  const int rem = n - ib;
  const bool full = n >= (wv + 1) * (64 * V_R);
  int32_t* oi = idx_out + t * top_k;
  int32_t* os = score_out ? score_out + t * top_k : nullptr;
  int need, bstar;
  uint32_t lo;
  {
    uint32_t v[V_R];
    row_load(v, row, n, ib, 0);
    // while the row is in flight: the cut bin b* from the histogram the indexer accumulated
    const int* gh = ws.hist + t * TOPK_BINS;
    for (int i = threadIdx.x; i < TOPK_BINS; i += NT_R) hist[i] = gh[i];
    if (threadIdx.x == 0) nk = 0;
    __syncthreads();
    find_cut<NT_R>(hist, TOPK_BINS, top_k, red, cut);
    bstar = cut[0];
    need = top_k - cut[1];
    lo = (uint32_t)topk_bin_lo(bstar);
    const uint32_t hm1 = (uint32_t)min(topk_bin_lo(bstar + 1) - 1, (uint64_t)0xFFFFFFFFu);
    const int above = full ? row_pass1<true>(v, ib, rem, lo, hm1, klo, khi, &nk)
                           : row_pass1<false>(v, ib, rem, lo, hm1, klo, khi, &nk);
    if (lane == 0) wsel[wv] = above;
  }
  __syncthreads();

  const int ncand = nk;
  if (ncand <= TOPK_CAND_CAP) {
    // pass 2's loads go out before the cut so their latency hides behind it
    uint32_t v[V_R];
    row_load(v, row, n, ib, 1);  // glc: a distinct load the compiler cannot merge with pass 1
    if (wv == 0) {
      uint64_t pf, mk;
      wave_radix_cut([&](int i) { return ((uint64_t)khi[i] << 32) | klo[i]; }, ncand, need, hist2,
                     &pf, &mk);
      // Keys are unique, so the cut is a threshold: the selected elements are exactly those whose
      // key (score, then lower index) is at least the cut key. When every candidate is taken the
      // cut is the bottom of bin b*.
      if (lane == 0) pm[0] = max(pf, (uint64_t)lo << 32);
      (void)mk;
    }
    __syncthreads();
    const uint64_t cutkey = pm[0];
    // selected candidates per owning wave (the index says which wave holds the score)
    for (int c = threadIdx.x; c < ncand; c += NT_R) {
      const uint64_t key = ((uint64_t)khi[c] << 32) | klo[c];
      if (key >= cutkey) atomicAdd(&wsel[(int)(0xFFFFFFFFu - klo[c]) / (64 * V_R)], 1);
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
    const uint32_t th = (uint32_t)(cutkey >> 32), tl = (uint32_t)cutkey;
    const int pos = __builtin_amdgcn_readfirstlane(woff[wv]);
    if (full)
      row_pass2<true>(v, ib, rem, th, tl, pos, top_k, oi, os);
    else
      row_pass2<false>(v, ib, rem, th, tl, pos, top_k, oi, os);
    return;
  }
  // more candidates than LDS holds (heavy ties): cut and emit straight from the score row
  radix_cut<NT_R>(
      n, need, [&](int i) { return sel_key(row[i], i); },
      [&](int i) { return score_bin((uint32_t)row[i]) == bstar; }, hist2, red, cut, pm);
  const uint64_t prefix = pm[0], mask = pm[1];
  const int c0 = wv * (64 * V_R);
  const int c1 = min(n, c0 + 64 * V_R);
  int cp = 0;
  for (int i = c0 + lane; i < c1; i += 64) {
    const int x = row[i];
    const int bn = score_bin((uint32_t)x);
    cp += bn > bstar || (bn == bstar && (sel_key(x, i) & mask) >= prefix);
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
    const int x = i < c1 ? row[i] : 0;
    const int bn = i < c1 ? score_bin((uint32_t)x) : -1;
    const bool f = bn > bstar || (bn == bstar && (sel_key(x, i) & mask) >= prefix);
    const uint64_t m = __ballot(f);
    if (f) {
      const int p = pos + __popcll(m & ((1ull << lane) - 1));
      if (p < top_k) {
        oi[p] = i;
        if (os) os[p] = x;
      }
    }
    pos += __popcll(m);
  }
}

// ---- rows of n > TOPK_ROW_MAX: segments of TOPK_SEG candidates over three kernels ---------
// count: per segment, the elements above b* and the b* candidates (appended to the row's
// candidate buffer); resolve: one workgroup per row finds the exact cut among the candidates and
// turns the per-segment counts into output offsets; emit: each segment writes its selected
// indices at their ranks. Kernel boundaries order the three, not device-wide fences.
__global__ __launch_bounds__(NT_B) void topk_seg_count_kernel(const Tok* __restrict__ toks,
                                                              const int32_t* __restrict__ scores,
                                                              int top_k, TopkWs ws) {
  __shared__ int hist[TOPK_BINS];
  __shared__ int red[NT_B / 64 + 1];
  __shared__ int cut[2];
  const int64_t t = blockIdx.y;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  const int g = blockIdx.x;
  const int s0 = g * TOPK_SEG;
  if (n <= TOPK_ROW_MAX || s0 >= n) return;
  const int s1 = min(n, s0 + TOPK_SEG);
  const int* gh = ws.hist + t * TOPK_BINS;
  for (int i = threadIdx.x; i < TOPK_BINS; i += NT_B) hist[i] = gh[i];
  __syncthreads();
  find_cut<NT_B>(hist, TOPK_BINS, top_k, red, cut);
  const int bstar = cut[0];
  int* rec = ws.rec + t * TOPK_REC;
  uint64_t* cand = ws.cand + t * TOPK_CAND_CAP;
  const int32_t* row = scores + tk.cand_off;
  const int lane = threadIdx.x & 63;
  constexpr int PER = TOPK_SEG / NT_B;
  int vals[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {  // every load of the segment in flight before any is used
    const int i = s0 + j * NT_B + threadIdx.x;
    vals[j] = i < s1 ? row[i] : 0;
  }
  int sel = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = s0 + j * NT_B + threadIdx.x;
    const int bn = i < s1 ? score_bin((uint32_t)vals[j]) : -1;
    sel += bn > bstar;
    const uint64_t m = __ballot(bn == bstar);
    if (m) {  // wave-aggregated append of this wave's b* candidates
      int base = 0;
      const int leader = __builtin_ctzll(m);
      if (lane == leader) base = atomicAdd(&rec[0], __popcll(m));
      base = __shfl(base, leader);
      if (bn == bstar) {
        const int slot = base + __popcll(m & ((1ull << lane) - 1));
        if (slot < TOPK_CAND_CAP) cand[slot] = sel_key(vals[j], i);
      }
    }
  }
  block_incl_scan<NT_B>(sel, red);
  if (threadIdx.x == 0) ws.seg[t * ws.nseg + g] = red[NT_B / 64];
}

__global__ __launch_bounds__(NT_B) void topk_resolve_kernel(const Tok* __restrict__ toks,
                                                            const int32_t* __restrict__ scores,
                                                            int top_k, TopkWs ws) {
  __shared__ int hist[TOPK_BINS];
  __shared__ uint64_t keys[TOPK_CAND_CAP];
  __shared__ int hist2[256];
  __shared__ int red[NT_B / 64 + 1];
  __shared__ int cut[2];
  __shared__ uint64_t pm[2];
  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  if (n <= TOPK_ROW_MAX) return;
  const int nseg_t = (n + TOPK_SEG - 1) / TOPK_SEG;
  const int* gh = ws.hist + t * TOPK_BINS;
  for (int i = threadIdx.x; i < TOPK_BINS; i += NT_B) hist[i] = gh[i];
  __syncthreads();
  find_cut<NT_B>(hist, TOPK_BINS, top_k, red, cut);
  const int bstar = cut[0];
  const int need = top_k - cut[1];
  int* rec = ws.rec + t * TOPK_REC;
  int* segc = ws.seg + t * ws.nseg;
  const int32_t* row = scores + tk.cand_off;
  const int ncand = rec[0];
  uint64_t prefix = 0, mask = 0;
  if (ncand <= TOPK_CAND_CAP) {
    const uint64_t* cand = ws.cand + t * TOPK_CAND_CAP;
    for (int i = threadIdx.x; i < ncand; i += NT_B) keys[i] = cand[i];
    __syncthreads();
    if (threadIdx.x < 64) {
      uint64_t pf, mk;
      wave_radix_cut([&](int i) { return keys[i]; }, ncand, need, hist2, &pf, &mk);
      if (threadIdx.x == 0) {
        pm[0] = pf;
        pm[1] = mk;
      }
    }
    __syncthreads();
    prefix = pm[0];
    mask = pm[1];
    for (int i = threadIdx.x; i < ncand; i += NT_B) {
      const uint64_t key = keys[i];
      if ((key & mask) >= prefix) atomicAdd(&segc[(int)(0xFFFFFFFFu - (uint32_t)key) / TOPK_SEG], 1);
    }
  } else {
    // more candidates than the buffer holds (heavy ties): cut straight from the score row
    radix_cut<NT_B>(
        n, need, [&](int i) { return sel_key(row[i], i); },
        [&](int i) { return score_bin((uint32_t)row[i]) == bstar; }, hist2, red, cut, pm);
    prefix = pm[0];
    mask = pm[1];
    for (int i = threadIdx.x; i < n; i += NT_B) {
      const int v = row[i];
      if (score_bin((uint32_t)v) == bstar && (sel_key(v, i) & mask) >= prefix)
        atomicAdd(&segc[i / TOPK_SEG], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the per-segment counts -> output offsets
  int carry = 0;
  for (int c0 = 0; c0 < nseg_t; c0 += NT_B) {
    const int c = c0 + threadIdx.x;
    const int v = c < nseg_t ? atomicAdd(&segc[c], 0) : 0;
    const int incl = block_incl_scan<NT_B>(v, red);
    const int tot = red[NT_B / 64];
    if (c < nseg_t) segc[c] = carry + incl - v;
    carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    rec[2] = bstar;
    rec[4] = (int)(uint32_t)prefix;
    rec[5] = (int)(uint32_t)(prefix >> 32);
    rec[6] = (int)(uint32_t)mask;
    rec[7] = (int)(uint32_t)(mask >> 32);
  }
}

// Pass 2: every segment writes its selected indices at their ranks (ascending index order).
__global__ __launch_bounds__(NT_B) void topk_emit_kernel(const Tok* __restrict__ toks,
                                                         const int32_t* __restrict__ scores,
                                                         int top_k, TopkWs ws,
                                                         int32_t* __restrict__ idx_out,
                                                         int32_t* __restrict__ score_out) {
  __shared__ int sc[TOPK_SEG];
  const int64_t t = blockIdx.y;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  const int g = blockIdx.x;
  const int s0 = g * TOPK_SEG;
  if (n <= TOPK_ROW_MAX || s0 >= n) return;
  const int s1 = min(n, s0 + TOPK_SEG);
  const int len = s1 - s0;
  const int* rec = ws.rec + t * TOPK_REC;
  const int bstar = rec[2];
  const uint64_t prefix = (uint64_t)(uint32_t)rec[4] | ((uint64_t)(uint32_t)rec[5] << 32);
  const uint64_t mask = (uint64_t)(uint32_t)rec[6] | ((uint64_t)(uint32_t)rec[7] << 32);
  const int off = ws.seg[t * ws.nseg + g];
  const int32_t* row = scores + tk.cand_off + s0;
  {
    constexpr int PER = TOPK_SEG / NT_B;
    int vals[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = j * NT_B + threadIdx.x;
      vals[j] = i < len ? row[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) sc[j * NT_B + threadIdx.x] = vals[j];
  }
  __syncthreads();
  __shared__ int wcnt[NT_B / 64];
  int32_t* oi = idx_out + t * top_k;
  int32_t* os = score_out ? score_out + t * top_k : nullptr;
  emit_in_order<NT_B>(
      len, off,
      [&](int i) {
        const int bn = score_bin((uint32_t)sc[i]);
        return bn > bstar || (bn == bstar && (sel_key(sc[i], s0 + i) & mask) >= prefix);
      },
      [&](int i, int pos) {
        if (pos < top_k) {  // exactly top_k are selected per row; the guard only bounds writes
          oi[pos] = s0 + i;
          if (os) os[pos] = sc[i];
        }
      },
      wcnt);
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

hipError_t topk_prepare(const smla_batch& b, const TopkWs& w, hipStream_t s) {
  if (b.max_kv <= TOPK_LDS_MAX) return hipSuccess;
  // histogram (filled by the indexer) and per-row counters start at zero; they are adjacent
  const int64_t n = (reinterpret_cast<const char*>(w.rec) - reinterpret_cast<const char*>(w.hist)) / 4 +
                    (int64_t)TOPK_REC * b.total_q;
  return launch_fill_i32(w.hist, n, 0, s);
}

hipError_t launch_topk(const smla_batch& b, const int32_t* scores, int32_t top_k, int32_t* idx,
                       int32_t* score, const TopkWs& w, hipStream_t s) {
  TableView tv = table_view(b.table, b.batch, b.total_q);
  const size_t lds_a = sizeof(int) * (TOPK_LDS_MAX + TOPK_BINS);
  static const bool lds_set = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_lds_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_a);
    return true;
  }();
  (void)lds_set;
  hipError_t e = hipSuccess;
  if (b.min_cand <= TOPK_LDS_MAX) {
    hipLaunchKernelGGL(topk_lds_kernel, dim3(b.total_q), dim3(NT_A), lds_a, s, tv.tok, scores,
                       top_k, idx, score);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (b.max_kv <= TOPK_LDS_MAX) return e;
  hipLaunchKernelGGL(topk_row_kernel, dim3(b.total_q), dim3(NT_R), 0, s, tv.tok, scores, top_k, w,
                     idx, score);
  if ((e = hipGetLastError()) != hipSuccess || b.max_kv <= TOPK_ROW_MAX) return e;
  const unsigned nseg = (unsigned)topk_nseg(b);
  hipLaunchKernelGGL(topk_seg_count_kernel, dim3(nseg, b.total_q), dim3(NT_B), 0, s, tv.tok,
                     scores, top_k, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_resolve_kernel, dim3(b.total_q), dim3(NT_B), 0, s, tv.tok, scores, top_k,
                     w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_emit_kernel, dim3(nseg, b.total_q), dim3(NT_B), 0, s, tv.tok, scores,
                     top_k, w, idx, score);
  return hipGetLastError();
}

}  // namespace smla
