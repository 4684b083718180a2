// topk.hip — exact per-query top-k over int32 indexer scores on gfx950.
//
// The indexer keeps, for every query token, the 2,048 earlier tokens with the largest scores
// ("Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "Why DP8 and TP8 fall short"); ties
// go to the lower token index, and every s <= p is kept when p + 1 <= k.
//
// Selection order is the total order of the unique 64-bit key (score << 32) | ~s, so the top-k
// set is unique. A select finds it without sorting:
//  1. a 4096-bin histogram of a monotone, floating-point-like code of the score (5-bit exponent,
//     7 bits below the leading one) locates the bin b* that holds the k-th largest key;
//     everything in higher bins is selected;
//  2. inside b* an MSD radix select over 8-bit digits of the 64-bit key finds the exact cut.
// Rows of up to 32,768 candidates are selected by one workgroup with the scores held in LDS.
// Longer rows are cut into 8,192-candidate segments: per-segment histograms meet in a global
// per-row histogram, every segment emits its elements above b* and its b* candidates, and one
// workgroup per row resolves the candidates. Selected indices are emitted in ascending order.
#include "smla_internal.h"

namespace smla {

namespace {

__device__ __forceinline__ int score_bin(uint32_t s) {
  if (s < 128u) return (int)s;
  const int e = 31 - __builtin_clz(s);  // 7..30
  return 128 * (e - 6) + (int)((s >> (e - 7)) & 127u);
}

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
  for (int i = threadIdx.x; i < n; i += NT_A) {
    const int v = row[i];
    sc[i] = v;
    atomicAdd(&hist[score_bin((uint32_t)v)], 1);
  }
  __syncthreads();
  find_cut<NT_A>(hist, TOPK_BINS, top_k, red, cut);
  const int bstar = cut[0];
  const int above = cut[1];
  const int need = top_k - above;
  __syncthreads();
  uint64_t prefix = 0, mask = 0;
  if (hist[bstar] != need) {
    radix_cut<NT_A>(
        n, need, [&](int i) { return sel_key(sc[i], i); },
        [&](int i) { return score_bin((uint32_t)sc[i]) == bstar; }, hist2, red, cut, pm);
    prefix = pm[0];
    mask = pm[1];
  }
  // emit in ascending index order: thread i owns the contiguous range [c0, c1)
  const int per = (n + NT_A - 1) / NT_A;
  const int c0 = min(n, (int)threadIdx.x * per), c1 = min(n, c0 + per);
  auto selected = [&](int i) {
    const int bn = score_bin((uint32_t)sc[i]);
    return bn > bstar || (bn == bstar && (sel_key(sc[i], i) & mask) >= prefix);
  };
  int cnt = 0;
  for (int i = c0; i < c1; ++i) cnt += selected(i);
  int pos = block_incl_scan<NT_A>(cnt, red) - cnt;
  for (int i = c0; i < c1; ++i)
    if (selected(i)) {
      if (pos < top_k) {  // exactly top_k are selected; the guard only bounds the writes
        oi[pos] = i;
        if (os) os[pos] = sc[i];
      }
      ++pos;
    }
}

// ---- path B: rows of n > TOPK_LDS_MAX ----------------------------------------------------
// Workspace per row: hist [TOPK_BINS] int, rec [4] int (out count, cand count, b*, above),
// cand [TOPK_CAND_CAP] uint64.
constexpr int NT_B = 256;

struct TopkWs {
  int* hist;
  int* rec;
  uint64_t* cand;
};

__host__ __device__ inline TopkWs topk_ws(void* base, int64_t total_q) {
  char* p = static_cast<char*>(base);
  TopkWs w;
  w.hist = reinterpret_cast<int*>(p);
  p += align_up(sizeof(int) * TOPK_BINS * (size_t)total_q, 256);
  w.rec = reinterpret_cast<int*>(p);
  p += align_up(sizeof(int) * 4 * (size_t)total_q, 256);
  w.cand = reinterpret_cast<uint64_t*>(p);
  return w;
}

__global__ __launch_bounds__(NT_B) void topk_hist_kernel(const Tok* __restrict__ toks,
                                                         const int32_t* __restrict__ scores,
                                                         TopkWs ws) {
  __shared__ int hist[TOPK_BINS];
  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  const int s0 = blockIdx.y * TOPK_SEG;
  if (n <= TOPK_LDS_MAX || s0 >= n) return;
  const int s1 = min(n, s0 + TOPK_SEG);
  for (int i = threadIdx.x; i < TOPK_BINS; i += NT_B) hist[i] = 0;
  __syncthreads();
  const int32_t* row = scores + tk.cand_off;
  for (int i = s0 + threadIdx.x; i < s1; i += NT_B) atomicAdd(&hist[score_bin((uint32_t)row[i])], 1);
  __syncthreads();
  int* g = ws.hist + t * TOPK_BINS;
  for (int i = threadIdx.x; i < TOPK_BINS; i += NT_B)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

__global__ __launch_bounds__(NT_B) void topk_filter_kernel(const Tok* __restrict__ toks,
                                                           const int32_t* __restrict__ scores,
                                                           int top_k, TopkWs ws,
                                                           int32_t* __restrict__ idx_out,
                                                           int32_t* __restrict__ score_out) {
  __shared__ int hist[TOPK_BINS];
  __shared__ int red[NT_B / 64 + 1];
  __shared__ int cut[2];
  __shared__ int cnt[2], base[2];
  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  const int s0 = blockIdx.y * TOPK_SEG;
  if (n <= TOPK_LDS_MAX || s0 >= n) return;
  const int s1 = min(n, s0 + TOPK_SEG);
  const int* g = ws.hist + t * TOPK_BINS;
  for (int i = threadIdx.x; i < TOPK_BINS; i += NT_B) hist[i] = g[i];
  if (threadIdx.x < 2) cnt[threadIdx.x] = 0;
  __syncthreads();
  find_cut<NT_B>(hist, TOPK_BINS, top_k, red, cut);
  const int bstar = cut[0];
  int* rec = ws.rec + t * 4;
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    rec[2] = bstar;
    rec[3] = cut[1];
  }
  const int32_t* row = scores + tk.cand_off;
  // count this segment's selected and candidate elements, reserve global ranges, then write
  for (int i = s0 + threadIdx.x; i < s1; i += NT_B) {
    const int bn = score_bin((uint32_t)row[i]);
    if (bn > bstar) atomicAdd(&cnt[0], 1);
    else if (bn == bstar) atomicAdd(&cnt[1], 1);
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    base[threadIdx.x] = cnt[threadIdx.x] ? atomicAdd(&rec[threadIdx.x], cnt[threadIdx.x]) : 0;
    cnt[threadIdx.x] = 0;
  }
  __syncthreads();
  int32_t* oi = idx_out + t * top_k;
  int32_t* os = score_out ? score_out + t * top_k : nullptr;
  uint64_t* cand = ws.cand + t * TOPK_CAND_CAP;
  for (int i = s0 + threadIdx.x; i < s1; i += NT_B) {
    const int v = row[i];
    const int bn = score_bin((uint32_t)v);
    if (bn > bstar) {
      const int slot = base[0] + atomicAdd(&cnt[0], 1);  // < above < top_k
      if (slot < top_k) {
        oi[slot] = i;
        if (os) os[slot] = v;
      }
    } else if (bn == bstar) {
      const int slot = base[1] + atomicAdd(&cnt[1], 1);
      if (slot < TOPK_CAND_CAP) cand[slot] = sel_key(v, i);
    }
  }
}

// Bitonic sort of m (power of two, <= 2 * NT) keys in LDS, ascending.
template <int NT>
__device__ void bitonic_sort(uint64_t* a, int m) {
  for (int k = 2; k <= m; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < m; i += NT) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t x = a[i], y = a[l];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      __syncthreads();
    }
}

constexpr int NT_R = 1024;

__global__ __launch_bounds__(NT_R) void topk_resolve_kernel(const Tok* __restrict__ toks,
                                                            const int32_t* __restrict__ scores,
                                                            int top_k, TopkWs ws,
                                                            int32_t* __restrict__ idx_out,
                                                            int32_t* __restrict__ score_out) {
  extern __shared__ uint64_t smem64[];
  uint64_t* keys = smem64;                 // [TOPK_CAND_CAP] candidate keys
  uint64_t* outk = smem64 + TOPK_CAND_CAP; // [TOPK_MAX_K] the row's result, (index << 32) | score
  __shared__ int hist2[256];
  __shared__ int red[NT_R / 64 + 1];
  __shared__ int cut[2];
  __shared__ uint64_t pm[2];
  __shared__ int wpos;

  const int64_t t = blockIdx.x;
  const Tok tk = toks[t];
  const int n = tk.pos + 1;
  if (n <= TOPK_LDS_MAX) return;
  const int* rec = ws.rec + t * 4;
  const int bstar = min(max(rec[2], 0), TOPK_BINS - 1);
  const int above = min(max(rec[3], 0), top_k - 1);
  const int ncand = rec[1];
  const int need = top_k - above;
  const int32_t* row = scores + tk.cand_off;
  int32_t* oi = idx_out + t * top_k;
  int32_t* os = score_out ? score_out + t * top_k : nullptr;
  if (threadIdx.x == 0) wpos = above;
  __syncthreads();

  if (ncand <= TOPK_CAND_CAP) {
    const uint64_t* cand = ws.cand + t * TOPK_CAND_CAP;
    for (int i = threadIdx.x; i < ncand; i += NT_R) keys[i] = cand[i];
    __syncthreads();
    uint64_t prefix = 0, mask = 0;
    if (ncand != need) {
      radix_cut<NT_R>(
          ncand, need, [&](int i) { return keys[i]; }, [&](int) { return true; }, hist2, red, cut,
          pm);
      prefix = pm[0];
      mask = pm[1];
    }
    for (int i = threadIdx.x; i < ncand; i += NT_R) {
      const uint64_t key = keys[i];
      if ((key & mask) >= prefix) {
        const int slot = atomicAdd(&wpos, 1);
        if (slot < top_k) outk[slot] = ((uint64_t)(0xFFFFFFFFu - (uint32_t)key) << 32) | (key >> 32);
      }
    }
  } else {
    // more candidates than the buffer holds (heavy ties): select straight from the score row
    radix_cut<NT_R>(
        n, need, [&](int i) { return sel_key(row[i], i); },
        [&](int i) { return score_bin((uint32_t)row[i]) == bstar; }, hist2, red, cut, pm);
    const uint64_t prefix = pm[0], mask = pm[1];
    for (int i = threadIdx.x; i < n; i += NT_R) {
      const int v = row[i];
      if (score_bin((uint32_t)v) == bstar && (sel_key(v, i) & mask) >= prefix) {
        const int slot = atomicAdd(&wpos, 1);
        if (slot < top_k) outk[slot] = ((uint64_t)(uint32_t)i << 32) | (uint32_t)v;
      }
    }
  }
  // the filter pass wrote the elements above b* to slots [0, above) of the output row
  for (int i = threadIdx.x; i < above; i += NT_R)
    outk[i] = ((uint64_t)(uint32_t)oi[i] << 32) | (os ? (uint32_t)os[i] : 0u);
  int m = 1;
  while (m < top_k) m <<= 1;
  for (int i = top_k + threadIdx.x; i < m; i += NT_R) outk[i] = ~0ull;
  __syncthreads();
  // ascending index order (indices are unique, so the score bits never decide)
  bitonic_sort<NT_R>(outk, m);
  for (int i = threadIdx.x; i < top_k; i += NT_R) {
    oi[i] = (int)(outk[i] >> 32);
    if (os) os[i] = (int)(uint32_t)outk[i];
  }
}

}  // namespace

size_t topk_workspace_bytes(const smla_batch& b, int32_t /*top_k*/) {
  if (b.max_kv <= TOPK_LDS_MAX) return 0;
  const size_t tq = (size_t)b.total_q;
  return align_up(sizeof(int) * TOPK_BINS * tq, 256) + align_up(sizeof(int) * 4 * tq, 256) +
         align_up(sizeof(uint64_t) * TOPK_CAND_CAP * tq, 256);
}

hipError_t launch_topk(const smla_batch& b, const int32_t* scores, int32_t top_k, int32_t* idx,
                       int32_t* score, void* ws, hipStream_t s) {
  TableView tv = table_view(b.table, b.batch, b.total_q);
  const size_t lds_a = sizeof(int) * (TOPK_LDS_MAX + TOPK_BINS);
  const size_t lds_r = sizeof(uint64_t) * (TOPK_CAND_CAP + TOPK_MAX_K);
  // dynamic LDS above 64 KiB: raise the per-kernel limit once
  static const bool lds_set = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_lds_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_a);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_resolve_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_r);
    return true;
  }();
  (void)lds_set;
  hipLaunchKernelGGL(topk_lds_kernel, dim3(b.total_q), dim3(NT_A), lds_a, s, tv.tok, scores,
                     top_k, idx, score);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || b.max_kv <= TOPK_LDS_MAX) return e;
  TopkWs w = topk_ws(ws, b.total_q);
  // histogram and per-row counters start at zero
  e = launch_fill_i32(w.hist, (int64_t)TOPK_BINS * b.total_q, 0, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32(w.rec, (int64_t)4 * b.total_q, 0, s);
  if (e != hipSuccess) return e;
  const unsigned nseg = (unsigned)((b.max_kv + TOPK_SEG - 1) / TOPK_SEG);
  hipLaunchKernelGGL(topk_hist_kernel, dim3(b.total_q, nseg), dim3(NT_B), 0, s, tv.tok, scores, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_filter_kernel, dim3(b.total_q, nseg), dim3(NT_B), 0, s, tv.tok, scores,
                     top_k, w, idx, score);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_resolve_kernel, dim3(b.total_q), dim3(NT_R), lds_r, s, tv.tok, scores,
                     top_k, w, idx, score);
  return hipGetLastError();
}

}  // namespace smla
