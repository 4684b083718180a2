// hot_resolve.hip — top-k resolution against a per-request hot buffer (hybrid offload).
//
// Under memory pressure the pages move a request's older KV pages to host memory and keep only
// its tail resident; the rows the indexer selects from the offloaded part live in a small GPU
// "hot buffer" managed least-recently-used. One fused kernel resolves a step's top-k: resident
// rows are read in place, a selected row already in the buffer refreshes its slot's last use,
// and a miss copies the row from pinned host memory into the least recently used slot ("vLLM
// GLM 5.3 ... Hybrid HiSparse", technical implementation; the buffer defaults to twice top-k
// rows per request, architectural details).
//
// Reading of the order inside one step (the pages give none): the distinct offloaded
// selections of all of a request's query tokens are taken in ascending token order; hits keep
// their slot; misses, ascending, take the slots not hit in this step in (last use, slot)
// order. The result is the same for any order of the selections within the step.
//
// One 1024-thread workgroup per request, everything in LDS:
//   1. the offloaded selections (others as +inf), sorted unless already ascending (a decode
//      token's top-k is), and marked at first occurrences;
//   2. the slot table in an LDS hash table (token -> slot); each distinct selection looked up;
//   3. if there are misses: the slots not hit as (last use, slot), sorted — miss number r takes
//      the r-th; the miss rows are copied host -> hot slot by whole waves, 16 bytes a lane;
//   4. every selection rewritten: -1 stays, a resident row stays, an offloaded row becomes
//      hot_base + its slot.
// Nothing in the request changes when its distinct offloaded selections outnumber the slots or
// its hot buffer / host rows fall outside their bounds (status < 0, selections set to -1).
#include "hot_resolve.h"

namespace smla {

namespace {

constexpr int HR_THREADS = 1024;
constexpr uint64_t HR_NONE = ~0ull;

__device__ __forceinline__ int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Ascending bitonic sort of a[0, n), n a power of two, by the whole workgroup.
template <typename T>
__device__ void bitonic_sort_lds(T* a, int n) {
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += HR_THREADS) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo + j;
        const bool up = (lo & k) == 0;
        const T x = a[lo], y = a[hi];
        if ((x > y) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
}

// Exclusive prefix sum of one value per thread over the workgroup; returns the thread's offset
// and writes the total to *total. `part` holds HR_THREADS / 64 + 1 ints.
__device__ int block_exclusive_scan(int v, int* part, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) part[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < HR_THREADS / 64; ++w) {
      const int c = part[w];
      part[w] = run;
      run += c;
    }
    part[HR_THREADS / 64] = run;
  }
  __syncthreads();
  *total = part[HR_THREADS / 64];
  const int r = part[wave] + x - v;
  __syncthreads();  // part may be reused by the caller
  return r;
}

struct HrLds {
  int sel[HOT_MAX_SEL];    // offloaded selections (else INT_MAX), sorted
  int res[HOT_MAX_SEL];    // slot of the distinct selection at a first occurrence
  uint64_t key[2 * HOT_MAX_SLOTS];  // slot hash table, then victims, then the misses' (token, slot)
  int part[HR_THREADS / 64 + 1];
};

__global__ __launch_bounds__(HR_THREADS) void hot_resolve_kernel(
    const Req* __restrict__ reqs, const Tok* __restrict__ toks, const int32_t* __restrict__ idx,
    int top_k,
    const int32_t* __restrict__ resident_from, const int32_t* __restrict__ hot_base, int n_slots,
    int32_t* __restrict__ hot_tok, int32_t* __restrict__ hot_age, int step,
    const unsigned char* __restrict__ host_rows, int64_t host_n_rows,
    const int64_t* __restrict__ host_row0, int row_bytes, unsigned char* __restrict__ kv,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ n_copied) {
  extern __shared__ __align__(16) unsigned char hr_smem[];
  HrLds& L = *reinterpret_cast<HrLds*>(hr_smem);
  const int b = blockIdx.x;
  const Req rq = reqs[b];
  const int n = rq.n_q * top_k;
  const int32_t* in = idx + (int64_t)rq.q_start * top_k;
  int32_t* out = idx_out + (int64_t)rq.q_start * top_k;
  const int rf = resident_from[b];
  const int hb = hot_base[b];
  const int64_t hr0 = host_row0[b];
  int32_t* tok = hot_tok + (int64_t)b * n_slots;
  int32_t* age = hot_age + (int64_t)b * n_slots;

  int status = 0;
  // the offloaded prefix (and the hot buffer inside it) must end at or before the first query
  // token's position (kv_len - n_q by default): every token of the request sees every hot row
  if (rf < 0 || rf > toks[rq.q_start].pos + 1) status = -2;
  else if (rf > 0 && (hb < 0 || (int64_t)hb + n_slots > rf)) status = -2;
  else if (rf > 0 && (hr0 < 0 || hr0 + rf > host_n_rows)) status = -3;
  if (status < 0 || rf == 0) {  // nothing offloaded, or a bad request: no state is touched
    for (int i = threadIdx.x; i < n; i += HR_THREADS) {
      const int v = in[i];
      out[i] = status < 0 || v < 0 ? -1 : v;
    }
    if (threadIdx.x == 0) n_copied[b] = status;
    return;
  }

  // 1. offloaded selections, sorted, first occurrences counted
  const int P = next_pow2(max(n, 1));
  bool unsorted = false;
  for (int i = threadIdx.x; i < P; i += HR_THREADS) {
    const int v = i < n ? in[i] : -1;
    L.sel[i] = v >= 0 && v < rf ? v : INT_MAX;
  }
  __syncthreads();
  for (int i = threadIdx.x + 1; i < P; i += HR_THREADS) unsorted |= L.sel[i - 1] > L.sel[i];
  if (__syncthreads_or(unsorted)) bitonic_sort_lds(L.sel, P);
  int n_first = 0;
  for (int i = threadIdx.x; i < P; i += HR_THREADS)
    n_first += L.sel[i] != INT_MAX && (i == 0 || L.sel[i - 1] != L.sel[i]);
  int m;
  (void)block_exclusive_scan(n_first, L.part, &m);
  if (m > n_slots) {  // the distinct offloaded rows do not fit: nothing changes
    for (int i = threadIdx.x; i < n; i += HR_THREADS) out[i] = -1;
    if (threadIdx.x == 0) n_copied[b] = -1;
    return;
  }

  // 2. hits: the slot table goes into an LDS hash table of 2 x PH entries (token << 32 | slot,
  // open addressing, at most half full), probed once per distinct selection. Each thread owns
  // the contiguous chunk [c0, c1) of the sorted selections, so miss ranks follow token order.
  const int PH = next_pow2(n_slots);
  const int TB = 2 * PH, tb_shift = 32 - __builtin_ctz((unsigned)TB);
  auto home = [&](uint32_t t) { return (int)((t * 2654435761u) >> tb_shift) & (TB - 1); };
  for (int j = threadIdx.x; j < TB; j += HR_THREADS) L.key[j] = HR_NONE;
  __syncthreads();
  for (int j = threadIdx.x; j < n_slots; j += HR_THREADS) {
    const int t = tok[j];
    if (t < 0) continue;
    const uint64_t e = ((uint64_t)(uint32_t)t << 32) | (uint32_t)j;
    for (int h = home((uint32_t)t), probe = 0; probe < TB; h = (h + 1) & (TB - 1), ++probe) {
      const uint64_t old = atomicCAS(reinterpret_cast<unsigned long long*>(&L.key[h]),
                                     (unsigned long long)HR_NONE, (unsigned long long)e);
      if (old == HR_NONE) break;
      if ((old >> 32) == (uint64_t)(uint32_t)t) {  // the token twice: the lower slot wins
        atomicMin(reinterpret_cast<unsigned long long*>(&L.key[h]), (unsigned long long)e);
        break;
      }
    }
  }
  __syncthreads();
  const int chunk = (P + HR_THREADS - 1) / HR_THREADS;
  const int c0 = min((int)threadIdx.x * chunk, P), c1 = min(c0 + chunk, P);
  auto first = [&](int i) { return L.sel[i] != INT_MAX && (i == 0 || L.sel[i - 1] != L.sel[i]); };
  int my_miss = 0;
  for (int i = c0; i < c1; ++i) {
    if (!first(i)) continue;
    const uint32_t v = (uint32_t)L.sel[i];
    int slot = -1;
    for (int h = home(v), probe = 0; probe < TB; h = (h + 1) & (TB - 1), ++probe) {
      const uint64_t e = L.key[h];
      if (e == HR_NONE) break;
      if ((uint32_t)(e >> 32) == v) {
        slot = (int)(uint32_t)e;
        break;
      }
    }
    L.res[i] = slot;
    my_miss += slot < 0;
  }
  int n_miss;
  const int rank0 = block_exclusive_scan(my_miss, L.part, &n_miss);  // also: searches done

  // 3. victims: the slots not hit, by (last use, slot); miss number r takes the r-th, and its
  // owner then stores (token << 32 | slot) at r for the copy loop
  if (n_miss > 0) {
    for (int j = threadIdx.x; j < PH; j += HR_THREADS) L.key[j] = j < n_slots ? 0 : HR_NONE;
    __syncthreads();
    for (int i = c0; i < c1; ++i)
      if (first(i) && L.res[i] >= 0) L.key[L.res[i]] = HR_NONE;
    __syncthreads();
    for (int j = threadIdx.x; j < n_slots; j += HR_THREADS)
      if (L.key[j] != HR_NONE)
        L.key[j] = ((uint64_t)((uint32_t)age[j] ^ 0x80000000u) << 32) | (uint32_t)j;
    __syncthreads();
    bitonic_sort_lds(L.key, PH);
    int r = rank0;
    for (int i = c0; i < c1; ++i) {
      if (!first(i) || L.res[i] >= 0) continue;
      const uint32_t s = (uint32_t)L.key[r];
      L.res[i] = (int)s;
      L.key[r] = ((uint64_t)(uint32_t)L.sel[i] << 32) | s;
      ++r;
    }
  }
  __syncthreads();

  // state: every distinct selection's slot was used at this step and holds its token
  for (int i = c0; i < c1; ++i) {
    if (!first(i)) continue;
    const int s = L.res[i];
    age[s] = step;
    tok[s] = L.sel[i];
  }
  // copies host -> hot slot: wave w takes misses w, w + 16, ...; a lane moves 16 bytes
  if (n_miss > 0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int vec = row_bytes >> 4;
    for (int r = wave; r < n_miss; r += HR_THREADS / 64) {
      const uint64_t e = L.key[r];
      const int64_t t = (int64_t)(e >> 32), s = (int64_t)(uint32_t)e;
      const uint4* src = reinterpret_cast<const uint4*>(host_rows + (hr0 + t) * row_bytes);
      uint4* dst = reinterpret_cast<uint4*>(kv + (rq.row_start + hb + s) * row_bytes);
      for (int c = lane; c < vec; c += 64) dst[c] = src[c];
    }
  }
  // 4. every selection: -1 stays, a resident row stays, an offloaded row names its slot
  for (int i = threadIdx.x; i < n; i += HR_THREADS) {
    const int v = in[i];
    if (v < 0 || v >= rf) {
      out[i] = v < 0 ? -1 : v;
      continue;
    }
    int lo = 0, hi = P;  // first occurrence of v in the sorted selections
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (L.sel[mid] < v) lo = mid + 1;
      else hi = mid;
    }
    out[i] = hb + L.res[lo];
  }
  if (threadIdx.x == 0) n_copied[b] = n_miss;
}

}  // namespace

size_t hot_resolve_lds_bytes() { return sizeof(HrLds); }

hipError_t launch_hot_resolve(const void* table, int32_t batch, const int32_t* idx, int32_t top_k,
                              const int32_t* resident_from, const int32_t* hot_base,
                              int32_t n_slots, int32_t* hot_tok, int32_t* hot_age, int32_t step,
                              const void* host_rows, int64_t host_n_rows, const int64_t* host_row0,
                              int32_t row_bytes, void* kv, int32_t* idx_out, int32_t* n_copied,
                              hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&hot_resolve_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(HrLds));
    attr = true;
  }
  hipLaunchKernelGGL(hot_resolve_kernel, dim3((unsigned)batch), dim3(HR_THREADS), sizeof(HrLds), s,
                     reinterpret_cast<const Req*>(table), table_view(table, batch, 0).tok, idx, top_k,
                     resident_from, hot_base,
                     n_slots, hot_tok, hot_age, step, static_cast<const unsigned char*>(host_rows),
                     host_n_rows, host_row0, row_bytes, static_cast<unsigned char*>(kv), idx_out,
                     n_copied);
  return hipGetLastError();
}

}  // namespace smla
