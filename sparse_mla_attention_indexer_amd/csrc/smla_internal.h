// smla_internal.h — layouts and constants shared by the library's host code and its gfx950
// kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla.h"

namespace smla {

// ---- device batch table (written by smla_batch_build, read by every kernel) --------------
// Layout inside the caller's table buffer: [Req x batch][Tok x total_q][Item x n_items].
struct alignas(16) Req {
  int64_t row_start;  // first row of the request in k_idx / kv
  int64_t kv_len;     // rows of the request (cached + its own queries)
  int32_t q_start;    // first global query token
  int32_t n_q;        // query tokens
  int64_t _pad;
};
struct alignas(16) Tok {
  int64_t row_start;  // row_start of the token's request
  int64_t cand_off;   // offset of the token's causal score row in compact layout
  int32_t pos;        // position p: rows s <= p are visible
  int32_t req;        // request id
  int64_t _pad;
};
// One indexer workgroup's work: up to two segments (a front query tile and a back query tile
// of the same request), each `nq` consecutive query tokens from global token `q0` against the
// keys [s0, s1) of their request.
struct alignas(16) Seg {
  int32_t q0, nq, s0, s1;
};
struct alignas(32) Item {
  Seg a, b;
};

// Indexer planning: query tiles of up to QT tokens; each front/back pair of tiles is cut into
// chunks of KEY_CHUNK keys of combined work, or of KEY_CHUNK_SMALL keys when that would give
// fewer than ITEMS_FILL workgroups (decode batches: a few long rows), so that the chip gets
// several workgroups per CU to balance.
constexpr int QT = 4;
constexpr int KEY_CHUNK = 4096;
constexpr int KEY_CHUNK_SMALL = 2048;
constexpr int ITEMS_FILL = 1024;

// Top-k: rows with n <= TOPK_LDS_MAX candidates are selected by one workgroup in LDS; longer
// rows by one workgroup each (up to TOPK_ROW_MAX) or by count / resolve / emit kernels over
// segments of TOPK_SEG candidates.
constexpr int TOPK_MAX_K = 2048;
constexpr int TOPK_LDS_MAX = 32768;
constexpr int TOPK_ROW_MAX = 73728;  // 1024 threads x 72 scores in registers
constexpr int TOPK_SEG = 4096;       // 256 threads x 16 scores in registers
constexpr int TOPK_SEG_MAX = 2048;   // segments per row: rows of up to 8,388,608 candidates
constexpr int TOPK_SEG_ALL_MAX_Q = 160;  // up to this many query tokens, all long rows segmented
// Rows whose selection reads the score histogram the indexer fills while scoring: the segmented
// top-k takes every row longer than TOPK_LDS_MAX in batches of at most TOPK_SEG_ALL_MAX_Q query
// tokens, and otherwise only rows longer than TOPK_ROW_MAX (shorter rows take their threshold
// from a sample of their own scores). The indexer histograms rows of more candidates than this.
inline int topk_hist_min_n(int64_t total_q) {
  return total_q <= TOPK_SEG_ALL_MAX_Q ? TOPK_LDS_MAX : TOPK_ROW_MAX;
}
constexpr int TOPK_BINS = 2048;
constexpr int TOPK_CAND_CAP = 4096;
// per row: [0] candidate counter, [1] b*, [2] count above b*, [4..5] cut key (low, high word)
constexpr int TOPK_REC = 8;

// Monotone 11-bit code of a non-negative score: values below 64 map to themselves, larger
// values to (leading-one position - 5) * 64 + the 6 bits below the leading one. Shared by the
// indexer (which accumulates the histogram of long rows while scoring) and the top-k kernels.
__device__ __forceinline__ int topk_bin(uint32_t s) {
  if (s < 64u) return (int)s;
  const int e = 31 - __builtin_clz(s);  // 6..31
  return 64 * (e - 5) + (int)((s >> (e - 6)) & 63u);
}

// Monotone 11-bit code of a non-negative fp32 score given as its bit pattern (FP8 keys): 64 bins
// per binade over [2^-16, 2^16); smaller scores share bin 0, larger ones bin 2047. Any monotone
// code selects exactly; a range that puts a row's scores into few bins only costs speed.
constexpr uint32_t TOPK_FBIN_BASE = 0x37800000u;  // 2^-16
__device__ __forceinline__ int topk_fbin(uint32_t s) {
  if (s < TOPK_FBIN_BASE) return 0;
  const uint32_t b = (s - TOPK_FBIN_BASE) >> 17;
  return b > 2047u ? 2047 : (int)b;
}
__device__ __forceinline__ uint64_t topk_fbin_lo(int b) {
  if (b <= 0) return 0;
  if (b >= TOPK_BINS) return 1ull << 32;
  return TOPK_FBIN_BASE + ((uint64_t)b << 17);
}

// Word of bin b in a row's histogram in device memory. A row's scores cluster in a few binades,
// so its busy bins are neighbours, and every workgroup that scores part of the row adds to them;
// many writers to one 128-byte line serialise, so bins less than 64 apart go to different lines.
__device__ __forceinline__ int topk_hist_slot(int b) { return (b & 63) * 32 + (b >> 6); }

// Smallest score whose code is b (the inverse of topk_bin on bin boundaries), as a 64-bit
// value so that the bound past the last bin is representable.
__device__ __forceinline__ uint64_t topk_bin_lo(int b) {
  if (b < 64) return (uint64_t)b;
  const int e = b / 64 + 5;
  return (uint64_t)(64 + b % 64) << (e - 6);
}

// Top-k workspace for rows longer than TOPK_LDS_MAX. The histogram and the candidate counters
// must be zero when a call starts: the kernels that consume them clear them again, so a
// workspace zero-filled once stays ready for every later call.
struct TopkWs {
  int* hist;       // [total_q][TOPK_BINS] score histogram of each row, bin b at word
                   // topk_hist_slot(b) (the indexer fills it)
  int* rec;        // [total_q][TOPK_REC]
  int* seg;        // [total_q][nseg] per-segment counts above b*, then output offsets
  uint64_t* cand;  // [total_q][TOPK_CAND_CAP] keys of the b* candidates
  int64_t nseg;
};

// Sparse MLA (big shape): heads, dims, rows per tile, decode splits.
constexpr int MLA_H = 64;
constexpr int MLA_DQK = 576;
constexpr int MLA_DV = 512;
constexpr int MLA_ROW_BYTES = 656;

inline __host__ __device__ size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct TableView {
  const Req* req;
  const Tok* tok;
  const Item* item;
};

inline __host__ __device__ TableView table_view(const void* base, int32_t batch, int32_t total_q) {
  const char* p = static_cast<const char*>(base);
  TableView v;
  v.req = reinterpret_cast<const Req*>(p);
  v.tok = reinterpret_cast<const Tok*>(p + align_up(sizeof(Req) * batch, 256));
  v.item = reinterpret_cast<const Item*>(p + align_up(sizeof(Req) * batch, 256) +
                                         align_up(sizeof(Tok) * (size_t)total_q, 256));
  return v;
}

// ---- optional per-stage events (smla_set_stage_events) -------------------------------------
enum Stage { STAGE_INDEXER = 0, STAGE_TOPK = 1, STAGE_MLA = 2, STAGE_COMBINE = 3, N_STAGES = 4 };
// Record the begin (end = false) or end event of stage s on stream st, if one is set.
void mark_stage(int s, bool end, hipStream_t st);

// ---- kernel launchers (defined in the .hip files) -----------------------------------------
// Each returns hipSuccess or the launch error; arguments were validated by the caller.
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t s);

// `hist` (optional, TopkWs::hist): histogram of every row longer than TOPK_LDS_MAX.
hipError_t launch_indexer_mfma(const smla_batch& b, const int8_t* q_idx, const int8_t* k_idx,
                               const int32_t* w, int32_t* scores, int compact, int* hist,
                               hipStream_t s);
// FP8 keys: q (E4M3 codes) [total_q, 64, 128], k (E4M3 codes) [total_rows, 128], k_scale
// [total_rows] fp32, w [total_q, 64] fp32; scores are fp32 bit patterns.
hipError_t launch_indexer_fp8(const smla_batch& b, const uint8_t* q, const uint8_t* k,
                              const float* k_scale, const float* w, int32_t* scores, int compact,
                              int* hist, hipStream_t s);
hipError_t launch_indexer_generic(const smla_batch& b, const int8_t* q_idx, const int8_t* k_idx,
                                  const int32_t* w, int32_t H_I, int32_t D_I, int32_t* scores,
                                  int compact, int* hist, hipStream_t s);

size_t topk_workspace_bytes(const smla_batch& b, int32_t top_k);
TopkWs topk_workspace(const smla_batch& b, void* ws);
// fscores: the scores are bit patterns of non-negative fp32 values (FP8 keys); padding scores
// are then -1.0f instead of -1.
hipError_t launch_topk(const smla_batch& b, const int32_t* scores_compact, int32_t top_k,
                       int32_t* idx, int32_t* score, const TopkWs& w, hipStream_t s,
                       bool fscores = false);

size_t mla_workspace_bytes(const smla_batch& b, int32_t H, int32_t D_v, int32_t top_k, int decode);
int mla_decode_splits(const smla_batch& b, int32_t top_k);
hipError_t launch_mla_fp8(const smla_batch& b, const void* q, const void* kv, const int32_t* idx,
                          int32_t top_k, float sm_scale, void* out, float* lse, void* ws,
                          int decode, hipStream_t s);
// The decode split-partial scratch of the allocation-free entry point: its size, and its address
// on the current device (looked up once per device).
size_t mla_scratch_bytes();
hipError_t mla_scratch(void** ptr);
hipError_t launch_kv_append(int64_t n, const void* latent, const int64_t* rows, void* kv,
                            const int8_t* k_new, int32_t D_I, int8_t* k_idx, hipStream_t s);
// DCP merges on one GPU (topk.hip, dcp.hip). The top-k merge holds at most MERGE_MAX_CAND
// candidates; fscores: the scores are fp32 bit patterns. Its per-shard local lists (local_idx,
// optional) are supported up to MERGE_FAST_LISTS lists, the most its search-based order handles.
constexpr int MERGE_MAX_CAND = 16384;
constexpr int MERGE_FAST_LISTS = 64;
hipError_t launch_topk_merge(int32_t total_q, int32_t n_lists, int32_t k_in, const int32_t* idx_lists,
                             const int32_t* score_lists, int64_t list_stride, int32_t top_k,
                             int32_t* idx, int32_t* score, int32_t* local_idx, bool fscores,
                             hipStream_t s);
hipError_t launch_local_indices(int32_t total_q, int32_t top_k, const int32_t* idx, int32_t n_shards,
                                int32_t* local_idx, hipStream_t s);
hipError_t launch_lse_merge(int32_t total_q, int32_t H, int32_t D_v, int32_t n_parts,
                            const void* outs, const float* lses, void* out, float* lse,
                            hipStream_t s);
hipError_t launch_mla_generic(const smla_batch& b, const void* q, const void* kv, int32_t H,
                              int32_t D_qk, int32_t D_v, const int32_t* idx, int32_t top_k,
                              float sm_scale, void* out, float* lse, hipStream_t s);

}  // namespace smla
