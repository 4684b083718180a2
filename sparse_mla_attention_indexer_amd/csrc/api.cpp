// api.cpp — host side of the C ABI (include/smla.h): argument validation, the batch table and
// indexer work plan, workspace sizing and kernel launches. Every check runs before anything is
// enqueued; failures set a thread-local message and return a negative status.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <algorithm>
#include <vector>

#include "smla.h"
#include "smla_internal.h"
#include "hot_resolve.h"

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SMLA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_batch(const smla_batch* b) {
  if (!b) return fail(SMLA_E_INVALID, "batch is NULL");
  if (b->batch < 1 || b->total_q < 1 || b->max_q < 1 || b->max_kv < 1 || b->total_rows < 1 ||
      b->n_items < 0 || b->min_cand < 1 || !b->table)
    return fail(SMLA_E_INVALID, "batch descriptor is not initialised (call smla_batch_build)");
  if (!aligned(b->table, 16)) return fail(SMLA_E_INVALID, "batch table is not 16-byte aligned");
  return SMLA_OK;
}

int check_indexer_args(const smla_batch* b, const int8_t* q_idx, const int8_t* k_idx,
                       const int32_t* w, int32_t H_I, int32_t D_I, bool* mfma) {
  int rc = check_batch(b);
  if (rc) return rc;
  if (!q_idx || !k_idx || !w) return fail(SMLA_E_INVALID, "q_idx, k_idx and w must be non-NULL");
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(w, 4))
    return fail(SMLA_E_INVALID, "q_idx and k_idx must be 16-byte aligned, w 4-byte aligned");
  if (H_I == 64 && D_I == 128) {
    *mfma = true;
    return SMLA_OK;
  }
  if (H_I >= 1 && H_I <= 16 && D_I >= 4 && D_I <= 256 && D_I % 4 == 0) {
    *mfma = false;
    return SMLA_OK;
  }
  return fail(SMLA_E_UNSUPPORTED,
              "indexer shape H_I=%d D_I=%d unsupported (64x128, or H_I<=16 with D_I%%4==0<=256)",
              H_I, D_I);
}

int check_mla_args(const smla_batch* b, const void* q, const void* kv, int32_t fmt, int32_t H,
                   int32_t D_qk, int32_t D_v, const int32_t* idx, int32_t top_k, const void* out,
                   bool* fp8) {
  int rc = check_batch(b);
  if (rc) return rc;
  if (!q || !kv || !idx || !out) return fail(SMLA_E_INVALID, "q, kv, idx and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(idx, 4) || !aligned(out, 16))
    return fail(SMLA_E_INVALID, "q, kv and out must be 16-byte aligned, idx 4-byte aligned");
  if (top_k < 1 || top_k > smla::TOPK_MAX_K)
    return fail(SMLA_E_UNSUPPORTED, "top_k=%d outside [1, %d]", top_k, smla::TOPK_MAX_K);
  if (fmt == SMLA_KV_FP8_656) {
    if (H != 64 || D_qk != 576 || D_v != 512)
      return fail(SMLA_E_UNSUPPORTED, "FP8_656 rows need H=64, D_qk=576, D_v=512 (got %d, %d, %d)",
                  H, D_qk, D_v);
    *fp8 = true;
    return SMLA_OK;
  }
  if (fmt == SMLA_KV_BF16) {
    if (H < 1 || H > 16 || D_qk < 1 || D_qk > 256 || D_v < 1 || D_v > D_qk)
      return fail(SMLA_E_UNSUPPORTED, "BF16 rows need H<=16, D_qk<=256, D_v<=D_qk (got %d, %d, %d)",
                  H, D_qk, D_v);
    *fp8 = false;
    return SMLA_OK;
  }
  return fail(SMLA_E_INVALID, "unknown kv_format %d", fmt);
}

// Indexer work plan: query tiles of up to QT tokens, tile i paired with tile n-1-i, each pair's
// combined key range (front tile's keys, then back tile's) cut into C-key items; a remainder
// under C / 4 keys joins the item before it. pos: every token's position (non-decreasing within a
// request).
void plan_items_chunk(int32_t batch, const int32_t* n_q, const std::vector<int32_t>& pos,
                      const std::vector<int32_t>& q_start, int64_t C, std::vector<smla::Item>* items) {
  using smla::Item;
  using smla::Seg;
  for (int32_t b = 0; b < batch; ++b) {
    const size_t first_item = items->size();
    const int32_t nt = (n_q[b] + smla::QT - 1) / smla::QT;
    auto tile = [&](int32_t i, int64_t* extent, int32_t* q0, int32_t* nq) {
      const int32_t lo = i * smla::QT;
      const int32_t hi = std::min<int32_t>(n_q[b], lo + smla::QT);
      *q0 = q_start[b] + lo;
      *nq = hi - lo;
      *extent = (int64_t)pos[(size_t)(q_start[b] + hi - 1)] + 1;  // keys [0, extent) cover the tile
    };
    for (int32_t i = 0; i < (nt + 1) / 2; ++i) {
      const int32_t j = nt - 1 - i;
      int64_t ea, eb = 0;
      int32_t qa, na, qb = 0, nb = 0;
      tile(i, &ea, &qa, &na);
      if (j != i) tile(j, &eb, &qb, &nb);
      const int64_t E = ea + eb;
      for (int64_t c0 = 0; c0 < E;) {
        int64_t c1 = std::min(E, c0 + C);
        if (E - c1 < C / 4) c1 = E;  // a short remainder joins this item instead of its own
        Seg segs[2];
        int ns = 0;
        if (c0 < ea) segs[ns++] = Seg{qa, na, (int32_t)c0, (int32_t)std::min(c1, ea)};
        if (c1 > ea && nb > 0)
          segs[ns++] = Seg{qb, nb, (int32_t)(std::max(c0, ea) - ea), (int32_t)(c1 - ea)};
        Item it;
        it.a = segs[0];
        it.b = ns > 1 ? segs[1] : Seg{0, 0, 0, 0};
        items->push_back(it);
        c0 = c1;
      }
    }
    // key range first: the workgroups that run at the same time then share a few key ranges,
    // which stay in their XCD's L2 instead of streaming from the last-level cache
    std::stable_sort(items->begin() + first_item, items->end(),
                     [](const Item& x, const Item& y) { return x.a.s0 < y.a.s0; });
  }
}

void plan_items(int32_t batch, const int32_t* n_q, const std::vector<int32_t>& pos,
                const std::vector<int32_t>& q_start, std::vector<smla::Item>* items) {
  plan_items_chunk(batch, n_q, pos, q_start, smla::KEY_CHUNK, items);
  if ((int64_t)items->size() < smla::ITEMS_FILL) {
    items->clear();
    plan_items_chunk(batch, n_q, pos, q_start, smla::KEY_CHUNK_SMALL, items);
  }
}

size_t table_layout(int32_t batch, int32_t total_q, int64_t n_items) {
  return smla::align_up(sizeof(smla::Req) * batch, 256) +
         smla::align_up(sizeof(smla::Tok) * (size_t)total_q, 256) +
         smla::align_up(sizeof(smla::Item) * (size_t)(n_items > 0 ? n_items : 1), 256);
}

hipEvent_t g_stage_begin[smla::N_STAGES] = {};
hipEvent_t g_stage_end[smla::N_STAGES] = {};

}  // namespace

void smla::mark_stage(int s, bool end, hipStream_t st) {
  hipEvent_t e = end ? g_stage_end[s] : g_stage_begin[s];
  if (e) (void)hipEventRecord(e, st);
}

extern "C" {

int smla_set_stage_events(void* const* begin, void* const* end, int32_t n) {
  g_err.clear();
  if (n < 0 || n > smla::N_STAGES || (n > 0 && (!begin || !end)))
    return fail(SMLA_E_INVALID, "stage events: 0 <= n <= %d with non-NULL arrays", smla::N_STAGES);
  for (int s = 0; s < smla::N_STAGES; ++s) {
    g_stage_begin[s] = s < n ? static_cast<hipEvent_t>(begin[s]) : nullptr;
    g_stage_end[s] = s < n ? static_cast<hipEvent_t>(end[s]) : nullptr;
  }
  return SMLA_OK;
}

size_t smla_batch_table_bytes(int32_t batch, int32_t total_q, int64_t max_kv) {
  if (batch < 1 || total_q < 1 || max_kv < 1) return 0;
  // every tile pair contributes at most ceil(E / C) <= E / C + 1 items, E <= 2 * max_kv
  const int64_t tiles = (int64_t)total_q / smla::QT + batch;
  const int64_t items = tiles * (max_kv / smla::KEY_CHUNK_SMALL + 2);
  return table_layout(batch, total_q, items);
}

int smla_batch_build(int32_t batch, const int32_t* n_q, const int64_t* kv_len, void* table,
                     size_t table_bytes, void* stream, smla_batch* out) {
  return smla_batch_build_pos(batch, n_q, kv_len, nullptr, nullptr, table, table_bytes, stream, out);
}

int smla_batch_build_pos(int32_t batch, const int32_t* n_q, const int64_t* kv_len,
                         const int64_t* pos, void* host_staging, void* table, size_t table_bytes,
                         void* stream, smla_batch* out) {
  g_err.clear();
  if (batch < 1 || !n_q || !kv_len || !table || !out)
    return fail(SMLA_E_INVALID, "batch >= 1 and non-NULL n_q, kv_len, table, out required");
  if (!aligned(table, 256)) return fail(SMLA_E_INVALID, "table must be 256-byte aligned");
  int64_t total_q = 0, total_rows = 0, max_kv = 0;
  int32_t max_q = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (n_q[b] < 1 || kv_len[b] < n_q[b] || kv_len[b] >= (int64_t(1) << 31))
      return fail(SMLA_E_INVALID, "request %d: need 1 <= n_q (%d) <= kv_len (%lld) < 2^31", b, n_q[b],
                  (long long)kv_len[b]);
    total_q += n_q[b];
    total_rows += kv_len[b];
    max_kv = std::max<int64_t>(max_kv, kv_len[b]);
    max_q = std::max(max_q, n_q[b]);
  }
  if (total_q >= (int64_t(1) << 31)) return fail(SMLA_E_INVALID, "too many query tokens");
  if (total_rows >= (int64_t(1) << 40)) return fail(SMLA_E_INVALID, "too many rows");
  // every token's position: given, or kv_len - n_q + j; token t sees (p + 1) candidates
  std::vector<int32_t> P((size_t)total_q);
  int64_t total_cand = 0, min_cand = INT64_MAX;
  {
    int64_t t = 0;
    for (int32_t b = 0; b < batch; ++b)
      for (int32_t j = 0; j < n_q[b]; ++j, ++t) {
        const int64_t p = pos ? pos[t] : kv_len[b] - n_q[b] + j;
        if (p < 0 || p >= kv_len[b] || (j > 0 && p < P[(size_t)t - 1]))
          return fail(SMLA_E_INVALID,
                      "request %d token %d: position %lld outside [0, kv_len) or below the token "
                      "before it", b, j, (long long)p);
        P[(size_t)t] = (int32_t)p;
        total_cand += p + 1;
        min_cand = std::min<int64_t>(min_cand, p + 1);
      }
  }
  std::vector<smla::Req> req(batch);
  std::vector<smla::Tok> tok((size_t)total_q);
  std::vector<int32_t> q_start(batch);
  int64_t q0 = 0, r0 = 0, cand = 0;
  for (int32_t b = 0; b < batch; ++b) {
    q_start[b] = (int32_t)q0;
    req[b] = smla::Req{r0, kv_len[b], (int32_t)q0, n_q[b], 0};
    for (int32_t j = 0; j < n_q[b]; ++j) {
      const int32_t p = P[(size_t)(q0 + j)];
      tok[(size_t)(q0 + j)] = smla::Tok{r0, cand, p, b, 0};
      cand += (int64_t)p + 1;
    }
    q0 += n_q[b];
    r0 += kv_len[b];
  }
  std::vector<smla::Item> items;
  plan_items(batch, n_q, P, q_start, &items);
  const size_t need = table_layout(batch, (int32_t)total_q, (int64_t)items.size());
  if (table_bytes < need)
    return fail(SMLA_E_WORKSPACE, "table needs %zu bytes, got %zu", need, table_bytes);
  // the table is assembled in the caller's staging buffer (copied without waiting), or in a
  // buffer of the call's own (then the call waits for the copy)
  std::vector<unsigned char> own;
  unsigned char* host = static_cast<unsigned char*>(host_staging);
  if (!host) {
    own.resize(need);
    host = own.data();
  }
  memset(host, 0, need);
  const size_t off_tok = smla::align_up(sizeof(smla::Req) * batch, 256);
  const size_t off_item = off_tok + smla::align_up(sizeof(smla::Tok) * (size_t)total_q, 256);
  memcpy(host, req.data(), sizeof(smla::Req) * batch);
  memcpy(host + off_tok, tok.data(), sizeof(smla::Tok) * (size_t)total_q);
  if (!items.empty()) memcpy(host + off_item, items.data(), sizeof(smla::Item) * items.size());
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(table, host, need, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(batch table)");
  if (!host_staging) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize(batch table)");
  }
  out->batch = batch;
  out->total_q = (int32_t)total_q;
  out->max_q = max_q;
  out->n_items = (int32_t)items.size();
  out->max_kv = max_kv;
  out->total_rows = total_rows;
  out->total_cand = total_cand;
  out->min_cand = min_cand;
  out->table = table;
  out->table_bytes = need;
  return SMLA_OK;
}

int smla_indexer_scores(const smla_batch* b, const int8_t* q_idx, const int8_t* k_idx,
                        const int32_t* w, int32_t H_I, int32_t D_I, int32_t* scores, void* stream) {
  g_err.clear();
  bool mfma = false;
  int rc = check_indexer_args(b, q_idx, k_idx, w, H_I, D_I, &mfma);
  if (rc) return rc;
  if (!scores || !aligned(scores, 16)) return fail(SMLA_E_INVALID, "scores must be non-NULL, 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = smla::launch_fill_i32(scores, (int64_t)b->total_q * b->max_kv, -1, s);
  if (e == hipSuccess)
    e = mfma ? smla::launch_indexer_mfma(*b, q_idx, k_idx, w, scores, 0, nullptr, s)
             : smla::launch_indexer_generic(*b, q_idx, k_idx, w, H_I, D_I, scores, 0, nullptr, s);
  return e == hipSuccess ? SMLA_OK : hip_fail(e, "indexer launch");
}

size_t smla_indexer_topk_workspace_bytes(const smla_batch* b, int32_t /*H_I*/, int32_t /*D_I*/,
                                         int32_t top_k) {
  if (!b || b->total_q < 1) return 0;
  return smla::align_up(sizeof(int32_t) * (size_t)b->total_cand, 256) +
         smla::topk_workspace_bytes(*b, top_k);
}

int smla_indexer_scores_topk(const smla_batch* b, const int8_t* q_idx, const int8_t* k_idx,
                             const int32_t* w, int32_t H_I, int32_t D_I, int32_t top_k,
                             int32_t* idx, int32_t* score, void* ws, size_t ws_bytes,
                             void* stream) {
  g_err.clear();
  bool mfma = false;
  int rc = check_indexer_args(b, q_idx, k_idx, w, H_I, D_I, &mfma);
  if (rc) return rc;
  if (top_k < 1 || top_k > smla::TOPK_MAX_K)
    return fail(SMLA_E_UNSUPPORTED, "top_k=%d outside [1, %d]", top_k, smla::TOPK_MAX_K);
  if (b->max_kv > (int64_t)smla::TOPK_SEG * smla::TOPK_SEG_MAX)
    return fail(SMLA_E_UNSUPPORTED, "kv_len %lld above the top-k limit %lld", (long long)b->max_kv,
                (long long)smla::TOPK_SEG * smla::TOPK_SEG_MAX);
  if (!idx || !aligned(idx, 4) || (score && !aligned(score, 4)))
    return fail(SMLA_E_INVALID, "idx must be non-NULL; idx and score 4-byte aligned");
  const size_t need = smla_indexer_topk_workspace_bytes(b, H_I, D_I, top_k);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(SMLA_E_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", need, ws_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* scores = static_cast<int32_t*>(ws);
  void* tws = static_cast<char*>(ws) + smla::align_up(sizeof(int32_t) * (size_t)b->total_cand, 256);
  const smla::TopkWs tw = smla::topk_workspace(*b, tws);
  smla::mark_stage(smla::STAGE_INDEXER, false, s);
  hipError_t e = mfma ? smla::launch_indexer_mfma(*b, q_idx, k_idx, w, scores, 1, tw.hist, s)
           : smla::launch_indexer_generic(*b, q_idx, k_idx, w, H_I, D_I, scores, 1, tw.hist, s);
  smla::mark_stage(smla::STAGE_INDEXER, true, s);
  if (e != hipSuccess) return hip_fail(e, "indexer launch");
  smla::mark_stage(smla::STAGE_TOPK, false, s);
  e = smla::launch_topk(*b, scores, top_k, idx, score, tw, s);
  smla::mark_stage(smla::STAGE_TOPK, true, s);
  return e == hipSuccess ? SMLA_OK : hip_fail(e, "top-k launch");
}

static int check_indexer_fp8_args(const smla_batch* b, const uint8_t* q, const uint8_t* k,
                                  const float* k_scale, const float* w, int32_t H_I, int32_t D_I) {
  int rc = check_batch(b);
  if (rc) return rc;
  if (!q || !k || !k_scale || !w) return fail(SMLA_E_INVALID, "q, k, k_scale and w must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(k_scale, 4) || !aligned(w, 4))
    return fail(SMLA_E_INVALID, "q and k must be 16-byte aligned, k_scale and w 4-byte aligned");
  if (H_I != 64 || D_I != 128)
    return fail(SMLA_E_UNSUPPORTED, "FP8 indexer shape H_I=%d D_I=%d unsupported (64x128 only)", H_I, D_I);
  return SMLA_OK;
}

int smla_indexer_scores_fp8(const smla_batch* b, const uint8_t* q, const uint8_t* k,
                            const float* k_scale, const float* w, int32_t H_I, int32_t D_I,
                            float* scores, void* stream) {
  g_err.clear();
  int rc = check_indexer_fp8_args(b, q, k, k_scale, w, H_I, D_I);
  if (rc) return rc;
  if (!scores || !aligned(scores, 16)) return fail(SMLA_E_INVALID, "scores must be non-NULL, 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* out = reinterpret_cast<int32_t*>(scores);
  hipError_t e = smla::launch_fill_i32(out, (int64_t)b->total_q * b->max_kv, (int32_t)0xBF800000u, s);
  if (e == hipSuccess) e = smla::launch_indexer_fp8(*b, q, k, k_scale, w, out, 0, nullptr, s);
  return e == hipSuccess ? SMLA_OK : hip_fail(e, "indexer launch");
}

int smla_indexer_scores_topk_fp8(const smla_batch* b, const uint8_t* q, const uint8_t* k,
                                 const float* k_scale, const float* w, int32_t H_I, int32_t D_I,
                                 int32_t top_k, int32_t* idx, float* score, void* ws,
                                 size_t ws_bytes, void* stream) {
  g_err.clear();
  int rc = check_indexer_fp8_args(b, q, k, k_scale, w, H_I, D_I);
  if (rc) return rc;
  if (top_k < 1 || top_k > smla::TOPK_MAX_K)
    return fail(SMLA_E_UNSUPPORTED, "top_k=%d outside [1, %d]", top_k, smla::TOPK_MAX_K);
  if (b->max_kv > (int64_t)smla::TOPK_SEG * smla::TOPK_SEG_MAX)
    return fail(SMLA_E_UNSUPPORTED, "kv_len %lld above the top-k limit %lld", (long long)b->max_kv,
                (long long)smla::TOPK_SEG * smla::TOPK_SEG_MAX);
  if (!idx || !aligned(idx, 4) || (score && !aligned(score, 4)))
    return fail(SMLA_E_INVALID, "idx must be non-NULL; idx and score 4-byte aligned");
  const size_t need = smla_indexer_topk_workspace_bytes(b, H_I, D_I, top_k);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(SMLA_E_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", need, ws_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* scores = static_cast<int32_t*>(ws);
  void* tws = static_cast<char*>(ws) + smla::align_up(sizeof(int32_t) * (size_t)b->total_cand, 256);
  const smla::TopkWs tw = smla::topk_workspace(*b, tws);
  smla::mark_stage(smla::STAGE_INDEXER, false, s);
  hipError_t e = smla::launch_indexer_fp8(*b, q, k, k_scale, w, scores, 1, tw.hist, s);
  smla::mark_stage(smla::STAGE_INDEXER, true, s);
  if (e != hipSuccess) return hip_fail(e, "indexer launch");
  smla::mark_stage(smla::STAGE_TOPK, false, s);
  e = smla::launch_topk(*b, scores, top_k, idx, reinterpret_cast<int32_t*>(score), tw, s, true);
  smla::mark_stage(smla::STAGE_TOPK, true, s);
  return e == hipSuccess ? SMLA_OK : hip_fail(e, "top-k launch");
}

int smla_topk_merge(int32_t total_q, int32_t n_lists, int32_t k_in, const int32_t* idx_lists,
                    const int32_t* score_lists, int64_t list_stride, int32_t float_scores,
                    int32_t top_k, int32_t* idx, int32_t* score, int32_t* local_idx, void* stream) {
  g_err.clear();
  if (total_q < 1 || n_lists < 1 || k_in < 1 || top_k < 1)
    return fail(SMLA_E_INVALID, "total_q, n_lists, k_in and top_k must be >= 1");
  if ((int64_t)n_lists * k_in > smla::MERGE_MAX_CAND || top_k > smla::TOPK_MAX_K)
    return fail(SMLA_E_UNSUPPORTED, "n_lists * k_in = %lld above %d or top_k = %d above %d",
                (long long)n_lists * k_in, smla::MERGE_MAX_CAND, top_k, smla::TOPK_MAX_K);
  if (list_stride < (int64_t)total_q * k_in)
    return fail(SMLA_E_INVALID, "list_stride %lld below total_q * k_in", (long long)list_stride);
  if (!idx_lists || !score_lists || !idx || !aligned(idx_lists, 4) || !aligned(score_lists, 4) ||
      !aligned(idx, 4) || (score && !aligned(score, 4)))
    return fail(SMLA_E_INVALID, "idx_lists, score_lists and idx must be non-NULL, all 4-byte aligned");
  if (float_scores != 0 && float_scores != 1) return fail(SMLA_E_INVALID, "float_scores must be 0 or 1");
  if (local_idx && !aligned(local_idx, 4)) return fail(SMLA_E_INVALID, "local_idx must be 4-byte aligned");
  if (local_idx && n_lists > smla::MERGE_FAST_LISTS)
    return fail(SMLA_E_UNSUPPORTED, "local_idx needs n_lists <= %d (got %d)", smla::MERGE_FAST_LISTS,
                n_lists);
  hipError_t e = smla::launch_topk_merge(total_q, n_lists, k_in, idx_lists, score_lists, list_stride,
                                         top_k, idx, score, local_idx, float_scores != 0,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMLA_OK : hip_fail(e, "top-k merge launch");
}

int smla_dcp_local_indices(int32_t total_q, int32_t top_k, const int32_t* idx, int32_t n_shards,
                           int32_t* local_idx, void* stream) {
  g_err.clear();
  if (total_q < 1 || top_k < 1 || top_k > smla::TOPK_MAX_K || n_shards < 1 || n_shards > 65535)
    return fail(SMLA_E_INVALID, "need total_q >= 1, 1 <= top_k <= %d, 1 <= n_shards <= 65535",
                smla::TOPK_MAX_K);
  if (!idx || !local_idx || !aligned(idx, 4) || !aligned(local_idx, 4))
    return fail(SMLA_E_INVALID, "idx and local_idx must be non-NULL, 4-byte aligned");
  hipError_t e = smla::launch_local_indices(total_q, top_k, idx, n_shards, local_idx,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMLA_OK : hip_fail(e, "local indices launch");
}

int smla_hot_resolve(const smla_batch* b, const int32_t* idx, int32_t top_k,
                     const int32_t* resident_from, const int32_t* hot_base, int32_t n_slots,
                     int32_t* hot_tok, int32_t* hot_age, int32_t step, const void* host_rows,
                     int64_t host_n_rows, const int64_t* host_row0, int32_t row_bytes, void* kv,
                     int32_t* idx_out, int32_t* n_copied, void* stream) {
  g_err.clear();
  int rc = check_batch(b);
  if (rc) return rc;
  if (top_k < 1 || (int64_t)b->max_q * top_k > smla::HOT_MAX_SEL)
    return fail(SMLA_E_UNSUPPORTED, "need top_k >= 1 and max n_q * top_k <= %d", smla::HOT_MAX_SEL);
  if (n_slots < 1 || n_slots > smla::HOT_MAX_SLOTS)
    return fail(SMLA_E_UNSUPPORTED, "n_slots=%d outside [1, %d]", n_slots, smla::HOT_MAX_SLOTS);
  if (step < 0) return fail(SMLA_E_INVALID, "step must be >= 0 (-1 marks a slot never used)");
  if (row_bytes < 16 || row_bytes > 65536 || row_bytes % 16 != 0)
    return fail(SMLA_E_INVALID, "row_bytes=%d must be a multiple of 16 in [16, 65536]", row_bytes);
  if (host_n_rows < 0) return fail(SMLA_E_INVALID, "host_n_rows must be >= 0");
  if (!idx || !resident_from || !hot_base || !hot_tok || !hot_age || !host_rows || !host_row0 ||
      !kv || !idx_out || !n_copied)
    return fail(SMLA_E_INVALID, "null pointer");
  if (!aligned(idx, 4) || !aligned(resident_from, 4) || !aligned(hot_base, 4) ||
      !aligned(hot_tok, 4) || !aligned(hot_age, 4) || !aligned(host_row0, 8) ||
      !aligned(idx_out, 4) || !aligned(n_copied, 4) || !aligned(host_rows, 16) || !aligned(kv, 16))
    return fail(SMLA_E_INVALID, "misaligned pointer (host_rows and kv: 16 bytes)");
  if (idx_out == idx) return fail(SMLA_E_INVALID, "idx_out must not alias idx");
  // the kernel reads host rows directly: they must be pinned, device-mapped host memory
  hipPointerAttribute_t attr{};
  hipError_t e = hipPointerGetAttributes(&attr, host_rows);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost || !attr.devicePointer) {
    (void)hipGetLastError();
    return fail(SMLA_E_INVALID, "host_rows must be pinned host memory (hipHostMalloc)");
  }
  const void* dev_rows = attr.devicePointer;
  e = smla::launch_hot_resolve(b->table, b->batch, idx, top_k, resident_from, hot_base, n_slots,
                               hot_tok, hot_age, step, dev_rows, host_n_rows, host_row0, row_bytes,
                               kv, idx_out, n_copied, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMLA_OK : hip_fail(e, "hot resolve launch");
}

int smla_lse_merge(int32_t total_q, int32_t H, int32_t D_v, int32_t n_parts, const void* outs,
                   const float* lses, void* out, float* lse, void* stream) {
  g_err.clear();
  if (total_q < 1 || H < 1 || D_v < 1 || D_v > 4096 || n_parts < 1 || n_parts > 64)
    return fail(SMLA_E_INVALID, "need total_q, H >= 1, 1 <= D_v <= 4096, 1 <= n_parts <= 64");
  if (!outs || !lses || !out || !aligned(outs, 2) || !aligned(lses, 4) || !aligned(out, 2) ||
      (lse && !aligned(lse, 4)))
    return fail(SMLA_E_INVALID, "outs, lses and out must be non-NULL and aligned");
  hipError_t e = smla::launch_lse_merge(total_q, H, D_v, n_parts, outs, lses, out, lse,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMLA_OK : hip_fail(e, "lse merge launch");
}

size_t smla_sparse_mla_workspace_bytes(const smla_batch* b, int32_t H, int32_t D_v, int32_t top_k,
                                       int32_t decode) {
  if (!b || b->total_q < 1 || top_k < 1) return 0;
  return smla::mla_workspace_bytes(*b, H, D_v, top_k, decode);
}

static int sparse_mla(const smla_batch* b, const void* q, const void* kv, int32_t kv_format,
                      int32_t H, int32_t D_qk, int32_t D_v, const int32_t* idx, int32_t top_k,
                      float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                      void* stream, int decode) {
  g_err.clear();
  bool fp8 = false;
  int rc = check_mla_args(b, q, kv, kv_format, H, D_qk, D_v, idx, top_k, out, &fp8);
  if (rc) return rc;
  if (lse && !aligned(lse, 4)) return fail(SMLA_E_INVALID, "lse must be 4-byte aligned");
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return fail(SMLA_E_INVALID, "sm_scale must be positive and finite");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (fp8) {
    const size_t need = smla::mla_workspace_bytes(*b, H, D_v, top_k, decode);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 256)))
      return fail(SMLA_E_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", need, ws_bytes);
    e = smla::launch_mla_fp8(*b, q, kv, idx, top_k, sm_scale, out, lse, ws, decode, s);
  } else {
    smla::mark_stage(smla::STAGE_MLA, false, s);
    e = smla::launch_mla_generic(*b, q, kv, H, D_qk, D_v, idx, top_k, sm_scale, out, lse, s);
    smla::mark_stage(smla::STAGE_MLA, true, s);
  }
  return e == hipSuccess ? SMLA_OK : hip_fail(e, "sparse MLA launch");
}

int smla_sparse_mla_prefill(const smla_batch* b, const void* q, const void* kv, int32_t kv_format,
                            int32_t H, int32_t D_qk, int32_t D_v, const int32_t* idx,
                            int32_t top_k, float sm_scale, void* out, float* lse, void* ws,
                            size_t ws_bytes, void* stream) {
  return sparse_mla(b, q, kv, kv_format, H, D_qk, D_v, idx, top_k, sm_scale, out, lse, ws,
                    ws_bytes, stream, 0);
}

int smla_sparse_mla_decode(const smla_batch* b, const void* q, const void* kv, int32_t kv_format,
                           int32_t H, int32_t D_qk, int32_t D_v, const int32_t* idx,
                           int32_t top_k, float sm_scale, void* out, float* lse, void* ws,
                           size_t ws_bytes, void* stream) {
  return sparse_mla(b, q, kv, kv_format, H, D_qk, D_v, idx, top_k, sm_scale, out, lse, ws,
                    ws_bytes, stream, 1);
}

int smla_sparse_mla_decode_noalloc(const smla_batch* b, const void* q, const void* kv,
                                   int32_t kv_format, int32_t H, int32_t D_qk, int32_t D_v,
                                   const int32_t* idx, int32_t top_k, float sm_scale, void* out,
                                   float* lse, void* stream) {
  g_err.clear();
  bool fp8 = false;
  int rc = check_mla_args(b, q, kv, kv_format, H, D_qk, D_v, idx, top_k, out, &fp8);
  if (rc) return rc;
  void* ws = nullptr;
  size_t need = 0;
  if (fp8) {
    need = smla::mla_workspace_bytes(*b, H, D_v, top_k, 1);
    if (need > smla::mla_scratch_bytes())
      return fail(SMLA_E_UNSUPPORTED, "decode split partials need %zu bytes, the built-in scratch holds %zu",
                  need, smla::mla_scratch_bytes());
    if (need) {
      hipError_t e = smla::mla_scratch(&ws);
      if (e != hipSuccess) return hip_fail(e, "scratch address");
    }
  }
  return sparse_mla(b, q, kv, kv_format, H, D_qk, D_v, idx, top_k, sm_scale, out, lse, ws, need,
                    stream, 1);
}

int smla_kv_append(int64_t n, const void* latent, const int8_t* k_new, int32_t D_I,
                   const int64_t* rows, void* kv, int8_t* k_idx, void* stream) {
  g_err.clear();
  if (n < 0 || n > (int64_t(1) << 33)) return fail(SMLA_E_INVALID, "n=%lld outside [0, 2^33]", (long long)n);
  if (n == 0) return SMLA_OK;
  if (!latent || !rows || !kv) return fail(SMLA_E_INVALID, "latent, rows and kv must be non-NULL");
  if (!aligned(latent, 16) || !aligned(kv, 16) || !aligned(rows, 8))
    return fail(SMLA_E_INVALID, "latent and kv must be 16-byte aligned, rows 8-byte aligned");
  if (k_new) {
    if (!k_idx) return fail(SMLA_E_INVALID, "k_idx must be non-NULL when k_new is given");
    if (D_I < 16 || D_I > 1024 || D_I % 16)
      return fail(SMLA_E_UNSUPPORTED, "D_I=%d: indexer keys must be a multiple of 16 bytes, at most 1024", D_I);
    if (!aligned(k_new, 16) || !aligned(k_idx, 16))
      return fail(SMLA_E_INVALID, "k_new and k_idx must be 16-byte aligned");
  }
  hipError_t e = smla::launch_kv_append(n, latent, rows, kv, k_new, D_I, k_idx,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMLA_OK : hip_fail(e, "kv append launch");
}

const char* smla_status_str(int status) {
  switch (status) {
    case SMLA_OK: return "SMLA_OK";
    case SMLA_E_INVALID: return "SMLA_E_INVALID";
    case SMLA_E_UNSUPPORTED: return "SMLA_E_UNSUPPORTED";
    case SMLA_E_WORKSPACE: return "SMLA_E_WORKSPACE";
    case SMLA_E_HIP: return "SMLA_E_HIP";
    default: return "SMLA_E_UNKNOWN";
  }
}

const char* smla_last_error(void) { return g_err.c_str(); }

int32_t smla_version(void) { return 100; }

}  // extern "C"
