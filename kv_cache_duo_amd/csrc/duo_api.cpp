// Host side of the C ABI declared in include/duo.h: validation, head
// partition, region layout, host length mirror and kernel launch ordering.
//
// Head kinds come from the offline identification that DuoAttention runs on
// synthetic data (sourcepulse card, "How It Works"); here they are an input.
// Retrieval KV heads get a full contiguous cache, streaming KV heads a
// constant-length sink + ring cache (DuoAttention abstract).  Every check
// runs before anything is enqueued, so a call that fails validation changes
// nothing; a call whose launch fails (DUO_ERR_HIP) keeps the handle's
// lengths and pages as they were.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "duo.h"
#include "duo_internal.h"

struct duo_cache {
  duo_config cfg;
  std::vector<uint8_t> mask;
  duo::Geom geom;
  duo_layout layout;
  std::vector<int64_t> len;  // host mirror of the stored tokens per sequence
  int32_t* buf_words;        // the device buffer, as int32 words
  // paged retrieval cache: free pool pages (used from the back) and the
  // pages of every sequence in position order (host mirror of page_table)
  std::vector<int32_t> free_pages;
  std::vector<std::vector<int32_t>> seq_pages;
  int32_t num_cus;  // compute units of the current device when the handle was made (decode split planning)
};

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kMaxLen = int64_t(1) << 30;

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Compute units of the current device, or 256 (an MI355X) when no device
// answers: the count only shapes how decode splits its rows.
int32_t device_compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || cus <= 0) {
    (void)hipGetLastError();  // clear the error the query left
    return 256;
  }
  return cus;
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

duo_status check_config(const duo_config* c) {
  if (c == nullptr) return DUO_ERR_INVALID_ARG;
  if (c->batch < 1 || c->num_kv_heads < 1 || c->num_q_heads < 1) return DUO_ERR_INVALID_ARG;
  if (c->num_q_heads % c->num_kv_heads != 0) return DUO_ERR_INVALID_ARG;
  if (c->sink < 0 || c->recent < 1 || c->max_len < 1) return DUO_ERR_INVALID_ARG;
  if (!(c->scale >= 0.f) || !std::isfinite(c->scale)) return DUO_ERR_INVALID_ARG;
  if (c->kv_head_is_retrieval == nullptr) return DUO_ERR_INVALID_ARG;
  if (c->kv_format != DUO_KV_BF16 && c->kv_format != DUO_KV_INT8 && c->kv_format != DUO_KV_FP8)
    return DUO_ERR_INVALID_ARG;
  for (float sc : {c->kv_scale_k, c->kv_scale_v}) {
    if (sc == 0.f) continue;
    int e = 0;
    if (!std::isfinite(sc) || !(sc > 0.f) || std::frexp(sc, &e) != 0.5f || e - 1 < -32 || e - 1 > 32)
      return DUO_ERR_INVALID_ARG;
  }
  if (c->fp8_prefill != DUO_FP8_PREFILL_EXACT && c->fp8_prefill != DUO_FP8_PREFILL_MFMA) return DUO_ERR_INVALID_ARG;
  if (c->decode_split != DUO_DECODE_STATIC && c->decode_split != DUO_DECODE_DYNAMIC) return DUO_ERR_INVALID_ARG;
  if (c->prefill_staging_bytes < 0 || (c->prefill_staging != nullptr && !aligned16(c->prefill_staging)))
    return DUO_ERR_INVALID_ARG;
  if (!(c->rope_base >= 0.f) || !std::isfinite(c->rope_base)) return DUO_ERR_INVALID_ARG;
  if (c->rope_base > 0.f && c->rope_style != DUO_ROPE_INTERLEAVED && c->rope_style != DUO_ROPE_HALF)
    return DUO_ERR_INVALID_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return DUO_ERR_UNSUPPORTED;
  if (c->batch > DUO_MAX_BATCH || c->num_kv_heads > duo::kMaxKvHeads) return DUO_ERR_UNSUPPORTED;
  if (c->max_len > kMaxLen || (int64_t)c->sink + c->recent > kMaxLen) return DUO_ERR_UNSUPPORTED;
  if (c->page_tokens != 0) {
    const int32_t p = c->page_tokens;
    if (p < 512 || p > 65536 || (p & (p - 1)) != 0) return DUO_ERR_INVALID_ARG;
    if (c->num_pages < 1 || c->num_pages > (int64_t(1) << 31) - 1) return DUO_ERR_INVALID_ARG;
  }
  return DUO_OK;
}

// Fill geometry and layout for a config (no device pointers yet).
void plan_layout(const duo_config* c, duo::Geom* g, duo_layout* L) {
  std::memset(g, 0, sizeof(*g));
  std::memset(L, 0, sizeof(*L));
  g->B = c->batch;
  g->Hq = c->num_q_heads;
  g->Hkv = c->num_kv_heads;
  g->G = c->num_q_heads / c->num_kv_heads;
  g->D = c->head_dim;
  g->S = c->sink;
  g->W = c->recent;
  g->slots = c->sink + c->recent;
  g->max_len = c->max_len;
  const float scale = c->scale > 0.f ? c->scale : 1.0f / std::sqrt((float)c->head_dim);
  g->scale_log2 = scale * 1.4426950408889634f;
  int nr = 0, ns = 0;
  for (int k = 0; k < c->num_kv_heads; ++k)
    if (c->kv_head_is_retrieval[k]) g->index_of_kv[k] = (uint8_t)nr++, g->is_retrieval[k] = 1;
  for (int k = 0; k < c->num_kv_heads; ++k)
    if (!c->kv_head_is_retrieval[k]) g->index_of_kv[k] = (uint8_t)ns++, g->is_retrieval[k] = 0;
  for (int k = 0; k < c->num_kv_heads; ++k)
    g->kv_of_unit[g->is_retrieval[k] ? g->index_of_kv[k] : nr + g->index_of_kv[k]] = (uint8_t)k;
  g->nR = nr;
  g->nS = ns;
  g->kv_int8 = c->kv_format == DUO_KV_INT8;
  g->kv_fp8 = c->kv_format == DUO_KV_FP8;
  g->fp8_mfma = g->kv_fp8 && c->fp8_prefill == DUO_FP8_PREFILL_MFMA;
  g->decode_dynamic = c->decode_split == DUO_DECODE_DYNAMIC;
  if ((g->kv_int8 || g->kv_fp8 || c->rope_base > 0.f) && c->prefill_staging != nullptr) {
    g->prefill_staging = static_cast<uint16_t*>(c->prefill_staging);
    g->prefill_staging_bytes = c->prefill_staging_bytes;
  }
  {
    const float sk = c->kv_scale_k > 0.f ? c->kv_scale_k : 1.f, sv = c->kv_scale_v > 0.f ? c->kv_scale_v : 1.f;
    int ek = 0, ev = 0;
    std::frexp(sk, &ek);
    std::frexp(sv, &ev);
    g->fp8_exp_k = ek - 1;
    g->fp8_exp_v = ev - 1;
    g->fp8_scale_k = sk;
    g->fp8_scale_v = sv;
    g->fp8_inv_k = 1.f / sk;  // exact: powers of two
    g->fp8_inv_v = 1.f / sv;
  }
  g->rope = c->rope_base > 0.f;
  g->rope_half = g->rope && c->rope_style == DUO_ROPE_HALF;
  g->rope_rho = g->rope ? std::pow((double)c->rope_base, -2.0 / c->head_dim) : 0.0;
  g->max_splits = duo::max_splits_for(c->max_len, g->slots, duo::decode_head_chunk(g->G, g->kv_int8 || g->kv_fp8));

  const int gc = duo::decode_head_chunk(g->G, g->kv_int8 || g->kv_fp8);
  const int64_t units = (int64_t)g->B * g->Hkv * (g->G / gc);
  int64_t off = 0;
  L->lengths_offset = off;
  off = align_up(off + 4 * (int64_t)g->B);
  // paged: page table right after the lengths (word indices stay small)
  L->page_table_offset = -1;
  g->paged = c->page_tokens > 0;
  // retrieval rows per head: max_len per sequence, or whole blocks of
  // 2^kBlockShift positions when longer than one block
  const int64_t blk = int64_t(1) << duo::kBlockShift;
  g->nblk = g->max_len > blk ? (int32_t)((g->max_len + blk - 1) / blk) : 1;
  L->block_tokens = g->nblk > 1 ? (int32_t)blk : 0;
  int64_t pool_rows = g->nblk > 1 ? (int64_t)g->B * g->nblk * blk : (int64_t)g->B * g->max_len;
  if (g->paged) {
    int shift = 0;
    while ((1 << shift) < c->page_tokens) ++shift;
    g->page_shift = shift;
    g->max_pages = (int32_t)((c->max_len + c->page_tokens - 1) / c->page_tokens);
    L->page_tokens = c->page_tokens;
    L->max_pages_per_seq = g->max_pages;
    L->num_pages = c->num_pages;
    L->page_table_offset = off;
    off = align_up(off + 4 * (int64_t)g->B * g->max_pages);
    pool_rows = c->num_pages * c->page_tokens;
    g->nblk = 1;
    L->block_tokens = 0;
  }
  L->work_offset = off;  // merge tickets, then the split records
  g->tickets_per_unit = duo::tickets_per_unit(g->max_splits);
  off = align_up(off + 4 * units * g->tickets_per_unit);
  L->work_records_offset = off;
  off = align_up(off + 4 * units * g->max_splits * gc * (g->D + 2));
  L->work_bytes = off - L->work_offset;
  const int64_t row = 2 * (int64_t)g->D;
  const int64_t rrow = (g->kv_int8 || g->kv_fp8) ? (int64_t)g->D : row;  // retrieval row bytes
  L->kv_format = c->kv_format;
  L->rk_offset = off;
  off = align_up(off + pool_rows * nr * rrow);
  L->rv_offset = off;
  off = align_up(off + pool_rows * nr * rrow);
  L->rks_offset = L->rvs_offset = -1;
  if (g->kv_int8) {
    L->rks_offset = off;
    off = align_up(off + pool_rows * nr * 4);
    L->rvs_offset = off;
    off = align_up(off + pool_rows * nr * 4);
  }
  L->sk_offset = off;
  off = align_up(off + (int64_t)g->B * ns * g->slots * row);
  L->sv_offset = off;
  off = align_up(off + (int64_t)g->B * ns * g->slots * row);
  L->total_bytes = off;
  // the staging workspace of a prefill that reads rows up to max_len: int8
  // rows as bf16 K and V, and with rotary embedding the streaming heads'
  // turned chunk K rows
  L->prefill_staging_bytes = ((g->kv_int8 || (g->kv_fp8 && !g->fp8_mfma)) ? 4 * (int64_t)g->B * nr * g->D * g->max_len
                                                                           : 0) +
                             (c->rope_base > 0.f ? 2 * (int64_t)g->B * ns * g->D * g->max_len : 0);
  L->n_retrieval = nr;
  L->n_streaming = ns;
  L->slots_per_streaming_head = g->slots;
}

void bind_device(duo::Geom* g, const duo_layout& L, void* buf) {
  char* base = static_cast<char*>(buf);
  g->lengths = reinterpret_cast<int32_t*>(base + L.lengths_offset);
  g->tickets = reinterpret_cast<uint32_t*>(base + L.work_offset);
  g->partials = reinterpret_cast<float*>(base + L.work_records_offset);
  g->rk = reinterpret_cast<uint16_t*>(base + L.rk_offset);
  g->rv = reinterpret_cast<uint16_t*>(base + L.rv_offset);
  g->rks = L.rks_offset >= 0 ? reinterpret_cast<float*>(base + L.rks_offset) : nullptr;
  g->rvs = L.rvs_offset >= 0 ? reinterpret_cast<float*>(base + L.rvs_offset) : nullptr;
  g->sk = reinterpret_cast<uint16_t*>(base + L.sk_offset);
  g->sv = reinterpret_cast<uint16_t*>(base + L.sv_offset);
  g->page_table = L.page_table_offset >= 0 ? reinterpret_cast<const int32_t*>(base + L.page_table_offset) : nullptr;
}

duo_status new_handle(const duo_config* cfg, void* buf, size_t bytes, const int64_t* lengths, duo_cache** out,
                      bool zero, void* stream) {
  duo_status st = check_config(cfg);
  if (st != DUO_OK) return st;
  if (out == nullptr) return DUO_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) % kAlign) != 0) return DUO_ERR_INVALID_ARG;
  duo::Geom g;
  duo_layout L;
  plan_layout(cfg, &g, &L);
  if ((int64_t)bytes < L.total_bytes) return DUO_ERR_BUFFER_TOO_SMALL;
  if (lengths != nullptr)
    for (int b = 0; b < cfg->batch; ++b)
      if (lengths[b] < 0 || lengths[b] > cfg->max_len || (cfg->page_tokens > 0 && lengths[b] != 0))
        return DUO_ERR_INVALID_ARG;
  duo_cache* h = new (std::nothrow) duo_cache;
  if (h == nullptr) return DUO_ERR_INVALID_ARG;
  h->cfg = *cfg;
  h->mask.assign(cfg->kv_head_is_retrieval, cfg->kv_head_is_retrieval + cfg->num_kv_heads);
  h->cfg.kv_head_is_retrieval = h->mask.data();
  h->geom = g;
  h->layout = L;
  bind_device(&h->geom, L, buf);
  h->len.assign(cfg->batch, 0);
  if (lengths != nullptr)
    for (int b = 0; b < cfg->batch; ++b) h->len[b] = lengths[b];
  h->buf_words = static_cast<int32_t*>(buf);
  h->num_cus = device_compute_units();
  h->seq_pages.assign(cfg->batch, {});
  if (h->geom.paged) {
    h->free_pages.resize((size_t)cfg->num_pages);
    for (int64_t i = 0; i < cfg->num_pages; ++i) h->free_pages[(size_t)i] = (int32_t)(cfg->num_pages - 1 - i);
  }
  if (zero) {
    // lengths, then the merge tickets (contiguous up to the split records)
    const int64_t words = (reinterpret_cast<char*>(h->geom.partials) - reinterpret_cast<char*>(h->geom.lengths)) / 4;
    hipError_t e = duo::launch_zero_words(reinterpret_cast<uint32_t*>(h->geom.lengths), words,
                                          static_cast<hipStream_t>(stream));
    // set up this device's static decode scratch now (look-up and zeroing,
    // once per device), so that duo_decode_static_scratch itself only uses it
    void* scratch = nullptr;
    if (e == hipSuccess) e = duo::static_decode_scratch(&scratch, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
      delete h;
      return DUO_ERR_HIP;
    }
  }
  *out = h;
  return DUO_OK;
}

}  // namespace

namespace duo {
void finish_seqs(Seqs& q, int32_t batch) {
  int32_t idx[DUO_MAX_BATCH];
  int32_t n = 0;
  for (int b = 0; b < batch; ++b)
    if (q.n[b] > 0) idx[n++] = b;
  // longest stored prefix first (then the most new tokens); stable
  for (int i = 1; i < n; ++i) {
    const int32_t x = idx[i];
    int j = i;
    while (j > 0 && (q.len[idx[j - 1]] < q.len[x] || (q.len[idx[j - 1]] == q.len[x] && q.n[idx[j - 1]] < q.n[x]))) {
      idx[j] = idx[j - 1];
      --j;
    }
    idx[j] = x;
  }
  q.nact = n;
  q.uniform = 1;
  for (int i = 0; i < n; ++i) {
    q.act[i] = idx[i];
    if (q.len[idx[i]] != q.len[idx[0]] || q.n[idx[i]] != q.n[idx[0]]) q.uniform = 0;
  }
}
}  // namespace duo

namespace {

// Shared validation of a chunk call; fills the sequence table.
duo_status check_chunk(const duo_cache* h, const int32_t* n_new, int32_t chunk, duo::Seqs* sq, int32_t* max_n) {
  if (chunk < 1) return DUO_ERR_INVALID_ARG;
  if (n_new == nullptr) return DUO_ERR_INVALID_ARG;
  if ((int64_t)h->cfg.batch * chunk > INT32_MAX) return DUO_ERR_UNSUPPORTED;  // row offsets b * chunk are int32
  int32_t mx = 0;
  for (int b = 0; b < h->cfg.batch; ++b) {
    if (n_new[b] < 0 || n_new[b] > chunk) return DUO_ERR_INVALID_ARG;
    if (h->len[b] + n_new[b] > h->cfg.max_len) return DUO_ERR_CAPACITY;
    mx = n_new[b] > mx ? n_new[b] : mx;
  }
  std::memset(sq, 0, sizeof(*sq));
  for (int b = 0; b < h->cfg.batch; ++b) {
    sq->len[b] = (int32_t)h->len[b];
    sq->n[b] = n_new[b];
    sq->off[b] = b * chunk;
  }
  duo::finish_seqs(*sq, h->cfg.batch);
  *max_n = mx;
  return DUO_OK;
}

// Packed inputs: cu_seqlens[B+1] host, from 0, nondecreasing.
duo_status check_varlen(const duo_cache* h, const int32_t* cu, duo::Seqs* sq, int32_t* max_n) {
  if (cu == nullptr || cu[0] != 0) return DUO_ERR_INVALID_ARG;
  int32_t mx = 0;
  for (int b = 0; b < h->cfg.batch; ++b) {
    const int64_t n = (int64_t)cu[b + 1] - cu[b];
    if (n < 0) return DUO_ERR_INVALID_ARG;
    if (h->len[b] + n > h->cfg.max_len) return DUO_ERR_CAPACITY;
    mx = n > mx ? (int32_t)n : mx;
  }
  std::memset(sq, 0, sizeof(*sq));
  for (int b = 0; b < h->cfg.batch; ++b) {
    sq->len[b] = (int32_t)h->len[b];
    sq->n[b] = cu[b + 1] - cu[b];
    sq->off[b] = cu[b];
  }
  duo::finish_seqs(*sq, h->cfg.batch);
  *max_n = mx;
  return DUO_OK;
}

// Paged cache: pages that the call's new tokens need, checked before
// anything is enqueued.
duo_status check_pages(const duo_cache* h, const duo::Seqs& sq) {
  if (!h->geom.paged) return DUO_OK;
  const int64_t p = h->cfg.page_tokens;
  int64_t need = 0;
  for (int b = 0; b < h->cfg.batch; ++b) {
    const int64_t pages = ((int64_t)sq.len[b] + sq.n[b] + p - 1) / p;
    need += pages - (int64_t)h->seq_pages[b].size();
  }
  return need <= (int64_t)h->free_pages.size() ? DUO_OK : DUO_ERR_CAPACITY;
}

// Page ownership before a call, to undo take_pages when a later launch of
// the same call fails: the handle then keeps its pages and lengths.
struct PageMark {
  std::vector<size_t> held;  // seq_pages[b].size() before the call
};
PageMark mark_pages(const duo_cache* h) {
  PageMark m;
  if (h->geom.paged) {
    m.held.resize(h->seq_pages.size());
    for (size_t b = 0; b < h->seq_pages.size(); ++b) m.held[b] = h->seq_pages[b].size();
  }
  return m;
}
// Give back the pages taken since `m`, restoring the free list's order
// (take_pages popped them from its back in sequence order).
void rollback_pages(duo_cache* h, const PageMark& m) {
  if (!h->geom.paged) return;
  for (size_t b = h->seq_pages.size(); b-- > 0;)
    while (h->seq_pages[b].size() > m.held[b]) {
      h->free_pages.push_back(h->seq_pages[b].back());
      h->seq_pages[b].pop_back();
    }
}

// Take the pages (check_pages passed) and enqueue the page-table writes.
// On a failed launch the caller rolls the host state back (rollback_pages);
// table entries already written name positions past the stored lengths,
// whose entries are unspecified.
hipError_t take_pages(duo_cache* h, const duo::Seqs& sq, hipStream_t s) {
  if (!h->geom.paged) return hipSuccess;
  const int64_t p = h->cfg.page_tokens;
  const int64_t table_word = h->layout.page_table_offset / 4;
  duo::WordWrites w;
  w.n = 0;
  for (int b = 0; b < h->cfg.batch; ++b) {
    const int64_t pages = ((int64_t)sq.len[b] + sq.n[b] + p - 1) / p;
    while ((int64_t)h->seq_pages[b].size() < pages) {
      const int32_t page = h->free_pages.back();
      h->free_pages.pop_back();
      w.index[w.n] = (int32_t)(table_word + (int64_t)b * h->geom.max_pages + (int64_t)h->seq_pages[b].size());
      w.value[w.n] = page;
      ++w.n;
      h->seq_pages[b].push_back(page);
      if (w.n == duo::kWordWritesPerLaunch) {
        hipError_t e = duo::launch_word_writes(h->buf_words, w, s);
        if (e != hipSuccess) return e;
        w.n = 0;
      }
    }
  }
  return w.n > 0 ? duo::launch_word_writes(h->buf_words, w, s) : hipSuccess;
}

// The kernels of one append call (validated: sq, max_n).
duo_status append_call(duo_cache* h, const duo::Seqs& sq, int32_t max_n, const void* k, const void* v, void* stream) {
  duo_status st = check_pages(h, sq);
  if (st != DUO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PageMark mark = mark_pages(h);
  hipError_t e = take_pages(h, sq, s);
  if (e == hipSuccess)
    e = duo::launch_append(h->geom, sq, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), max_n, s);
  if (e != hipSuccess) {
    rollback_pages(h, mark);
    return DUO_ERR_HIP;
  }
  for (int b = 0; b < h->cfg.batch; ++b) h->len[b] += sq.n[b];
  return DUO_OK;
}

// The kernels of one prefill call (validated: sq, max_n).
duo_status prefill_call(duo_cache* h, const duo::Seqs& sq, int32_t max_n, const void* q, const void* k, const void* v,
                        void* out, void* stream) {
  duo_status st = check_pages(h, sq);
  if (st != DUO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PageMark mark = mark_pages(h);
  hipError_t e = take_pages(h, sq, s);
  if (e != hipSuccess) {
    rollback_pages(h, mark);
    return DUO_ERR_HIP;
  }
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  // Streaming heads read ring slots that this chunk's append overwrites, so
  // their rows are stored after the attention.  With rotary embedding the
  // retrieval rows are stored (rotated) first and the attention reads every
  // retrieval key from the cache; streaming heads rotate their chunk rows
  // as they load them.
  // A bf16 or fp8 cache stores the retrieval rows first as well: its
  // prefill reads every retrieval key and value as stored (contiguous rows
  // of one head, rather than rows strided by the input's heads).  An int8
  // cache without rotary embedding attends its chunk's own rows at input
  // precision, read from the input.
  const bool store_first = h->geom.rope || !h->geom.kv_int8;
  if (store_first) e = duo::launch_append(h->geom, sq, kk, vv, max_n, s, duo::kAppendRetrieval);
  if (e == hipSuccess)
    e = duo::launch_prefill(h->geom, sq, static_cast<const uint16_t*>(q), kk, vv, max_n, static_cast<uint16_t*>(out),
                            s);
  if (e == hipSuccess)
    e = duo::launch_append(h->geom, sq, kk, vv, max_n, s,
                           store_first ? duo::kAppendStreaming : duo::kAppendRetrieval | duo::kAppendStreaming);
  if (e != hipSuccess) {
    rollback_pages(h, mark);
    return DUO_ERR_HIP;
  }
  for (int b = 0; b < h->cfg.batch; ++b) h->len[b] += sq.n[b];
  return DUO_OK;
}

// One decode call.  static_scratch: the split counters and records live in
// the library's static device array (duo_decode_static_scratch) instead of
// the cache buffer's work region.
duo_status decode_call(duo_cache* h, const void* q, const void* k, const void* v, void* out, void* stream,
                       bool static_scratch) {
  if (h == nullptr || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return DUO_ERR_INVALID_ARG;
  for (int b = 0; b < h->cfg.batch; ++b)
    if (h->len[b] + 1 > h->cfg.max_len) return DUO_ERR_CAPACITY;
  duo::Seqs sq;
  std::memset(&sq, 0, sizeof(sq));
  for (int b = 0; b < h->cfg.batch; ++b) {
    sq.len[b] = (int32_t)h->len[b];
    sq.n[b] = 1;
    sq.off[b] = b;
  }
  duo::finish_seqs(sq, h->cfg.batch);
  duo_status st = check_pages(h, sq);
  if (st != DUO_OK) return st;
  duo::Geom g = h->geom;
  if (static_scratch) {
    const int64_t units = (int64_t)g.B * g.Hkv * (g.G / duo::decode_head_chunk(g.G, g.kv_int8 || g.kv_fp8));
    const int64_t gc = duo::decode_head_chunk(g.G, g.kv_int8 || g.kv_fp8);
    if (4 * units * g.tickets_per_unit > duo::kStaticTicketBytes ||
        4 * units * g.max_splits * gc * (g.D + 2) > duo::kStaticRecordBytes)
      return DUO_ERR_UNSUPPORTED;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PageMark mark = mark_pages(h);
  hipError_t e = hipSuccess;
  if (static_scratch) {
    void* base = nullptr;
    e = duo::static_decode_scratch(&base, s);
    if (e == hipSuccess) {
      g.tickets = static_cast<uint32_t*>(base);
      g.partials = reinterpret_cast<float*>(static_cast<char*>(base) + duo::kStaticTicketBytes);
    }
  }
  if (e == hipSuccess) e = take_pages(h, sq, s);
  if (e == hipSuccess) {
    const duo::DecodePlan p = duo::plan_decode(g, sq, h->num_cus);
    e = duo::launch_decode(g, sq, p, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), s);
  }
  if (e != hipSuccess) {
    rollback_pages(h, mark);
    return DUO_ERR_HIP;
  }
  for (int b = 0; b < h->cfg.batch; ++b) h->len[b] += 1;
  return DUO_OK;
}

}  // namespace

extern "C" {

const char* duo_status_string(duo_status s) {
  switch (s) {
    case DUO_OK: return "ok";
    case DUO_ERR_INVALID_ARG: return "invalid argument";
    case DUO_ERR_UNSUPPORTED: return "unsupported configuration";
    case DUO_ERR_BUFFER_TOO_SMALL: return "device buffer too small";
    case DUO_ERR_CAPACITY: return "sequence would exceed max_len (or the page pool is used up)";
    case DUO_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

duo_status duo_cache_init(const duo_config* cfg, void* dev_buf, size_t buf_bytes, size_t* required_bytes,
                          duo_cache** out, void* stream) {
  duo_status st = check_config(cfg);
  if (st != DUO_OK) return st;
  duo::Geom g;
  duo_layout L;
  plan_layout(cfg, &g, &L);
  if (required_bytes != nullptr) *required_bytes = (size_t)L.total_bytes;
  if (dev_buf == nullptr) return required_bytes != nullptr ? DUO_OK : DUO_ERR_INVALID_ARG;
  return new_handle(cfg, dev_buf, buf_bytes, nullptr, out, true, stream);
}

duo_status duo_cache_attach(const duo_config* cfg, void* dev_buf, size_t buf_bytes, const int64_t* lengths,
                            duo_cache** out) {
  if (dev_buf == nullptr || lengths == nullptr) return DUO_ERR_INVALID_ARG;
  return new_handle(cfg, dev_buf, buf_bytes, lengths, out, false, nullptr);
}

void duo_cache_destroy(duo_cache* h) { delete h; }

duo_status duo_cache_release(duo_cache* h, int32_t b, void* stream) {
  if (h == nullptr || b < 0 || b >= h->cfg.batch) return DUO_ERR_INVALID_ARG;
  duo::WordWrites w;
  w.n = 1;
  w.index[0] = (int32_t)(h->layout.lengths_offset / 4 + b);
  w.value[0] = 0;
  if (duo::launch_word_writes(h->buf_words, w, static_cast<hipStream_t>(stream)) != hipSuccess) return DUO_ERR_HIP;
  for (auto it = h->seq_pages[b].rbegin(); it != h->seq_pages[b].rend(); ++it) h->free_pages.push_back(*it);
  h->seq_pages[b].clear();
  h->len[b] = 0;
  return DUO_OK;
}

duo_status duo_cache_append(duo_cache* h, const void* k, const void* v, const int32_t* n_new, int32_t chunk,
                            void* stream) {
  if (h == nullptr || !aligned16(k) || !aligned16(v)) return DUO_ERR_INVALID_ARG;
  duo::Seqs sq;
  int32_t max_n = 0;
  duo_status st = check_chunk(h, n_new, chunk, &sq, &max_n);
  if (st != DUO_OK) return st;
  return append_call(h, sq, max_n, k, v, stream);
}

duo_status duo_cache_append_varlen(duo_cache* h, const void* k, const void* v, const int32_t* cu_seqlens,
                                   void* stream) {
  if (h == nullptr) return DUO_ERR_INVALID_ARG;
  duo::Seqs sq;
  int32_t max_n = 0;
  duo_status st = check_varlen(h, cu_seqlens, &sq, &max_n);
  if (st != DUO_OK) return st;
  if (max_n == 0) return DUO_OK;  // no rows: nothing to do (the pointers may be null)
  if (!aligned16(k) || !aligned16(v)) return DUO_ERR_INVALID_ARG;
  return append_call(h, sq, max_n, k, v, stream);
}

duo_status duo_prefill(duo_cache* h, const void* q, const void* k, const void* v, const int32_t* n_new,
                       int32_t chunk, void* out, void* stream) {
  if (h == nullptr || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return DUO_ERR_INVALID_ARG;
  duo::Seqs sq;
  int32_t max_n = 0;
  duo_status st = check_chunk(h, n_new, chunk, &sq, &max_n);
  if (st != DUO_OK) return st;
  return prefill_call(h, sq, max_n, q, k, v, out, stream);
}

duo_status duo_prefill_varlen(duo_cache* h, const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                              void* out, void* stream) {
  if (h == nullptr) return DUO_ERR_INVALID_ARG;
  duo::Seqs sq;
  int32_t max_n = 0;
  duo_status st = check_varlen(h, cu_seqlens, &sq, &max_n);
  if (st != DUO_OK) return st;
  if (max_n == 0) return DUO_OK;  // no rows: nothing to do (the pointers may be null)
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return DUO_ERR_INVALID_ARG;
  return prefill_call(h, sq, max_n, q, k, v, out, stream);
}

duo_status duo_decode(duo_cache* h, const void* q, const void* k, const void* v, void* out, void* stream) {
  return decode_call(h, q, k, v, out, stream, false);
}

duo_status duo_decode_static_scratch(duo_cache* h, const void* q, const void* k, const void* v, void* out,
                                     void* stream) {
  return decode_call(h, q, k, v, out, stream, true);
}

duo_status duo_cache_lengths(const duo_cache* h, int64_t* out) {
  if (h == nullptr || out == nullptr) return DUO_ERR_INVALID_ARG;
  for (int b = 0; b < h->cfg.batch; ++b) out[b] = h->len[b];
  return DUO_OK;
}

duo_status duo_cache_layout(const duo_cache* h, duo_layout* out) {
  if (h == nullptr || out == nullptr) return DUO_ERR_INVALID_ARG;
  *out = h->layout;
  return DUO_OK;
}

duo_status duo_cache_head_index(const duo_cache* h, int32_t* out) {
  if (h == nullptr || out == nullptr) return DUO_ERR_INVALID_ARG;
  for (int k = 0; k < h->cfg.num_kv_heads; ++k) out[k] = h->geom.index_of_kv[k];
  return DUO_OK;
}

duo_status duo_cache_pages(const duo_cache* h, int32_t b, int32_t* out, int32_t cap, int32_t* n, int64_t* free_pages) {
  if (h == nullptr || b < 0 || b >= h->cfg.batch || n == nullptr || cap < 0 || (cap > 0 && out == nullptr))
    return DUO_ERR_INVALID_ARG;
  const std::vector<int32_t>& pg = h->seq_pages[b];
  *n = (int32_t)pg.size();
  for (int32_t i = 0; i < *n && i < cap; ++i) out[i] = pg[i];
  if (free_pages != nullptr) *free_pages = (int64_t)h->free_pages.size();
  return DUO_OK;
}

}  // extern "C"
