/*
 * duo.h -- C ABI of a gfx950 (AMD MI355X) library for DuoAttention's
 * per-head mixed attention over a head-split KV cache.
 *
 * The method (DuoAttention, arXiv 2410.10819; abstract as reproduced on the
 * pith.science review page, and the sourcepulse.org project card, "How It
 * Works"): attention heads are of two kinds.  Retrieval heads keep the full
 * KV cache and attend to every earlier token.  Streaming heads keep a
 * constant-length cache and attend only to the attention sinks and the most
 * recent tokens.  Both prefill (many new tokens at once) and decoding (one
 * new token per sequence) use the split.  Which heads are retrieval heads is
 * decided offline (the pages' optimisation on synthetic data) and is an
 * INPUT here: one flag per KV head.
 *
 * Readings of points the pages leave open (the pith.science referee report,
 * minor comment 3, notes that the cache size and sink handling have no
 * equation):
 *   - sinks are the first `sink` positions of each sequence;
 *   - a streaming query at position t sees positions t-recent+1 .. t (the
 *     window includes the query) and the sinks, i.e. min(t+1, sink+recent)
 *     positions -- exactly what sink+recent cache slots hold after the new
 *     token is stored;
 *   - query head h uses KV head h / (num_q_heads / num_kv_heads) (grouped
 *     query attention) and inherits that KV head's kind;
 *   - positional encoding: none by default (q and k arrive positioned), or
 *     rotary position embedding applied by the library (duo_rope_style);
 *   - retrieval heads never evict: running out of `max_len` is an error.
 *
 * Conventions for every call:
 *   - Tensors are bf16 (bfloat16: the top 16 bits of an IEEE binary32), dense,
 *     row-major, in DEVICE memory, 16-byte aligned.  The caller owns every
 *     buffer; the library never allocates or frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it and never synchronise; DUO_OK means the
 *     work was enqueued.  Results are visible after the caller synchronises.
 *   - All arguments are validated before anything is enqueued; a call that
 *     returns a validation error (INVALID_ARG, UNSUPPORTED, BUFFER_TOO_SMALL,
 *     CAPACITY) leaves the device buffer and the handle unchanged.  A call
 *     that returns DUO_ERR_HIP (a launch failed) leaves the handle unchanged
 *     -- stored lengths, and in a paged cache every page's owner -- but
 *     kernels launched before the failing one may have written device memory
 *     that no stored length covers (rows past a sequence's length, page-table
 *     entries of pages it does not hold); nothing a later call reads.
 *   - A handle is not thread-safe; use one stream per handle, calls in order.
 *   - No exception crosses the ABI and nothing aborts.
 */
#ifndef DUO_H
#define DUO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DUO_MAX_BATCH 128

typedef enum duo_status {
  DUO_OK = 0,
  DUO_ERR_INVALID_ARG = 1,      /* null/misaligned pointer, bad size or shape */
  DUO_ERR_UNSUPPORTED = 2,      /* head_dim not 64 or 128, batch > DUO_MAX_BATCH */
  DUO_ERR_BUFFER_TOO_SMALL = 3, /* buf_bytes < required bytes */
  DUO_ERR_CAPACITY = 4,         /* a sequence would exceed max_len tokens */
  DUO_ERR_HIP = 5               /* a HIP launch failed (hipGetLastError) */
} duo_status;

/* Storage format of the retrieval heads' cached K and V rows.
 *   DUO_KV_BF16: bf16 rows, as the inputs.
 *   DUO_KV_INT8: one int8 code per element and one fp32 scale per row (a row
 *     is the head_dim values of one sequence, KV head and position).  The
 *     pages only say that DuoAttention reaches a 3.3M-token context combined
 *     with quantization (abstract on the pith.science review page); the
 *     scheme is this library's reading: scale = max|x| / 127 and code =
 *     clamp(rint(x / scale), -127, 127), both in fp32 with round to nearest
 *     even (a zero row: scale 0, codes 0); stored as the byte code + 128.
 *     A call attends to rows stored by earlier calls through code * scale,
 *     and to the rows of its own chunk (or decode token) as given.
 *   DUO_KV_FP8: one OCP E4M3 8-bit float per element (largest finite 448)
 *     and one power-of-two scale per tensor for the whole cache
 *     (duo_config.kv_scale_k / kv_scale_v): code = e4m3(x / scale), which
 *     clamps to [-448, 448] and rounds to nearest even.  Every row a call
 *     attends to -- its own new rows included, which are stored first -- is
 *     seen through code * scale.  How retrieval heads' prefill computes over
 *     those values is duo_fp8_prefill.
 * Streaming heads' caches are bf16 in every format. */
typedef enum duo_kv_format { DUO_KV_BF16 = 0, DUO_KV_INT8 = 1, DUO_KV_FP8 = 2 } duo_kv_format;

/* Retrieval heads' prefill over a DUO_KV_FP8 cache.
 *   DUO_FP8_PREFILL_EXACT: every stored e4m3 value times its power-of-two
 *     scale is decoded to bf16 -- exactly: an e4m3 value has 4 significant
 *     bits -- and the products run on the bf16 matrix cores, so the only
 *     rounding beyond the stored K and V is that of the bf16 path (q, the
 *     softmax weights, the output).
 *   DUO_FP8_PREFILL_MFMA: the products run on the fp8 matrix cores at twice
 *     the bf16 rate; q is rounded to e4m3 (with a power-of-two scale per
 *     query row) and the softmax weights too, so results carry fp8 rounding
 *     (up to 2^-4 relative per rounded element) beyond the stored K and V. */
typedef enum duo_fp8_prefill { DUO_FP8_PREFILL_EXACT = 0, DUO_FP8_PREFILL_MFMA = 1 } duo_fp8_prefill;

/* How a decode call splits a retrieval head's rows over work-groups.
 *   DUO_DECODE_STATIC: work-group s of a (sequence, KV head) takes the fixed
 *     row batches s, s + n, s + 2n, ... (n work-groups), and the partial
 *     results are merged in work-group order: two runs on the same inputs
 *     give bitwise equal outputs.
 *   DUO_DECODE_DYNAMIC: after its first batch a work-group claims the next
 *     unclaimed one from a counter, so work-groups that get less memory
 *     bandwidth take fewer rows; which work-group sums which rows, and so
 *     the fp32 summation order, then depends on timing, and two runs may
 *     differ in the last bits (within the fp32 rounding of the softmax sums,
 *     a few units of the bf16 output's last place at most). */
typedef enum duo_decode_split { DUO_DECODE_STATIC = 0, DUO_DECODE_DYNAMIC = 1 } duo_decode_split;

/* Rotary position embedding applied inside the library (RoFormer, cited in
 * the reference list of the pith.science review page), when
 * duo_config.rope_base > 0.  q and k are then passed UN-rotated.  Pair i of
 * a head turns by p * theta_i, theta_i = rope_base^(-2i/head_dim), where p is
 * the token's position in its sequence (len_b + i for chunk row i; the
 * streaming cache keeps original positions); (a, b) -> (a cos - b sin,
 * a sin + b cos).  K is stored rotated, rounded to bf16 (nearest even), and
 * every key is attended through that stored value; q is rotated at its
 * position before the product; V is not rotated.  Angles are formed in fp64
 * and reduced before the fp32 sine and cosine, so positions in the millions
 * keep their accuracy.  With an 8-bit format the rotated bf16 K row is what
 * gets encoded; DUO_KV_INT8 still attends the call's own rows through their
 * (rotated) bf16 values and stored rows through their codes, DUO_KV_FP8 every
 * retrieval row through its codes.
 *   DUO_ROPE_INTERLEAVED: pair i = dims (2i, 2i+1) (the RoFormer form);
 *   DUO_ROPE_HALF: pair i = dims (i, i + head_dim/2). */
typedef enum duo_rope_style { DUO_ROPE_INTERLEAVED = 0, DUO_ROPE_HALF = 1 } duo_rope_style;

/* Configuration of one attention layer's cache. */
typedef struct duo_config {
  int32_t batch;        /* B, 1..DUO_MAX_BATCH sequences */
  int32_t num_q_heads;  /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* D: 64 or 128 */
  int64_t max_len;      /* token capacity per sequence of the retrieval cache */
  int32_t sink;         /* S >= 0 attention-sink positions kept by streaming heads */
  int32_t recent;       /* W >= 1 recent positions kept by streaming heads */
  float scale;          /* softmax scale; 0 selects 1/sqrt(head_dim) */
  const uint8_t* kv_head_is_retrieval; /* HOST [Hkv]: nonzero = retrieval; copied */
  int32_t kv_format;    /* duo_kv_format of the retrieval cache */
  float rope_base;      /* 0: no rotary embedding; > 0: its base (e.g. 10000) */
  int32_t rope_style;   /* duo_rope_style (read when rope_base > 0) */
  /* Paged retrieval cache (0 = contiguous rows, see duo_layout).  With
   * page_tokens > 0 the retrieval rows live in a pool of num_pages pages of
   * page_tokens positions each, shared by all sequences; a sequence takes
   * pages as it grows (one page covers page_tokens positions of every
   * retrieval head) and gives them back with duo_cache_release.  max_len
   * still bounds each sequence.  page_tokens: a power of two, 512..65536
   * (a page holds whole decode row batches and prefill tiles). */
  int32_t page_tokens;
  int64_t num_pages;
  /* DUO_KV_FP8: the K and V scales, powers of two in [2^-32, 2^32]; 0 = 1 */
  float kv_scale_k;
  float kv_scale_v;
  int32_t fp8_prefill;  /* duo_fp8_prefill (read with DUO_KV_FP8) */
  int32_t decode_split; /* duo_decode_split */
  /* An optional caller-owned DEVICE workspace (16-byte aligned,
   * prefill_staging_bytes long, must outlive the handle) where a prefill
   * call first writes, once per call, rows its attention would otherwise
   * prepare in every tile that reads them:
   *   - DUO_KV_INT8: the stored retrieval rows it reads, decoded to bf16 K
   *     and V (with rotary embedding also its own chunk's rows, K turned):
   *     4 * batch * retrieval KV heads * head_dim * rows bytes, rows = the
   *     largest len_b (len_b + n_new[b] with rotary embedding) among the
   *     sequences it extends;
   *   - DUO_KV_FP8 with DUO_FP8_PREFILL_EXACT: every retrieval row it reads,
   *     its own chunk's among them (stored first), as code * scale in bf16
   *     (exact): 4 * batch * retrieval KV heads * head_dim * rows bytes, rows
   *     = the largest len_b + n_new[b];
   *   - rotary embedding (any format): the chunk's K rows of every streaming
   *     head, turned: 2 * batch * streaming KV heads * head_dim * chunk
   *     bytes, after the 8-bit rows.
   * Each part is used when the workspace has room for it (and, for the
   * turned rows, when the int8 rows are staged or the cache is not int8);
   * otherwise the tiles prepare those rows themselves.  duo_layout.
   * prefill_staging_bytes is the most any call needs.  Both ways attend the
   * same values (a stored int8 row as code * scale rounded once to bf16, an
   * fp8 row as code * scale, a key turned as every K rotation turns it) and
   * give bitwise equal outputs.
   * Caches whose calls run in order on one stream may share one workspace.
   * NULL / 0: no workspace. */
  void* prefill_staging;
  int64_t prefill_staging_bytes;
} duo_config;

/* Opaque host-side handle: configuration, head maps, region offsets and the
 * host mirror of every sequence's length. */
typedef struct duo_cache duo_cache;

/* Byte offsets of the regions inside the caller's device buffer (all 256-byte
 * aligned).  With a paged retrieval cache (page_tokens > 0) rk / rv (and
 * rks / rvs) are page pools [num_pages][nR][page_tokens][D] (scales
 * [num_pages][nR][page_tokens]) and page_table int32 [B][max_pages_per_seq]
 * names the pool page holding positions [j P, (j+1) P) of sequence b
 * (entries past a sequence's length are unspecified).  nR / nS = number of retrieval / streaming KV heads; retrieval
 * KV head k is stored at index head_index[k] among the retrieval heads
 * (in increasing k), likewise for streaming heads.
 *   lengths  int32 [B]                     tokens stored per sequence
 *   rk, rv   bf16  [B][nR][max_len][D]     retrieval cache, row = position,
 *            when max_len <= 1024 (block_tokens = 0); longer contiguous caches
 *            hold [B][nblk][nR][block_tokens][D] with block_tokens = 1024 and
 *            nblk = ceil(max_len / 1024): block j of sequence b holds
 *            positions [1024 j, 1024 (j+1)) of each retrieval head in turn
 *            (DUO_KV_INT8: uint8 codes, DUO_KV_FP8: e4m3 codes, same shape)
 *   rks, rvs fp32  the rows' scales, same layout without D
 *            (DUO_KV_INT8 only; offset -1 otherwise)
 *   sk, sv   bf16  [B][nS][sink+recent][D] streaming cache, slot map:
 *            slot(p) = p for p < sink, else sink + (p - sink) mod recent
 *   work     uint32 split counters and fp32 split-K partial results of
 *            decoding (library-private; the counters are zero between calls) */
typedef struct duo_layout {
  int64_t lengths_offset;
  int64_t rk_offset, rv_offset;
  int64_t sk_offset, sv_offset;
  int64_t work_offset, work_bytes;
  int64_t total_bytes;
  int32_t n_retrieval, n_streaming;
  int32_t slots_per_streaming_head; /* sink + recent */
  int32_t kv_format;                /* duo_kv_format */
  int64_t rks_offset, rvs_offset;
  int64_t page_table_offset;        /* -1 for a contiguous cache */
  int32_t page_tokens, max_pages_per_seq;
  int64_t num_pages;
  int32_t block_tokens;             /* contiguous cache: 1024 if its rows are blocked, else 0 (also when paged) */
  int64_t work_records_offset;      /* decoding's split-K partial results, up to work_offset + work_bytes
                                       (written by a decode call before it reads them; their contents
                                       between calls are unspecified) */
  int64_t prefill_staging_bytes;    /* the duo_config.prefill_staging size that serves every prefill call:
                                       4 * B * nR * D * max_len for DUO_KV_INT8 and for DUO_KV_FP8 with exact
                                       prefill, plus 2 * B * nS * D * max_len with rotary embedding; 0 when
                                       none applies */
} duo_layout;

/* Lay out a new, empty cache in `dev_buf`.  The head-split layout is the
 * method's memory saving: a full cache only for retrieval heads and a
 * constant-length sink + recent cache for streaming heads (sourcepulse.org
 * project card, "How It Works"; abstract on the pith.science review page).
 * dev_buf == NULL: only writes *required_bytes (no device work); *out untouched.
 * Otherwise dev_buf (256-byte aligned, buf_bytes long, caller-owned, must
 * outlive the handle) receives the layout above; the lengths and the split
 * counters are zeroed on `stream` by a fill kernel; *out gets a new handle.
 * Errors: INVALID_ARG (null cfg / mask / out, B < 1, Hkv < 1, Hq % Hkv != 0,
 * sink < 0, recent < 1, max_len < 1, misaligned dev_buf, scale < 0 or not
 * finite, kv_format not a duo_kv_format, rope_base < 0 or not finite,
 * rope_style not a duo_rope_style, page_tokens not 0 or a power of two in
 * 512..65536, page_tokens > 0 with num_pages < 1, kv_scale_k / kv_scale_v
 * not 0 or a power of two in [2^-32, 2^32], fp8_prefill not a
 * duo_fp8_prefill, decode_split not a duo_decode_split, prefill_staging
 * misaligned or prefill_staging_bytes < 0), UNSUPPORTED (head_dim, batch,
 * num_kv_heads, max_len or sink + recent beyond the library's limits),
 * BUFFER_TOO_SMALL, HIP. */
duo_status duo_cache_init(const duo_config* cfg, void* dev_buf, size_t buf_bytes,
                          size_t* required_bytes, duo_cache** out, void* stream);

/* Wrap a buffer that already holds a cache laid out for `cfg` (for example a
 * copy of another handle's buffer: checkpoint / resume), with the host
 * lengths `lengths[B]` (each 0..max_len).  Enqueues nothing.  Same errors as
 * duo_cache_init, plus INVALID_ARG for null or out-of-range lengths, and for
 * a paged cache any nonzero length (the page table is not recoverable from
 * the buffer alone). */
duo_status duo_cache_attach(const duo_config* cfg, void* dev_buf, size_t buf_bytes,
                            const int64_t* lengths, duo_cache** out);

/* Free the host handle only (the device buffer stays the caller's). */
void duo_cache_destroy(duo_cache* h);

/* Sequence b ends: its length becomes 0 and, in a paged cache, its pages go
 * back to the pool; the slot can start a new sequence.  Enqueues a small
 * kernel (the device copy of the length) on `stream`.
 * Errors: INVALID_ARG (null handle, b out of range), HIP. */
duo_status duo_cache_release(duo_cache* h, int32_t b, void* stream);

/* Append n_new[b] tokens to every sequence without attending.  Retrieval
 * heads keep every token and streaming heads only the sinks and the most
 * recent ones, evicting the oldest (sourcepulse.org project card, "How It
 * Works"; the ajithp.com blog, "How DuoAttention Works").
 * k, v: bf16 [B][chunk][Hkv][D]; rows i >= n_new[b] of sequence b are
 * ignored.  Token i of sequence b gets position len_b + i (with rotary
 * embedding, k is stored rotated at that position).  Retrieval heads
 * store it at row len_b + i; streaming heads store positions < sink in their
 * sink slot and the last `recent` non-sink positions in their ring slot
 * (older ones would be overwritten at once).  Lengths advance by n_new.
 * n_new: HOST int32 [B], each in [0, chunk].
 * Errors: INVALID_ARG (null handle/k/v/n_new, misaligned, chunk < 1,
 * n_new out of range), UNSUPPORTED (B * chunk > 2^31 - 1 input rows),
 * CAPACITY (len_b + n_new[b] > max_len, or a paged cache without enough
 * free pages), HIP. */
duo_status duo_cache_append(duo_cache* h, const void* k, const void* v,
                            const int32_t* n_new, int32_t chunk, void* stream);

/* Packed (variable-length) inputs: the new rows of all sequences back to
 * back, sequence b's in rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of
 * k, v: bf16 [cu_seqlens[B]][Hkv][D] (q, out: [cu_seqlens[B]][Hq][D]).
 * cu_seqlens: HOST int32 [B+1], cu_seqlens[0] = 0, nondecreasing; a
 * sequence with no rows is skipped; a call with no rows at all does
 * nothing and accepts null tensor pointers.  Otherwise as duo_cache_append
 * and duo_prefill (INVALID_ARG also for a bad cu_seqlens). */
duo_status duo_cache_append_varlen(duo_cache* h, const void* k, const void* v,
                                   const int32_t* cu_seqlens, void* stream);
duo_status duo_prefill_varlen(duo_cache* h, const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens, void* out, void* stream);

/* Pre-filling (the abstract on the pith.science review page: the head split
 * speeds up pre-filling as well as decoding; retrieval heads attend to every
 * token, streaming heads to the attention sinks and recent tokens).
 * For every new token i < n_new[b] of sequence b at position
 * p = len_b + i and every query head, out = softmax(scale * q k^T) v over
 * the positions that head may see (retrieval: 0..p; streaming: sinks and
 * p-recent+1..p), where earlier positions come from the cache and the rest
 * from this chunk; then the chunk is appended as by duo_cache_append.  A
 * sequence may be prefilled in several chunks; the result equals one call
 * with the whole sequence.  n_new[b] = 0 skips sequence b.
 * q, out: bf16 [B][chunk][Hq][D]; k, v: bf16 [B][chunk][Hkv][D]; output
 * rows i >= n_new[b] are left untouched.  n_new: HOST int32 [B].
 * Errors: as duo_cache_append, plus null/misaligned q or out. */
duo_status duo_prefill(duo_cache* h, const void* q, const void* k, const void* v,
                       const int32_t* n_new, int32_t chunk, void* out, void* stream);

/* Decoding (the abstract on the pith.science review page: full attention
 * over the full cache for retrieval heads, the constant-length cache for
 * streaming heads).  Append one token per sequence at p = len_b and attend from it
 * (itself included), exactly as duo_prefill with n_new[b] = 1 for all b.
 * With decode_split = DUO_DECODE_STATIC (the default) two calls on equal
 * caches and inputs give bitwise equal outputs (duo_decode_split).
 * q, out: bf16 [B][Hq][D]; k, v: bf16 [B][Hkv][D].
 * Errors: INVALID_ARG (null/misaligned pointers), CAPACITY, HIP. */
duo_status duo_decode(duo_cache* h, const void* q, const void* k, const void* v,
                      void* out, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): decoding exactly as
 * duo_decode -- same kernels, same results bit for bit -- but the split-K
 * partial results and counters live in a static device array of the
 * library instead of the cache buffer's work region.  The array is 64 MiB
 * per GPU (4 MiB of counters, 60 MiB of partial results), held until the
 * process ends; duo_cache_init looks it up and zeroes its counters once per
 * device (on its stream), and every completed call leaves them at zero.
 * The call allocates and frees nothing.  All calls on one GPU share the
 * array: calls that overlap on one GPU (concurrent streams, or another
 * thread) race and must not be issued.
 * Errors: as duo_decode, plus UNSUPPORTED when the handle's decode needs
 * more counters (units x counters per unit) or partial results (units x
 * max splits x heads per work-group x (head_dim + 2) floats) than the
 * array holds -- e.g. 256 KV heads x 128 sequences. */
duo_status duo_decode_static_scratch(duo_cache* h, const void* q, const void* k, const void* v,
                                     void* out, void* stream);

/* Introspection (host only, no device work). */
const char* duo_status_string(duo_status s);
duo_status duo_cache_lengths(const duo_cache* h, int64_t* out /* [B] */);
duo_status duo_cache_layout(const duo_cache* h, duo_layout* out);
/* out[k] = index of KV head k among the heads of its own kind. */
duo_status duo_cache_head_index(const duo_cache* h, int32_t* out /* [Hkv] */);
/* Paged cache: *n = pages held by sequence b, and their pool indices in
 * out[0 .. min(*n, cap)) (in position order); *free_pages = pages left in
 * the pool.  A contiguous cache reports 0 pages. */
duo_status duo_cache_pages(const duo_cache* h, int32_t b, int32_t* out, int32_t cap, int32_t* n,
                           int64_t* free_pages);

#ifdef __cplusplus
}
#endif

#endif /* DUO_H */
