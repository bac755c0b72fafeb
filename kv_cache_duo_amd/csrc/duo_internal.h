// Internal definitions shared by the host library (duo_api.cpp) and the
// gfx950 kernels (*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "duo.h"

namespace duo {

constexpr int kMaxKvHeads = 256;  // kv head ids are stored as uint8
// Contiguous caches longer than 2^kBlockShift positions keep their retrieval
// rows in blocks of that many positions, the retrieval heads of a sequence
// interleaved block by block ([B][blocks][nR][2^kBlockShift][D]): streaming
// a step's rows then spreads over HBM like a paged pool does, which measured
// ~4% faster decode than one long region per head.  Shorter caches have one
// block per sequence, [B][nR][max_len][D].
constexpr int kBlockShift = 10;

// Geometry of one cache, passed by value to every kernel.
struct Geom {
  int32_t B, Hq, Hkv, G, D;
  int32_t S, W, slots;        // sink, recent, sink+recent
  int32_t nR, nS;             // retrieval / streaming KV heads
  int32_t kv_int8;            // retrieval rows stored as int8 codes + fp32 scales
  int32_t kv_fp8;             // retrieval rows stored as e4m3 codes, per-tensor power-of-two scales
  int32_t fp8_mfma;           // kv_fp8: retrieval prefill on fp8 matrix cores (else exact bf16 decoding)
  int32_t decode_dynamic;     // decode work-groups claim row batches from a counter (else a fixed stride)
  int32_t fp8_exp_k, fp8_exp_v;  // log2 of the K / V scales
  float fp8_scale_k, fp8_scale_v, fp8_inv_k, fp8_inv_v;
  int64_t max_len;
  float scale_log2;           // softmax scale * log2(e): scores in base-2 units
  uint16_t* prefill_staging;     // kv_int8 or rope: caller's workspace for bf16 rows a prefill stages (or null)
  int64_t prefill_staging_bytes;
  int32_t rope;               // rotary position embedding applied to q and k
  int32_t rope_half;          // pairs (i, i + D/2) instead of (2i, 2i + 1)
  double rope_rho;            // rotary base^(-2/D): pair i turns by rho^i per position
  uint16_t* rk;               // bf16 bits, rows as retrieval_row0 places them (kv_int8 / kv_fp8: D bytes per row)
  uint16_t* rv;
  float* rks;                 // kv_int8: fp32 row scales of rk / rv, one per row
  int32_t nblk;               // contiguous caches: blocks of 2^kBlockShift positions per sequence (1: unblocked)
  float* rvs;
  uint16_t* sk;               // bf16 bits [B][nS][slots][D]
  uint16_t* sv;
  int32_t* lengths;           // [B]
  // Paged retrieval cache (paged != 0): rk / rv (rks / rvs) are pools
  // [num_pages][nR][1 << page_shift][D]; page_table[b * max_pages + j] is
  // the pool page of positions [j << page_shift, (j + 1) << page_shift).
  int32_t paged;
  int32_t page_shift;
  int32_t max_pages;
  const int32_t* page_table;
  float* partials;            // split-K records, see decode.hip
  uint32_t* tickets;          // [units][tickets_per_unit] split counters (zero between calls)
  int32_t tickets_per_unit;   // words: arrivals, pair claims, then one line per group of kMergeGroup splits
  int32_t max_splits;         // capacity of the partial records per unit
  // unit u < nR is retrieval KV head kv_of_unit[u]; unit nR+s is streaming
  // KV head kv_of_unit[nR+s]; index_of_kv[k] is k's index within its kind.
  uint8_t kv_of_unit[kMaxKvHeads];
  uint8_t index_of_kv[kMaxKvHeads];
  uint8_t is_retrieval[kMaxKvHeads];
};

static_assert(offsetof(Geom, kv_of_unit) % 4 == 0, "kv_of_unit is read as 32-bit words");

// Row index (in rows of D elements) of retrieval row p of (sequence b,
// retrieval index idx), minus p: adding p to it gives the row, for every p
// of the page (paged caches) or block (blocked contiguous caches) holding
// `p_page`.  Hot loops take it once per page-aligned batch of rows.
__device__ __forceinline__ int64_t retrieval_row0(const Geom& g, int b, int idx, int p_page) {
  if (!g.paged) {
    if (g.nblk == 1) return ((int64_t)b * g.nR + idx) * g.max_len;
    const int j = p_page >> kBlockShift;  // blocked contiguous layout: blocks of sequence b in order
    return ((((int64_t)b * g.nblk + j) * g.nR + idx) << kBlockShift) - ((int64_t)j << kBlockShift);
  }
  const int j = p_page >> g.page_shift;
  const int64_t page = g.page_table[(int64_t)b * g.max_pages + j];
  return ((page * g.nR + idx) << g.page_shift) - ((int64_t)j << g.page_shift);
}

// The same for arguments that are uniform across the work-group: the
// page-table entry comes through the scalar cache and is waited for in
// place.  A vector load there would make its wait also wait for every load
// the kernel has in flight.  (Page tables are written by earlier launches;
// each launch starts with the scalar cache invalidated.)
__device__ __forceinline__ int32_t load_uniform_i32(const int32_t* p) {
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}
__device__ __forceinline__ int64_t retrieval_row0_uniform(const Geom& g, int b, int idx, int p_page) {
  if (!g.paged) return retrieval_row0(g, b, idx, p_page);  // no table
  const int j = p_page >> g.page_shift;
  const int64_t page = load_uniform_i32(g.page_table + (int64_t)b * g.max_pages + j);
  return ((page * g.nR + idx) << g.page_shift) - ((int64_t)j << g.page_shift);
}

// KV head of unit u.  Read as a 32-bit word of the kernel argument: for a
// work-group-uniform u that is a scalar load, where a byte load of the
// argument would be a vector memory round trip.
__device__ __forceinline__ int kv_head_of_unit(const Geom& g, int u) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(g.kv_of_unit)[u >> 2];
  return (int)((w >> (8 * (u & 3))) & 0xffu);
}

// Per-call sequence table: tokens already stored, tokens added, and the
// input row of sequence b's first new token (b * chunk for padded inputs,
// cu_seqlens[b] for packed ones).
struct Seqs {
  int32_t len[DUO_MAX_BATCH];
  int32_t n[DUO_MAX_BATCH];
  int32_t off[DUO_MAX_BATCH];
  // Sequences with new tokens, the longest stored prefix first (prefill
  // work-groups index them), and whether every one of them has the same
  // stored and new lengths (equal work per unit).
  int32_t nact;
  int32_t uniform;
  int32_t act[DUO_MAX_BATCH];
};
// Fill nact / uniform / act from len and n.
void finish_seqs(Seqs& q, int32_t batch);

// Sequence of active slot i (i work-group uniform).
__host__ __device__ __forceinline__ int active_seq(const Seqs& q, int i) { return q.act[i]; }

// Prefill work over sequences of different lengths, dealt to the 8 XCDs of
// an MI355X (work-group i runs on XCD i mod 8).  Units u = 0 .. units-1
// (units_per_seq per active sequence, active slot u / units_per_seq, so the
// longest stored prefix first) go to the XCDs in snake order: round j deals
// units 8j .. 8j+7, every other round in reverse.  Each XCD runs its units
// one after another, a unit's query tiles (tq rows) longest first, so its
// resident work-groups share one unit's K/V tiles in its L2.
constexpr int kPrefillXcds = 8;
__host__ __device__ __forceinline__ int snake_unit(int j, int x) {
  return kPrefillXcds * j + ((j & 1) ? kPrefillXcds - 1 - x : x);
}
// Work-group count of the deal (8 x the largest XCD's tile count), or 0 when
// it would leave the XCDs' work (keys summed over query tiles) more than 10%
// from even, or there are fewer than 16 units.
int64_t snake_deal_items(const Seqs& q, int units_per_seq, int tq);
// Work item `id` of the deal: query tile t of unit u; false past the end of
// its XCD's units.
__host__ __device__ __forceinline__ bool snake_deal_item(const Seqs& sq, int id, int units, int units_per_seq, int tq,
                                                         int& t, int& u) {
  const int x = id % kPrefillXcds;
  int k = id / kPrefillXcds;
  for (int j = 0;; ++j) {
    const int v = snake_unit(j, x);
    if (v >= units) return false;
    const int tiles = (sq.n[active_seq(sq, v / units_per_seq)] + tq - 1) / tq;
    if (k < tiles) {
      t = tiles - 1 - k;
      u = v;
      return true;
    }
    k -= tiles;
  }
}

// Writes of int32 words of the cache buffer (page-table entries, device
// lengths), carried in the kernel arguments.
constexpr int kWordWritesPerLaunch = 448;
struct WordWrites {
  int32_t n;
  int32_t index[kWordWritesPerLaunch];  // word index from the buffer start
  int32_t value[kWordWritesPerLaunch];
};
hipError_t launch_word_writes(int32_t* base, const WordWrites& w, hipStream_t s);

// Launchers (each returns hipGetLastError() after the launch).
hipError_t launch_zero_words(uint32_t* p, int64_t words, hipStream_t s);

// kinds: kAppendRetrieval | kAppendStreaming, the heads whose rows are stored
constexpr int kAppendRetrieval = 1, kAppendStreaming = 2;
hipError_t launch_append(const Geom& g, const Seqs& q, const uint16_t* k, const uint16_t* v,
                         int32_t max_n, hipStream_t s,
                         int kinds = kAppendRetrieval | kAppendStreaming);

struct DecodePlan {
  int32_t split_tokens;      // rows per work-group on average (a multiple of the pair rows)
  int32_t splits_r;          // max splits over retrieval units
  int32_t splits_s;          // max splits over streaming units
  int32_t head_chunk;        // query heads handled per work-group (divides G)
};
// num_cus: compute units of the device (work-groups per call are sized to it)
DecodePlan plan_decode(const Geom& g, const Seqs& q, int32_t num_cus);
hipError_t launch_decode(const Geom& g, const Seqs& q, const DecodePlan& p,
                         const uint16_t* qin, const uint16_t* kin, const uint16_t* vin,
                         uint16_t* out, hipStream_t s);

// Retrieval heads of an fp8 cache (DUO_KV_FP8), on fp8 matrix cores; the
// chunk's retrieval rows must be stored first.
// Stage the retrieval rows [0, len_b) of an int8 cache (with_chunk: also
// the chunk's rows, K turned when g.rope) as bf16 rows
// [B][nR][rows][D] at st_k / st_v.
hipError_t launch_stage(const Geom& g, const Seqs& q, const uint16_t* k, const uint16_t* v, uint16_t* st_k,
                        uint16_t* st_v, int64_t rows, bool with_chunk, hipStream_t s);
// With rotary embedding: the chunk's K rows of every streaming head turned
// (as every K rotation turns them) into rot [B][nS][rows][D].
hipError_t launch_turn(const Geom& g, const Seqs& q, const uint16_t* k, uint16_t* rot, int32_t rows, hipStream_t s);
hipError_t launch_prefill_fp8(const Geom& g, const Seqs& q, const uint16_t* qin, int32_t max_n, uint16_t* out,
                              hipStream_t s);

hipError_t launch_prefill(const Geom& g, const Seqs& q, const uint16_t* qin, const uint16_t* kin,
                          const uint16_t* vin, int32_t max_n, uint16_t* out, hipStream_t s);

// The library's own decode scratch for callers that cannot allocate
// (duo_decode_static_scratch): one static device array per GPU, split into
// a counter region (zero between calls) and a partial-result region.
constexpr int64_t kStaticTicketBytes = int64_t(4) << 20;
constexpr int64_t kStaticRecordBytes = int64_t(60) << 20;
// Device address of this GPU's array (the current device's), looked up once
// per device; the first call on a device also enqueues the zeroing of its
// counter region on `s`.  Returns the HIP error of the look-up or launch.
hipError_t static_decode_scratch(void** base, hipStream_t s);

// Query heads of one KV group handled together by a decode work-group (at
// most 4 with an int8 retrieval cache, whose lanes hold 16 dims each).
inline int decode_head_chunk(int G, bool kv_int8) {
  for (int c : {8, 4, 2, 1})
    if (G % c == 0 && !(kv_int8 && c > 4)) return c;
  return 1;
}

// Decode splits arrive in groups of this many; the last arrival of each
// group moves on to the unit's counter.  Every counter sits on its own
// 128-byte line (kTicketStride words): atomics to one line are serialised
// where they are performed.
constexpr int kMergeGroup = 16;
constexpr int kTicketStride = 32;
// per unit: the arrivals counter, the pair-claim counter, a counter per group
inline int32_t tickets_per_unit(int32_t max_splits) {
  return kTicketStride * (2 + (max_splits + kMergeGroup - 1) / kMergeGroup);
}

// Rows of a decode pair of batches (the unit of dynamic claiming): 4 waves,
// 64 / (D/8) rows per wave load, 4 loads in flight per lane (2 for chunks of
// 4 or more query heads), two batches.
constexpr int decode_pair_rows(int D, int head_chunk) { return 2 * 4 * (64 / (D / 8)) * (head_chunk >= 4 ? 2 : 4); }
// int8 retrieval rows: a lane loads 16 codes, so a pair holds twice the rows.
constexpr int decode_pair_rows_int8(int D, int head_chunk) { return 2 * decode_pair_rows(D, head_chunk); }

// Split-K record capacity per (sequence, KV head, head chunk): enough for
// splits of >= 256 rows, and at most 1024 / head_chunk records so that the
// merging work-group can stage every (m, l) pair in LDS.
int32_t max_splits_for(int64_t max_len, int32_t slots, int head_chunk);

}  // namespace duo
