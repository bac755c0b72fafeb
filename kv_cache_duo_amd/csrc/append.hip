// Cache append / evict kernel.
//
// DuoAttention (abstract; sourcepulse card, "How It Works"): retrieval heads
// keep every token, streaming heads keep a constant-length cache of the
// attention sinks and the recent tokens.  Storing a token therefore means:
//   retrieval KV head: row `position` of its contiguous cache;
//   streaming KV head: slot(p) = p for p < sink, else sink + (p-sink) mod
//   recent -- which overwrites (evicts) the token `recent` positions older.
// Within one call only the last `recent` non-sink positions of a chunk are
// written to the ring: older ones would be overwritten by the same call.
// With an int8 retrieval cache (duo_kv_format DUO_KV_INT8) retrieval rows
// are quantized as they are stored (fp8 cache, DUO_KV_FP8: e4m3 codes).  With rotary position embedding, K rows
// are turned to their position as they are stored (RoFormer, cited in the
// pith.science review page's reference list).
#include "device_util.h"
#include "duo_internal.h"

namespace duo {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kRowsPerBlock = 64;

__global__ __launch_bounds__(kAppendThreads) void zero_words_kernel(uint32_t* p, int64_t words) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < words; i += stride) p[i] = 0u;
}

// One block copies up to 64 token rows of one (sequence, KV head).
// Blocks [0, nr_blocks) handle retrieval heads, the rest streaming heads
// (nr_blocks = 0 when only streaming heads are stored).
template <int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(Geom g, Seqs q, const uint16_t* __restrict__ k,
                                                                const uint16_t* __restrict__ v, int32_t xr,
                                                                int32_t xs, int32_t nr_blocks) {
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int ROWS_PER_PASS = kAppendThreads / CH;
  int id = blockIdx.x;
  const int retrieval_blocks = nr_blocks;
  bool retrieval = id < retrieval_blocks;
  int b, idx, x;
  if (retrieval) {
    x = id % xr;
    idx = (id / xr) % g.nR;
    b = id / (xr * g.nR);
  } else {
    id -= retrieval_blocks;
    x = id % xs;
    idx = (id / xs) % g.nS;
    b = id / (xs * g.nS);
  }
  const int len = q.len[b];
  const int n = q.n[b];
  const int kvh = kv_head_of_unit(g, retrieval ? idx : g.nR + idx);

  // Lengths: written once per sequence, by the first block of its first head.
  if (x == 0 && idx == 0 && threadIdx.x == 0 && (retrieval || g.nR == 0)) g.lengths[b] = len + n;

  // Rows of this call that the head stores.
  int count, first_ring, sinks_here = 0;
  if (retrieval) {
    count = n;
    first_ring = 0;
  } else {
    sinks_here = min(max(g.S - len, 0), n);          // chunk rows that are sinks
    first_ring = max(sinks_here, n - g.W);           // first row kept in the ring
    count = sinks_here + (n - first_ring);
  }
  const int c = threadIdx.x % CH;
  for (int j = x * kRowsPerBlock + threadIdx.x / CH; j < min(count, (x + 1) * kRowsPerBlock);
       j += ROWS_PER_PASS) {
    int i = retrieval ? j : (j < sinks_here ? j : first_ring + (j - sinks_here));
    int64_t p = (int64_t)len + i;
    uint16_t *dk, *dv;
    int64_t rrow = 0;  // retrieval row (contiguous or through the page table)
    if (retrieval) {
      rrow = retrieval_row0(g, b, idx, (int)p) + p;
      dk = g.rk + rrow * D;
      dv = g.rv + rrow * D;
    } else {
      int64_t slot = p < g.S ? p : g.S + (p - g.S) % g.W;
      int64_t row = ((int64_t)b * g.nS + idx) * g.slots + slot;
      dk = g.sk + row * D;
      dv = g.sv + row * D;
    }
    int64_t src = (((int64_t)q.off[b] + i) * g.Hkv + kvh) * D;
    uint4 kx = reinterpret_cast<const uint4*>(k + src)[c];
    const uint4 vx = reinterpret_cast<const uint4*>(v + src)[c];
    if (g.rope) {
      float cs[8], sn[8];
      rope_angles8_key<D>((int)p, c, g.rope_half, g.rope_rho, cs, sn);
      kx = rope_apply8<CH>(kx, cs, sn, g.rope_half, c);
    }
    if (retrieval && g.kv_fp8) {
      store_fp8_row8(reinterpret_cast<uint8_t*>(g.rk) + rrow * D, kx, c, g.fp8_inv_k);
      store_fp8_row8(reinterpret_cast<uint8_t*>(g.rv) + rrow * D, vx, c, g.fp8_inv_v);
    } else if (retrieval && g.kv_int8) {
      // int8 row: the CH lanes of the row agree on its scale (group max)
      store_int8_row<CH>(reinterpret_cast<uint8_t*>(g.rk) + rrow * D, g.rks + rrow, kx, c);
      store_int8_row<CH>(reinterpret_cast<uint8_t*>(g.rv) + rrow * D, g.rvs + rrow, vx, c);
    } else {
      reinterpret_cast<uint4*>(dk)[c] = kx;
      reinterpret_cast<uint4*>(dv)[c] = vx;
    }
  }
}

// The retrieval rows that a prefill over an 8-bit cache reads, written once
// per call as bf16 into a staging area [B][nR][rows][D] (K and V apart).
// int8: the stored prefix [0, len) decoded (code * scale rounded to bf16,
// the value a tile decoded in the attention kernel would hold), and with
// rotary embedding the chunk's own rows too, K turned to its position, V as
// given.  fp8 (exact prefill): every row [0, len + n), the call's own rows
// stored before the attention, as code * scale (exact in bf16).
// One block per (sequence, retrieval head, 64 rows); sequences without new
// rows in the call are skipped.
template <int D>
__global__ __launch_bounds__(kAppendThreads) void stage_kernel(Geom g, Seqs q, const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               uint16_t* __restrict__ st_k,
                                                               uint16_t* __restrict__ st_v, int64_t rows,
                                                               int32_t xr, int32_t with_chunk) {
  constexpr int CH = D / 8;
  constexpr int ROWS_PER_PASS = kAppendThreads / CH;
  const int id = blockIdx.x;
  const int x = id % xr;
  const int idx = (id / xr) % g.nR;
  const int b = id / (xr * g.nR);
  const int len = q.len[b];
  const int n = q.n[b];
  if (n <= 0) return;
  // fp8: the call's own rows are stored before the attention, so every row
  // comes from the cache
  const int stored = g.kv_fp8 ? len + n : len;
  const int count = g.kv_fp8 ? len + n : len + (with_chunk ? n : 0);
  const int kvh = kv_head_of_unit(g, idx);
  const int c = threadIdx.x % CH;
  const int64_t base = ((int64_t)b * g.nR + idx) * rows;
  const uint8_t* rk8 = reinterpret_cast<const uint8_t*>(g.rk);
  const uint8_t* rv8 = reinterpret_cast<const uint8_t*>(g.rv);
  for (int p = x * kRowsPerBlock + threadIdx.x / CH; p < min(count, (x + 1) * kRowsPerBlock); p += ROWS_PER_PASS) {
    uint4 kx, vx;
    if (p < stored) {
      const int64_t rrow = retrieval_row0(g, b, idx, p) + p;
      const uint2 kc = reinterpret_cast<const uint2*>(rk8 + rrow * D)[c];
      const uint2 vc = reinterpret_cast<const uint2*>(rv8 + rrow * D)[c];
      if (g.kv_fp8) {  // code * scale: exact in bf16 (4 significant bits, a power-of-two scale)
        kx = fp8_to_bf16x8(kc.x, kc.y, g.fp8_scale_k);
        vx = fp8_to_bf16x8(vc.x, vc.y, g.fp8_scale_v);
      } else {
        kx = int8_dequant8(kc.x, kc.y, g.rks[rrow]);
        vx = int8_dequant8(vc.x, vc.y, g.rvs[rrow]);
      }
    } else {
      const int64_t src = (((int64_t)q.off[b] + (p - len)) * g.Hkv + kvh) * D;
      kx = reinterpret_cast<const uint4*>(k + src)[c];
      vx = reinterpret_cast<const uint4*>(v + src)[c];
      if (g.rope) {
        float cs[8], sn[8];
        rope_angles8_key<D>(p, c, g.rope_half, g.rope_rho, cs, sn);
        kx = rope_apply8<CH>(kx, cs, sn, g.rope_half, c);
      }
    }
    reinterpret_cast<uint4*>(st_k + (base + p) * D)[c] = kx;
    reinterpret_cast<uint4*>(st_v + (base + p) * D)[c] = vx;
  }
}

// With rotary embedding: the chunk's K rows of every streaming head turned
// to their positions once per call, into [B][nS][rows][D] (the prefill's
// tiles then load them as they are, instead of turning them in every
// work-group that reads them).  One block per (sequence, streaming head,
// 64 rows); sequences without new rows are skipped.
template <int D>
__global__ __launch_bounds__(kAppendThreads) void turn_kernel(Geom g, Seqs q, const uint16_t* __restrict__ k,
                                                              uint16_t* __restrict__ rot, int32_t rows, int32_t xr) {
  constexpr int CH = D / 8;
  constexpr int ROWS_PER_PASS = kAppendThreads / CH;
  const int id = blockIdx.x;
  const int x = id % xr;
  const int idx = (id / xr) % g.nS;
  const int b = id / (xr * g.nS);
  const int len = q.len[b];
  const int n = q.n[b];
  if (n <= 0) return;
  const int kvh = kv_head_of_unit(g, g.nR + idx);
  const int c = threadIdx.x % CH;
  const int64_t base = ((int64_t)b * g.nS + idx) * rows;
  for (int i = x * kRowsPerBlock + threadIdx.x / CH; i < min(n, (x + 1) * kRowsPerBlock); i += ROWS_PER_PASS) {
    const int64_t src = (((int64_t)q.off[b] + i) * g.Hkv + kvh) * D;
    float cs[8], sn[8];
    rope_angles8_key<D>(len + i, c, g.rope_half, g.rope_rho, cs, sn);
    reinterpret_cast<uint4*>(rot + (base + i) * D)[c] =
        rope_apply8<CH>(reinterpret_cast<const uint4*>(k + src)[c], cs, sn, g.rope_half, c);
  }
}

// Page-table entries and device lengths written by the host's calls.
__global__ __launch_bounds__(kAppendThreads) void word_writes_kernel(int32_t* base, WordWrites w) {
  for (int i = threadIdx.x; i < w.n; i += blockDim.x) base[w.index[i]] = w.value[i];
}

}  // namespace

hipError_t launch_word_writes(int32_t* base, const WordWrites& w, hipStream_t s) {
  if (w.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(word_writes_kernel, dim3(1), dim3(kAppendThreads), 0, s, base, w);
  return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t* p, int64_t words, hipStream_t s) {
  if (words <= 0) return hipSuccess;
  int64_t blocks = (words + kAppendThreads - 1) / kAppendThreads;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(kAppendThreads), 0, s, p, words);
  return hipGetLastError();
}

hipError_t launch_append(const Geom& g, const Seqs& q, const uint16_t* k, const uint16_t* v, int32_t max_n,
                         hipStream_t s, int kinds) {
  int32_t xr = (max_n + kRowsPerBlock - 1) / kRowsPerBlock;
  int32_t xs = (min(max_n, g.slots) + kRowsPerBlock - 1) / kRowsPerBlock;
  if (xr < 1) xr = 1;  // still one block per head so that the lengths are written
  if (xs < 1) xs = 1;
  const int64_t nr_blocks = (kinds & kAppendRetrieval) ? (int64_t)g.B * g.nR * xr : 0;
  const int64_t ns_blocks = (kinds & kAppendStreaming) ? (int64_t)g.B * g.nS * xs : 0;
  const int64_t blocks = nr_blocks + ns_blocks;
  if (blocks <= 0) return hipSuccess;
  if (g.D == 128)
    hipLaunchKernelGGL(append_kernel<128>, dim3((unsigned)blocks), dim3(kAppendThreads), 0, s, g, q, k, v, xr, xs,
                       (int32_t)nr_blocks);
  else
    hipLaunchKernelGGL(append_kernel<64>, dim3((unsigned)blocks), dim3(kAppendThreads), 0, s, g, q, k, v, xr, xs,
                       (int32_t)nr_blocks);
  return hipGetLastError();
}

hipError_t launch_stage(const Geom& g, const Seqs& q, const uint16_t* k, const uint16_t* v, uint16_t* st_k,
                        uint16_t* st_v, int64_t rows, bool with_chunk, hipStream_t s) {
  if (rows <= 0 || g.nR <= 0) return hipSuccess;
  const int32_t xr = (int32_t)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  const int64_t blocks = (int64_t)g.B * g.nR * xr;
  if (g.D == 128)
    hipLaunchKernelGGL(stage_kernel<128>, dim3((unsigned)blocks), dim3(kAppendThreads), 0, s, g, q, k, v, st_k, st_v,
                       rows, xr, (int32_t)with_chunk);
  else
    hipLaunchKernelGGL(stage_kernel<64>, dim3((unsigned)blocks), dim3(kAppendThreads), 0, s, g, q, k, v, st_k, st_v,
                       rows, xr, (int32_t)with_chunk);
  return hipGetLastError();
}

hipError_t launch_turn(const Geom& g, const Seqs& q, const uint16_t* k, uint16_t* rot, int32_t rows, hipStream_t s) {
  if (rows <= 0 || g.nS <= 0) return hipSuccess;
  const int32_t xr = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t blocks = (int64_t)g.B * g.nS * xr;
  if (g.D == 128)
    hipLaunchKernelGGL(turn_kernel<128>, dim3((unsigned)blocks), dim3(kAppendThreads), 0, s, g, q, k, rot, rows, xr);
  else
    hipLaunchKernelGGL(turn_kernel<64>, dim3((unsigned)blocks), dim3(kAppendThreads), 0, s, g, q, k, rot, rows, xr);
  return hipGetLastError();
}

}  // namespace duo
