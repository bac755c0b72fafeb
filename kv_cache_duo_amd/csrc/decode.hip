// Mixed retrieval/streaming decoding (one new token per sequence).
//
// DuoAttention (abstract, as reproduced on the pith.science review page):
// retrieval heads attend over their full KV cache, streaming heads over the
// constant-length cache of sinks + recent tokens.  Decoding is memory-bound:
// every cached K/V byte of a retrieval head is read once per step.
//
// One launch per step.  A unit is (sequence b, KV head, query-head chunk);
// its rows are the cache rows (retrieval: positions 0..L; streaming: the
// min(L+1, sink+recent) occupied slots), cut into pairs of batches.  Every
// unit gets ns work-groups.  Work-group `split` of a unit takes pair `split`
// first.  With the static split (the default) it then takes pairs split +
// ns, split + 2 ns, ...: which rows a work-group sums, and in what order, is
// fixed, and the records are merged in work-group order, so outputs are
// bitwise reproducible.  With the dynamic split it claims further pairs
// from the unit's counter (one claim ahead of use), so work-groups that get
// less bandwidth take fewer rows, at the price of a timing-dependent fp32
// summation order.
// The new token's row is read from the input and stored to the cache by the
// work-group whose pair holds it; no other work-group reads that row.  Each
// work-group streams its rows with coalesced 16-byte loads (a row of D bf16
// is read by D/8 lanes; one wave instruction reads 1 KB of consecutive
// rows), scores every query head of the KV group from the same K bytes with
// bf16 dot2 + DPP group sums, and keeps an online softmax (running max m,
// sum l, unnormalised o) per head.  A unit with one work-group writes the
// output; otherwise each work-group writes a record and the last one to
// arrive merges:  M = max m_k, L = sum l_k 2^(m_k-M), O = sum o_k 2^(m_k-M) / L.
// Records and tickets use agent-coherent (sc1) accesses without fences: an
// agent-scope fence on gfx950 writes back and invalidates the whole L2.
// Scores are kept in base-2 units (scale * log2 e folded in), so exp2 is the
// only transcendental of the row loop.  With rotary position embedding q
// and the new K row are turned to position L once, in the prologue, and the
// new token is scored outside the row loop (by work-group 0 of the unit).
#include <cfloat>
#include <mutex>
#include <type_traits>

#include "device_util.h"
#include "duo_internal.h"

namespace duo {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr int kMaxMergeRecords = 1024;  // (m, l) pairs the merge stages in LDS
// Pairs of batches per work-group, at least, on average (bf16 rows; 8-bit
// rows, whose pairs hold twice the rows), under the ~2048-work-group rule of
// plan_decode for work-groups that serve several query heads (a sweep on the
// 32K MHA layer picked these before that layer moved to one work-group per CU)
constexpr int kMinPairs = 3, kMinPairsInt8 = 2;

struct DecodeArgs {
  const uint16_t* q;  // [B][Hq][D]
  const uint16_t* k;  // [B][Hkv][D]
  const uint16_t* v;
  uint16_t* out;      // [B][Hq][D]
  int32_t split_tokens, splits_r, splits_s;
};

// Agent-coherent (cross-XCD) accesses without fences: on gfx950 relaxed
// atomics at agent scope are plain loads/stores with the sc1 bit, which
// bypass the non-coherent cache levels.  Only fences at agent scope write
// back / invalidate a whole L2, which would cost far more than the merge.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_agent2(const float* p) {  // p 8-byte aligned
  const uint64_t x = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(float2, x);
}

__device__ __forceinline__ float max_or_zero(float m) { return m == -INFINITY ? 0.f : m; }


__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

// Records of one unit (b, kv head, head chunk): o [max_splits][GC][D] fp32,
// then (m, l) [max_splits][GC].
template <int D, int GC>
__device__ __forceinline__ float* unit_records(const Geom& g, int64_t pu) {
  return g.partials + pu * g.max_splits * GC * (D + 2);
}

// Merge `cnt` records of one unit (slots first, first+step, ...) with
// agent-coherent loads, into either the outputs or the record slot `first`
// (o relative to the new max M, with m = M and l = sum).  All threads of the
// work-group call it.  lds must hold kMergeLdsBytes.
constexpr int kMergeBatch = 16;  // record loads in flight per thread
template <int GC>
constexpr int merge_lds_bytes() { return kMaxMergeRecords * 8 + kThreads * 8 + 2 * GC * 4; }

// Single-pass merge: when a unit's records fit, the last work-group loads
// every o value at once (kSingleLoads 64-bit loads per thread, issued together
// with the (m, l) loads), so the merge costs one memory round trip after the
// ticket.  Records of GC*D floats are read as GC*D/2 float2 chunks; KL
// records are summed in parallel.
constexpr int kSingleLoads = 36;
// Units of at most this many splits skip the group counters: their
// arrivals go straight to the unit's counter.
constexpr int kDirectArrivals = 32;
template <int D, int GC>
constexpr int single_merge_max() {
  return GC * D / 2 > kThreads ? 0 : (kThreads / (GC * D / 2)) * kSingleLoads;
}

template <int D, int GC>
__device__ void merge_single(const Geom& g, const DecodeArgs& a, char* lds, const float* rec_o, const float* rec_ml,
                             int cnt, int b, int h0) {
  constexpr int E = GC * D;
  constexpr int C2 = E / 2;            // float2 chunks per record
  constexpr int KL = kThreads / C2;    // records summed in parallel
  static_assert(C2 <= kThreads && kThreads % C2 == 0, "single-pass merge layout");
  float2* st_ml = reinterpret_cast<float2*>(lds);                           // [cnt * GC]
  float2* st_acc = reinterpret_cast<float2*>(lds + kMaxMergeRecords * 8);   // [kThreads]
  float* st_L = reinterpret_cast<float*>(st_acc + kThreads);                // [GC]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cc = threadIdx.x % C2;
  const int kl = threadIdx.x / C2;
  float2 v[kSingleLoads];
#pragma unroll
  for (int u = 0; u < kSingleLoads; ++u)
    if (u * KL < cnt) v[u] = load_agent2(rec_o + (int64_t)min(kl + u * KL, cnt - 1) * E + 2 * cc);
  for (int i = threadIdx.x; i < cnt * GC; i += kThreads) st_ml[i] = load_agent2(rec_ml + 2 * i);
  __syncthreads();
  for (int gg = wave; gg < GC; gg += kWaves) {
    float mx = -INFINITY;
    for (int k = lane; k < cnt; k += 64) mx = fmaxf(mx, st_ml[k * GC + gg].x);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float mu = max_or_zero(mx);
    float ls = 0.f;
    for (int k = lane; k < cnt; k += 64) {
      const float2 ml = st_ml[k * GC + gg];
      const float f = exp2_fast(ml.x - mu);
      st_ml[k * GC + gg].x = f;
      ls += ml.y * f;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off);
    if (lane == 0) st_L[gg] = ls;
  }
  __syncthreads();
  const int gg = 2 * cc / D;
  float2 acc = make_float2(0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kSingleLoads; ++u) {
    const int k = kl + u * KL;
    if (u * KL < cnt && k < cnt) {
      const float f = st_ml[k * GC + gg].x;
      acc.x = fmaf(v[u].x, f, acc.x);
      acc.y = fmaf(v[u].y, f, acc.y);
    }
  }
  if (KL > 1) {
    st_acc[threadIdx.x] = acc;
    __syncthreads();
    if (kl == 0)
      for (int j = 1; j < KL; ++j) {
        const float2 x = st_acc[j * C2 + cc];
        acc.x += x.x;
        acc.y += x.y;
      }
  }
  if (kl == 0) {
    const float inv = 1.0f / st_L[gg];
    *reinterpret_cast<uint32_t*>(a.out + ((int64_t)b * g.Hq + h0 + gg) * D + (2 * cc) % D) =
        pack_bf16x2(acc.x * inv, acc.y * inv);
  }
}

template <int D, int GC>
__device__ void merge_records(const Geom& g, const DecodeArgs& a, char* lds, float* rec_o, float* rec_ml, int first,
                              int step, int cnt, bool to_output, int b, int h0) {
  constexpr int E = GC * D;                               // outputs of the unit
  constexpr int KL = E >= kThreads ? 1 : kThreads / E;    // records summed in parallel
  constexpr int EB = kThreads / KL;                       // outputs per pass
  float2* st_ml = reinterpret_cast<float2*>(lds);                              // [cnt * GC]
  float* st_acc = reinterpret_cast<float*>(lds + kMaxMergeRecords * 8);        // [kThreads]
  float* st_M = st_acc + kThreads;                                             // [GC]
  float* st_L = st_M + GC;                                                     // [GC]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // The first batch of o loads goes out together with the (m, l) loads, so
  // a merge of up to KL * kMergeBatch records costs one memory round trip.
  float v0[kMergeBatch];
  {
    const int e = threadIdx.x % EB;
    const int kl = threadIdx.x / EB;
#pragma unroll
    for (int u2 = 0; u2 < kMergeBatch; ++u2) {
      const int k = min(kl + u2 * KL, cnt - 1);
      v0[u2] = load_agent(rec_o + (int64_t)(first + k * step) * E + e);
    }
  }
  for (int i = threadIdx.x; i < cnt * GC; i += kThreads) {
    const int s = first + (i / GC) * step;
    const float* ml = rec_ml + 2 * ((int64_t)s * GC + i % GC);
    st_ml[i] = make_float2(load_agent(ml), load_agent(ml + 1));
  }
  __syncthreads();
  for (int gg = wave; gg < GC; gg += kWaves) {
    float mx = -INFINITY;
    for (int k = lane; k < cnt; k += 64) mx = fmaxf(mx, st_ml[k * GC + gg].x);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float mu = max_or_zero(mx);
    float ls = 0.f;
    for (int k = lane; k < cnt; k += 64) {
      const float2 ml = st_ml[k * GC + gg];
      const float f = exp2_fast(ml.x - mu);
      st_ml[k * GC + gg].x = f;
      ls += ml.y * f;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off);
    if (lane == 0) {
      st_M[gg] = mx;
      st_L[gg] = ls;
    }
  }
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += EB) {
    const int e = e0 + threadIdx.x % EB;
    const int kl = threadIdx.x / EB;
    const int gg = e / D;
    float acc = 0.f;
    for (int k0 = kl; k0 < cnt; k0 += KL * kMergeBatch) {
      float v[kMergeBatch];
      if (e0 == 0 && k0 == kl) {
#pragma unroll
        for (int u2 = 0; u2 < kMergeBatch; ++u2) v[u2] = v0[u2];
      } else {
#pragma unroll
        for (int u2 = 0; u2 < kMergeBatch; ++u2) {
          const int k = min(k0 + u2 * KL, cnt - 1);
          v[u2] = load_agent(rec_o + (int64_t)(first + k * step) * E + e);
        }
      }
#pragma unroll
      for (int u2 = 0; u2 < kMergeBatch; ++u2) {
        const int k = k0 + u2 * KL;
        acc = fmaf(v[u2], k < cnt ? st_ml[k * GC + gg].x : 0.f, acc);
      }
    }
    if (KL > 1) {
      st_acc[threadIdx.x] = acc;
      __syncthreads();
      if (kl == 0)
        for (int j = 1; j < KL; ++j) acc += st_acc[j * EB + threadIdx.x];
    }
    if (kl == 0) {
      if (to_output) {
        a.out[((int64_t)b * g.Hq + h0 + gg) * D + e % D] = (uint16_t)f32_to_bf16_bits(acc / st_L[gg]);
      } else {
        store_agent(rec_o + (int64_t)first * E + e, acc);
        if (e % D == 0) {
          store_agent(rec_ml + 2 * ((int64_t)first * GC + gg), st_M[gg]);
          store_agent(rec_ml + 2 * ((int64_t)first * GC + gg) + 1, st_L[gg]);
        }
      }
    }
    if (KL > 1) __syncthreads();
  }
}

// 8-bit decode rows: the softmax reference moves only when a score passes
// it by more than this (log2 units), so the weights stay below 2^8.
constexpr float kDecodeSlack = 8.f;

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// FMT: the cache's retrieval rows are bf16 (0), int8 codes with fp32 row
// scales (1, DUO_KV_INT8) or e4m3 codes with per-tensor power-of-two scales
// (2, DUO_KV_FP8)
// (DUO_KV_INT8); streaming units of the same launch stay bf16.
template <int D, int GC, int FMT>
__global__ __launch_bounds__(kThreads) void decode_kernel(Geom g, Seqs sq, DecodeArgs a) {
  constexpr int LPR = D / 8;                  // lanes per row (8 bf16 each)
  constexpr int RPW = 64 / LPR;               // rows per wave per load
  // K and V rows each lane loads per batch (two batches in flight); fewer
  // when more query heads per work-group need registers.
  constexpr int kInFlight = GC >= 4 ? 2 : 4;
  constexpr int ROWS_ITER = kWaves * RPW * kInFlight;  // rows per batch
  constexpr int PAIR = 2 * ROWS_ITER;                   // rows per claimed pair of batches
  static_assert(PAIR == decode_pair_rows(D, GC), "host and kernel pair sizes");
  // the cross-wave partials [kWaves][GC][D] share LDS with the merge staging
  // area of the last work-group
  constexpr int kCombineBytes = kWaves * GC * D * 4;
  constexpr int kMergeLds = merge_lds_bytes<GC>();
  __shared__ __attribute__((aligned(16))) char sm_raw[kCombineBytes > kMergeLds ? kCombineBytes : kMergeLds];
  float(*sm_o)[GC][D] = reinterpret_cast<float(*)[GC][D]>(sm_raw);
  __shared__ float sm_m[kWaves][GC];
  __shared__ float sm_l[kWaves][GC];
  __shared__ int sm_flag;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane / LPR;
  const int c = lane % LPR;

  // ---- work item
  const int n_hc = g.G / GC;
  int id = blockIdx.x;
  const int items_r = g.B * g.nR * n_hc * a.splits_r;
  const bool retrieval = id < items_r;
  int splits = a.splits_r;
  if (!retrieval) {
    id -= items_r;
    splits = a.splits_s;
  }
  const int split = id % splits;
  int u = id / splits;
  const int hc = u % n_hc;
  u /= n_hc;
  const int nkind = retrieval ? g.nR : g.nS;
  const int idx = u % nkind;
  const int b = u / nkind;

  const int L = sq.len[b];
  const int T = retrieval ? L + 1 : min(L + 1, g.slots);
  const int new_row = retrieval ? L : (L < g.S ? L : g.S + (L - g.S) % g.W);
  const int ns = (T + a.split_tokens - 1) / a.split_tokens;  // work-groups of this unit
  if (split >= ns) return;
  const int kvh = kv_head_of_unit(g, retrieval ? idx : g.nR + idx);
  const int64_t unit_rows = retrieval ? g.max_len : (int64_t)g.slots;
  const int64_t unit_row0 = ((int64_t)b * nkind + idx) * unit_rows;  // contiguous rows of the unit
  // Row base of the pair of batches starting at row `base` (rows past
  // `rows` - 1 read row rows - 1): a page or block of the retrieval cache
  // holds whole pairs; streaming units are contiguous.
  auto pair_row0 = [&](int base, int rows) __attribute__((always_inline)) -> int64_t {
    return retrieval ? retrieval_row0_uniform(g, b, idx, min(base, rows - 1)) : unit_row0;
  };
  const uint16_t* nk = a.k + ((int64_t)b * g.Hkv + kvh) * D;
  const uint16_t* nv = a.v + ((int64_t)b * g.Hkv + kvh) * D;
  const int h0 = kvh * g.G + hc * GC;
  const int64_t pu = ((int64_t)b * g.Hkv + kvh) * n_hc + hc;
  uint32_t* t_unit = g.tickets + pu * g.tickets_per_unit;  // line 0: arrivals, line 1: pair claims
  uint32_t* t_claim = t_unit + kTicketStride;
  // Dynamic split: thread 0 claims for the work-group, one atomic per pair;
  // the claim for the second pair goes out before anything else.
  auto claim = [&]() {
    return __hip_atomic_fetch_add(t_claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  uint32_t claimed = 0;
  const bool dynamic = g.decode_dynamic != 0;
  if (dynamic && threadIdx.x == 0) claimed = claim();

  // ---- queries of the GC heads: this lane's 8 dims of each
  uint32_t qw[GC][4];
#pragma unroll
  for (int gg = 0; gg < GC; ++gg) {
    uint4 t = reinterpret_cast<const uint4*>(a.q + ((int64_t)b * g.Hq + h0 + gg) * D)[c];
    qw[gg][0] = t.x; qw[gg][1] = t.y; qw[gg][2] = t.z; qw[gg][3] = t.w;
  }

  // The new token's K chunk c, turned to position L with rotary embedding
  // (rows are stored rotated: the cached rows already are); q turned by the
  // same angles.
  uint4 knew = reinterpret_cast<const uint4*>(nk)[c];
  if (g.rope) {
    float cs[8], sn[8];
    rope_angles8_key<D>(L, c, g.rope_half, g.rope_rho, cs, sn);
#pragma unroll
    for (int gg = 0; gg < GC; ++gg) {
      const uint4 t = rope_apply8<LPR>(make_uint4(qw[gg][0], qw[gg][1], qw[gg][2], qw[gg][3]), cs, sn, g.rope_half, c);
      qw[gg][0] = t.x; qw[gg][1] = t.y; qw[gg][2] = t.z; qw[gg][3] = t.w;
    }
    knew = rope_apply8<LPR>(knew, cs, sn, g.rope_half, c);
  }
  // Rows streamed by the row loop.  With rotary embedding the new token is
  // scored separately: retrieval units stream rows 0..L-1, streaming units
  // mask the new token's slot (its load reads the input row: finite).
  const int Tst = (g.rope && retrieval) ? L : T;
  const int skip_row = (g.rope && !retrieval) ? new_row : -1;

  float m[GC], l[GC], o[GC][8];
#pragma unroll
  for (int gg = 0; gg < GC; ++gg) {
    m[gg] = -INFINITY;
    l[gg] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[gg][e] = 0.f;
  }

  // Row j of a batch starting at `base`: consecutive rows per load
  // instruction of a wave, so each instruction reads RPW * D * 2 = 1 KB.
  auto row_of = [&](int base, int j) { return base + (j * kWaves + wave) * RPW + grp; };
  // Loads are unconditional per lane (rows past the unit's end re-read its
  // last row and get a -inf score), so the compiler can count outstanding
  // loads and wait only for the older batch.
  auto load = [&](uint4 (&kr)[kInFlight], uint4 (&vr)[kInFlight], int base, int64_t r0) {
    const uint16_t* ckp = (retrieval ? g.rk : g.sk) + r0 * D;
    const uint16_t* cvp = (retrieval ? g.rv : g.sv) + r0 * D;
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) {
      const int row = min(row_of(base, j), Tst - 1);
      const uint16_t* pk = row == new_row ? nk : ckp + (int64_t)row * D;
      const uint16_t* pv = row == new_row ? nv : cvp + (int64_t)row * D;
      kr[j] = load_nt(reinterpret_cast<const uint4*>(pk) + c);  // streamed once: non-temporal
      vr[j] = load_nt(reinterpret_cast<const uint4*>(pv) + c);
    }
  };
  auto process = [&](const uint4 (&kr)[kInFlight], const uint4 (&vr)[kInFlight], int base) {
    float s[kInFlight][GC];
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) {
      const int rj = row_of(base, j);
      const bool valid = rj < Tst && rj != skip_row;
#pragma unroll
      for (int gg = 0; gg < GC; ++gg) {
        float acc = dot2_bf16(kr[j].x, qw[gg][0], 0.f);
        acc = dot2_bf16(kr[j].y, qw[gg][1], acc);
        acc = dot2_bf16(kr[j].z, qw[gg][2], acc);
        acc = dot2_bf16(kr[j].w, qw[gg][3], acc);
        acc = group_sum<LPR>(acc);
        s[j][gg] = valid ? acc * g.scale_log2 : -INFINITY;
      }
    }
    // With several query heads per KV head (GC >= 4) the V products
    // dominate the loop's vector work: dim d of rows 2t and 2t + 1 then goes
    // as one bf16 pair (v_perm of their words) into one v_dot2 per dim and
    // head.  (For one head per KV head the plain FMAs measured faster.)
    constexpr bool kPairV = GC >= 4;
    uint32_t vpair[kPairV ? kInFlight / 2 : 1][8];
#pragma unroll
    for (int t = 0; t < (kPairV ? kInFlight / 2 : 0); ++t) {
      const uint32_t w0[4] = {vr[2 * t].x, vr[2 * t].y, vr[2 * t].z, vr[2 * t].w};
      const uint32_t w1[4] = {vr[2 * t + 1].x, vr[2 * t + 1].y, vr[2 * t + 1].z, vr[2 * t + 1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vpair[t][2 * e] = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);      // low halves
        vpair[t][2 * e + 1] = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);  // high halves
      }
    }
    // the batch's max per head; rescale only when some lane's max moved (one
    // wave vote for all heads): elsewhere the factor is exactly 1 (or l and
    // o are still 0), so skipping it changes nothing, and past the first
    // rows the max rarely moves
    float mn[GC], mu[GC];
    bool moved = false;
#pragma unroll
    for (int gg = 0; gg < GC; ++gg) {
      float mx = s[0][gg];
#pragma unroll
      for (int j = 1; j < kInFlight; ++j) mx = fmaxf(mx, s[j][gg]);
      mn[gg] = fmaxf(m[gg], mx);
      mu[gg] = max_or_zero(mn[gg]);
      moved = moved || mn[gg] > m[gg];
    }
    if (__any(moved)) {
#pragma unroll
      for (int gg = 0; gg < GC; ++gg) {
        const float alpha = exp2_fast(m[gg] - mu[gg]);
        l[gg] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[gg][e] *= alpha;
      }
    }
#pragma unroll
    for (int gg = 0; gg < GC; ++gg) {
      if constexpr (kPairV) {
        // rows in pairs: the two weights as one bf16 pair (l sums those same
        // values), one v_dot2 per dim with the two rows' values of that dim
#pragma unroll
        for (int t = 0; t < kInFlight / 2; ++t) {
          const uint32_t pw = pack_bf16x2(exp2_fast(s[2 * t][gg] - mu[gg]), exp2_fast(s[2 * t + 1][gg] - mu[gg]));
          l[gg] = dot2_bf16(pw, 0x3f803f80u, l[gg]);  // (1, 1)
#pragma unroll
          for (int e = 0; e < 8; ++e) o[gg][e] = dot2_bf16(vpair[t][e], pw, o[gg][e]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
          const float p = exp2_fast(s[j][gg] - mu[gg]);
          l[gg] += p;
          const uint32_t w[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[gg][2 * e] = fmaf(p, bf16_lo(w[e]), o[gg][2 * e]);
            o[gg][2 * e + 1] = fmaf(p, bf16_hi(w[e]), o[gg][2 * e + 1]);
          }
        }
      }
      m[gg] = mn[gg];
    }
  };

  // ---- stream the pairs: pair `split`, then (static split) pairs
  // split + ns, split + 2 ns, ..., or (dynamic split) claimed pairs ns,
  // ns+1, ...  While a pair's two batches are processed, the next pair's
  // loads go out batch by batch.  A dynamic claim for the pair after it is
  // in flight meanwhile and reaches the other waves through a
  // double-buffered LDS slot (one barrier per pair).  `rows` bounds the
  // streamed rows, `npr` the pairs; past the last pair the loads re-read the
  // last row (cached): unconditional loads keep the outstanding-load count
  // static.
  __shared__ int sm_claim[2];
  bool own_new = false;  // this work-group's rows hold the new token
  auto stream_pairs = [&](auto& ka, auto& va, auto& kb, auto& vb, auto&& ld, auto&& pr, int rows, int npr,
                          auto pair_c, auto iter_c, auto order_c) __attribute__((always_inline)) {
    constexpr int P = decltype(pair_c)::value, IT = decltype(iter_c)::value;  // rows per pair, per batch
    int base = split * P;
    int pair = split;
    const int64_t r0 = pair_row0(base, rows);
    ld(ka, va, base, r0);
    ld(kb, vb, base + IT, r0);
    for (int it = 0;; it ^= 1) {
      int p_next = pair + ns;
      if (dynamic) {
        if (threadIdx.x == 0) {
          sm_claim[it] = ns + (int)claimed;
          claimed = claim();
        }
        __syncthreads();
        p_next = __builtin_amdgcn_readfirstlane(sm_claim[it]);
      }
      pair = p_next;
      const bool more = p_next < npr;
      const int nbase = more ? p_next * P : rows;
      const int64_t nr0 = pair_row0(nbase, rows);  // page lookup: in flight while this pair is scored
      pr(ka, va, base);
      ld(ka, va, nbase, nr0);
      // 8-bit rows: keep these loads ahead of the second batch's work (left
      // to itself the compiler sinks them below it, and every pair then
      // waits out its whole load latency)
      if constexpr (decltype(order_c)::value) __builtin_amdgcn_sched_barrier(0);
      pr(kb, vb, base + IT);
      ld(kb, vb, nbase + IT, nr0);
      own_new = own_new || (new_row >= base && new_row < base + P);
      if (!more) break;
      base = nbase;
    }
  };
  auto stream_bf16 = [&]() __attribute__((always_inline)) {
    if (Tst > 0) {
      uint4 ka[kInFlight], va[kInFlight], kb[kInFlight], vb[kInFlight];
      stream_pairs(ka, va, kb, vb, load, process, Tst, (Tst + PAIR - 1) / PAIR, std::integral_constant<int, PAIR>(),
                   std::integral_constant<int, ROWS_ITER>(), std::false_type());
    }
  };
  const bool q8 = FMT != 0 && retrieval;  // 8-bit retrieval rows
  if constexpr (FMT != 0) {
    if (retrieval) {
      // int8 rows 0..L-1 of the cache; the new token (row L) is scored from
      // the input below.  A row of D codes is read by LPR8 = D/16 lanes with
      // 16-byte loads (one wave instruction: 1 KB of consecutive rows, as in
      // the bf16 path).  K: the codes b (stored code + 128) become the f16
      // values 1024 + b (byte b under the exponent byte 0x64, one v_perm per
      // two codes) and meet q in v_dot2_f32_f16; q is held in f16 scaled by a
      // power of two (2^(15 - e), amax = m 2^e over the head: no overflow,
      // bf16 values stay exact), and the 1024 + 128 offset comes back as one
      // per-lane constant -1152 * sum(q).  V: a lane's rows are taken in
      // pairs, and one v_dot2 per dim adds both rows' products: the bytes b
      // as exact bf16 values against p * scale_v rounded to bf16, with
      // 128 * sum(p * scale_v) taken off once at the end.
      // fp8 (FMT 2): K codes become exact f16 pairs (v_cvt_scalef32_pk_f16_fp8)
      // for the same dot2 with no offset; V codes exact f16 pairs of a row
      // pair against the two weights in f16; the K tensor scale folds into
      // the score constant, the V scale multiplies the sums at the end.
      constexpr int LPR8 = D / 16;
      constexpr int RPW8 = 64 / LPR8;
      constexpr int ITER8 = kWaves * RPW8 * kInFlight;
      constexpr int PAIR8 = 2 * ITER8;
      static_assert(PAIR8 == decode_pair_rows_int8(D, GC), "host and kernel int8 pair sizes");
      const int grp8 = lane / LPR8, c8 = lane % LPR8;
      const int Tc = L;
      typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
      const f16x2_t ones16 = {(_Float16)1.0f, (_Float16)1.0f};
      uint32_t q16[GC][8];  // f16 pairs of dims 16 c8 .. 16 c8 + 15
      float qoff[GC], qsc[GC], cacc[GC], o8[GC][16];
#pragma unroll
      for (int gg = 0; gg < GC; ++gg) {
        const uint4* src = reinterpret_cast<const uint4*>(a.q + ((int64_t)b * g.Hq + h0 + gg) * D) + 2 * c8;
        uint4 x0, x1;
        if (g.rope) {  // the rotated q of the 8-dims-per-lane layout: its chunks 2 c8 and 2 c8 + 1
          auto from = [&](int src_lane) __attribute__((always_inline)) {
            return make_uint4((uint32_t)__shfl((int)qw[gg][0], src_lane), (uint32_t)__shfl((int)qw[gg][1], src_lane),
                              (uint32_t)__shfl((int)qw[gg][2], src_lane), (uint32_t)__shfl((int)qw[gg][3], src_lane));
          };
          x0 = from(2 * c8);
          x1 = from(2 * c8 + 1);
        } else {
          x0 = src[0];
          x1 = src[1];
        }
        const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
        amax = group_max<LPR8>(amax);
        int ex;
        frexpf(amax, &ex);  // amax = m 2^ex, m in [0.5, 1) (ex = 0 for a zero head)
        const float up = ldexpf(1.0f, 15 - ex);
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const f16x2_t hq = {(_Float16)(bf16_lo(w[e]) * up), (_Float16)(bf16_hi(w[e]) * up)};
          q16[gg][e] = __builtin_bit_cast(uint32_t, hq);
          sum += (float)hq.x + (float)hq.y;
        }
        qoff[gg] = FMT == 1 ? -1152.0f * sum : 0.f;
        qsc[gg] = ldexpf(FMT == 1 ? g.scale_log2 : g.scale_log2 * g.fp8_scale_k, ex - 15);
        cacc[gg] = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) o8[gg][e] = 0.f;
      }
      struct Rows8 {
        u32x4_t k, v;
        float ks, vs;
      };
      auto row_of8 = [&](int base, int j) __attribute__((always_inline)) {
        return base + (j * kWaves + wave) * RPW8 + grp8;
      };
      // rows of a batch from a uniform base row (the batch's first row, or
      // the last stored row when the batch starts past it) plus a lane
      // offset, clamped to the last stored row
      const int lane_row8 = wave * RPW8 + grp8;
      auto load8 = [&](Rows8 (&r)[kInFlight], Rows8 (&)[kInFlight], int base, int64_t r0) __attribute__((always_inline)) {
        const int bb = min(base, Tc - 1);
        const uint8_t* kb = reinterpret_cast<const uint8_t*>(g.rk) + (r0 + bb) * D;
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(g.rv) + (r0 + bb) * D;
        const char* ksb = reinterpret_cast<const char*>(g.rks + r0 + bb);
        const char* vsb = reinterpret_cast<const char*>(g.rvs + r0 + bb);
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
          const uint32_t rel = (uint32_t)min(lane_row8 + j * (kWaves * RPW8) + (base - bb), Tc - 1 - bb);
          r[j].k = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + (rel * D + c8 * 16)));
          r[j].v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + (rel * D + c8 * 16)));
          if constexpr (FMT == 1) {
            r[j].ks = *reinterpret_cast<const float*>(ksb + 4 * rel);
            r[j].vs = *reinterpret_cast<const float*>(vsb + 4 * rel);
          }
        }
      };
      auto process8 = [&](const Rows8 (&r)[kInFlight], const Rows8 (&)[kInFlight], int base)
          __attribute__((always_inline)) {
        float s[kInFlight][GC];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
          const bool valid = row_of8(base, j) < Tc;
          uint32_t kh[8];  // f16 pairs of the 16 codes: 1024 + b (int8), the e4m3 values (fp8)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (FMT == 1) {
              kh[2 * e] = __builtin_amdgcn_perm(0x64646464u, r[j].k[e], 0x04010400u);
              kh[2 * e + 1] = __builtin_amdgcn_perm(0x64646464u, r[j].k[e], 0x04030402u);
            } else {
              kh[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[j].k[e], 1.0f, false));
              kh[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[j].k[e], 1.0f, true));
            }
          }
#pragma unroll
          for (int gg = 0; gg < GC; ++gg) {
            float acc = qoff[gg];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, kh[e]), __builtin_bit_cast(f16x2_t, q16[gg][e]),
                                           acc, false);
            acc = group_sum<LPR8>(acc);
            s[j][gg] = valid ? acc * (FMT == 1 ? r[j].ks * qsc[gg] : qsc[gg]) : -INFINITY;
          }
        }
        // fp8: the codes of rows 2t and 2t + 1 for dim 4e + k as one exact
        // f16 pair (bytes interleaved by v_perm, then converted two at a time);
        // int8: their stored bytes b (0..255, exact in bf16) as one bf16 pair
        f16x2_t vh[FMT == 2 ? kInFlight / 2 : 1][16];
        uint32_t vb[FMT == 1 ? kInFlight / 2 : 1][16];
        if constexpr (FMT == 1) {
#pragma unroll
          for (int t = 0; t < kInFlight / 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int k = 0; k < 4; ++k)
                vb[t][4 * e + k] = pack_bf16x2((float)((r[2 * t].v[e] >> (8 * k)) & 0xffu),
                                               (float)((r[2 * t + 1].v[e] >> (8 * k)) & 0xffu));
        }
        if constexpr (FMT == 2) {
#pragma unroll
          for (int t = 0; t < kInFlight / 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t a0 = r[2 * t].v[e], a1 = r[2 * t + 1].v[e];
              const uint32_t lo = __builtin_amdgcn_perm(a1, a0, 0x05010400u);  // bytes a0.0 a1.0 a0.1 a1.1
              const uint32_t hi = __builtin_amdgcn_perm(a1, a0, 0x07030602u);  // bytes a0.2 a1.2 a0.3 a1.3
              vh[t][4 * e] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
              vh[t][4 * e + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
              vh[t][4 * e + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
              vh[t][4 * e + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
            }
        }
#pragma unroll
        for (int gg = 0; gg < GC; ++gg) {
          float mx = s[0][gg];
#pragma unroll
          for (int j = 1; j < kInFlight; ++j) mx = fmaxf(mx, s[j][gg]);
          // m is the reference the weights are taken against; it moves (and
          // l, cacc, o8 with it) only when a score passes it by more than the
          // slack (wave vote): exact, since they always share it, and it
          // saves the 8-bit rows' VALU-bound loop most of its rescales
          if (__any(mx > m[gg] + kDecodeSlack)) {
            const float mn = fmaxf(m[gg], mx);
            const float alpha = exp2_fast(m[gg] - max_or_zero(mn));
            l[gg] *= alpha;
            cacc[gg] *= alpha;
#pragma unroll
            for (int e = 0; e < 16; ++e) o8[gg][e] *= alpha;
            m[gg] = mn;
          }
          const float mu = max_or_zero(m[gg]);
          if constexpr (FMT == 2) {
            // rows in pairs: the two weights (at most 2^8) as one f16 pair,
            // l summed from those same values, and one v_dot2 per dim with
            // the pair's two codes of that dim (the exact f16 values of
            // vh); the V scale, one per tensor, comes in at the end
#pragma unroll
            for (int t = 0; t < kInFlight / 2; ++t) {
              const f16x2_t ph = {(_Float16)exp2_fast(s[2 * t][gg] - mu), (_Float16)exp2_fast(s[2 * t + 1][gg] - mu)};
              l[gg] = __builtin_amdgcn_fdot2(ph, ones16, l[gg], false);
#pragma unroll
              for (int e = 0; e < 16; ++e)
                o8[gg][e] = __builtin_amdgcn_fdot2(vh[t][e], ph, o8[gg][e], false);
            }
          } else {
            // int8, rows in pairs: the weights times the rows' V scales as
            // one bf16 pair (range of any scale), one v_dot2 per dim with the
            // pair's two bytes of that dim (vb); 128 * sum of those same
            // rounded products comes off once at the end
#pragma unroll
            for (int t = 0; t < kInFlight / 2; ++t) {
              const float p0 = exp2_fast(s[2 * t][gg] - mu), p1 = exp2_fast(s[2 * t + 1][gg] - mu);
              l[gg] += p0 + p1;
              const uint32_t pw = pack_bf16x2(p0 * r[2 * t].vs, p1 * r[2 * t + 1].vs);
              cacc[gg] = dot2_bf16(pw, 0x3f803f80u, cacc[gg]);  // (1, 1)
#pragma unroll
              for (int e = 0; e < 16; ++e) o8[gg][e] = dot2_bf16(vb[t][e], pw, o8[gg][e]);
            }
          }
        }
      };
      if (Tc > 0) {
        Rows8 ra[kInFlight], rb[kInFlight];
        stream_pairs(ra, ra, rb, rb, load8, process8, Tc, (Tc + PAIR8 - 1) / PAIR8,
                     std::integral_constant<int, PAIR8>(), std::integral_constant<int, ITER8>(), std::true_type());
      }
      // merge the row groups of the wave (16 dims per lane), then hand the
      // wave's state to the 8-dims-per-lane layout of the code below: lane
      // c < LPR takes dims 8c .. 8c+7 (half c mod 2 of lane c/2); the other
      // row groups are left empty
      if constexpr (FMT == 1) {
#pragma unroll
        for (int gg = 0; gg < GC; ++gg)
#pragma unroll
          for (int e = 0; e < 16; ++e) o8[gg][e] = fmaf(-128.0f, cacc[gg], o8[gg][e]);
      } else {
#pragma unroll
        for (int gg = 0; gg < GC; ++gg)
#pragma unroll
          for (int e = 0; e < 16; ++e) o8[gg][e] *= g.fp8_scale_v;  // a power of two: exact
      }
#pragma unroll
      for (int off = LPR8; off < 64; off <<= 1) {
#pragma unroll
        for (int gg = 0; gg < GC; ++gg) {
          const float mo = __shfl_xor(m[gg], off);
          const float lo = __shfl_xor(l[gg], off);
          const float mn = fmaxf(m[gg], mo);
          const float mu = max_or_zero(mn);
          const float a1 = exp2_fast(m[gg] - mu);
          const float a2 = exp2_fast(mo - mu);
          l[gg] = l[gg] * a1 + lo * a2;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float oo = __shfl_xor(o8[gg][e], off);
            o8[gg][e] = o8[gg][e] * a1 + oo * a2;
          }
          m[gg] = mn;
        }
      }
      const int src_lane = c >> 1;
      const bool keep = grp == 0;
#pragma unroll
      for (int gg = 0; gg < GC; ++gg) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float lo8 = __shfl(o8[gg][e], src_lane);
          const float hi8 = __shfl(o8[gg][8 + e], src_lane);
          o[gg][e] = keep ? ((c & 1) ? hi8 : lo8) : 0.f;
        }
        const float mw = __shfl(m[gg], src_lane), lw = __shfl(l[gg], src_lane);
        m[gg] = keep ? mw : -INFINITY;
        l[gg] = keep ? lw : 0.f;
      }
    } else {
      stream_bf16();
    }
  } else {
    stream_bf16();
  }
  // The new token, scored outside the row loop (int8 retrieval rows: at
  // input precision; rotary embedding: rotated): work-group 0, one lane
  // group of wave 0.
  if (q8 || g.rope) {
    own_new = split == 0;
    if (own_new) {
      uint4 vx = reinterpret_cast<const uint4*>(nv)[c];
      uint4 kx = knew;
      if (FMT == 2 && retrieval) {  // attended through its stored fp8 value (exact in bf16)
        kx = fp8_roundtrip8(kx, g.fp8_inv_k, g.fp8_scale_k);
        vx = fp8_roundtrip8(vx, g.fp8_inv_v, g.fp8_scale_v);
      }
      const bool mine = wave == 0 && grp == 0;
      const uint32_t kw[4] = {kx.x, kx.y, kx.z, kx.w}, vw[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
      for (int gg = 0; gg < GC; ++gg) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = dot2_bf16(kw[e], qw[gg][e], acc);
        acc = group_sum<LPR>(acc);
        const float sc = mine ? acc * g.scale_log2 : -INFINITY;
        const float mn = fmaxf(m[gg], sc);
        const float mu = max_or_zero(mn);
        const float alpha = exp2_fast(m[gg] - mu);
        const float p = exp2_fast(sc - mu);
        l[gg] = l[gg] * alpha + p;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[gg][2 * e] = fmaf(p, bf16_lo(vw[e]), o[gg][2 * e] * alpha);
          o[gg][2 * e + 1] = fmaf(p, bf16_hi(vw[e]), o[gg][2 * e + 1] * alpha);
        }
        m[gg] = mn;
      }
    }
  }

  // ---- merge the row groups of the wave (same head, different rows)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int gg = 0; gg < GC; ++gg) {
      const float mo = __shfl_xor(m[gg], off);
      const float lo = __shfl_xor(l[gg], off);
      const float mn = fmaxf(m[gg], mo);
      const float mu = max_or_zero(mn);
      const float a1 = exp2_fast(m[gg] - mu);
      const float a2 = exp2_fast(mo - mu);
      l[gg] = l[gg] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float oo = __shfl_xor(o[gg][e], off);
        o[gg][e] = o[gg][e] * a1 + oo * a2;
      }
      m[gg] = mn;
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int gg = 0; gg < GC; ++gg) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wave][gg][c * 8 + e] = o[gg][e];
      if (lane == 0) {
        sm_m[wave][gg] = m[gg];
        sm_l[wave][gg] = l[gg];
      }
    }
  }

  // ---- the owner of the new token stores it (one head chunk does it)
  if (hc == 0 && own_new && threadIdx.x < LPR) {
    const uint4 kx = knew;  // threads 0..LPR-1 hold chunks c = 0..LPR-1
    const uint4 vx = reinterpret_cast<const uint4*>(nv)[threadIdx.x];
    const int64_t row = retrieval ? retrieval_row0(g, b, idx, new_row) + new_row : unit_row0 + new_row;
    if (q8 && FMT == 2) {
      store_fp8_row8(reinterpret_cast<uint8_t*>(g.rk) + row * D, kx, threadIdx.x, g.fp8_inv_k);
      store_fp8_row8(reinterpret_cast<uint8_t*>(g.rv) + row * D, vx, threadIdx.x, g.fp8_inv_v);
    } else if (q8) {
      store_int8_row<LPR>(reinterpret_cast<uint8_t*>(g.rk) + row * D, g.rks + row, kx, threadIdx.x);
      store_int8_row<LPR>(reinterpret_cast<uint8_t*>(g.rv) + row * D, g.rvs + row, vx, threadIdx.x);
    } else {
      reinterpret_cast<uint4*>((retrieval ? g.rk : g.sk) + row * D)[threadIdx.x] = kx;
      reinterpret_cast<uint4*>((retrieval ? g.rv : g.sv) + row * D)[threadIdx.x] = vx;
    }
    if (threadIdx.x == 0 && kvh == 0) g.lengths[b] = L + 1;
  }
  __syncthreads();

  // ---- merge the waves; write the output or this work-group's record
  float* rec_o = unit_records<D, GC>(g, pu);
  float* rec_ml = rec_o + (int64_t)g.max_splits * GC * D;  // (m, l) pairs
  for (int t = threadIdx.x; t < GC * D; t += kThreads) {
    const int gg = t / D, d = t % D;
    float mw = sm_m[0][gg];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mw = fmaxf(mw, sm_m[w][gg]);
    const float mu = max_or_zero(mw);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2_fast(sm_m[w][gg] - mu);
      lsum += sm_l[w][gg] * f;
      osum += sm_o[w][gg][d] * f;
    }
    if (ns == 1) {
      a.out[((int64_t)b * g.Hq + h0 + gg) * D + d] = (uint16_t)f32_to_bf16_bits(osum / lsum);
    } else {
      store_agent(&rec_o[((int64_t)split * GC + gg) * D + d], osum);
      if (d == 0) {
        store_agent(&rec_ml[2 * (split * GC + gg)], mw);
        store_agent(&rec_ml[2 * (split * GC + gg) + 1], lsum);
      }
    }
  }
  if (ns == 1) {  // the only claimer of this unit
    if (dynamic && threadIdx.x == 0) __hip_atomic_store(t_claim, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // ---- merge.  Each work-group's record stores are complete (at the
  // agent-coherent level) before its ticket increment.  The work-groups of
  // a unit arrive in groups of kMergeGroup; the last arrival of a group
  // arrives at the unit's counter, and the last arrival there (after which
  // no work-group of the unit claims any more) resets the claim counter and
  // merges.  Up to single_merge_max records it merges them all in one pass;
  // beyond that the last arrival of each group first merges its group into
  // the group's first record slot.
  __builtin_amdgcn_s_waitcnt(0);
  const int mgrp = split / kMergeGroup;
  const int ng = (ns + kMergeGroup - 1) / kMergeGroup;
  const int g0 = mgrp * kMergeGroup;
  const int gsz = min(kMergeGroup, ns - g0);
  uint32_t* t_group = t_unit + kTicketStride * (2 + mgrp);  // arrivals of this group
  // True in the work-group that completes n arrivals at *t (which it resets).
  auto last_arrival = [&](uint32_t* t, int n) {
    __syncthreads();  // also: sm_flag of an earlier call has been read
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm_flag = prev == (uint32_t)(n - 1);
      if (sm_flag) __hip_atomic_store(t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return sm_flag != 0;
  };
  auto reset_claims = [&]() {
    if (dynamic && threadIdx.x == 0) __hip_atomic_store(t_claim, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if constexpr (single_merge_max<D, GC>() > 0) {
    if (ns <= single_merge_max<D, GC>()) {
      // a few dozen arrivals go straight to the unit's counter (one atomic
      // round trip less for the last one)
      const bool grouped = ns > kDirectArrivals;
      if (grouped && !last_arrival(t_group, gsz)) return;
      if (!last_arrival(t_unit, grouped ? ng : ns)) return;
      reset_claims();
      merge_single<D, GC>(g, a, sm_raw, rec_o, rec_ml, ns, b, h0);
      return;
    }
  }
  if (!last_arrival(t_group, gsz)) return;
  merge_records<D, GC>(g, a, sm_raw, rec_o, rec_ml, g0, 1, gsz, ng == 1, b, h0);
  if (ng == 1) {
    reset_claims();
    return;
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (!last_arrival(t_unit, ng)) return;
  reset_claims();
  merge_records<D, GC>(g, a, sm_raw, rec_o, rec_ml, 0, kMergeGroup, ng, true, b, h0);
}

}  // namespace

// Scratch of duo_decode_static_scratch: counters first, partial results
// after them.  In host code `scratch` names a host-side stand-in; its device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kStaticTicketBytes + kStaticRecordBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t static_decode_scratch(void** base, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // every call that completes leaves the counters it used at zero; they
    // start at zero here, on the caller's stream, before its first decode
    e = launch_zero_words(static_cast<uint32_t*>(p), kStaticTicketBytes / 4, s);
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *base = g_scratch[dev];
  return hipSuccess;
}

int32_t max_splits_for(int64_t max_len, int32_t slots, int head_chunk) {
  const int64_t rows = max_len > slots ? max_len : slots;
  const int64_t s = (rows + 255) / 256;
  const int64_t cap = kMaxMergeRecords / head_chunk;
  return (int32_t)(s < cap ? s : cap);
}

namespace {
template <int DD, int GG>
const void* decode_fn(const Geom& g) {
  if constexpr (GG <= 4) {
    if (g.kv_int8) return reinterpret_cast<const void*>(&decode_kernel<DD, GG, 1>);
    if (g.kv_fp8) return reinterpret_cast<const void*>(&decode_kernel<DD, GG, 2>);
  }
  return reinterpret_cast<const void*>(&decode_kernel<DD, GG, 0>);
}
std::mutex g_occ_mu;
int32_t g_occ[2][4][3] = {};  // [D 64/128][head chunk 1/2/4/8][format]: 0 = not yet queried
}  // namespace

// Decode work-groups of the instance that `g` launches with `head_chunk`
// that one CU holds at once (its occupancy), queried once per instance;
// 4 when no device answers.
int32_t decode_wgs_per_cu(const Geom& g, int head_chunk) {
  const int di = g.D == 128 ? 1 : 0;
  const int ci = head_chunk == 8 ? 3 : head_chunk == 4 ? 2 : head_chunk == 2 ? 1 : 0;
  const int fi = g.kv_int8 ? 1 : g.kv_fp8 ? 2 : 0;
  std::lock_guard<std::mutex> lock(g_occ_mu);
  int32_t& slot = g_occ[di][ci][fi];
  if (slot == 0) {
    const void* fn = nullptr;
#define DUO_OCC_CASE(DD, GG) \
    if (g.D == DD && head_chunk == GG) fn = decode_fn<DD, GG>(g);
    DUO_OCC_CASE(128, 1) DUO_OCC_CASE(128, 2) DUO_OCC_CASE(128, 4) DUO_OCC_CASE(128, 8)
    DUO_OCC_CASE(64, 1) DUO_OCC_CASE(64, 2) DUO_OCC_CASE(64, 4) DUO_OCC_CASE(64, 8)
#undef DUO_OCC_CASE
    int n = 0;
    if (fn == nullptr || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, 0) != hipSuccess || n < 1) {
      (void)hipGetLastError();
      return 4;
    }
    slot = n;
  }
  return slot;
}

DecodePlan plan_decode(const Geom& g, const Seqs& q, int32_t num_cus) {
  DecodePlan p;
  const bool byte_rows = g.kv_int8 || g.kv_fp8;
  p.head_chunk = decode_head_chunk(g.G, byte_rows);
  const int n_hc = g.G / p.head_chunk;
  // the larger pair when the retrieval rows are int8 (a multiple of the bf16 one)
  const int64_t pair = byte_rows ? decode_pair_rows_int8(g.D, p.head_chunk) : decode_pair_rows(g.D, p.head_chunk);
  int64_t total = 0;
  int32_t tmax = 1;
  for (int b = 0; b < g.B; ++b) {
    total += (int64_t)(q.len[b] + 1) * g.nR * n_hc;
    tmax = q.len[b] + 1 > tmax ? q.len[b] + 1 : tmax;
  }
  // Rows per work-group on average (work-groups of a unit share its rows
  // dynamically): about 2048 work-groups over the retrieval rows, at least
  // kMinPairs pairs each, and few enough work-groups per unit for its records.
  auto round_pair = [&](int64_t x) { return (x + pair - 1) / pair * pair; };
  int64_t ts = round_pair((total + 2047) / 2048);
  const int min_pairs = byte_rows ? kMinPairsInt8 : kMinPairs;
  // One query head per work-group: a work-group scores each row it reads
  // once and keeps 64 KB of loads in flight, as much as one CU's share of
  // HBM bandwidth needs, so the call gets about one work-group per CU.  More
  // work-groups only add split records to merge and stretch the end of the
  // stream (the last claimed pair of a unit runs on a CU shared with other
  // work-groups); on the 32K MHA layer one per CU beats the ~2000-work-group
  // rule by 6%.  With several query heads per work-group each row costs
  // several dot products, and the ~2000-work-group rule stays (the 8-by-128K
  // GQA batch runs 9% slower at half as many work-groups).
  if (p.head_chunk == 1 && g.nR > 0) {
    const int64_t units_r = (int64_t)g.B * g.nR * n_hc;
    const int64_t wg_s = (int64_t)g.B * g.nS * n_hc;  // about one per streaming unit
    const int64_t per_unit = ((int64_t)num_cus - wg_s) / units_r;
    if (per_unit >= 1) ts = round_pair(((int64_t)tmax + per_unit - 1) / per_unit);
  }
  if (ts < min_pairs * pair) ts = min_pairs * pair;
  const int64_t ts_cap = round_pair(((int64_t)tmax + g.max_splits - 1) / g.max_splits);
  if (ts < ts_cap) ts = ts_cap;
  // Several query heads per work-group: size the split so that the call's
  // work-groups fill a whole number of rounds of the resident work-groups
  // (CUs x the instance's occupancy), the streaming units' short work-groups
  // counted in: the smallest split whose work-groups fit.
  if (p.head_chunk > 1 && g.nR > 0) {
    const int64_t slots = (int64_t)num_cus * decode_wgs_per_cu(g, p.head_chunk);
    int64_t wg_s = 0;
    for (int b = 0; b < g.B; ++b) wg_s += (int64_t)g.nS * n_hc * (q.len[b] + 1 > 0 ? 1 : 0);
    // Measured (sweep of 1-3 rounds): for sequences of equal length two
    // rounds, which is what the ~2048 rule gave already (the 8 x 128K GQA
    // batch: 354 us at one, two or that rule, 369 at three); three when
    // lengths differ (the mixed batch of 32, U[4096, 65536]: 0.70-0.75 of
    // HBM peak at three against 0.56-0.74 by that rule and 0.54-0.73 at two),
    // where every unit ends in a partial work-group and finer splits balance
    // them better.
    bool same_len = true;
    for (int b = 1; b < g.B; ++b) same_len = same_len && q.len[b] == q.len[0];
    const int rounds = same_len ? 2 : 3;
    const int64_t target = rounds * slots - wg_s;
    if (target >= (int64_t)g.B * g.nR * n_hc) {
      auto wgs = [&](int64_t t) {
        int64_t n = 0;
        for (int b = 0; b < g.B; ++b) n += (int64_t)g.nR * n_hc * (((int64_t)q.len[b] + 1 + t - 1) / t);
        return n;
      };
      // smallest multiple of the pair size, at least the minimum split and
      // the record cap's split, whose work-groups fit the target
      // (wgs() does not grow with the split: a binary search over pairs)
      int64_t lo = round_pair((total + target - 1) / target);
      if (lo < min_pairs * pair) lo = min_pairs * pair;
      if (lo < ts_cap) lo = ts_cap;
      int64_t hi = round_pair(tmax) > lo ? round_pair(tmax) : lo;  // one work-group per unit fits
      while (lo < hi) {
        const int64_t mid = lo + ((hi - lo) / pair / 2) * pair;
        if (wgs(mid) <= target) hi = mid;
        else lo = mid + pair;
      }
      ts = lo;
    }
  }
  p.split_tokens = (int32_t)ts;
  p.splits_r = (int32_t)((tmax + ts - 1) / ts);
  const int32_t smax = tmax < g.slots ? tmax : g.slots;
  p.splits_s = (int32_t)((smax + ts - 1) / ts);
  return p;
}

// int8 retrieval caches use head chunks of at most 4 (decode_head_chunk).
template <int DD, int GG>
hipError_t launch_dg(const Geom& g, const Seqs& q, const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if constexpr (GG <= 4) {
    if (g.kv_int8) {
      hipLaunchKernelGGL((decode_kernel<DD, GG, 1>), grid, block, 0, s, g, q, a);
      return hipGetLastError();
    }
    if (g.kv_fp8) {
      hipLaunchKernelGGL((decode_kernel<DD, GG, 2>), grid, block, 0, s, g, q, a);
      return hipGetLastError();
    }
  }
  if (g.kv_int8 || g.kv_fp8) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_kernel<DD, GG, 0>), grid, block, 0, s, g, q, a);
  return hipGetLastError();
}

hipError_t launch_decode(const Geom& g, const Seqs& q, const DecodePlan& p, const uint16_t* qin,
                         const uint16_t* kin, const uint16_t* vin, uint16_t* out, hipStream_t s) {
  DecodeArgs a{qin, kin, vin, out, p.split_tokens, p.splits_r, p.splits_s};
  const int n_hc = g.G / p.head_chunk;
  const int64_t items = (int64_t)g.B * g.nR * n_hc * p.splits_r + (int64_t)g.B * g.nS * n_hc * p.splits_s;
  if (items <= 0) return hipSuccess;
  const dim3 grid((unsigned)items), block(kThreads);
#define DUO_DECODE_CASE(DD, GG) \
  if (g.D == DD && p.head_chunk == GG) return launch_dg<DD, GG>(g, q, a, grid, block, s);
  DUO_DECODE_CASE(128, 1)
  DUO_DECODE_CASE(128, 2)
  DUO_DECODE_CASE(128, 4)
  DUO_DECODE_CASE(128, 8)
  DUO_DECODE_CASE(64, 1)
  DUO_DECODE_CASE(64, 2)
  DUO_DECODE_CASE(64, 4)
  DUO_DECODE_CASE(64, 8)
#undef DUO_DECODE_CASE
  return hipErrorInvalidValue;
}

}  // namespace duo
