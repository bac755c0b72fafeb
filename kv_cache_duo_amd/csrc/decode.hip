// Mixed retrieval/streaming decoding (one new token per sequence).
//
// DuoAttention (abstract, as reproduced on the pith.science review page):
// retrieval heads attend over their full KV cache, streaming heads over the
// constant-length cache of sinks + recent tokens.  Decoding is memory-bound:
// every cached K/V byte of a retrieval head is read once per step.
//
// One launch does everything for a step:
//   * work item = (sequence b, KV head, query-head chunk, split).  A split is
//     a contiguous range of cache rows (retrieval: rows = positions 0..L;
//     streaming: the min(L+1, sink+recent) occupied slots).  The new token's
//     row is read from the input and written to the cache by its owner, so
//     no work item ever reads a row that is being written;
//   * each work-group streams its rows with coalesced 16-byte loads (a row of
//     D bf16 is read by D/8 lanes), scores all query heads of the KV group
//     from the same K bytes with bf16 dot2 + DPP group sums, and keeps an
//     online softmax (running max m, sum l, unnormalised o) per head;
//   * splits of one unit are merged by the last work-group to finish (agent
//     -scope atomic ticket): M = max m_k, L = sum l_k 2^(m_k-M),
//     O = sum o_k 2^(m_k-M) / L.  A unit with one split writes directly.
// Scores are kept in base-2 units (scale * log2 e folded in), so exp2 is the
// only transcendental.
#include <cfloat>
#include <cstdlib>

#include "device_util.h"
#include "duo_internal.h"

namespace duo {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr int kInFlight = 4;   // K rows and V rows loaded per lane before use

struct DecodeArgs {
  const uint16_t* q;  // [B][Hq][D]
  const uint16_t* k;  // [B][Hkv][D]
  const uint16_t* v;
  uint16_t* out;      // [B][Hq][D]
  int32_t split_tokens, splits_r, splits_s;
};

__device__ __forceinline__ float max_or_zero(float m) { return m == -INFINITY ? 0.f : m; }

template <int D, int GC>
__global__ __launch_bounds__(kThreads) void decode_kernel(Geom g, Seqs sq, DecodeArgs a) {
  constexpr int LPR = D / 8;                  // lanes per row (8 bf16 each)
  constexpr int RPW = 64 / LPR;               // rows per wave per load
  constexpr int ROWS_ITER = kWaves * RPW * kInFlight;
  __shared__ float sm_o[kWaves][GC][D];
  __shared__ float sm_m[kWaves][GC];
  __shared__ float sm_l[kWaves][GC];
  __shared__ int sm_last;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane / LPR;
  const int c = lane % LPR;

  // ---- work item
  const int n_hc = g.G / GC;
  int id = blockIdx.x;
  const int items_r = g.B * g.nR * n_hc * a.splits_r;
  bool retrieval = id < items_r;
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
  const int ns = (T + a.split_tokens - 1) / a.split_tokens;
  if (split >= ns) return;
  const int r0 = split * a.split_tokens;
  const int r1 = min(r0 + a.split_tokens, T);
  const int kvh = g.kv_of_unit[retrieval ? idx : g.nR + idx];
  const int64_t unit_rows = retrieval ? g.max_len : (int64_t)g.slots;
  const int64_t cache_off = ((int64_t)b * nkind + idx) * unit_rows * D;
  uint16_t* ck = (retrieval ? g.rk : g.sk) + cache_off;
  uint16_t* cv = (retrieval ? g.rv : g.sv) + cache_off;
  const uint16_t* nk = a.k + ((int64_t)b * g.Hkv + kvh) * D;
  const uint16_t* nv = a.v + ((int64_t)b * g.Hkv + kvh) * D;
  const int h0 = kvh * g.G + hc * GC;

  // ---- queries of the GC heads: this lane's 8 dims of each
  uint32_t qw[GC][4];
#pragma unroll
  for (int gg = 0; gg < GC; ++gg) {
    uint4 t = reinterpret_cast<const uint4*>(a.q + ((int64_t)b * g.Hq + h0 + gg) * D)[c];
    qw[gg][0] = t.x; qw[gg][1] = t.y; qw[gg][2] = t.z; qw[gg][3] = t.w;
  }

  float m[GC], l[GC], o[GC][8];
#pragma unroll
  for (int gg = 0; gg < GC; ++gg) {
    m[gg] = -INFINITY;
    l[gg] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[gg][e] = 0.f;
  }

  for (int base = r0; base < r1; base += ROWS_ITER) {
    uint4 kr[kInFlight], vr[kInFlight];
    bool valid[kInFlight];
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) {
      const int row = base + (j * kWaves + wave) * RPW + grp;
      valid[j] = row < r1;
      const uint16_t* pk = row == new_row ? nk : ck + (int64_t)row * D;
      const uint16_t* pv = row == new_row ? nv : cv + (int64_t)row * D;
      if (valid[j]) {
        kr[j] = reinterpret_cast<const uint4*>(pk)[c];
        vr[j] = reinterpret_cast<const uint4*>(pv)[c];
      } else {
        kr[j] = make_uint4(0, 0, 0, 0);
        vr[j] = make_uint4(0, 0, 0, 0);
      }
    }
    float s[kInFlight][GC];
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) {
#pragma unroll
      for (int gg = 0; gg < GC; ++gg) {
        float acc = dot2_bf16(kr[j].x, qw[gg][0], 0.f);
        acc = dot2_bf16(kr[j].y, qw[gg][1], acc);
        acc = dot2_bf16(kr[j].z, qw[gg][2], acc);
        acc = dot2_bf16(kr[j].w, qw[gg][3], acc);
        acc = group_sum<LPR>(acc);
        s[j][gg] = valid[j] ? acc * g.scale_log2 : -INFINITY;
      }
    }
#pragma unroll
    for (int gg = 0; gg < GC; ++gg) {
      float mx = s[0][gg];
#pragma unroll
      for (int j = 1; j < kInFlight; ++j) mx = fmaxf(mx, s[j][gg]);
      const float mn = fmaxf(m[gg], mx);
      const float mu = max_or_zero(mn);
      const float alpha = exp2_fast(m[gg] - mu);
      l[gg] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[gg][e] *= alpha;
#pragma unroll
      for (int j = 0; j < kInFlight; ++j) {
        const float p = exp2_fast(s[j][gg] - mu);
        l[gg] += p;
        const uint32_t w[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[gg][2 * e] = fmaf(p, bf16_lo(w[e]), o[gg][2 * e]);
          o[gg][2 * e + 1] = fmaf(p, bf16_hi(w[e]), o[gg][2 * e + 1]);
        }
      }
      m[gg] = mn;
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
  if (hc == 0 && new_row >= r0 && new_row < r1 && threadIdx.x < LPR) {
    const int64_t off = (int64_t)new_row * D;
    reinterpret_cast<uint4*>(ck + off)[threadIdx.x] = reinterpret_cast<const uint4*>(nk)[threadIdx.x];
    reinterpret_cast<uint4*>(cv + off)[threadIdx.x] = reinterpret_cast<const uint4*>(nv)[threadIdx.x];
    if (threadIdx.x == 0 && kvh == 0) g.lengths[b] = L + 1;
  }
  __syncthreads();

  // ---- merge the waves; write the output or this split's partial record
  const int64_t pu = ((int64_t)b * g.Hkv + kvh) * n_hc + hc;
  float* recs = g.partials + pu * g.max_splits * GC * (D + 2);
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
      float* rec = recs + ((int64_t)split * GC + gg) * (D + 2);
      rec[d] = osum;
      if (d == 0) {
        rec[D] = mw;
        rec[D + 1] = lsum;
      }
    }
  }
  if (ns == 1) return;

  // ---- last work-group of the unit merges all splits
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(&g.tickets[pu], 1u);
    sm_last = prev == (uint32_t)(ns - 1);
  }
  __syncthreads();
  if (!sm_last) return;
  __threadfence();
  for (int t = threadIdx.x; t < GC * D; t += kThreads) {
    const int gg = t / D, d = t % D;
    float mx = -INFINITY;
    for (int k = 0; k < ns; ++k) mx = fmaxf(mx, recs[((int64_t)k * GC + gg) * (D + 2) + D]);
    const float mu = max_or_zero(mx);
    float lsum = 0.f, osum = 0.f;
    for (int k = 0; k < ns; ++k) {
      const float* rec = recs + ((int64_t)k * GC + gg) * (D + 2);
      const float f = exp2_fast(rec[D] - mu);
      lsum += rec[D + 1] * f;
      osum += rec[d] * f;
    }
    a.out[((int64_t)b * g.Hq + h0 + gg) * D + d] = (uint16_t)f32_to_bf16_bits(osum / lsum);
  }
  if (threadIdx.x == 0) g.tickets[pu] = 0u;  // ready for the next call
}

}  // namespace

int32_t max_splits_for(int64_t max_len, int32_t slots) {
  int64_t rows = max_len > slots ? max_len : slots;
  int64_t s = (rows + 255) / 256;
  return (int32_t)(s < 1024 ? s : 1024);
}

static int head_chunk_for(int G) {
  for (int c : {8, 4, 2, 1})
    if (G % c == 0) return c;
  return 1;
}

DecodePlan plan_decode(const Geom& g, const Seqs& q) {
  DecodePlan p;
  p.head_chunk = head_chunk_for(g.G);
  const int n_hc = g.G / p.head_chunk;
  int64_t total = 0;
  int32_t tmax = 1;
  for (int b = 0; b < g.B; ++b) {
    total += (int64_t)(q.len[b] + 1) * g.nR * n_hc;
    tmax = q.len[b] + 1 > tmax ? q.len[b] + 1 : tmax;
  }
  auto round64 = [](int64_t x) { return (x + 63) / 64 * 64; };
  int64_t ts = round64((total + 2047) / 2048);
  if (ts < 256) ts = 256;
  const int64_t ts_cap = round64(((int64_t)tmax + g.max_splits - 1) / g.max_splits);
  if (ts < ts_cap) ts = ts_cap;
  static const int64_t env_ts = [] {
    const char* e = getenv("DUO_DECODE_SPLIT_TOKENS");
    return e ? (int64_t)atoll(e) : (int64_t)0;
  }();
  if (env_ts >= 64 && env_ts % 64 == 0 && env_ts >= ts_cap) ts = env_ts;
  p.split_tokens = (int32_t)ts;
  p.splits_r = (int32_t)((tmax + ts - 1) / ts);
  const int32_t smax = tmax < g.slots ? tmax : g.slots;
  p.splits_s = (int32_t)((smax + ts - 1) / ts);
  return p;
}

hipError_t launch_decode(const Geom& g, const Seqs& q, const DecodePlan& p, const uint16_t* qin,
                         const uint16_t* kin, const uint16_t* vin, uint16_t* out, hipStream_t s) {
  DecodeArgs a{qin, kin, vin, out, p.split_tokens, p.splits_r, p.splits_s};
  const int n_hc = g.G / p.head_chunk;
  const int64_t items = (int64_t)g.B * g.nR * n_hc * p.splits_r + (int64_t)g.B * g.nS * n_hc * p.splits_s;
  if (items <= 0) return hipSuccess;
  const dim3 grid((unsigned)items), block(kThreads);
#define DUO_DECODE_CASE(DD, GG)                                                   \
  if (g.D == DD && p.head_chunk == GG) {                                          \
    hipLaunchKernelGGL((decode_kernel<DD, GG>), grid, block, 0, s, g, q, a);      \
    return hipGetLastError();                                                     \
  }
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
