// Mixed retrieval/streaming pre-filling on bf16 MFMA (gfx950).
//
// DuoAttention (abstract, as reproduced on the pith.science review page)
// speeds up pre-filling as well as decoding: retrieval heads run full causal
// attention over every earlier position, streaming heads only over the
// attention sinks and the recent window.  Per query at position p:
//   retrieval: keys 0..p;   streaming: keys j <= p with j < sink or j > p-recent.
// Earlier positions come from the cache (retrieval rows, or the sink / ring
// slots of streaming heads), positions of this chunk from the inputs, so a
// sequence may be prefilled in chunks.  The append of the chunk runs after
// this kernel (streaming ring slots read here may be overwritten by it).
//
// Tile engine (flash-style online softmax, fp32 accumulation):
//   * work-group = 4 waves; each wave owns 32 query rows of one query head
//     (the work-group covers 128 rows: 128/gh tokens x gh heads of one KV
//     group, so every K/V tile staged in LDS serves gh query heads);
//   * K/V tiles of 64 keys are gathered row by row (any mix of cache rows,
//     ring slots and chunk rows) with 16-byte loads into registers while the
//     previous tile is computed, then stored to a double-buffered LDS: K as
//     rows, V transposed so that both MFMA operands are 16-byte LDS reads;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q
//     held in registers), so each lane holds 32 scores of ONE query: the
//     row max and sum need only in-lane work plus one exchange with lane^32;
//   * P (bf16) feeds O^T += V^T P^T straight from the S^T registers: the key
//     order inside a 16-key MFMA step is permuted identically in P and in the
//     transposed V tile, which is legal because keys are the contracted axis.
//   * keys are processed longest-q-tile-first, t-major and unit-minor, so the
//     work-groups resident on one XCD share a KV head and its L2 lines.
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "duo_internal.h"

namespace duo {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBN = 64;      // keys per tile
constexpr int kRowsWave = 32;

struct PrefillArgs {
  const uint16_t* q;  // [B][chunk][Hq][D]
  const uint16_t* k;  // [B][chunk][Hkv][D]
  const uint16_t* v;
  uint16_t* out;      // [B][chunk][Hq][D]
  int32_t chunk;
  int32_t tiles_max;  // query tiles per sequence, max over sequences
  int32_t gh;         // query heads per work-group (1, 2 or 4)
  int32_t tq;         // tokens per query tile = 128 / gh
  int32_t n_hc;       // G / gh
  int32_t items_r;    // work-groups of retrieval heads
};

template <int D>
struct Lds {
  static constexpr int KSTRIDE = D * 2 + 16;        // bytes per K row (padded)
  static constexpr int VSTRIDE = kBN * 2 + 16;      // bytes per V^T row (padded)
  static constexpr int KBYTES = kBN * KSTRIDE;
  static constexpr int VBYTES = D * VSTRIDE;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int TOTAL = 2 * BUF;
};

// Position inside a 16-key block of the transposed V tile where key `kk`
// (0..15) is stored: 4-key groups 1 and 2 swap places, matching the order in
// which the S^T accumulator registers hold keys.
__device__ __forceinline__ int vt_pos(int kk) {
  const int b16 = kk >> 4, g4 = (kk >> 2) & 3;
  const int sw = g4 == 1 ? 2 : (g4 == 2 ? 1 : g4);
  return b16 * 16 + sw * 4 + (kk & 3);
}

__device__ __forceinline__ uint32_t word_of(const uint4& x, int i) {
  return i == 0 ? x.x : (i == 1 ? x.y : (i == 2 ? x.z : x.w));
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(Geom g, Seqs sq, PrefillArgs a) {
  using LD = Lds<D>;
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int RPT = kBN * CH / kThreads;  // tile rows loaded per thread (4 or 2)
  constexpr int QC = D / 16;                // MFMA k-steps of Q K^T
  constexpr int DB = D / 32;                // 32-wide column blocks of O
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;   // query row of the wave held by this lane
  const int half = lane >> 5;  // which 8-wide k slice / 4-row group

  // ---- work item: t-major (longest tiles first), unit-minor
  int id = blockIdx.x;
  const bool retrieval = id < a.items_r;
  if (!retrieval) id -= a.items_r;
  const int nkind = retrieval ? g.nR : g.nS;
  const int per_t = g.B * nkind * a.n_hc;
  const int t = a.tiles_max - 1 - id / per_t;
  int rest = id % per_t;
  const int hc = rest % a.n_hc;
  rest /= a.n_hc;
  const int idx = rest % nkind;
  const int b = rest / nkind;
  const int n = sq.n[b];
  if (t * a.tq >= n) return;
  const int L = sq.len[b];
  const int kvh = g.kv_of_unit[retrieval ? idx : g.nR + idx];
  const int64_t unit_rows = retrieval ? g.max_len : (int64_t)g.slots;
  const int64_t cache_off = ((int64_t)b * nkind + idx) * unit_rows * D;
  const uint16_t* ck = (retrieval ? g.rk : g.sk) + cache_off;
  const uint16_t* cv = (retrieval ? g.rv : g.sv) + cache_off;

  // query positions of the work-group and of this wave
  const int i_lo = t * a.tq;                          // first chunk row
  const int i_hi = min(i_lo + a.tq, n) - 1;           // last chunk row
  const int qmin = L + i_lo, qmax = L + i_hi;
  const int waves_per_head = kWaves / a.gh;
  const int gg = wave / waves_per_head;
  const int wi0 = i_lo + (wave % waves_per_head) * kRowsWave;  // wave's first chunk row
  const int wqmin = L + wi0;
  const int wqmax = L + min(wi0 + kRowsWave, n) - 1;
  const int h = kvh * g.G + hc * a.gh + gg;
  const int my_i = wi0 + col;                          // this lane's query row
  const int my_q = L + my_i;

  // ---- key tiles: retrieval 0..qmax; streaming sinks + window
  int tA = 0, tB0 = 0, tB1 = qmax / kBN;  // tiles [0,tA) then [tB0,tB1]
  if (!retrieval) {
    const int sink_end = min(g.S, qmax + 1);
    tA = (sink_end + kBN - 1) / kBN;
    tB0 = max(qmin - g.W + 1, 0) / kBN;
    if (tB0 <= tA) {
      tA = 0;
      tB0 = 0;
    }
  }
  const int ntiles = tA + (tB1 - tB0 + 1);
  auto tile_of = [&](int k) { return k < tA ? k : tB0 + (k - tA); };

  // ---- Q operand (B of S^T = K Q^T): lane holds row `col`, k slice `half`
  bf16x8_t qreg[QC];
  {
    const bool ok = wave < kWaves && my_i <= i_hi;
    const uint4* src = reinterpret_cast<const uint4*>(a.q + (((int64_t)b * a.chunk + my_i) * g.Hq + h) * D);
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      uint4 x = ok ? src[2 * c + half] : make_uint4(0, 0, 0, 0);
      qreg[c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // ---- tile loader: thread -> RPT consecutive keys at one 16-byte chunk
  const int ch = threadIdx.x % CH;
  const int rg = threadIdx.x / CH;
  uint4 kbuf[RPT], vbuf[RPT];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int kp = tile * kBN + rg * RPT + i;
      const uint16_t* pk = nullptr;
      const uint16_t* pv = nullptr;
      if (kp <= qmax) {
        if (kp >= L) {
          const int64_t o = (((int64_t)b * a.chunk + (kp - L)) * g.Hkv + kvh) * D;
          pk = a.k + o;
          pv = a.v + o;
        } else if (retrieval || kp < g.S) {
          pk = ck + (int64_t)kp * D;
          pv = cv + (int64_t)kp * D;
        } else if (kp >= L - g.W) {
          const int64_t slot = g.S + (kp - g.S) % g.W;
          pk = ck + slot * D;
          pv = cv + slot * D;
        }
      }
      if (pk != nullptr) {
        kbuf[i] = reinterpret_cast<const uint4*>(pk)[ch];
        vbuf[i] = reinterpret_cast<const uint4*>(pv)[ch];
      } else {
        kbuf[i] = make_uint4(0, 0, 0, 0);
        vbuf[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* kb = smem + buf * LD::BUF;
    char* vb = kb + LD::KBYTES;
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<uint4*>(kb + (rg * RPT + i) * LD::KSTRIDE + ch * 16) = kbuf[i];
    const int pos = vt_pos(rg * RPT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      char* dst = vb + (ch * 8 + e) * LD::VSTRIDE + pos * 2;
      const uint32_t lo = __builtin_amdgcn_perm(word_of(vbuf[1], e >> 1), word_of(vbuf[0], e >> 1), sel);
      if constexpr (RPT == 4) {
        const uint32_t hi = __builtin_amdgcn_perm(word_of(vbuf[3], e >> 1), word_of(vbuf[2], e >> 1), sel);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<uint32_t*>(dst) = lo;
      }
    }
  };

  // ---- softmax state: this lane's query (m, partial l) and O^T columns
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = g.scale_log2;

  load_tile(tile_of(0));
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    const int tile = tile_of(kt);
    const int k0 = tile * kBN;
    if (kt + 1 < ntiles) load_tile(tile_of(kt + 1));

    // wave-uniform: can this tile hold a key any of the wave's queries see?
    bool live = k0 <= wqmax;
    if (!retrieval && k0 >= g.S && k0 + kBN - 1 < wqmin - g.W + 1) live = false;
    if (live) {
      const char* kb = smem + cur * LD::BUF;
      const char* vb = kb + LD::KBYTES;
      f32x16_t sacc[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb2][r] = 0.f;
#pragma unroll
        for (int c = 0; c < QC; ++c) {
          const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kb + (kb2 * 32 + col) * LD::KSTRIDE + (2 * c + half) * 16);
          sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[c], sacc[kb2], 0, 0, 0);
        }
      }
      // masks: causal for the diagonal tiles, band for streaming heads
      const bool need_mask = !retrieval || k0 + kBN - 1 > wqmin;
      if (need_mask) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kp = k0 + kb2 * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            bool ok = kp <= my_q;
            if (!retrieval) ok = ok && (kp < g.S || kp > my_q - g.W);
            if (!ok) sacc[kb2][r] = -INFINITY;
          }
      }
      float mt = sacc[0][0];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb2][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt * c2);
      const float mu = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - mu);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          bf16x8_t pb;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const float p = exp2_fast(fmaf(sacc[kb2][st * 8 + r], c2, -mu));
            l_run += p;
            pb[r] = (__bf16)p;
          }
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(vb + (db * 32 + col) * LD::VSTRIDE +
                                                                   (kb2 * 32 + st * 16 + 8 * half) * 2);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
          }
        }
      }
    }
    if (kt + 1 < ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- normalise and store this lane's query row
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_i <= i_hi) {
    const float inv = 1.0f / l_tot;
    uint16_t* dst = a.out + (((int64_t)b * a.chunk + my_i) * g.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * half;
        const uint32_t w0 = pack_bf16x2(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2*>(dst + d0) = make_uint2(w0, w1);
      }
  }
}

int heads_per_group(int G) {
  for (int c : {4, 2, 1})
    if (G % c == 0) return c;
  return 1;
}

template <int D>
hipError_t launch_t(const Geom& g, const Seqs& q, const PrefillArgs& a, int64_t blocks, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Lds<D>::TOTAL);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(prefill_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), Lds<D>::TOTAL, s, g, q, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const Geom& g, const Seqs& q, const uint16_t* qin, const uint16_t* kin,
                          const uint16_t* vin, int32_t chunk, int32_t max_n, uint16_t* out, hipStream_t s) {
  if (max_n <= 0) return hipSuccess;
  PrefillArgs a;
  a.q = qin;
  a.k = kin;
  a.v = vin;
  a.out = out;
  a.chunk = chunk;
  a.gh = heads_per_group(g.G);
  a.tq = kWaves * kRowsWave / a.gh;
  a.n_hc = g.G / a.gh;
  a.tiles_max = (max_n + a.tq - 1) / a.tq;
  a.items_r = a.tiles_max * g.B * g.nR * a.n_hc;
  const int64_t blocks = (int64_t)a.items_r + (int64_t)a.tiles_max * g.B * g.nS * a.n_hc;
  if (blocks <= 0) return hipSuccess;
  return g.D == 128 ? launch_t<128>(g, q, a, blocks, s) : launch_t<64>(g, q, a, blocks, s);
}

}  // namespace duo
