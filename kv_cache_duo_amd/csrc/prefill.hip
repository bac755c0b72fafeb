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
//   * work-group = 4 waves; each wave owns QB blocks of 32 query rows of one
//     query head; the work-group covers gh query heads of one KV group, so
//     every K/V tile staged in LDS serves all of them;
//   * K/V tiles of 64 keys are gathered row by row (any mix of cache rows,
//     ring slots and chunk rows) with 16-byte loads into registers while the
//     previous tile is computed, then stored to a double-buffered LDS: K as
//     rows (padded to 272 B), V transposed (rows of 144 B) so that both MFMA
//     operands are 16-byte LDS reads.  The V tile is loaded with the row
//     group varying fastest across lanes, which makes the transposed stores
//     bank-conflict free;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q
//     held in registers): each lane holds 32 scores of ONE query, so row max
//     and sum need in-lane work plus one exchange with lane^32.  Each K
//     fragment read from LDS feeds QB MFMAs;
//   * P (bf16) feeds O^T += V^T P^T straight from the S^T registers: the key
//     order inside a 16-key MFMA step is permuted identically in P and in the
//     transposed V tile, which is legal because keys are the contracted axis;
//   * the running max is only moved (and O, l rescaled) when a tile's max
//     exceeds it by more than 2^8; the result is exact because l and O always
//     share the same reference;
//   * l sums the bf16 P that the MFMA consumes (v_dot2 with ones);
//   * work-groups run longest query tile first, t-major and unit-minor.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "device_util.h"
#include "duo_internal.h"

namespace duo {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBN = 64;             // keys per tile
constexpr float kRescaleSlack = 8.f;  // log2 units: rescale when the max grows by > 2^8

struct PrefillArgs {
  const uint16_t* q;  // [B][chunk][Hq][D]
  const uint16_t* k;  // [B][chunk][Hkv][D]
  const uint16_t* v;
  uint16_t* out;      // [B][chunk][Hq][D]
  int32_t chunk;
  int32_t tiles_max;  // query tiles per sequence, max over sequences
  int32_t gh;         // query heads per work-group (1, 2 or 4)
  int32_t tq;         // tokens per query tile
  int32_t n_hc;       // G / gh
  int32_t items_r;    // work-groups of retrieval heads
};

template <int D>
struct Lds {
  static constexpr int KSTRIDE = D * 2;             // bytes per K row (XOR-swizzled chunks)
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

// Dynamic LDS of the prefill kernel (two K/V tile buffers).
extern __shared__ __attribute__((aligned(16))) char prefill_smem[];

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes bytes [lds_off + 16 l, lds_off + 16 l + 16); lds_off is wave-uniform.
// (Kept out of the kernel template: the host pass must not see the builtin
// in a template body, or the kernel's host stub is not emitted.)
__device__ __forceinline__ void global_to_lds16(const void* src, int lds_off) {
  __builtin_amdgcn_global_load_lds(src, prefill_smem + lds_off, 16, 0, 0);
}

__device__ __forceinline__ uint4 select4(bool ok, const uint4& x) {
  return make_uint4(ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u);
}

template <int D, int QB>
__global__ __launch_bounds__(kThreads, QB == 1 ? 2 : 1)
void prefill_kernel(Geom g, Seqs sq, PrefillArgs a) {
  using LD = Lds<D>;
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int RPT = kBN * CH / kThreads;  // tile rows loaded per thread (4 or 2)
  constexpr int RG = kBN / RPT;             // row groups per tile
  constexpr int QC = D / 16;                // MFMA k-steps of Q K^T
  constexpr int DB = D / 32;                // 32-wide column blocks of O
  constexpr int ROWS_WAVE = 32 * QB;
  char* const smem = prefill_smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int col = lane & 31;   // query row of a 32-row block held by this lane
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
  const int64_t in_base = ((int64_t)b * a.chunk * g.Hkv + kvh) * D;  // chunk row 0
  const int64_t in_stride = (int64_t)g.Hkv * D;

  // query positions of the work-group and of this wave's blocks
  const int i_lo = t * a.tq;                          // first chunk row
  const int i_hi = min(i_lo + a.tq, n) - 1;           // last chunk row
  const int qmin = L + i_lo, qmax = L + i_hi;
  const int waves_per_head = kWaves / a.gh;
  const int gg = wave / waves_per_head;
  const int wi0 = i_lo + (wave % waves_per_head) * ROWS_WAVE;  // wave's first chunk row
  const int h = kvh * g.G + hc * a.gh + gg;
  int blo[QB], bhi[QB], my_i[QB], my_q[QB];  // block position range (wave-uniform), lane row
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    blo[qb] = L + wi0 + 32 * qb;
    bhi[qb] = L + min(wi0 + 32 * qb + 32, n) - 1;  // < blo: block has no rows
    my_i[qb] = wi0 + 32 * qb + col;
    my_q[qb] = L + my_i[qb];
  }

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
  bf16x8_t qreg[QB][QC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bool ok = my_i[qb] <= i_hi;
    const uint4* src = reinterpret_cast<const uint4*>(a.q + (((int64_t)b * a.chunk + (ok ? my_i[qb] : i_lo)) * g.Hq + h) * D);
#pragma unroll
    for (int c = 0; c < QC; ++c) qreg[qb][c] = __builtin_bit_cast(bf16x8_t, select4(ok, src[2 * c + half]));
  }

  // ---- tile loader.
  // K goes straight from global memory to LDS (global_load_lds_dwordx4): each
  // wave instruction fills 1 KB of the tile, lane l the 16-byte chunk l of
  // it.  Chunk c of row r is stored at chunk c ^ (r mod CH) of the row, which
  // keeps the MFMA operand reads (32 rows, same chunk) bank-conflict free.
  // Rows that no query of this work-group may use load an arbitrary valid
  // row: their scores are always masked.
  // V goes through registers, is zeroed where unusable, and is stored
  // transposed; it is loaded with the row group varying fastest across
  // lanes, which makes the transposed stores bank-conflict free.
  const int rgV = threadIdx.x % RG, chV = threadIdx.x / RG;
  uint4 vbuf[RPT];
  bool vok[RPT];
  auto ring_slot = [&](int kp) {  // valid for kp >= S
    return g.S + (kp - g.S) % g.W;
  };
  // Element offset of position kp's row and whether this work-group may use it.
  auto row_src = [&](int kp, int slot, int64_t& off, bool& from_cache) -> bool {
    const bool in_chunk = kp >= L;
    const bool ok = kp <= qmax && (in_chunk || retrieval || kp < g.S || kp >= L - g.W);
    const int64_t cache_row = (retrieval || kp < g.S) ? (int64_t)kp : (int64_t)slot;
    off = in_chunk ? in_base + (int64_t)(kp - L) * in_stride : cache_row * D;
    from_cache = !in_chunk && ok;
    if (!ok) off = in_base;  // chunk row 0 of this head: always readable
    return ok;
  };
  // Per-lane element offsets of this lane's rows inside a tile, for a tile
  // that lies wholly in the chunk input (row stride Hkv*D) or wholly in the
  // retrieval cache (row stride D); such tiles need one uniform base each.
  // K: the lane's j-th direct load covers row r0k + j*KROWS_J with the same
  // swizzled chunk for every j; V: rows rgV*RPT + i.
  constexpr int KROWS_J = kWaves * 64 / CH;  // tile rows between a lane's K loads
  const int r0k = (wave * 64 + lane) / CH;
  const int lck = ((wave * 64 + lane) % CH) ^ (r0k & (CH - 1));
  const int koff_in = r0k * (int)in_stride + lck * 8, koff_c = r0k * D + lck * 8;
  const int voff_in = rgV * RPT * (int)in_stride + chV * 8, voff_c = rgV * RPT * D + chV * 8;
  auto load_tile = [&](int tile, int buf) {
    const int k0 = tile * kBN;
    const bool all_in = k0 >= L && k0 + kBN - 1 <= qmax;           // every row in the chunk
    const bool all_cache = retrieval && k0 + kBN - 1 < L;          // every row cached
    if (all_in || all_cache) {
      const int64_t stride = all_in ? in_stride : D;
      const uint16_t* kbase = (all_in ? a.k + in_base + (int64_t)(k0 - L) * in_stride : ck + (int64_t)k0 * D) +
                              (all_in ? koff_in : koff_c);
      const uint16_t* vbase = (all_in ? a.v + in_base + (int64_t)(k0 - L) * in_stride : cv + (int64_t)k0 * D) +
                              (all_in ? voff_in : voff_c);
#pragma unroll
      for (int j = 0; j < RPT; ++j)
        global_to_lds16(kbase + j * KROWS_J * stride, buf * LD::BUF + (j * kWaves + wave) * 1024);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        vok[i] = true;
        vbuf[i] = *reinterpret_cast<const uint4*>(vbase + i * stride);
      }
      return;
    }
    // general tile: any mix of cache rows, ring slots, chunk rows, unusable rows
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int p = (j * kWaves + wave) * 64 + lane;  // 16-byte chunk index in the tile
      const int r = p / CH;
      const int lc = (p % CH) ^ (r & (CH - 1));
      const int kp = k0 + r;
      int64_t off;
      bool from_cache;
      row_src(kp, retrieval || kp < g.S ? 0 : ring_slot(kp), off, from_cache);
      const uint16_t* src = (from_cache ? ck : a.k) + off + lc * 8;
      global_to_lds16(src, buf * LD::BUF + (j * kWaves + wave) * 1024);
    }
    const int kp0 = k0 + rgV * RPT;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int kp = kp0 + i;
      int64_t off;
      bool from_cache;
      vok[i] = row_src(kp, retrieval || kp < g.S ? 0 : ring_slot(kp), off, from_cache);
      vbuf[i] = reinterpret_cast<const uint4*>((from_cache ? cv : a.v) + off)[chV];  // zeroed at the store
    }
  };
  auto store_tile = [&](int buf) {
    char* vb = smem + buf * LD::BUF + LD::KBYTES;
#pragma unroll
    for (int i = 0; i < RPT; ++i) vbuf[i] = select4(vok[i], vbuf[i]);
    const int pos = vt_pos(rgV * RPT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      char* dst = vb + (chV * 8 + e) * LD::VSTRIDE + pos * 2;
      const uint32_t lo = __builtin_amdgcn_perm(word_of(vbuf[1], e >> 1), word_of(vbuf[0], e >> 1), sel);
      if constexpr (RPT == 4) {
        const uint32_t hi = __builtin_amdgcn_perm(word_of(vbuf[3], e >> 1), word_of(vbuf[2], e >> 1), sel);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<uint32_t*>(dst) = lo;
      }
    }
  };

  // ---- softmax state per block: this lane's query (m, partial l), O^T
  f32x16_t oacc[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
  }
  const float c2 = g.scale_log2;
  const uint32_t ones = 0x3f803f80u;  // bf16 pair (1, 1)

  load_tile(tile_of(0), 0);
  store_tile(0);
  __builtin_amdgcn_s_waitcnt(0);  // the direct-to-LDS loads of K
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    const int tile = tile_of(kt);
    const int k0 = tile * kBN;
    if (kt + 1 < ntiles) load_tile(tile_of(kt + 1), cur ^ 1);

    // wave-uniform: can any block of this wave see a key of this tile?
    bool any_live = false, need_mask = !retrieval;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      bool live = bhi[qb] >= blo[qb] && k0 <= bhi[qb];
      if (!retrieval && k0 >= g.S && k0 + kBN - 1 < blo[qb] - g.W + 1) live = false;
      any_live = any_live || live;
      need_mask = need_mask || k0 + kBN - 1 > blo[qb];
    }
    if (any_live) {
      const char* kb = smem + cur * LD::BUF;
      const char* vb = kb + LD::KBYTES;
      f32x16_t sacc[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[qb][kb2][r] = 0.f;
#pragma unroll
      for (int c = 0; c < QC; ++c) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const int kr = kb2 * 32 + col;
          const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kb + kr * LD::KSTRIDE + (((2 * c + half) ^ (kr & (CH - 1))) * 16));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sacc[qb][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][c], sacc[qb][kb2], 0, 0, 0);
        }
      }
      // masks: causal on the diagonal, band for streaming heads (branch-free)
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int lo_win = retrieval ? -1 : max(my_q[qb] - g.W, g.S - 1);  // keep kp > lo_win ...
          const int sink_end = retrieval ? 0 : g.S;                        // ... or kp < sink_end
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kp = k0 + kb2 * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
              const bool ok = (kp <= my_q[qb]) & ((kp > lo_win) | (kp < sink_end));
              sacc[qb][kb2][r] = ok ? sacc[qb][kb2][r] : -INFINITY;
            }
        }
      }
      float mu[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mt = fmaxf(sacc[qb][0][0], sacc[qb][1][0]);
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[qb][kb2][r]);
        mt = fmaxf(mt, __shfl_xor(mt, 32)) * c2;
        // move the reference only when some query's max grew by > 2^8
        if (__any(mt > m_run[qb] + kRescaleSlack)) {
          const float m_new = fmaxf(m_run[qb], mt);
          const float alpha = exp2_fast(m_run[qb] - (m_new == -INFINITY ? 0.f : m_new));
          m_run[qb] = m_new;
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
        }
        mu[qb] = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
      }
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          bf16x8_t pb[QB];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            uint32_t w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float p0 = exp2_fast(fmaf(sacc[qb][kb2][st * 8 + 2 * r], c2, -mu[qb]));
              const float p1 = exp2_fast(fmaf(sacc[qb][kb2][st * 8 + 2 * r + 1], c2, -mu[qb]));
              w[r] = pack_bf16x2(p0, p1);
              l_run[qb] = dot2_bf16(w[r], ones, l_run[qb]);
            }
            pb[qb] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
          }
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(vb + (db * 32 + col) * LD::VSTRIDE +
                                                                   (kb2 * 32 + st * 16 + 8 * half) * 2);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qb], oacc[qb][db], 0, 0, 0);
          }
        }
    }
    if (kt + 1 < ntiles) store_tile(cur ^ 1);
    __builtin_amdgcn_s_waitcnt(0);  // the direct-to-LDS loads of K
    __syncthreads();
  }

  // ---- normalise and store this lane's query rows
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    if (my_i[qb] <= i_hi) {
      const float inv = 1.0f / l_tot;
      uint16_t* dst = a.out + (((int64_t)b * a.chunk + my_i[qb]) * g.Hq + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = db * 32 + 8 * r4 + 4 * half;
          const uint32_t w0 = pack_bf16x2(oacc[qb][db][4 * r4] * inv, oacc[qb][db][4 * r4 + 1] * inv);
          const uint32_t w1 = pack_bf16x2(oacc[qb][db][4 * r4 + 2] * inv, oacc[qb][db][4 * r4 + 3] * inv);
          *reinterpret_cast<uint2*>(dst + d0) = make_uint2(w0, w1);
        }
    }
  }
}

int heads_per_group(int G) {
  for (int c : {4, 2, 1})
    if (G % c == 0) return c;
  return 1;
}

template <int D, int QB>
hipError_t launch_t(const Geom& g, const Seqs& q, PrefillArgs a, int32_t max_n, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, QB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Lds<D>::TOTAL);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  a.tq = kWaves * 32 * QB / a.gh;
  a.tiles_max = (max_n + a.tq - 1) / a.tq;
  a.items_r = a.tiles_max * g.B * g.nR * a.n_hc;
  const int64_t blocks = (int64_t)a.items_r + (int64_t)a.tiles_max * g.B * g.nS * a.n_hc;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<D, QB>), dim3((unsigned)blocks), dim3(kThreads), Lds<D>::TOTAL, s, g, q, a);
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
  a.n_hc = g.G / a.gh;
  static const int qb_env = [] {
    const char* e = getenv("DUO_PREFILL_QB");
    return e ? atoi(e) : 1;
  }();
  if (g.D == 128) return qb_env == 1 ? launch_t<128, 1>(g, q, a, max_n, s) : launch_t<128, 2>(g, q, a, max_n, s);
  return qb_env == 1 ? launch_t<64, 1>(g, q, a, max_n, s) : launch_t<64, 2>(g, q, a, max_n, s);
}

}  // namespace duo
