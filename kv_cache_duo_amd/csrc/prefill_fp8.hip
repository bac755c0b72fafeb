// Retrieval heads' pre-filling on fp8 matrix cores, over an fp8 retrieval
// cache (duo_kv_format DUO_KV_FP8).
//
// DuoAttention (abstract, as reproduced on the pith.science review page):
// retrieval heads run full causal attention in pre-filling too; the pages
// tie the method's longest contexts to quantization.  Here the K and V rows
// of a retrieval head are e4m3 codes with one power-of-two scale per tensor,
// and the chunk's own rows were stored before this kernel, so every key and
// value comes from the cache as e4m3.  Per query row at position p, over keys
// 0..p: O = softmax(scale * q k^T) v, with
//   * q rounded to e4m3 after multiplying by scale * log2 e and by a power
//     of two 2^-eq per query row (its largest magnitude lands in [224, 448));
//     eq and the K scale go back in through the matrix instruction's E8M0
//     scale operands, so S^T = K Q^T comes out in base-2 units;
//   * the softmax weights rounded to e4m3 as 2^(s - mu + 7) (at most
//     2^(7 + 1.75) < 448 with the reference mu moved whenever a tile max
//     exceeds it by more than 1.75; weights down to 2^-16 stay representable);
//   * O^T += V^T P^T with the V scale as the instruction's A scale, and the
//     weights' sum l from the same rounded weights through one more (16x16x128)
//     matrix instruction whose A operand selects each query's weights, so
//     that the output is exactly a convex combination of V rows (and the
//     vector ALUs are spared 31 adds per tile).
// v_mfma_scale_f32_32x32x64_f8f6f4: 32x32 outputs per 64-deep contraction,
// the C layout of the bf16 32x32 instructions; per 64-key tile a wave issues
// 4 (D = 128) QK and 4 PV instructions instead of 16 + 16 bf16 ones.
// Three waves per SIMD (at most 168 VGPRs at D = 128): the MFMA C operand
// that carries 7 - mu and the row-sum selector are built right before use,
// so that neither stays live across the tile loop.  A third wave hides more
// of each wave's dependency stalls (MFMA results, LDS reads, the end-of-tile
// barrier) than the software pipelining within a wave that was tried.
//
// Tiles (64 keys, D bytes per row) go global -> LDS directly (16 bytes per
// lane), double-buffered in four distinct LDS objects.  Operand reads:
//   * K (A of S^T): two 16-byte reads per instruction, 32 consecutive bytes
//     of one key row; granules XOR-swizzled by row so 16 lanes hit 16 bank
//     groups;
//   * V^T (A of O^T): ds_read_b64_tr_b8, which inside each 16-lane group
//     gives out lane i, byte j the byte i mod 8 of the 8 bytes addressed by
//     lane 2j + i/8 (pinned with a probe); each lane names 8 bytes of one key
//     row so that lane (d, half) receives V[key][d] for the 32 keys of the P
//     operand in the order the S^T accumulator hands them over (keys
//     32*(j/16) + 8*((j%16)/4) + 4*half + j%4 for byte j), a permutation of
//     the contracted axis shared by both operands.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_util.h"
#include "duo_internal.h"

namespace duo {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBN = 64;           // keys per tile
constexpr int kXcds = 8;
constexpr float kPOffset = 7.f;   // weights are 2^(s - mu + 7)
constexpr float kSlack = 1.75f;   // move mu when a tile max exceeds it by more

struct Fp8Args {
  const uint16_t* q;  // [rows][Hq][D] bf16
  uint16_t* out;      // [rows][Hq][D] bf16
  int32_t tiles_max, gh, tq, n_hc;
  int32_t xcd_plan;  // 1: the snake deal of units to XCDs (sequences of different lengths)
};

// 16-byte granule swizzles (by row) of the K and V tiles in LDS.
template <int D>
__device__ __forceinline__ int k_swz(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
template <int D>
__device__ __forceinline__ int v_swz(int r) { return D == 128 ? (2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1)) : 2 * ((r >> 3) & 1); }

__device__ __forceinline__ void g2l16(const void* src, char* lds) {
  typedef __attribute__((address_space(3))) void lds_void_t;
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds, 16, 0, 0);
}
__device__ __forceinline__ i32x2_t lds_read_tr8(const char* lds) {
  typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)lds);
}
// e4m3 codes of 4 values known to lie within +-448 (both halves of the word
// are written, so its old contents are left unspecified).
__device__ __forceinline__ uint32_t pack4_in_range(float a, float b, float c, float d) {
  const uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_nondeterministic_value(0u), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D>
__global__ __launch_bounds__(kThreads, 3) void prefill_fp8_kernel(Geom g, Seqs sq, Fp8Args a) {
  constexpr int TILE = kBN * D;           // bytes of a K or V tile
  __shared__ __attribute__((aligned(16))) char lds_k0[TILE];
  __shared__ __attribute__((aligned(16))) char lds_v0[TILE];
  __shared__ __attribute__((aligned(16))) char lds_k1[TILE];
  __shared__ __attribute__((aligned(16))) char lds_v1[TILE];
  constexpr int CH = D / 16;              // 16-byte granules per row
  constexpr int RPC = 64 / CH;            // rows per 1 KB wave load
  constexpr int ROWS_J = RPC * kWaves;    // tile rows between a lane's loads
  constexpr int NJ = kBN / ROWS_J;        // wave loads per tile and operand
  constexpr int KS = D / 64;              // 64-deep contraction steps of Q K^T
  constexpr int DB = D / 32;              // 32-wide column blocks of O
  static_assert(NJ >= 1 && KS >= 1, "tile shape");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;

  // ---- work item: retrieval units of the sequences with new tokens
  // (longest stored prefix first), longest query tiles first.  When every
  // unit does the same work and the units split evenly over the XCDs
  // (blockIdx mod 8), each unit stays on one XCD and each XCD runs its units
  // one after another; with sequences of different lengths the snake deal of
  // units to XCDs when it balances, else t-major, unit-minor over all XCDs
  const int id = blockIdx.x;
  const int per_t = sq.nact * g.nR * a.n_hc;
  int t, rest;
  if (sq.uniform && per_t % kXcds == 0) {
    const int x = id % kXcds, k = id / kXcds;
    t = a.tiles_max - 1 - k % a.tiles_max;
    rest = x + kXcds * (k / a.tiles_max);
  } else if (a.xcd_plan) {
    if (!snake_deal_item(sq, id, per_t, g.nR * a.n_hc, a.tq, t, rest)) return;
  } else {
    t = a.tiles_max - 1 - id / per_t;
    rest = id % per_t;
  }
  const int hc = rest % a.n_hc;
  rest /= a.n_hc;
  const int idx = rest % g.nR;
  const int b = active_seq(sq, rest / g.nR);
  const int n = sq.n[b];
  if (t * a.tq >= n) return;
  const int L = sq.len[b];
  const int kvh = kv_head_of_unit(g, idx);
  const int i_lo = t * a.tq;
  const int i_hi = min(i_lo + a.tq, n) - 1;
  const int qmax = L + i_hi;
  const int waves_per_head = kWaves / a.gh;
  const int gg = wave / waves_per_head;
  const int wi0 = i_lo + (wave % waves_per_head) * 32;
  const int h = kvh * g.G + hc * a.gh + gg;
  const int blo = L + wi0;
  const int bhi = L + min(wi0 + 32, n) - 1;
  const int my_i = wi0 + col;
  const int my_q = L + my_i;
  const int ntiles = qmax / kBN + 1;

  // ---- Q operand (B of S^T = K Q^T): query `col`, dims 64c + 32 half + 0..31
  // (rotated to the query's position first with rotary embedding)
  i32x8_t qreg[KS];
  int eq = 0;
  {
    const bool ok = my_i <= i_hi;
    const uint4* src = reinterpret_cast<const uint4*>(a.q + (((int64_t)sq.off[b] + (ok ? my_i : i_lo)) * g.Hq + h) * D);
    float x[KS][4][8];  // x[c][u]: dims 64c + 32 half + 8u + 0..7, the row's 8-dim chunk 8c + 4 half + u
#pragma unroll
    for (int c = 0; c < KS; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 t = src[(64 * c + 32 * half) / 8 + u];
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[c][u][2 * e] = bf16_lo(w[e]);
          x[c][u][2 * e + 1] = bf16_hi(w[e]);
        }
      }
    if (g.rope) {
      float cs[8], sn[8];
      if (!g.rope_half) {  // pairs (2i, 2i + 1) inside a chunk
#pragma unroll
        for (int c = 0; c < KS; ++c)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            rope_angles8<D>(my_q, 8 * c + 4 * half + u, false, g.rope_rho, cs, sn);
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const float p0 = x[c][u][e], p1 = x[c][u][e + 1];
              x[c][u][e] = fmaf(p0, cs[e], -p1 * sn[e]);
              x[c][u][e + 1] = fmaf(p0, sn[e], p1 * cs[e]);
            }
          }
      } else if constexpr (KS >= 2) {  // pairs (d, d + D/2): c = 0 with c = 1 (D = 128), same lane
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          rope_angles8<D>(my_q, 4 * half + u, true, g.rope_rho, cs, sn);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p0 = x[0][u][e], p1 = x[1][u][e];
            x[0][u][e] = fmaf(p0, cs[e], -p1 * sn[e]);
            x[1][u][e] = fmaf(p0, sn[e], p1 * cs[e]);
          }
        }
      } else {  // D = 64: pairs (d, d + 32) join the two halves, lanes l and l ^ 32
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          rope_angles8<D>(my_q, 4 * half + u, true, g.rope_rho, cs, sn);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float mine = x[0][u][e], other = __shfl_xor(mine, 32);
            x[0][u][e] = half == 0 ? fmaf(mine, cs[e], -other * sn[e]) : fmaf(other, sn[e], mine * cs[e]);
          }
        }
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < KS; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[c][u][e]));
    amax = fmaxf(amax, __shfl_xor(amax, 32)) * g.scale_log2;  // the whole row (both halves)
    if (amax > 0.f) frexpf(amax * (1.0f / 448.0f), &eq);      // amax 2^-eq in [224, 448)
    eq = min(max(eq, -126), 127);                              // an E8M0 scale byte (255 is NaN)
    const float s = ok ? ldexpf(g.scale_log2, -eq) : 0.f;
#pragma unroll
    for (int c = 0; c < KS; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* y = x[c][u];
        qreg[c][2 * u] = (int)fp8_pack4(y[0] * s, y[1] * s, y[2] * s, y[3] * s);
        qreg[c][2 * u + 1] = (int)fp8_pack4(y[4] * s, y[5] * s, y[6] * s, y[7] * s);
      }
  }
  const int scale_q = 127 + eq;                // E8M0: 2^eq back onto the query column
  const int scale_k = 127 + g.fp8_exp_k;       // K tensor scale
  const int scale_v = 127 + g.fp8_exp_v;       // V tensor scale

  // ---- tile loader: a lane's byte offsets inside a tile are fixed; the
  // tile's base address is uniform (scalar registers)
  const int r0 = wave * RPC + lane / CH;
  const int pch = lane % CH;
  const uint32_t koff = (uint32_t)(r0 * D + (pch ^ k_swz<D>(r0)) * 16);  // rows r0 + j ROWS_J swizzle like r0
  const uint32_t voff = (uint32_t)(r0 * D + (pch ^ v_swz<D>(r0)) * 16);
  auto load_tile = [&](int tile, char* kbuf, char* vbuf) __attribute__((always_inline)) {
    const int k0 = tile * kBN;
    const int64_t row0 = retrieval_row0_uniform(g, b, idx, k0) + k0;  // row of position k0
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(g.rk) + row0 * D;
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(g.rv) + row0 * D;
    if (k0 + kBN - 1 <= qmax) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        g2l16(kb + j * ROWS_J * D + koff, kbuf + (j * kWaves + wave) * 1024);
        g2l16(vb + j * ROWS_J * D + voff, vbuf + (j * kWaves + wave) * 1024);
      }
    } else {  // last tile: rows past qmax read the last granule of row qmax instead
      const uint32_t lim = (uint32_t)(qmax - k0 + 1) * D - 16;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        g2l16(kb + min(koff + j * ROWS_J * D, lim), kbuf + (j * kWaves + wave) * 1024);
        g2l16(vb + min(voff + j * ROWS_J * D, lim), vbuf + (j * kWaves + wave) * 1024);
      }
    }
  };

  // ---- LDS operand addresses (bytes inside a tile)
  auto k_addr = [&](int kb2, int c, int u) __attribute__((always_inline)) {
    return (kb2 * 32 + col) * D + (((4 * c + 2 * half + u) ^ k_swz<D>(col)) * 16);
  };
  const int grp = lane >> 4, gi = lane & 15;  // 16-lane group, lane in group
  auto v_addr = [&](int db, int tt) __attribute__((always_inline)) {
    const int jj = gi >> 1;  // byte j' of the read that this lane names
    const int key = 32 * (tt >> 1) + 16 * (tt & 1) + 8 * (jj >> 2) + 4 * (grp >> 1) + (jj & 3);
    const int gd = 2 * db + (grp & 1);
    return key * D + ((gd ^ v_swz<D>(key)) * 16) + 8 * (gi & 1);
  };

  // ---- softmax state, O^T
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  // Row sums through v_mfma_scale_f32_16x16x128_f8f6f4 with the weights as
  // its B operand: lane l holds column l % 16 and contraction group l / 16,
  // so groups 0 and 2 carry query l % 16 (both halves of the keys) and
  // groups 1 and 3 query l % 16 + 16.  A row 0 of ones over groups 0, 2 and
  // a row 1 of ones over groups 1, 3 give the two queries' sums in
  // registers 0 and 1 of lanes 0..15.
  f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};
  const int sel_row = lane & 15, sel_grp = (lane >> 4) & 1;
  const int one_w = (sel_row == sel_grp && sel_row < 2) ? 0x38383838 : 0;  // e4m3 1.0

  float m_run = -INFINITY, mu = 0.f, thr = -INFINITY;
  float negm_s = kPOffset;

  auto compute_tile = [&](int kt, auto cur_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    char* const kcur = cur ? lds_k1 : lds_k0;
    char* const vcur = cur ? lds_v1 : lds_v0;
    char* const knext = cur ? lds_k0 : lds_k1;
    char* const vnext = cur ? lds_v0 : lds_v1;
    const int k0 = kt * kBN;
    if (kt + 1 < ntiles) load_tile(kt + 1, knext, vnext);
    const bool live = bhi >= blo && k0 <= bhi;
    if (live) {
      f32x16_t sacc[2];
      f32x16_t negm;
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[r] = negm_s;
#pragma unroll
      for (int c = 0; c < KS; ++c)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(kcur + k_addr(kb2, c, 0));
          const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(kcur + k_addr(kb2, c, 1));
          const i32x8_t ka = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          sacc[kb2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qreg[c], c == 0 ? negm : sacc[kb2], 0, 0, 0,
                                                                      scale_k, 0, scale_q);
        }
      if (k0 + kBN - 1 > blo) {  // causal mask on the diagonal tiles
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kp = k0 + kb2 * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            sacc[kb2][r] = kp <= my_q ? sacc[kb2][r] : -INFINITY;
          }
      }
      float mt = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[kb2][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32)) - kPOffset;  // tile max relative to mu
      if (__any(mt > thr)) {
        const float m_new = fmaxf(m_run, mu + mt);
        const float mu_new = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - mu_new);
        const float delta = mu_new - mu;
        m_run = m_new;
        mu = mu_new;
        thr = m_new == -INFINITY ? -INFINITY : kSlack;
        {  // lane c < 16 holds the sums of queries c (register 0) and c + 16 (register 1)
          const float alpha_hi = __shfl(alpha, (lane & 15) + 16);
          lacc[0] *= alpha;
          lacc[1] *= alpha_hi;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb2][r] -= delta;
        negm_s = kPOffset - mu;
      }
      // weights 2^(s - mu + 7) as the B operand of O^T += V^T P^T: byte
      // j = 16 kb2 + r holds register r of block kb2
      i32x8_t pb;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const float p0 = exp2_fast(sacc[kb2][4 * w4]), p1 = exp2_fast(sacc[kb2][4 * w4 + 1]);
          const float p2 = exp2_fast(sacc[kb2][4 * w4 + 2]), p3 = exp2_fast(sacc[kb2][4 * w4 + 3]);
          pb[4 * kb2 + w4] = (int)pack4_in_range(p0, p1, p2, p3);
        }
      {
        const i32x8_t ones = {one_w, one_w, one_w, one_w, one_w, one_w, one_w, one_w};
        lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pb, lacc, 0, 0, 0, 127, 0, 127);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        i32x8_t va;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const i32x2_t r2 = lds_read_tr8(vcur + v_addr(db, tt));
          va[2 * tt] = r2.x;
          va[2 * tt + 1] = r2.y;
        }
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, oacc[db], 0, 0, 0, scale_v, 0, 127);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next tile's direct-to-LDS loads
    __syncthreads();
  };

  load_tile(0, lds_k0, lds_v0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; kt += 2) {
    compute_tile(kt, std::integral_constant<int, 0>());
    if (kt + 1 < ntiles) compute_tile(kt + 1, std::integral_constant<int, 1>());
  }

  // ---- normalise and store this lane's query row
  // query col's sum: register (col >= 16) of lane col % 16
  const float l_a = __shfl(lacc[0], col & 15), l_b = __shfl(lacc[1], col & 15);
  const float l_tot = col < 16 ? l_a : l_b;
  if (my_i <= i_hi) {
    const float inv = 1.0f / l_tot;
    uint16_t* dst = a.out + (((int64_t)sq.off[b] + my_i) * g.Hq + h) * D;
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

int heads_per_group_fp8(int G) {
  for (int c : {4, 2, 1})
    if (G % c == 0) return c;
  return 1;
}

}  // namespace

hipError_t launch_prefill_fp8(const Geom& g, const Seqs& q, const uint16_t* qin, int32_t max_n, uint16_t* out,
                              hipStream_t s) {
  if (max_n <= 0 || g.nR == 0) return hipSuccess;
  Fp8Args a;
  a.q = qin;
  a.out = out;
  a.gh = heads_per_group_fp8(g.G);
  a.n_hc = g.G / a.gh;
  a.tq = kWaves * 32 / a.gh;
  a.tiles_max = (max_n + a.tq - 1) / a.tq;
  int64_t blocks = (int64_t)a.tiles_max * q.nact * g.nR * a.n_hc;
  a.xcd_plan = 0;
  if (!(q.uniform && (q.nact * g.nR * a.n_hc) % kXcds == 0)) {
    const int64_t items = snake_deal_items(q, g.nR * a.n_hc, a.tq);
    if (items > 0) {
      a.xcd_plan = 1;
      blocks = items;
    }
  }
  if (blocks <= 0) return hipSuccess;
  if (g.D == 128)
    hipLaunchKernelGGL(prefill_fp8_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, s, g, q, a);
  else
    hipLaunchKernelGGL(prefill_fp8_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, s, g, q, a);
  return hipGetLastError();
}

}  // namespace duo
