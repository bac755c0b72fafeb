// Mixed retrieval/streaming pre-filling on bf16 MFMA (gfx950).
//
// DuoAttention (abstract, as reproduced on the pith.science review page)
// speeds up pre-filling as well as decoding: retrieval heads run full causal
// attention over every earlier position, streaming heads only over the
// attention sinks and the recent window.  Per query at position p:
//   retrieval: keys 0..p;   streaming: keys j <= p with j < sink or j > p-recent.
// Earlier positions come from the cache (retrieval rows, or the sink / ring
// slots of streaming heads), positions of this chunk from the inputs, so a
// sequence may be prefilled in chunks.  The streaming heads' rows of the
// chunk are appended after this kernel (ring slots read here may be
// overwritten by it); the retrieval rows of a bf16 or fp8 cache, and of any
// cache with rotary embedding, are stored before it, and the retrieval tiles
// then read every row from the cache (contiguous rows of one head).
//
// Tile engine (flash-style online softmax, fp32 accumulation):
//   * work-group = 4 waves; each wave owns 32 query rows of one query head;
//     the work-group covers gh query heads of one KV group, so every K/V tile
//     staged in LDS serves all of them;
//   * K and V tiles of 64 keys go from global memory straight into a
//     double-buffered LDS (global_load_lds_dwordx4, 1 KB per wave
//     instruction) while the previous tile is computed; rows may be any mix
//     of cache rows, ring slots and chunk rows.  Both tiles keep the natural
//     [key][d] layout with the 16-byte granules of a row XOR-swizzled so that
//     the operand reads below are free of bank conflicts;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q
//     in registers, pre-multiplied by scale * log2 e): each lane holds 32
//     scores of ONE query, so row max and sum need in-lane work plus one
//     exchange with lane^32.  The accumulator starts at minus the running
//     max, so the MFMA output is already the exponent of the softmax term;
//   * P (bf16) feeds O^T += V^T P^T straight from the S^T registers.  The
//     V^T operand comes from ds_read_b64_tr_b16, which transposes 4x4 blocks
//     of 16-bit elements across each 16-lane group; the key order of P inside
//     a 16-key MFMA step (groups of 4 keys interleaved by lane half) is
//     reproduced by the read addresses, legal because keys are the
//     contracted axis;
//   * the running max is only moved (and O, l rescaled) when a tile's max
//     exceeds it by more than 2^8; the result is exact because l and O always
//     share the same reference;
//   * l sums the bf16 P that the MFMA consumes (v_dot2 with ones);
//   * work-groups run longest query tile first; on each XCD one unit (head
//     group of one sequence) at a time where the work allows it (see the
//     work-item mapping), so the resident work-groups share its K/V in L2;
//   * the wave priority is raised over the matrix-core blocks and lowered
//     for the softmax.
// With rotary position embedding (RoFormer, cited in the pith.science review
// page's reference list) q is turned to its position in the prologue; the
// chunk's retrieval rows are stored (rotated) before this kernel, so every
// retrieval key comes from the cache; the streaming heads' chunk K rows come
// turned from the call's staging workspace, or are staged through registers
// and turned in the tiles that hold them.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_util.h"
#include "duo_internal.h"

namespace duo {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X, each with its own L2
constexpr int kBN = 64;               // keys per tile
constexpr float kRescaleSlack = 8.f;  // log2 units: rescale when the max grows by > 2^8

struct PrefillArgs {
  const uint16_t* q;  // [rows][Hq][D]: sequence b's new rows from Seqs::off[b]
  const uint16_t* k;  // [rows][Hkv][D]
  const uint16_t* v;
  uint16_t* out;      // [rows][Hq][D]
  int32_t tiles_max;  // query tiles per sequence, max over sequences
  int32_t gh;         // query heads per work-group (1, 2 or 4)
  int32_t tq;         // tokens per query tile
  int32_t n_hc;       // G / gh
  int32_t items_r;    // work-groups of retrieval heads
  int32_t xcd_plan;   // 1: retrieval units dealt to the XCDs in snake order (sequences of different lengths)
  // rotary embedding with the staging workspace: the chunk's K rows of every
  // streaming head, turned once per call, [B][nS][rot_n][D] (null: turned
  // in every tile that holds them)
  const uint16_t* rot_k;
  int32_t rot_n;
};

// LDS has 64 banks of 4 bytes; a wave's 16-byte reads are served 16 lanes
// at a time, 8-byte reads 32 lanes at a time.  Granule swizzles (granule =
// 16 bytes of a row) that keep the operand reads below conflict-free:
//   K row r: granule g stored at g ^ k_swizzle(r)  (the 16 rows one read
//     serves fall on 16 distinct 16-byte bank groups);
//   V row r: granule g stored at g ^ v_swizzle(r)  (the 4 rows x 4 granules
//     of a transposing read's 32 lanes do likewise).
template <int D>
__device__ __forceinline__ int k_swizzle(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_swizzle(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

template <int D>
struct Lds {
  static constexpr int ROW = D * 2;       // bytes per K or V row
  static constexpr int TILE = kBN * ROW;  // one K or V tile
};

// The helpers below wrap target builtins that take LDS pointers; they stay
// out of the kernel template, whose host-side stub is otherwise not emitted.

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes bytes [lds + 16 l, lds + 16 l + 16); lds is wave-uniform.
__device__ __forceinline__ void global_to_lds16(const void* src, char* lds) {
  typedef __attribute__((address_space(3))) void lds_void_t;
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds, 16, 0, 0);
}

// ds_read_b64_tr_b16: every lane names 8 bytes (four 16-bit elements) of
// LDS; inside each group of 16 lanes, lane i receives as element j the
// element (i mod 4) of the 8 bytes named by lane 4 j + i / 4 of its group.
__device__ __forceinline__ uint2 lds_read_tr16(const char* lds) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)lds);
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ uint32_t scaled_pair(uint32_t w, float s) {
  return pack_bf16x2(bf16_lo(w) * s, bf16_hi(w) * s);
}

// Q8: the retrieval cache holds int8 rows (DUO_KV_INT8) and some sequence
// has a stored prefix; tiles with stored retrieval rows are then staged
// through registers and dequantized into the bf16 LDS layout.
// ROPE: rotary position embedding; q is turned in the prologue.  ROPE 1:
// every turned key comes from memory (retrieval rows from the cache, which
// holds them turned; the streaming heads' chunk rows from the call's turned
// copy, PrefillArgs::rot_k), so tiles load straight into LDS as without
// rotation.  ROPE 2: the streaming heads' chunk rows are turned in each tile
// that holds them (staged through registers), and with Q8 as well (an int8
// cache with rotary embedding, prefix or not) every retrieval tile is
// staged: stored rows dequantized, the chunk's rows turned to their
// positions.
// ROPE 3: no rotation, and every retrieval key and value row comes from the
// cache, the call's own rows too (they were stored first): a bf16 cache, and
// the exact fp8 prefill over rows staged as bf16 in the caller's workspace.
// F8: the retrieval cache holds e4m3 rows (DUO_KV_FP8, exact prefill); the
// call's own rows are stored first, so every retrieval tile is staged from
// the cache: codes through registers, decoded at unit scale -- exactly, an
// e4m3 value has 4 significant bits -- into the bf16 LDS layout.  The K
// scale joins q's pre-multiplication and the V scale the final
// normalisation; both are powers of two, so the result is the bf16 tile
// engine's over the stored values, bit for bit.
template <int D, bool Q8, int ROPE, bool F8 = false>
__global__ __launch_bounds__(kThreads, 2)
void prefill_kernel(Geom g, Seqs sq, PrefillArgs a) {
  // The K and V tiles of the two pipeline stages are four distinct LDS
  // objects: the compiler then knows that the next tile's direct-to-LDS
  // loads cannot alias the transposing reads of the current one, and does
  // not wait for those loads before the P V products.
  __shared__ __attribute__((aligned(16))) char lds_k0[Lds<D>::TILE];
  __shared__ __attribute__((aligned(16))) char lds_v0[Lds<D>::TILE];
  __shared__ __attribute__((aligned(16))) char lds_k1[Lds<D>::TILE];
  __shared__ __attribute__((aligned(16))) char lds_v1[Lds<D>::TILE];
  // ROPE: cos (first D) and sin (next D) of the turn of the ROWS_J positions
  // between the rows a lane stages, per dim
  __shared__ __attribute__((aligned(16))) float lds_step[ROPE == 2 ? 2 * D : 4];
  using LD = Lds<D>;
  constexpr int CH = D / 8;                 // 16-byte granules per row
  constexpr int RPC = 64 / CH;              // rows per 1 KB wave load (4 or 8)
  constexpr int ROWS_J = RPC * kWaves;      // tile rows between a lane's loads
  constexpr int NJ = kBN / ROWS_J;          // wave loads per tile and operand (4 or 2)
  constexpr int QC = D / 16;                // MFMA k-steps of Q K^T
  constexpr int DB = D / 32;                // 32-wide column blocks of O

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int col = lane & 31;   // query row of the 32-row block held by this lane
  const int half = lane >> 5;  // which 8-wide k slice / 4-row group

  // ---- work item: longest query tiles first, over the sequences that have
  // new tokens (longest stored prefix first).  Work-groups go to the 8 XCDs
  // round-robin (blockIdx mod 8).  When every unit (sequence, KV head, head
  // chunk) does the same work and the units of a kind split evenly over the
  // XCDs, every unit stays on one XCD, and each XCD runs its units one after
  // another, a unit's query tiles longest first: the XCD's resident
  // work-groups then belong to one unit, start nearly together and take
  // nearly the same time, so they stream the same K/V tiles nearly together
  // and share them in the XCD's L2.  Otherwise (sequences of different
  // lengths: pinned units would load some XCDs far more than others)
  // t-major, unit-minor, which spreads every unit over all XCDs.
  int id = blockIdx.x;
  const bool retrieval = id < a.items_r;
  if (!retrieval) id -= a.items_r;
  const int nkind = retrieval ? g.nR : g.nS;
  const int per_t = sq.nact * nkind * a.n_hc;
  int t, rest;
  if (sq.uniform && per_t % kXcds == 0 && (retrieval || a.items_r % kXcds == 0)) {
    const int x = id % kXcds, k = id / kXcds;
    t = a.tiles_max - 1 - k % a.tiles_max;
    rest = x + kXcds * (k / a.tiles_max);
  } else if (retrieval && a.xcd_plan) {
    // sequences of different lengths: the snake deal of the retrieval units
    if (!snake_deal_item(sq, id, per_t, nkind * a.n_hc, a.tq, t, rest)) return;
  } else {
    t = a.tiles_max - 1 - id / per_t;
    rest = id % per_t;
  }
  const int hc = rest % a.n_hc;
  rest /= a.n_hc;
  const int idx = rest % nkind;
  const int b = active_seq(sq, rest / nkind);
  const int n = sq.n[b];
  if (t * a.tq >= n) return;
  const int L = sq.len[b];
  const int kvh = kv_head_of_unit(g, retrieval ? idx : g.nR + idx);
  const int64_t unit_rows = retrieval ? g.max_len : (int64_t)g.slots;
  const int64_t cache_off = ((int64_t)b * nkind + idx) * unit_rows * D;
  const uint16_t* ck = (retrieval ? g.rk : g.sk) + cache_off;
  const uint16_t* cv = (retrieval ? g.rv : g.sv) + cache_off;
  const int64_t in_base = ((int64_t)sq.off[b] * g.Hkv + kvh) * D;  // chunk row 0
  const int in_stride = g.Hkv * D;

  // query positions of the work-group and of this wave's block
  const int i_lo = t * a.tq;                 // first chunk row
  const int i_hi = min(i_lo + a.tq, n) - 1;  // last chunk row
  const int qmin = L + i_lo, qmax = L + i_hi;
  const int waves_per_head = kWaves / a.gh;
  const int gg = wave / waves_per_head;
  const int wi0 = i_lo + (wave % waves_per_head) * 32;  // wave's first chunk row
  const int h = kvh * g.G + hc * a.gh + gg;
  const int blo = L + wi0;                   // block position range (wave-uniform)
  const int bhi = L + min(wi0 + 32, n) - 1;  // < blo: the block has no rows
  const int my_i = wi0 + col;
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
  auto tile_of = [&](int k) __attribute__((always_inline)) { return k < tA ? k : tB0 + (k - tA); };

  // ---- Q operand (B of S^T = K Q^T), scaled by scale * log2 e: lane holds
  // row `col`, k slice `half`
  const float c2 = (F8 && retrieval) ? g.scale_log2 * g.fp8_scale_k : g.scale_log2;
  bf16x8_t qreg[QC];
  {
    const bool ok = my_i <= i_hi;
    const uint4* src = reinterpret_cast<const uint4*>(a.q + (((int64_t)sq.off[b] + (ok ? my_i : i_lo)) * g.Hq + h) * D);
    const float s = ok ? c2 : 0.f;
    if constexpr (ROPE == 1 || ROPE == 2) {
      // k-step c holds dims 16c + 8 half + 0..7 (chunk 2c + half of the
      // row): interleaved pairs lie inside it; half-split pairs join k-step c
      // with c + QC/2 (dims d and d + D/2), in this same lane.
      float x[QC][8];
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const uint4 t = src[2 * c + half];
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[c][2 * e] = bf16_lo(w[e]);
          x[c][2 * e + 1] = bf16_hi(w[e]);
        }
      }
      if (!g.rope_half) {
#pragma unroll
        for (int c = 0; c < QC; ++c) {
          float cs[8], sn[8];
          rope_angles8<D>(my_q, 2 * c + half, false, g.rope_rho, cs, sn);
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float u = x[c][e], w = x[c][e + 1];
            x[c][e] = fmaf(u, cs[e], -w * sn[e]);
            x[c][e + 1] = fmaf(u, sn[e], w * cs[e]);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < QC / 2; ++c) {
          float cs[8], sn[8];
          rope_angles8<D>(my_q, 2 * c + half, true, g.rope_rho, cs, sn);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float u = x[c][e], w = x[c + QC / 2][e];
            x[c][e] = fmaf(u, cs[e], -w * sn[e]);
            x[c + QC / 2][e] = fmaf(u, sn[e], w * cs[e]);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < QC; ++c)
        qreg[c] = __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2(x[c][0] * s, x[c][1] * s),
                                                          pack_bf16x2(x[c][2] * s, x[c][3] * s),
                                                          pack_bf16x2(x[c][4] * s, x[c][5] * s),
                                                          pack_bf16x2(x[c][6] * s, x[c][7] * s)));
    } else {
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const uint4 x = src[2 * c + half];
        qreg[c] = __builtin_bit_cast(bf16x8_t, make_uint4(scaled_pair(x.x, s), scaled_pair(x.y, s),
                                                          scaled_pair(x.z, s), scaled_pair(x.w, s)));
      }
    }
  }

  // ---- tile loader.  Wave load j of wave w fills 1 KB chunk j*4+w of the
  // K (or V) tile: tile rows r0 + j*ROWS_J, lane l the physical granule l mod
  // CH of its row, which holds logical granule gK (gV) of that row.  Rows no
  // query of this work-group may use load chunk row 0 of this KV head
  // instead: their scores are always masked, so P is exactly 0 there and the
  // (finite) V row adds nothing.
  const int r0 = wave * RPC + lane / CH;
  const int pch = lane % CH;
  const int gK = pch ^ k_swizzle<D>(r0);  // the swizzles of rows r0 + j*ROWS_J equal r0's
  const int gV = pch ^ v_swizzle<D>(r0);
  auto ring_slot = [&](int kp) __attribute__((always_inline)) {  // valid for kp >= S
    return g.S + (kp - g.S) % g.W;
  };
  // Element offset of position kp's row and whether it comes from the cache.
  auto row_src = [&](int kp, int64_t& off, bool& from_cache) __attribute__((always_inline)) {
    const bool in_chunk = kp >= L;
    const bool ok = kp <= qmax && (in_chunk || retrieval || kp < g.S || kp >= L - g.W);
    const int64_t cache_row = (retrieval || kp < g.S) ? (int64_t)kp : (int64_t)ring_slot(kp);
    off = in_chunk ? in_base + (int64_t)(kp - L) * in_stride : cache_row * D;
    from_cache = !in_chunk && ok;
    if (!ok) off = in_base;  // chunk row 0 of this head: always readable
  };
  const int koff_in = r0 * in_stride + gK * 8, koff_c = r0 * D + gK * 8;
  const int voff_in = r0 * in_stride + gV * 8, voff_c = r0 * D + gV * 8;
  // int8 retrieval rows (Q8): codes of granule g of row r at byte
  // r*D + 8g, row scales apart; a staged tile's 16-byte granules wait in
  // kst / vst (bit j of q8rows: row j holds codes + scale in .x .y .z).
  // (the retrieval pointers are set per tile: a paged cache keeps a tile's
  // 64 rows in one page)
  // ROPE: a staged tile's chunk rows wait in kst / vst as bf16 granules
  // (bit j of rotrows: row j is a chunk row whose K is turned in store_tile).
  // Both: retrieval tiles mix stored int8 rows and chunk rows to be turned.
  // F8: a staged retrieval tile's e4m3 granules wait in kst / vst (.x .y).
  u32x4_t kst[(Q8 || ROPE == 2 || F8) ? NJ : 1], vst[(Q8 || ROPE == 2 || F8) ? NJ : 1];
  uint32_t q8rows = 0, rotrows = 0;
  int st_k0 = 0;  // first key of the staged tile
  auto load_tile = [&](int tile, char* kbuf, char* vbuf) __attribute__((always_inline)) -> bool {  // true: staged, store_tile to follow
    const int k0 = tile * kBN;
    char* dst = kbuf + wave * 1024;   // K tile, this wave's 1 KB chunks
    char* vdst = vbuf + wave * 1024;  // V tile
    // retrieval rows of this tile: row r at (row0 + r) * D of the pool
    const uint16_t* ckr = ck;
    const uint16_t* cvr = cv;
    int64_t row0 = 0;
    if (retrieval) {
      row0 = retrieval_row0_uniform(g, b, idx, k0);
      ckr = g.rk + row0 * D;
      cvr = g.rv + row0 * D;
    }
    if constexpr (F8) {
      if (retrieval) {
        // every row up to qmax is stored; rows past it read row k0 (<= qmax,
        // the same page), whose scores are masked
        const uint8_t* ck8 = reinterpret_cast<const uint8_t*>(g.rk) + row0 * D;
        const uint8_t* cv8 = reinterpret_cast<const uint8_t*>(g.rv) + row0 * D;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int kp = k0 + r0 + j * ROWS_J;
          const int64_t row = kp <= qmax ? (int64_t)kp : (int64_t)k0;
          const u32x2_t kc = *reinterpret_cast<const u32x2_t*>(ck8 + row * D + gK * 8);
          const u32x2_t vc = *reinterpret_cast<const u32x2_t*>(cv8 + row * D + gV * 8);
          kst[j] = u32x4_t{kc.x, kc.y, 0u, 0u};
          vst[j] = u32x4_t{vc.x, vc.y, 0u, 0u};
        }
        return true;
      }
    }
    if constexpr (Q8 && ROPE == 2) {
      if (retrieval) {
        // stored rows (kp < L) as int8 codes + scale, the chunk's rows from
        // the input (turned in store_tile), rows past qmax chunk row 0
        const uint8_t* ck8 = reinterpret_cast<const uint8_t*>(g.rk) + row0 * D;
        const uint8_t* cv8 = reinterpret_cast<const uint8_t*>(g.rv) + row0 * D;
        st_k0 = k0;
        q8rows = 0;
        rotrows = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int kp = k0 + r0 + j * ROWS_J;
          if (kp < L) {
            const u32x2_t kc = *reinterpret_cast<const u32x2_t*>(ck8 + (int64_t)kp * D + gK * 8);
            const u32x2_t vc = *reinterpret_cast<const u32x2_t*>(cv8 + (int64_t)kp * D + gV * 8);
            kst[j] = u32x4_t{kc.x, kc.y, __float_as_uint(g.rks[row0 + kp]), 0u};
            vst[j] = u32x4_t{vc.x, vc.y, __float_as_uint(g.rvs[row0 + kp]), 0u};
            q8rows |= 1u << j;
          } else {
            const bool in = kp <= qmax;
            const int64_t off = in ? in_base + (int64_t)(kp - L) * in_stride : in_base;
            kst[j] = *reinterpret_cast<const u32x4_t*>(a.k + off + gK * 8);
            vst[j] = *reinterpret_cast<const u32x4_t*>(a.v + off + gV * 8);
            if (in) rotrows |= 1u << j;
          }
        }
        return true;
      }
    }
    if constexpr (ROPE != 0 && !Q8) {
      if (retrieval) {
        // every key row is in the cache (this chunk's rows were stored,
        // rotated or as fp8 values, before the kernel); rows past qmax read
        // row k0 instead
        if (k0 + kBN - 1 <= qmax) {
          const uint16_t* kb = ckr + (int64_t)k0 * D + koff_c;
          const uint16_t* vb = cvr + (int64_t)k0 * D + voff_c;
#pragma unroll
          for (int j = 0; j < NJ; ++j) global_to_lds16(kb + j * ROWS_J * D, dst + j * kWaves * 1024);
#pragma unroll
          for (int j = 0; j < NJ; ++j) global_to_lds16(vb + j * ROWS_J * D, vdst + j * kWaves * 1024);
        } else {
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int kp = k0 + r0 + j * ROWS_J;
            const int64_t row = kp <= qmax ? (int64_t)kp : (int64_t)k0;  // k0 <= qmax: same page
            global_to_lds16(ckr + row * D + gK * 8, dst + j * kWaves * 1024);
            global_to_lds16(cvr + row * D + gV * 8, vdst + j * kWaves * 1024);
          }
        }
        return false;
      }
    }
    if constexpr (ROPE == 1) {
      if (k0 + kBN - 1 >= L) {
        // a streaming tile with chunk rows whose K rows were turned once for
        // the call: straight into LDS, K of chunk rows from the turned copy
        // (rows no query may use read the copy's row 0: masked, finite)
        const uint16_t* rot = a.rot_k + ((int64_t)b * g.nS + idx) * a.rot_n * D;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int kp = k0 + r0 + j * ROWS_J;
          const bool in_chunk = kp >= L;
          const bool ok = kp <= qmax && (in_chunk || kp < g.S || kp >= L - g.W);
          const bool from_cache = !in_chunk && ok;
          const int64_t cache_row = kp < g.S ? (int64_t)kp : (int64_t)(g.S + (kp - g.S) % g.W);
          const int64_t ci = (ok && in_chunk) ? (int64_t)(kp - L) : 0;
          const uint16_t* ksrc = from_cache ? ck + cache_row * D : rot + ci * D;
          const uint16_t* vsrc = from_cache ? cv + cache_row * D : a.v + in_base + ci * in_stride;
          global_to_lds16(ksrc + gK * 8, dst + j * kWaves * 1024);
          global_to_lds16(vsrc + gV * 8, vdst + j * kWaves * 1024);
        }
        return false;
      }
    }
    if constexpr (ROPE == 2) {
      if (k0 + kBN - 1 >= L) {  // a streaming tile with chunk rows: stage it
        st_k0 = k0;
        rotrows = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          // row_src for a streaming head, written out (a second call of
          // that lambda makes the compiler copy the kernel arguments to
          // scratch)
          const int kp = k0 + r0 + j * ROWS_J;
          const bool in_chunk = kp >= L;
          const bool ok = kp <= qmax && (in_chunk || kp < g.S || kp >= L - g.W);
          const bool from_cache = !in_chunk && ok;
          const int64_t cache_row = kp < g.S ? (int64_t)kp : (int64_t)(g.S + (kp - g.S) % g.W);
          const int64_t off = !ok ? in_base : in_chunk ? in_base + (int64_t)(kp - L) * in_stride : cache_row * D;
          kst[j] = *reinterpret_cast<const u32x4_t*>((from_cache ? ck : a.k) + off + gK * 8);
          vst[j] = *reinterpret_cast<const u32x4_t*>((from_cache ? cv : a.v) + off + gV * 8);
          if (!from_cache && kp >= L && kp <= qmax) rotrows |= 1u << j;
        }
        return true;
      }
    }
    if constexpr (Q8) {
      if (retrieval && k0 < L) {
        const uint8_t* ck8 = reinterpret_cast<const uint8_t*>(g.rk) + row0 * D;
        const uint8_t* cv8 = reinterpret_cast<const uint8_t*>(g.rv) + row0 * D;
        const float* cks = g.rks + row0;
        const float* cvs = g.rvs + row0;
        q8rows = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          // a retrieval row: stored (kp < L), in the chunk, or past qmax
          // (unusable: chunk row 0 instead, as in row_src)
          const int kp = k0 + r0 + j * ROWS_J;
          const bool from_cache = kp < L;
          const int64_t off = (kp >= L && kp <= qmax) ? in_base + (int64_t)(kp - L) * in_stride : in_base;
          if (from_cache) {  // retrieval cache row kp
            const u32x2_t kc = *reinterpret_cast<const u32x2_t*>(ck8 + (int64_t)kp * D + gK * 8);
            const u32x2_t vc = *reinterpret_cast<const u32x2_t*>(cv8 + (int64_t)kp * D + gV * 8);
            kst[j] = u32x4_t{kc.x, kc.y, __float_as_uint(cks[kp]), 0u};
            vst[j] = u32x4_t{vc.x, vc.y, __float_as_uint(cvs[kp]), 0u};
            q8rows |= 1u << j;
          } else {
            kst[j] = *reinterpret_cast<const u32x4_t*>(a.k + off + gK * 8);
            vst[j] = *reinterpret_cast<const u32x4_t*>(a.v + off + gV * 8);
          }
        }
        return true;
      }
    }
    const bool all_in = k0 >= L && k0 + kBN - 1 <= qmax;   // every row in the chunk
    const bool all_cache = retrieval && k0 + kBN - 1 < L;  // every row cached
    if (all_in || all_cache) {
      const int64_t stride = all_in ? in_stride : D;
      const uint16_t* kb = all_in ? a.k + in_base + (int64_t)(k0 - L) * in_stride + koff_in : ckr + (int64_t)k0 * D + koff_c;
      const uint16_t* vb = all_in ? a.v + in_base + (int64_t)(k0 - L) * in_stride + voff_in : cvr + (int64_t)k0 * D + voff_c;
#pragma unroll
      for (int j = 0; j < NJ; ++j) global_to_lds16(kb + j * ROWS_J * stride, dst + j * kWaves * 1024);
#pragma unroll
      for (int j = 0; j < NJ; ++j) global_to_lds16(vb + j * ROWS_J * stride, vdst + j * kWaves * 1024);
      return false;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int64_t off;
      bool from_cache;
      row_src(k0 + r0 + j * ROWS_J, off, from_cache);
      global_to_lds16((from_cache ? ckr : a.k) + off + gK * 8, dst + j * kWaves * 1024);
      global_to_lds16((from_cache ? cvr : a.v) + off + gV * 8, vdst + j * kWaves * 1024);
    }
    return false;
  };
  // Write a staged tile: int8 granules become code * scale rounded to bf16.
  auto store_tile = [&](char* kbuf, char* vbuf) __attribute__((always_inline)) {
    auto granule = [&](const u32x4_t& x, bool q8) __attribute__((always_inline)) -> u32x4_t {
      if (!q8) return x;
      const uint4 r = int8_dequant8(x.x, x.y, __uint_as_float(x.z));
      return u32x4_t{r.x, r.y, r.z, r.w};
    };
    char* dst = kbuf + wave * 1024 + lane * 16;
    char* vdst = vbuf + wave * 1024 + lane * 16;
    if constexpr (F8) {
      if (retrieval) {  // e4m3 codes -> bf16 at unit scale (exact)
        auto dec = [](const u32x4_t& x) __attribute__((always_inline)) -> u32x4_t {
          return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false)),
                         __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true)),
                         __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false)),
                         __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true))};
        };
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          *reinterpret_cast<u32x4_t*>(dst + j * kWaves * 1024) = dec(kst[j]);
          *reinterpret_cast<u32x4_t*>(vdst + j * kWaves * 1024) = dec(vst[j]);
        }
        return;
      }
    }
    if constexpr (ROPE == 2) {
      // chunk K rows turned to their positions (every lane takes part: the
      // half-split pairs exchange values across lanes)
      // the angles of row r0 from fp64 turns; rows r0 + j ROWS_J by complex
      // multiplication with the angles of ROWS_J positions (NJ - 1 fp32
      // steps, a few 1e-7 on cos and sin, far below the bf16 rounding of K):
      // rope_angles8_key, which every other K rotation uses
      static_assert(ROWS_J == rope_key_step<D>(), "tile row groups and the key angles' steps");
      float cs[8], sn[8], cd[8], sd[8];
      rope_angles8<D>(st_k0 + r0, gK, g.rope_half, g.rope_rho, cs, sn);
      if constexpr (NJ > 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          cd[e] = lds_step[8 * gK + e];
          sd[e] = lds_step[D + 8 * gK + e];
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (j > 0) rope_step8(cs, sn, cd, sd);
        const uint4 x = make_uint4(kst[j].x, kst[j].y, kst[j].z, kst[j].w);
        const uint4 r = rope_apply8<CH>(x, cs, sn, g.rope_half, gK);
        const u32x4_t kr = ((rotrows >> j) & 1u) ? u32x4_t{r.x, r.y, r.z, r.w} : kst[j];
        const bool q8 = Q8 && ((q8rows >> j) & 1u);
        *reinterpret_cast<u32x4_t*>(dst + j * kWaves * 1024) = granule(kr, q8);
        *reinterpret_cast<u32x4_t*>(vdst + j * kWaves * 1024) = granule(vst[j], q8);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bool q8 = (q8rows >> j) & 1u;
      *reinterpret_cast<u32x4_t*>(dst + j * kWaves * 1024) = granule(kst[j], q8);
      *reinterpret_cast<u32x4_t*>(vdst + j * kWaves * 1024) = granule(vst[j], q8);
    }
  };

  // ---- LDS operand addresses (bytes inside a tile)
  // K rows kb2*32 + col, logical granule 2c + half
  auto k_addr = [&](int kb2, int c) __attribute__((always_inline)) { return (kb2 * 32 + col) * LD::ROW + (((2 * c + half) ^ k_swizzle<D>(col)) * 16); };
  // V^T operand of the 16-key step starting at key s16, rows d = db*32 + col:
  // lane l names key s16 + 8 t + 4 half + (l/4 mod 4), columns
  // db*32 + 16 ((l/16) mod 2) + 4 (l mod 4) .. +3, for t = 0, 1.
  const int vq = (lane >> 2) & 3;
  const int vg = 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
  auto v_addr = [&](int s16, int tt, int db) __attribute__((always_inline)) {
    return (s16 + 8 * tt + 4 * half + vq) * LD::ROW + (((4 * db + vg) ^ v_swizzle<D>(vq)) * 16) + 8 * (lane & 1);
  };

  // ---- softmax state: this lane's query (running max, partial l), O^T
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;  // running max (log2 units), -inf before any key
  float mu = 0.f;           // reference subtracted from the scores (m_run, or 0)
  float thr = -INFINITY;    // move the reference when a tile max (relative to mu) exceeds this
  float l_run = 0.f;
  f32x16_t negm;
#pragma unroll
  for (int r = 0; r < 16; ++r) negm[r] = 0.f;
  const uint32_t ones = 0x3f803f80u;  // bf16 pair (1, 1)

  auto compute_tile = [&](int kt, auto cur_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    const int k0 = tile_of(kt) * kBN;
    char* const kcur = cur ? lds_k1 : lds_k0;
    char* const vcur = cur ? lds_v1 : lds_v0;
    char* const knext = cur ? lds_k0 : lds_k1;
    char* const vnext = cur ? lds_v0 : lds_v1;
    const bool staged = kt + 1 < ntiles && load_tile(tile_of(kt + 1), knext, vnext);

    // wave-uniform: can the block see a key of this tile, and does any key
    // need a mask (causal diagonal, or outside the streaming band)
    bool live = bhi >= blo && k0 <= bhi;
    if (!retrieval && k0 >= g.S && k0 + kBN - 1 < blo - g.W + 1) live = false;
    const bool need_mask = k0 + kBN - 1 > blo || (!retrieval && k0 + kBN - 1 >= g.S && k0 < bhi - g.W + 1);
    if (live) {
      f32x16_t sacc[2];
      // wave priority: raised while this wave issues its matrix-core work
      // (S^T, then higher for the P V block) and back to 0 for the softmax,
      // so that the SIMD's other wave takes the vector ALU in between
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c = 0; c < QC; ++c)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kcur + k_addr(kb2, c));
          sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[c], c == 0 ? negm : sacc[kb2], 0, 0, 0);
        }
      __builtin_amdgcn_s_setprio(0);
      // masks: causal on the diagonal, band for streaming heads (branch-free)
      if (need_mask) {
        const int lo_win = retrieval ? -1 : max(my_q - g.W, g.S - 1);  // keep kp > lo_win ...
        const int sink_end = retrieval ? 0 : g.S;                       // ... or kp < sink_end
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kp = k0 + kb2 * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool ok = (kp <= my_q) & ((kp > lo_win) | (kp < sink_end));
            sacc[kb2][r] = ok ? sacc[kb2][r] : -INFINITY;
          }
      }
      float mt = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[kb2][r]);
      {  // max with lane ^ 32 (a VALU swap of the wave's halves, not an LDS round trip)
        const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));  // tile max relative to mu
      }
      if (__any(mt > thr)) {
        const float m_new = fmaxf(m_run, mu + mt);
        const float mu_new = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - mu_new);  // 0 while m_run = -inf
        const float delta = mu_new - mu;
        m_run = m_new;
        mu = mu_new;
        thr = m_new == -INFINITY ? -INFINITY : kRescaleSlack;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb2][r] -= delta;
#pragma unroll
        for (int r = 0; r < 16; ++r) negm[r] = -mu;
      }
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          uint32_t w[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            w[r] = pack_bf16x2(exp2_fast(sacc[kb2][st * 8 + 2 * r]), exp2_fast(sacc[kb2][st * 8 + 2 * r + 1]));
            l_run = dot2_bf16(w[r], ones, l_run);
          }
          const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const uint2 lo = lds_read_tr16(vcur + v_addr(kb2 * 32 + st * 16, 0, db));
            const uint2 hi = lds_read_tr16(vcur + v_addr(kb2 * 32 + st * 16, 1, db));
            const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
          }
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (Q8 || ROPE == 2 || F8) {
      if (staged) store_tile(knext, vnext);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the direct-to-LDS loads of the next tile
    __syncthreads();
  };

  if constexpr (ROPE == 2 && NJ > 1) {  // the turn of ROWS_J positions, per dim: the same for every staged tile
    if (threadIdx.x < D / 8) {
      float cs[8], sn[8];
      rope_angles8<D>(ROWS_J, threadIdx.x, g.rope_half, g.rope_rho, cs, sn);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lds_step[8 * threadIdx.x + e] = cs[e];
        lds_step[D + 8 * threadIdx.x + e] = sn[e];
      }
    }
    __syncthreads();
  }
  if (load_tile(tile_of(0), lds_k0, lds_v0)) store_tile(lds_k0, lds_v0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; kt += 2) {
    compute_tile(kt, std::integral_constant<int, 0>());
    if (kt + 1 < ntiles) compute_tile(kt + 1, std::integral_constant<int, 1>());
  }

  // ---- normalise and store this lane's query row
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_i <= i_hi) {
    float inv = 1.0f / l_tot;
    if (F8 && retrieval) inv *= g.fp8_scale_v;  // a power of two: exact
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

int heads_per_group(int G) {
  for (int c : {4, 2, 1})
    if (G % c == 0) return c;
  return 1;
}

template <int D, bool Q8, int ROPE, bool F8 = false>
hipError_t launch_t(const Geom& g, const Seqs& q, PrefillArgs a, int32_t max_n, hipStream_t s,
                    bool streaming_only = false) {
  a.tq = kWaves * 32 / a.gh;
  a.tiles_max = (max_n + a.tq - 1) / a.tq;
  a.items_r = streaming_only ? 0 : a.tiles_max * q.nact * g.nR * a.n_hc;
  a.xcd_plan = 0;
  const int units_r = q.nact * g.nR * a.n_hc;
  if (!streaming_only && !(q.uniform && units_r % kXcds == 0)) {
    const int64_t items = snake_deal_items(q, g.nR * a.n_hc, a.tq);
    if (items > 0) {
      a.xcd_plan = 1;
      a.items_r = (int32_t)items;
    }
  }
  const int64_t blocks = (int64_t)a.items_r + (int64_t)a.tiles_max * q.nact * g.nS * a.n_hc;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<D, Q8, ROPE, F8>), dim3((unsigned)blocks), dim3(kThreads), 0, s, g, q, a);
  return hipGetLastError();
}

}  // namespace

int64_t snake_deal_items(const Seqs& q, int units_per_seq, int tq) {
  const int units = q.nact * units_per_seq;
  if (units < 2 * kPrefillXcds) return 0;
  int64_t slots[kPrefillXcds] = {}, work[kPrefillXcds] = {};
  for (int j = 0; kPrefillXcds * j < units; ++j)
    for (int x = 0; x < kPrefillXcds; ++x) {
      const int u = snake_unit(j, x);
      if (u >= units) continue;
      const int b = q.act[u / units_per_seq];
      const int64_t tiles = (q.n[b] + tq - 1) / tq;
      slots[x] += tiles;
      work[x] += tiles * (2 * (int64_t)q.len[b] + q.n[b]);
    }
  int64_t max_slots = 0, max_work = 0, sum_work = 0;
  for (int x = 0; x < kPrefillXcds; ++x) {
    max_slots = slots[x] > max_slots ? slots[x] : max_slots;
    max_work = work[x] > max_work ? work[x] : max_work;
    sum_work += work[x];
  }
  return 10 * kPrefillXcds * max_work <= 11 * sum_work ? kPrefillXcds * max_slots : 0;
}

hipError_t launch_prefill(const Geom& g, const Seqs& q, const uint16_t* qin, const uint16_t* kin,
                          const uint16_t* vin, int32_t max_n, uint16_t* out, hipStream_t s) {
  if (max_n <= 0) return hipSuccess;
  PrefillArgs a;
  a.q = qin;
  a.k = kin;
  a.v = vin;
  a.out = out;
  a.gh = heads_per_group(g.G);
  a.n_hc = g.G / a.gh;
  a.rot_k = nullptr;
  a.rot_n = 0;
  // int8 retrieval rows are only read from a stored prefix
  bool prefix = false;
  for (int b = 0; b < g.B; ++b) prefix = prefix || (q.n[b] > 0 && q.len[b] > 0);
  // The staging workspace, per call: first the int8 rows (below), then the
  // streaming heads' turned chunk K rows, each only if the rest has room.
  uint16_t* ws = g.prefill_staging;
  const int64_t ws_bytes = ws != nullptr ? g.prefill_staging_bytes : 0;
  int64_t int8_elems = 0;  // per tensor, when the 8-bit rows are staged
  int64_t int8_rows = 0;
  const bool fp8_exact = g.kv_fp8 && !g.fp8_mfma;
  if (((g.kv_int8 && (prefix || g.rope)) || fp8_exact) && g.nR > 0 && ws != nullptr) {
    for (int i = 0; i < q.nact; ++i) {  // fp8: every row, the call's own stored first
      const int b = q.act[i];
      const int64_t r = (int64_t)q.len[b] + ((g.rope || fp8_exact) ? q.n[b] : 0);
      int8_rows = r > int8_rows ? r : int8_rows;
    }
    const int64_t elems = (int64_t)g.B * g.nR * int8_rows * g.D;
    if (int8_rows > 0 && 4 * elems <= ws_bytes) int8_elems = elems;
  }
  // the int8 kernel that stages its own tiles turns the chunk's rows itself
  const bool q8_tiles = g.kv_int8 && g.nR > 0 && (prefix || g.rope) && int8_elems == 0;
  if (g.rope && g.nS > 0 && ws != nullptr && !q8_tiles) {
    const int64_t rot_elems = (int64_t)g.B * g.nS * max_n * g.D;
    if (2 * (2 * int8_elems + rot_elems) <= ws_bytes) {
      uint16_t* rot = ws + 2 * int8_elems;
      const hipError_t e = launch_turn(g, q, kin, rot, max_n, s);
      if (e != hipSuccess) return e;
      a.rot_k = rot;
      a.rot_n = max_n;
    }
  }
  // rotary mode of the kernels: 1 when every turned key comes from memory
  // (no streaming heads, or their turned copy), 2 when tiles turn them; 3
  // (no rotation): every retrieval row from memory, the call's own among
  // them (a bf16 cache, or fp8 rows staged as bf16)
  const bool stored_bf16 = !g.kv_int8 && !g.kv_fp8;
  const int rope = !g.rope ? ((stored_bf16 || (fp8_exact && int8_elems > 0)) ? 3 : 0)
                           : (g.nS == 0 || a.rot_k != nullptr) ? 1 : 2;
  // launch_t for the cache format's flags and the rotary mode
  auto run = [&](const Geom& gg, auto q8_c, auto f8_c, bool streaming_only = false) -> hipError_t {
    constexpr bool Q8 = decltype(q8_c)::value, F8 = decltype(f8_c)::value;
    if (gg.D == 128) {
      if (rope == 0) return launch_t<128, Q8, 0, F8>(gg, q, a, max_n, s, streaming_only);
      if constexpr (!Q8) {
        if (rope == 1) return launch_t<128, Q8, 1, F8>(gg, q, a, max_n, s, streaming_only);
        if constexpr (!F8) {
          if (rope == 3) return launch_t<128, Q8, 3, F8>(gg, q, a, max_n, s, streaming_only);
        }
      }
      return launch_t<128, Q8, 2, F8>(gg, q, a, max_n, s, streaming_only);
    }
    if (rope == 0) return launch_t<64, Q8, 0, F8>(gg, q, a, max_n, s, streaming_only);
    if constexpr (!Q8) {
      if (rope == 1) return launch_t<64, Q8, 1, F8>(gg, q, a, max_n, s, streaming_only);
      if constexpr (!F8) {
        if (rope == 3) return launch_t<64, Q8, 3, F8>(gg, q, a, max_n, s, streaming_only);
      }
    }
    return launch_t<64, Q8, 2, F8>(gg, q, a, max_n, s, streaming_only);
  };
  using T = std::true_type;
  using F = std::false_type;
  if (fp8_exact && int8_elems == 0)  // stored e4m3 rows decoded exactly in the tiles, bf16 matrix cores
    return run(g, F(), T());
  if (g.kv_fp8 && !fp8_exact) {  // retrieval heads on fp8 matrix cores, streaming heads here
    const hipError_t e = launch_prefill_fp8(g, q, qin, max_n, out, s);
    if (e != hipSuccess) return e;
    return run(g, F(), F(), true);
  }
  if (int8_elems > 0) {
    // Stage the rows the call reads as bf16 in the caller's workspace (once
    // per call, instead of once per work-group and tile), then attend as
    // over a bf16 cache laid out [B][nR][rows][D]; with rotary embedding the
    // int8 chunk's rows are staged turned, as a bf16 cache would hold them
    // (fp8 values are staged times their power-of-two scales, exactly, so
    // the bf16 kernel attends the same values as the fp8 tiles would).
    Geom gs = g;
    gs.kv_int8 = 0;
    gs.kv_fp8 = 0;
    gs.rk = ws;
    gs.rv = ws + int8_elems;
    gs.rks = gs.rvs = nullptr;
    gs.paged = 0;
    gs.nblk = 1;
    gs.max_len = int8_rows;
    const hipError_t e = launch_stage(g, q, kin, vin, gs.rk, gs.rv, int8_rows, g.rope != 0, s);
    if (e != hipSuccess) return e;
    return run(gs, F(), F());
  }
  if (q8_tiles) return run(g, T(), F());  // stored rows as int8 (with rotary embedding: chunk rows turned per tile)
  return run(g, F(), F());
}

}  // namespace duo
