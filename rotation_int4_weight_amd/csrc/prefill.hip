// prefill.hip - many-token rotated W4A16 linear: MFMA GEMM over the rotated
// activations, with each packed weight tile dequantized once into LDS.
//
//   y[m][n] = sum_k x_r[m][k] * w[k][n] + b[n],   w[k][n] = (q[k][n] - z[g][n]) * s[g][n]
//
// ("ParoQuant" wiki, Activation and weight transforms: Y = X_r Q(W_r)^T + b;
// Triton plans and tuning: unpack the 4-bit tile, subtract zero points,
// multiply by group scales, accumulate in fp32.)
//
// A workgroup computes a BM=256 x BN=128 tile of y with 8 waves in two
// roles, one of each per SIMD:
//   * consumer waves 0..3 own rows 64c..64c+63 and all 128 columns (4 x 8
//     MFMA tiles, 32 v_mfma_f32_16x16x32 per 32-deep k step) and issue
//     nothing but their MFMAs, the LDS reads of the next step's B fragments
//     (each issued after the last MFMA that reads its register, with seven
//     column tiles of MFMAs to arrive in) and the loads of A four steps
//     ahead;
//   * producer waves 4..7 load the packed weight words eight steps before
//     they are needed, decode each group's scales and zero points and
//     dequantize each tile one super-step before its first reader, five to
//     eight steps ahead, into a ring of eight LDS tiles.
// On gfx950 a SIMD hides only about one VALU instruction per 16-cycle MFMA
// from the same wave but about two from a second wave, so the split keeps
// the matrix pipe fed while the dequantization runs beside it.  Both roles
// meet at one barrier per super-step of four k steps (128 MFMAs per consumer
// wave between barriers).
//
// Operand layouts are chosen for whole-cache-line loads (the texture/L1 path
// bounds this kernel otherwise):
//   * A comes in the fragment-major tiled layout (launch.hpp): one 16-byte
//     load per lane fetches a complete 16 x 32 MFMA fragment, 1 KB over 8
//     full cache lines.  The buffer descriptor's base moves along k in
//     scalar registers and its record count ends at the last row tile, so
//     tiles past the end read as zeros.
//   * B: a producer thread loads word t&15 of rows 2(t>>4), +1 (a wave's load
//     covers four rows of 64 contiguous bytes) and writes its 8 columns x 2
//     rows into the LDS tile [column][k].  fp16: a byte permute and an OR
//     with 0x6400 make 1024+q exactly, then one packed add of -(1024+z) and
//     one packed multiply by s give (q-z)*s rounded once, two weights per
//     instruction.  bf16 (no packed bf16 arithmetic): the same masks give
//     1024+q or 1024+16q per fp16 half, one v_fma_mix_f32 per weight turns
//     that into the exact fp32 (q-z)*s, and a paired round makes bf16.
//     Columns are 80 bytes apart and within each column the four 8-row
//     blocks of k are XOR-permuted by (column/16)&3, so each fragment read
//     (8 consecutive k) is one aligned 16-byte load.  (SQ_LDS_BANK_CONFLICT
//     reads about five times the cycles of 72-byte columns read as two
//     8-byte halves, with no measurable change in the kernel's time: LDS is
//     not what bounds it.)
#include <stdlib.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"

namespace paro {

// Optional per-wave timeline, compiled in only with PARO_PREFILL_TIMELINE
// (csrc/prefill_timeline.hip): lane 0 of a wave stores the 100 MHz realtime
// counter at fixed points into prefill_timeline_buf[workgroup][wave][48]:
// 0 entry, 1 pipeline primed (consumers: first B fragments read; producers:
// first super-step expanded), 46 producer done; consumer marks of tile it
// (it < 8) at 2 + 4 it: tile start, + 1 main loop done, + 2 MFMAs drained,
// + 3 epilogue stores issued.
#ifdef PARO_PREFILL_TIMELINE
__device__ unsigned long long *prefill_timeline_buf;
#define PREFILL_MARK(i)                                                                                 \
  do {                                                                                                  \
    if ((threadIdx.x & 63) == 0)                                                                        \
      prefill_timeline_buf[((size_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)) * 48 + (i)] =  \
          __builtin_amdgcn_s_memrealtime();                                                             \
  } while (0)
#else
#define PREFILL_MARK(i) \
  do {                  \
  } while (0)
#endif

constexpr int kBM = 256, kBN = 128, kBK = 32;  // kBM: the MoE grouped GEMM's rows per tile
constexpr int kCUs = 256;                       // compute units of an MI355X
constexpr int kWaves = 8, kThreads = 64 * kWaves;  // 4 consumer + 4 producer waves
constexpr int kBStride = kBK + 8;  // halves per LDS column (80 bytes: 16-byte aligned fragment reads)
constexpr int kTiles = 8;           // LDS ring of expanded weight tiles (k steps)
constexpr int kWordRing = 8;        // packed weight words in flight per producer thread (steps)
constexpr int kASlots = 4;          // A fragments in flight per consumer wave (steps)
constexpr int kGroupM = 2;          // M blocks per group of the tile order (dense layers)
static_assert(kTiles == 8 && kWordRing == 8, "the producer's ring slot arithmetic assumes rings of 8");
static_assert(kASlots == 4, "a tile's last super-step loads two A steps of the next tile, the epilogue the other two");

// Physical k-pair index of k-pair rp (k = 2rp, 2rp+1) in column col: the
// four 8-row blocks are XOR-permuted by (col/16)&3.
__device__ __forceinline__ int swz_pair(int col, int rp) { return rp ^ (4 * ((col >> 4) & 3)); }

// Per-group constants of one expansion thread, for the 8 nibble slots of its
// word (slot s = column 8w + awq_col(s)).  fp16: packed pairs -(1024+z) and
// (s, s); bf16: -z*s and s in fp32.
template <int DT>
struct GroupConsts;
template <>
struct GroupConsts<kF16> {
  f16x2 zo[8], sc[8];
  __device__ __forceinline__ void decode(u32x4 sw, uint32_t zw) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = awq_col(s);
      const uint32_t h = (sw[c >> 1] >> (16 * (c & 1))) & 0xffffu;
      const uint32_t z = 0xe400u | ((zw >> (4 * s)) & 0xfu);  // fp16 bits of -(1024 + z)
      sc[s] = __builtin_bit_cast(f16x2, h | (h << 16));
      zo[s] = __builtin_bit_cast(f16x2, z | (z << 16));
    }
  }
};
template <>
struct GroupConsts<kBF16> {
  // Slot s is the low nibble of its byte for even s and the high nibble for
  // odd s; expand_pair_to_lds builds the fp16 numbers 1024 + q and 1024 + 16q
  // from them.  b, c make b * that + c = (q - z) * s exactly in one fma:
  //   even: b = s,      c = -(1024 + z) * s   (11-bit x 11-bit: exact in fp32)
  //   odd:  b = s / 16, c = -(64 + z) * s     (a power-of-two scaling and a
  //                                            7-bit x 11-bit product: exact)
  // and (q - z) * s itself has at most 15 significant bits.
  float b[8], c[8];
  __device__ __forceinline__ void decode(u32x4 sw, uint32_t zw) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int col = awq_col(s);
      const float sc = f16_bits_to_f32((sw[col >> 1] >> (16 * (col & 1))) & 0xffffu);
      const uint32_t z = (zw >> (4 * s)) & 0xfu;
      b[s] = (s & 1) ? sc * 0.0625f : sc;
      c[s] = -(float)(((s & 1) ? 64u : 1024u) + z) * sc;
    }
  }
};

// Nibble masks and the fp16 exponent pattern, held in VGPRs for the whole
// producer: v_and_or_b32 takes no literal operand, and with the constants in
// registers each 1024+q (or 1024+16q) pair costs one instruction.
struct NibbleMasks {
  uint32_t lo, hi, e;
  __device__ __forceinline__ NibbleMasks() : lo(0x000f000fu), hi(0x00f000f0u), e(0x64006400u) {
    asm volatile("" : "+v"(lo), "+v"(hi), "+v"(e));
  }
};

// Dequantize one packed word of rows 2rp (ra) and 2rp+1 (rb) into the LDS
// tile: slot s goes to column 8w + awq_col(s), k-pair rp (swizzled) as one u32.
template <int DT>
__device__ __forceinline__ void expand_pair_to_lds(uint32_t ra, uint32_t rb, const GroupConsts<DT> &gc,
                                                   const NibbleMasks &nm, uint16_t *bl, int w, int rp) {
  uint32_t v[8];
  if constexpr (DT == kF16) {
    // P = [ra.b0, ra.b2, rb.b0, rb.b2], Q = [ra.b1, ra.b3, rb.b1, rb.b3]: after
    // the shifts below, bits 0..3 and 16..19 hold slot s of ra and of rb.
    const uint32_t P = __builtin_amdgcn_perm(ra, rb, 0x02000604u);
    const uint32_t Q = __builtin_amdgcn_perm(ra, rb, 0x03010705u);
    const uint32_t M = nm.lo, E = nm.e;
    const uint32_t e[8] = {(P & M) | E,         ((P >> 4) & M) | E, (Q & M) | E,         ((Q >> 4) & M) | E,
                           ((P >> 8) & M) | E, ((P >> 12) & M) | E, ((Q >> 8) & M) | E, ((Q >> 12) & M) | E};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      f16x2 h = __builtin_bit_cast(f16x2, e[s]) + gc.zo[s];  // q - z, exact
      h = h * gc.sc[s];                                      // one rounding
      v[s] = __builtin_bit_cast(uint32_t, h);
    }
  } else {
    // Same byte gathers as fp16: P's halves hold bytes 0 and 2 of ra (low
    // half) and of rb (high half), Q's bytes 1 and 3.  A low nibble masked in
    // and OR-ed with 0x6400 is the fp16 number 1024 + q, a high nibble
    // 1024 + 16q; v_fma_mix_f32 takes each half as an fp16 operand, so one
    // instruction per weight gives the exact fp32 (q - z) * s.
    const uint32_t P = __builtin_amdgcn_perm(ra, rb, 0x02000604u);
    const uint32_t Q = __builtin_amdgcn_perm(ra, rb, 0x03010705u);
    const uint32_t P8 = P >> 8, Q8 = Q >> 8;
    const uint32_t L = nm.lo, H = nm.hi, E = nm.e;
    const uint32_t e[8] = {(P & L) | E,  (P & H) | E,  (Q & L) | E,  (Q & H) | E,
                           (P8 & L) | E, (P8 & H) | E, (Q8 & L) | E, (Q8 & H) | E};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const f16x2 h = __builtin_bit_cast(f16x2, e[s]);
      const f32x2 d = {__builtin_fmaf((float)h[0], gc.b[s], gc.c[s]), __builtin_fmaf((float)h[1], gc.b[s], gc.c[s])};
      v[s] = __builtin_bit_cast(uint32_t, __builtin_convertvector(d, bf16x2));  // one paired RNE
    }
  }
  const int prp = swz_pair(8 * w, rp);  // the word's 8 columns share one 16-column block
#pragma unroll
  for (int s = 0; s < 8; ++s)
    *reinterpret_cast<uint32_t *>(bl + (8 * w + awq_col(s)) * kBStride + 2 * prp) = v[s];
}

// MOE: experts stacked in the weight tensors (qweight [E][I][O/8], qzeros
// [E][I/G][O/8], scales [E][I/G][O], bias [E][O]) share one rotation; the
// rows of expert e are [offsets[e], offsets[e+1]) of the rotated activations
// (rotated once for all experts).  An output tile is a 256-row block of one
// expert's rows, starting at the 16-row tile that holds the expert's first
// row: rows of neighbouring experts in its tiles are computed and dropped.
// Offsets are clamped into [0, tokens] and made nondecreasing, so no offsets
// can take a workgroup outside its buffers.
// RT: 16-row tiles per consumer wave, so the workgroup tile is BM = 64 RT
// rows: 4 (256 rows) by default, 2 (128 rows) for dense layers whose
// 256-row grid would leave CUs idle (each weight tile then serves half as
// many MFMAs, and twice as many workgroups fill the chip).
//
// Dense layers and the MoE run persistent workgroups: workgroup b takes the
// output tiles b, b + G, b + 2G, ... (G workgroups, at most one per CU) in
// turn.  Steps are numbered across its tiles, so the weight ring simply
// continues: while the consumers finish a tile (its epilogue), the producers
// already expand the first steps of the next one, and the consumers' A loads
// for it are in flight, instead of every tile starting from an empty
// pipeline.
template <int DT, int GK, bool MOE, int RT>
__global__ void __launch_bounds__(kThreads)
prefill_gemm_kernel(LinearArgs a, LayerTable lt) {
  static_assert(RT == 4 || (RT == 2 && !MOE), "256-row tiles, or 128-row tiles for dense layers");
  constexpr int BM = 64 * RT;
  __shared__ __attribute__((aligned(16))) uint16_t bl[kTiles][kBN * kBStride];
  // Every argument the kernel reads, named in one empty asm at the top, so
  // that their scalar loads go out together instead of in two dependent
  // round trips.
  asm volatile("" ::"s"(a.I), "s"(a.O), "s"(a.tokens), "s"(a.group), "s"(a.experts), "s"(a.expert_offsets),
               "s"(a.qweight), "s"(a.qzeros), "s"(a.scales), "s"(a.bias), "s"(a.y), "s"(a.y_dt), "s"(lt.n),
               "s"(lt.xt[0]), "s"(lt.y[0]), "s"(gridDim.x));
  const int lane = lane_id(), wave = wave_id();
  // the layer table is read where a tile is entered, from the argument
  // segment (a scalar load at the entry's offset), not held in registers
  const LayerTable *ltp = &lt;
  PREFILL_MARK(0);
  // dense layers of a table may differ in out_features (each tile carries
  // its layer's); a MoE launch has one
  const int64_t I = a.I, M = a.tokens;
  const int moe_n_tiles = (int)((a.O + kBN - 1) / kBN);
  // MoE: the experts' 256-row work items, counted from the offsets (each
  // expert's rows, clamped into [0, M] and made nondecreasing, start at the
  // 16-row tile that holds its first row)
  auto moe_items = [&]() -> int {
    int64_t cum = 0, prev = a.expert_offsets[0];
    prev = prev < 0 ? 0 : (prev > M ? M : prev);
    for (int k = 0; k < a.experts; ++k) {
      int64_t o1 = a.expert_offsets[k + 1];
      o1 = o1 < prev ? prev : (o1 > M ? M : o1);
      cum += o1 > prev ? (o1 - (prev & ~(int64_t)15) + kBM - 1) / kBM : 0;
      prev = o1;
    }
    return (int)cum;
  };
  const int m_tiles = MOE ? moe_items() : (int)((M + BM - 1) / BM);
  // dense: the layers of the table one after another in the tile order
  // (layer l's tiles start at tile0[l] = m_tiles times the column tiles of
  // the layers before it)
  const int total = MOE ? moe_n_tiles * m_tiles : ltp->tile0[lt.n];
  // tiles of this workgroup: b, b + G, ... (MoE: the grid is sized on the
  // host for the most work items the offsets can give, so a workgroup may
  // have none)
  const int my_tiles = (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  if (my_tiles <= 0) return;  // the whole workgroup leaves before any barrier
  // GK k-steps per quantization group (G = 32 * GK); I is a multiple of 128
  // (GK = 0: one quantization group over the whole row)
  const int nsteps = (int)(I / kBK), ngroups = GK ? (int)(I / (kBK * GK)) : 1;
  const int wg_steps = my_tiles * nsteps;

  // The output tile of this workgroup's iteration it (uniform values; the
  // tile indices go through readfirstlane so that everything derived from
  // them stays in scalar registers).
  struct Tile {
    int64_t n0, mb, row_lo, row_hi;
    int64_t O, W;  // the layer's out_features and packed words per row
    const uint16_t *xt;  // the layer's tiled activations (read at every k step)
    const int32_t *qweight, *qzeros;
    const uint16_t *scales, *bias;
    int layer;  // entry of the layer table (MoE: 0)
  };
  auto tile_of = [&](int it, Tile &t) -> bool {
    t.row_lo = 0;
    t.row_hi = M;
    // XCD-local order: consecutive logical tiles (the N tiles of one M block)
    // share an XCD and its L2.  Workgroup b's iteration it stands for launch
    // id b + it G, which lies on b's XCD when G is a multiple of 8.
    int lwg = xcd_local_order((int)blockIdx.x + it * (int)gridDim.x, total);
    int n_tiles = moe_n_tiles;
    if constexpr (MOE) {
      t.layer = 0;
      t.O = a.O;
      t.xt = lt.xt[0];
      t.qweight = a.qweight;
      t.qzeros = a.qzeros;
      t.scales = a.scales;
      t.bias = a.bias;
    } else {
      int l = 0;
      for (int k = 1; k < lt.n; ++k)
        if (lwg >= ltp->tile0[k]) l = k;
      t.layer = __builtin_amdgcn_readfirstlane(l);
      lwg -= ltp->tile0[t.layer];
      t.O = ltp->o[t.layer];
      t.xt = t.layer == 0 ? lt.xt[0] : ltp->xt[t.layer];
      n_tiles = (int)((t.O + kBN - 1) / kBN);
      if (t.layer == 0) {  // entry 0 is also in a (the single-layer launch)
        t.qweight = a.qweight;
        t.qzeros = a.qzeros;
        t.scales = a.scales;
        t.bias = a.bias;
      } else {
        t.qweight = ltp->qweight[t.layer];
        t.qzeros = ltp->qzeros[t.layer];
        t.scales = ltp->scales[t.layer];
        t.bias = ltp->bias[t.layer];
      }
    }
    t.W = t.O / 8;
    // Dense layers: logical tiles go in groups of kGroupM M blocks, the M
    // block fastest, so an XCD's share of consecutive tiles spans kGroupM
    // blocks of rows and 1/kGroupM as many weight columns as a row-major
    // order would.
    int tn = lwg % n_tiles, tm = lwg / n_tiles;
    if constexpr (!MOE) {
      const int first = (lwg / (kGroupM * n_tiles)) * kGroupM;
      const int gsz = m_tiles - first < kGroupM ? m_tiles - first : kGroupM;
      const int r = lwg % (kGroupM * n_tiles);
      tm = first + r % gsz;
      tn = r / gsz;
    }
    t.n0 = (int64_t)__builtin_amdgcn_readfirstlane(tn) * kBN;
    if constexpr (MOE) {
      // work item (expert, 256-row tile) number lwg / n_tiles, experts in order
      const int64_t wi = __builtin_amdgcn_readfirstlane(lwg / n_tiles);
      int64_t cum = 0, prev = a.expert_offsets[0];
      prev = prev < 0 ? 0 : (prev > M ? M : prev);
      int e = -1;
      int64_t lo = 0, hi = 0, j = 0;
      for (int k = 0; k < a.experts; ++k) {
        int64_t o1 = a.expert_offsets[k + 1];
        o1 = o1 < prev ? prev : (o1 > M ? M : o1);
        const int64_t c = o1 > prev ? (o1 - (prev & ~(int64_t)15) + kBM - 1) / kBM : 0;
        if (wi < cum + c) {
          e = k;
          lo = prev;
          hi = o1;
          j = wi - cum;
          break;
        }
        cum += c;
        prev = o1;
      }
      if (e < 0) {  // (not reached: every tile below total has its expert)
        t.mb = t.row_lo = t.row_hi = 0;
        return false;
      }
      t.mb = (lo & ~(int64_t)15) + j * kBM;
      t.row_lo = lo > t.mb ? lo : t.mb;
      t.row_hi = hi < t.mb + kBM ? hi : t.mb + kBM;
      const int64_t G = (int64_t)kBK * GK, O = a.O, W = O / 8;
      t.qweight += (int64_t)e * I * W;
      t.qzeros += (int64_t)e * (I / G) * W;
      t.scales += (int64_t)e * (I / G) * O;
      if (t.bias) t.bias += (int64_t)e * O;
    } else {
      t.mb = (int64_t)__builtin_amdgcn_readfirstlane(tm) * BM;
    }
    return true;
  };
  const uint32_t tile_bytes = (uint32_t)nsteps * 1024u;  // one row tile over all of k

  Tile t0;
  tile_of(0, t0);  // (every tile below total exists)
  auto tile_at = [&](int it, Tile &t) {
    if (it == 0)
      t = t0;
    else
      tile_of(it, t);
  };
  // A position in the workgroup's sequence of (tile, k step) or (tile,
  // group) pairs.  Every load stream below takes its positions in order, one
  // at a time, so each keeps its own cursor and looks a tile up only when
  // it enters one: no division in the loops.  Past the end a cursor stays
  // on the last position (in-bounds loads whose values are never used).
  struct Cursor {
    int it, pos;
    Tile t;
  };
  auto advance = [&](Cursor &c, int len) {
    if (c.pos + 1 < len) {
      ++c.pos;
    } else if (c.it + 1 < my_tiles) {
      ++c.it;
      c.pos = 0;
      tile_at(c.it, c.t);
    }
  };

  if (wave >= 4) {
    // ------------------------------ producer ------------------------------
    const int tp = threadIdx.x - 256;
    const int dw = tp & 15, drp = tp >> 4;  // word dw of the tile's 16, rows 2drp, 2drp+1 of a step
    // this thread's packed word of a tile's column block (tail tile: any
    // in-bounds word)
    auto word_of = [&](const Tile &t) -> uint32_t {
      const int64_t dword = t.n0 / 8 + dw;
      return (uint32_t)(dword < t.W ? dword : t.W - 1);
    };

    struct Words {
      uint32_t ra, rb;
    };
    // packed words of the next step of the sequence (steps in order).  The
    // thread's byte offset within a step's rows depends on the tile alone
    // (its column block and its layer's width), so it is formed where the
    // cursor enters a tile rather than at every step.
    Cursor cw{0, 0, t0};
    auto w_lane_of = [&](const Tile &t) { return (uint32_t)((2 * drp) * t.W + word_of(t)) * 4u; };
    uint32_t w_lane = w_lane_of(t0);
    auto load_words = [&](Words &wd) {
      const int64_t W = cw.t.W;
      const __amdgpu_buffer_rsrc_t r = raw_rsrc(cw.t.qweight + (int64_t)cw.pos * kBK * W, (uint32_t)(kBK * W * 4));
      wd.ra = __builtin_amdgcn_raw_buffer_load_b32(r, w_lane, 0, 0);
      wd.rb = __builtin_amdgcn_raw_buffer_load_b32(r, w_lane + (uint32_t)(W * 4), 0, 0);
      const int it0 = cw.it;
      advance(cw, nsteps);
      if (cw.it != it0) w_lane = w_lane_of(cw.t);
    };
    struct GroupRaw {
      u32x4 sw;
      uint32_t zw;
    };
    // scales and zeros of the next group of the sequence (groups in order)
    Cursor cg{0, 0, t0};
    uint32_t g_word = word_of(t0);
    auto load_group = [&](GroupRaw &gr) {
      const int64_t O = cg.t.O, W = cg.t.W;
      const __amdgpu_buffer_rsrc_t rs = raw_rsrc(cg.t.scales + (int64_t)cg.pos * O, (uint32_t)(O * 2));
      gr.sw = __builtin_amdgcn_raw_buffer_load_b128(rs, g_word * 16u, 0, 0);
      const __amdgpu_buffer_rsrc_t rz = raw_rsrc(cg.t.qzeros + (int64_t)cg.pos * W, (uint32_t)(W * 4));
      gr.zw = __builtin_amdgcn_raw_buffer_load_b32(rz, g_word * 4u, 0, 0);
      const int it0 = cg.it;
      advance(cg, ngroups);
      if (cg.it != it0) g_word = word_of(cg.t);
    };

    // Scales and zeros: a ring of NSLOT groups.  Group q sits in slot
    // q % NSLOT; it is decoded just before the first k-step of the group is
    // expanded, and the slot is refilled at once with group q + NSLOT.  Every
    // slot index below is a compile-time constant: the step's value mod 8 is
    // (nsteps is a multiple of 4 and of GK, so a group never straddles two
    // tiles).  One group over the whole row (GK = 0): decoded at the first
    // step of each tile, the next tile's loaded meanwhile.
    constexpr int NSLOT = GK == 0 ? 1 : GK == 1 ? 4 : 2;
    GroupConsts<DT> gc;
    const NibbleMasks nm;
    GroupRaw graw[NSLOT];
    Words wd[kWordRing];
#pragma unroll
    for (int q = 0; q < NSLOT; ++q) load_group(graw[q]);
#pragma unroll
    for (int k = 0; k < kWordRing; ++k) load_words(wd[k]);
    // The step being expanded (st % 8 == sm, steps in order): entering its
    // group if it is the group's first step.
    Cursor ce{0, 0, t0};
    auto enter_group = [&](int sm) {
      if constexpr (GK == 0) {
        if (ce.pos == 0) {  // a tile's first step
          gc.decode(graw[0].sw, graw[0].zw);
          load_group(graw[0]);
        }
      } else if (sm % GK == 0) {
        GroupRaw &gr = graw[(sm / GK) % NSLOT];
        gc.decode(gr.sw, gr.zw);
        load_group(gr);
      }
      advance(ce, nsteps);
    };
    // tiles 0..4 before the first barrier: the consumers' first super-step
    // computes steps 0..3 and reads the fragments of steps 1..4
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      enter_group(k);
      expand_pair_to_lds<DT>(wd[k].ra, wd[k].rb, gc, nm, bl[k], dw, drp);
      load_words(wd[k]);  // step k + kWordRing
      __builtin_amdgcn_sched_barrier(0);  // one expansion's temporaries live at a time
    }
    __syncthreads();
    // The consumers read tile 0 (slot 0) after that barrier, and super-step 0
    // below rewrites slot 0 with step 8: a second barrier, which they pass
    // once their reads of tile 0 have landed, keeps the two apart.  (From
    // super-step 1 on, a slot's previous tile was read a whole super-step
    // earlier.)
    __syncthreads();

    // Super-step S (the consumers' steps 4S..4S+3): expand steps 4S+5..4S+8
    // into tiles (4S+5..4S+8) % 8.  Their first reader runs in super-step
    // S+1, after the barrier that ends S.  Their slots' previous tiles
    // (4S-3..4S) were last read in super-step S-1 (tile 0: before the extra
    // barrier above), and the consumers wait for their own LDS reads before
    // each barrier.  Each word slot is refilled kWordRing steps ahead.  Steps
    // run on across the workgroup's tiles; past its last step everything
    // runs on clamped, in-bounds addresses into tiles no consumer uses.  kk:
    // parity of S in a two-super-step iteration, so that the ring slots
    // (4kk+5+u) % 8 are constants.
    auto psuper = [&](int kk) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int slot = (4 * kk + 5 + u) % kTiles;  // == (4S+5+u) % 8
        enter_group(slot);  // step 4S+5+u
        Words &w = wd[slot];
        expand_pair_to_lds<DT>(w.ra, w.rb, gc, nm, bl[slot], dw, drp);
        load_words(w);      // step 4S+5+u + kWordRing
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
    };
    const int nsuper = wg_steps / 4;  // I % 128 == 0
    for (int S0 = 0; S0 < nsuper; S0 += 2) {
      psuper(0);
      if (S0 == 0) PREFILL_MARK(1);
      if (S0 + 1 < nsuper) psuper(1);
    }
    PREFILL_MARK(46);
    return;
  }

  // ------------------------------ consumer ------------------------------
  const int fr = lane & 15, fk = (lane >> 4) * 8;  // lane row / k block of each 16 x 32 fragment
  // A fragment i of this wave: row tile wave RT + i (a scalar offset) and
  // lane's 16 bytes of it (the one per-lane offset)
  const uint32_t a_lane = (uint32_t)lane * 16u;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // in a scalar register
  const uint32_t a_wave = (uint32_t)wave_s * RT * tile_bytes;
  // A of k step ls of tile t: 16-row tiles from mb/16 of its M block, of
  // which those in the (16-row padded) tiled buffer exist; the buffer
  // descriptor ends there, so later ones read as zeros.
  auto load_a = [&](const Tile &t, int ls, u32x4 af[RT]) {
    const int64_t rtiles = (t.row_hi + 15) / 16 - t.mb / 16;
    const int tiles = (int)(rtiles < BM / 16 ? rtiles : BM / 16);
    const uint32_t kb = (uint32_t)ls * 1024u;
    const uint16_t *xt = t.xt;
    const char *a_base = reinterpret_cast<const char *>(xt + (t.mb / 16) * (I / 32) * 512);
    const __amdgpu_buffer_rsrc_t r = raw_rsrc(a_base + kb, (uint32_t)tiles * tile_bytes - kb);
#pragma unroll
    for (int i = 0; i < RT; ++i)
      af[i] = __builtin_amdgcn_raw_buffer_load_b128(r, a_lane, (int)(a_wave + (uint32_t)i * tile_bytes), 0);
  };
  // B fragment j of one k step: 16 of the tile's columns, k block fk
  // (physical block (fk/8) ^ ((column/16)&3)), one 16-byte LDS read.  The
  // weights are the MFMA's first operand, so a lane's results are four
  // consecutive fragment columns (4(lane/16) + r) of one token; fragment
  // column c of fragment j is tile column
  //     32 (j/2) + 8 (c/4) + 4 (j%2) + c%4,
  // which puts fragments 2s and 2s+1 of lane group g on the eight adjacent
  // columns 32s + 8g .. 32s + 8g + 7 (one 16-byte store in the epilogue).
  // Only the four lane offsets for j&3 live in registers; the tile and j>=4
  // (64 columns on) are constant offsets folded into the LDS instructions.
  uint32_t fcol[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int col = 32 * (jj >> 1) + 8 * (fr >> 2) + 4 * (jj & 1) + (fr & 3);
    fcol[jj] = (uint32_t)(col * kBStride + 8 * ((fk >> 3) ^ ((col >> 4) & 3)));
  }
  auto read_frag = [&](int tile, int j, u32x4 &b) {
    const uint16_t *col = &bl[0][0] + tile * (kBN * kBStride) + fcol[j & 3] + (j >> 2) * 64 * kBStride;
    b = *reinterpret_cast<const u32x4 *>(col);
  };

  u32x4 ab[kASlots][RT], bf[8];
#pragma unroll
  for (int k = 0; k < kASlots; ++k) load_a(t0, k, ab[k]);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) read_frag(0, j, bf[j]);
  // tile 0's slot is rewritten in the producer's first super-step
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  PREFILL_MARK(1);

  int step = 0;
  Tile t = t0;
  for (int it = 0;;) {
    // the next tile (this one again past the last: its A loads go unused)
    Tile tn;
    tile_at(it + 1 < my_tiles ? it + 1 : it, tn);
    // This tile's accumulators (AGPRs; declared per tile, so that nothing
    // carries them around the loop)
    f32x4 acc[RT][8];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_fence(acc[i][j]);
      }
    asm volatile("s_nop 7");  // accumulator writes -> first MFMA
    if (it < 8) PREFILL_MARK(2 + 4 * it);
    // Step s: for each column tile j, its four MFMAs on A slot s%4, then the
    // refill of fragment j with that of step s+1 (tile (s+1)%8, expanded at
    // least one barrier earlier), which has the other seven tiles' MFMAs to
    // arrive in; then the refill of the A slot with step s+4 (k step la of
    // tile ta), and after every fourth step a barrier, once this wave's LDS
    // reads have landed (the producer rewrites the slot of the last tile
    // read in the next super-step).  Halving the barriers of a two-step
    // super-step measured 202 -> 197.5 us at 2048 x 14336 -> 4096.  The
    // scheduling barriers keep each refill after the MFMAs that read the old
    // fragment (an MFMA reads its sources when issued).  Steps and ring
    // slots run on across the workgroup's tiles: the last step of a tile
    // refills with the first of the next.
    auto cstep = [&](int step, u32x4(&A)[RT], bool barrier, const Tile &ta, int la, bool reload_a = true) {
      const int next = (step + 1) % kTiles;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int i = 0; i < RT; ++i) mfma_acc<DT>(bf[j], A[i], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
        read_frag(next, j, bf[j]);
      }
      if (reload_a) load_a(ta, la, A);
      if (barrier) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // When both waves of a SIMD are ready, issue the consumer's MFMAs first;
    // the producer's VALU work fills the cycles in between.
    __builtin_amdgcn_s_setprio(2);
    // Super-steps of 4 (the A slots need constant indices; nsteps is a
    // positive multiple of 4).  All but the last load A of this tile four
    // steps ahead; the last one loads the next tile's first four steps, so
    // no branch on the tile sits inside the loop.
    int ls = 0;
    while (ls + kASlots < nsteps) {
#pragma unroll
      for (int k = 0; k < kASlots; ++k) cstep(step + k, ab[k], k == 3, t, ls + kASlots + k);
      step += kASlots;
      ls += kASlots;
    }
    if (it < 8) PREFILL_MARK(3 + 4 * it);
    // (the B fragments of the next tile's first step are read here, before
    // the barrier after which the producers rewrite their slot; of its A
    // steps only the first two are loaded before the epilogue, the other two
    // after it, so that fewer registers are live through it)
    // The tile's bias: lane l loads columns 2l, 2l+1 (one dword; the
    // epilogue hands each lane its eight columns per group by bpermute),
    // before the next tile's first A loads, so that waiting for it does not
    // wait for them.  The lane index is recomputed here by a volatile asm,
    // so that the compiler derives the epilogue's addresses per tile
    // instead of holding them (or spilling them) through the main loop.
    int el;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(el));
    uint32_t bw = 0u;
    if (t.bias && t.n0 + 2 * el < t.O) bw = *reinterpret_cast<const uint32_t *>(t.bias + t.n0 + 2 * el);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kASlots; ++k) cstep(step + k, ab[k], k == 3, tn, k, k < 2);
    step += kASlots;
    __builtin_amdgcn_s_setprio(0);
    mfma_drain();
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc_fence(acc[i][j]);
    if (it < 8) PREFILL_MARK(4 + 4 * it);

    asm volatile("" : "+v"(el));
    const int erow = el & 15, eg = el >> 4;
    // Epilogue, straight from the accumulators: lane (g, t) = (lane/16,
    // lane%16) holds, for each 16-row block i and column group s, the eight
    // outputs 32s + 8g .. 32s + 8g + 7 of row 16i + t (fragments 2s, 2s+1):
    // bias added in fp32, one rounding, one 16-byte store (two for fp32
    // output); the four lanes of a row write its 64 contiguous bytes.  No
    // LDS staging, so nothing waits here on the producers' LDS traffic.
    const int64_t m0 = t.mb + wave_s * 16 * RT;
    // rows m0 + lo .. m0 + hi - 1 of this wave's 16 RT are stored
    const int64_t lo64 = t.row_lo - m0, hi64 = t.row_hi - m0;
    const int lo = (int)(lo64 < 0 ? 0 : lo64 > 16 * RT ? 16 * RT : lo64);
    const int hi = (int)(hi64 < 0 ? 0 : hi64 > 16 * RT ? 16 * RT : hi64);
    // (1 through an empty asm: the compiler would fold acc * 1 + bias into
    // a convert and an add)
    float one = 1.0f;
    asm volatile("" : "+v"(one));
    // one copy per output dtype (no dtype test per store)
    auto epilogue = [&](auto ydt) {
      constexpr int YD = decltype(ydt)::value;
      typedef typename std::conditional<YD == kF32, float, uint16_t>::type YT;
      const int64_t O = t.O;
      YT *ybase = reinterpret_cast<YT *>(t.layer == 0 ? a.y : ltp->y[t.layer]) + (m0 + erow) * O + t.n0 + 8 * eg;
      // Two fp32 sums -> one packed pair, RNE.  For fp16 the conversion is
      // written as asm: the compiler would otherwise fuse it with the bias
      // fma into one mixed fma with an fp16 result (a single rounding),
      // whereas a 16-bit output is the rounding of the fp32 output.
      auto pk2 = [](float lo, float hi) -> uint32_t {
        if constexpr (YD == kF16) {
          uint32_t r;
          asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
          return r;
        } else {
          return pack2<YD>(lo, hi);
        }
      };
      // The lane's bias halves of column group s4: columns 32 s4 + 8 eg + 2q,
      // +1 are bias dword 16 s4 + 4 eg + q (bpermute), each added to its
      // output as the fp16 operand of one mixed fma.  The next block's are
      // fetched before this block's arithmetic, so that their latency is
      // hidden behind it.
      auto bias_of = [&](int s4, f16x2 (&b)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          b[q] = __builtin_bit_cast(f16x2, __builtin_amdgcn_ds_bpermute(4 * (16 * s4 + 4 * eg + q), (int)bw));
      };
      f16x2 bcur[4];
      bias_of(0, bcur);
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int row = 16 * i + erow;
        const bool row_ok = row >= lo && row < hi;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          f16x2 bnext[4];
          if (i + 1 < RT || s4 < 3) bias_of((s4 + 1) & 3, bnext);
          float v[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 &c = acc[i][2 * s4 + (q >> 1)];
            v[2 * q] = __builtin_fmaf(c[2 * (q & 1)], one, (float)bcur[q][0]);
            v[2 * q + 1] = __builtin_fmaf(c[2 * (q & 1) + 1], one, (float)bcur[q][1]);
          }
          if (row_ok && t.n0 + 32 * s4 + 8 * eg < O) {
            YT *dst = ybase + (int64_t)(16 * i) * O + 32 * s4;
            // ordinary (write-back) stores: a row's four 64-byte pieces meet
            // in L2 and leave as whole lines (streaming stores wrote 1.4x
            // the output bytes to HBM)
            if constexpr (YD == kF32) {
              *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
              *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
            } else {
              *reinterpret_cast<u32x4 *>(dst) = u32x4{pk2(v[0], v[1]), pk2(v[2], v[3]), pk2(v[4], v[5]), pk2(v[6], v[7])};
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) bcur[q] = bnext[q];
          __builtin_amdgcn_sched_barrier(0);  // one block's values live at a time
        }
      }
    };
    if (a.y_dt == kF32)
      epilogue(std::integral_constant<int, kF32>());
    else if (a.y_dt == kF16)
      epilogue(std::integral_constant<int, kF16>());
    else
      epilogue(std::integral_constant<int, kBF16>());
    if (it < 8) PREFILL_MARK(5 + 4 * it);
    if (++it >= my_tiles) break;
    t = tn;
    load_a(t, 2, ab[2]);
    load_a(t, 3, ab[3]);
  }
}

template <int GK, bool MOE, int RT>
static void launch_prefill_gk(const LinearArgs &a, const LayerTable &x, dim3 grid, hipStream_t st) {
  if (a.x_dt == kF16)
    hipLaunchKernelGGL((prefill_gemm_kernel<kF16, GK, MOE, RT>), grid, dim3(kThreads), 0, st, a, x);
  else
    hipLaunchKernelGGL((prefill_gemm_kernel<kBF16, GK, MOE, RT>), grid, dim3(kThreads), 0, st, a, x);
}

template <bool MOE, int RT>
static void launch_prefill_moe(const LinearArgs &a, const LayerTable &x, dim3 grid, hipStream_t st) {
  if constexpr (!MOE) {  // one group over the whole row (dense layers only)
    if (a.group == a.I && a.group > kG) {
      launch_prefill_gk<0, MOE, RT>(a, x, grid, st);
      return;
    }
  }
  if (a.group == 32) launch_prefill_gk<1, MOE, RT>(a, x, grid, st);
  else if (a.group == 64) launch_prefill_gk<2, MOE, RT>(a, x, grid, st);
  else launch_prefill_gk<4, MOE, RT>(a, x, grid, st);
}

// Rows per workgroup tile of a dense layer: 256, or 128 when a 256-row
// grid would not give every CU a workgroup (k_proj / v_proj of Llama-3-8B at
// 4096 tokens: 16 x 8 = 128 workgroups of 256 rows on 256 CUs).
// PARO_PREFILL_BM=128|256 forces one (tuning), read once per process.
static int dense_tile_rows(int64_t tokens, int64_t n_tiles) {
  static const int forced = [] {
    const char *v = getenv("PARO_PREFILL_BM");
    const int n = (v && *v) ? atoi(v) : 0;
    return (n == 128 || n == 256) ? n : 0;
  }();
  if (forced) return forced;
  return ((tokens + 255) / 256) * n_tiles < kCUs ? 128 : 256;
}

// Workgroups of a dense launch: one per CU, each taking every kCUs-th tile
// (a multiple of the 8 XCDs, so that a workgroup's tiles stay on its XCD in
// the tile order); fewer tiles than CUs give one tile per workgroup.
// PARO_PREFILL_PERSIST=0 gives every tile its own workgroup (tuning), read
// once per process.
static int64_t persistent_grid(int64_t tiles) {
  static const bool on = [] {
    const char *v = getenv("PARO_PREFILL_PERSIST");
    return !(v && *v && atoi(v) == 0);
  }();
  return on && tiles > kCUs ? kCUs : tiles;
}

int64_t moe_work_tiles(int64_t tokens, int experts) {
  // sum over experts of ceil((rows + up to 15 rows of the first 16-row tile) / 256)
  return (tokens + 15 * (int64_t)experts + kBM - 1) / kBM + experts;
}

hipError_t launch_prefill_gemm_multi(const LinearArgs &a, const LayerTable &lt_in, hipStream_t st) {
  LayerTable lt = lt_in;
  if (a.experts > 0) {
    const int64_t n_tiles = (a.O + kBN - 1) / kBN;
    // persistent: the workgroups take the tiles the offsets give in turn
    launch_prefill_moe<true, 4>(a, lt, dim3((unsigned)persistent_grid(n_tiles * moe_work_tiles(a.tokens, a.experts))),
                                st);
  } else {
    // the layers' column tiles one after another, each over all M blocks
    int64_t col_tiles = 0;
    for (int l = 0; l < lt.n; ++l) col_tiles += (lt.o[l] + kBN - 1) / kBN;
    const int bm = dense_tile_rows(a.tokens, col_tiles);
    const int64_t m_tiles = (a.tokens + bm - 1) / bm;
    lt.tile0[0] = 0;
    for (int l = 0; l < lt.n; ++l) lt.tile0[l + 1] = lt.tile0[l] + (int32_t)((lt.o[l] + kBN - 1) / kBN * m_tiles);
    const dim3 grid((unsigned)persistent_grid(lt.tile0[lt.n]));
    if (bm == 128)
      launch_prefill_moe<false, 2>(a, lt, grid, st);
    else
      launch_prefill_moe<false, 4>(a, lt, grid, st);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_gemm(const LinearArgs &a, const uint16_t *x, hipStream_t st) {
  LayerTable lt{};
  lt.n = 1;
  lt.qweight[0] = a.qweight;
  lt.qzeros[0] = a.qzeros;
  lt.scales[0] = a.scales;
  lt.bias[0] = a.bias;
  lt.xt[0] = x;
  lt.y[0] = a.y;
  lt.o[0] = a.O;
  return launch_prefill_gemm_multi(a, lt, st);
}

}  // namespace paro
