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
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"

namespace paro {

constexpr int kBM = 256, kBN = 128, kBK = 32;
constexpr int kWaves = 8, kThreads = 64 * kWaves;  // 4 consumer + 4 producer waves
constexpr int kStepsPerGroup = kG / kBK;
constexpr int kBStride = kBK + 8;  // halves per LDS column (80 bytes: 16-byte aligned fragment reads)
constexpr int kTiles = 8;           // LDS ring of expanded weight tiles (k steps)
constexpr int kWordRing = 8;        // packed weight words in flight per producer thread (steps)
constexpr int kASlots = 4;          // A fragments in flight per consumer wave (steps)
constexpr int kGroupM = 2;          // M blocks per group of the tile order (dense layers)
constexpr int kStageRS = kBN + 4;   // epilogue staging row stride (floats): the four row groups of a store hit distinct banks
static_assert(kTiles == 8 && kWordRing == 8, "the producer's ring slot arithmetic assumes rings of 8");

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
// (rotated once for all experts).  A workgroup takes one 256-row tile of one
// expert's rows, starting at the 16-row tile that holds the expert's first
// row: rows of neighbouring experts in its tiles are computed and dropped.
// Offsets are clamped into [0, tokens] and made nondecreasing, so no offsets
// can take a workgroup outside its buffers.
template <int DT, int GK, bool MOE>
__global__ void __launch_bounds__(kThreads)
prefill_gemm_kernel(LinearArgs a, const uint16_t *__restrict__ xt) {
  __shared__ __attribute__((aligned(16))) uint16_t bl[kTiles][kBN * kBStride];
  __shared__ __attribute__((aligned(16))) float stage[4][32 * kStageRS];  // epilogue, one per consumer wave
  const int lane = lane_id(), wave = wave_id();
  const int64_t I = a.I, O = a.O, W = O / 8, M = a.tokens;
  // XCD-local order: consecutive logical tiles (the N tiles of one M block)
  // share an XCD and its L2.  The tile indices are uniform; readfirstlane
  // moves them (computed with VALU division) to scalar registers so that the
  // buffer descriptors derived from them stay scalar too.
  const int n_tiles = (int)((O + kBN - 1) / kBN);
  const int m_tiles = MOE ? (int)(gridDim.x / n_tiles) : (int)((M + kBM - 1) / kBM);
  const int lwg = xcd_local_order((int)blockIdx.x, n_tiles * m_tiles);
  // Dense layers: logical tiles go in groups of kGroupM M blocks, the M block
  // fastest, so an XCD's share of consecutive tiles spans kGroupM blocks of
  // rows and 1/kGroupM as many weight columns as a row-major order would.
  int tn = lwg % n_tiles, tm = lwg / n_tiles;
  if constexpr (!MOE) {
    const int first = (lwg / (kGroupM * n_tiles)) * kGroupM;
    const int gsz = m_tiles - first < kGroupM ? m_tiles - first : kGroupM;
    const int r = lwg % (kGroupM * n_tiles);
    tm = first + r % gsz;
    tn = r / gsz;
  }
  const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane(tn) * kBN;
  int64_t mb, row_lo = 0, row_hi = M;
  const int32_t *qweight = a.qweight, *qzeros = a.qzeros;
  const uint16_t *scales = a.scales, *bias = a.bias;
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
      const int64_t t = o1 > prev ? (o1 - (prev & ~(int64_t)15) + kBM - 1) / kBM : 0;
      if (wi < cum + t) {
        e = k;
        lo = prev;
        hi = o1;
        j = wi - cum;
        break;
      }
      cum += t;
      prev = o1;
    }
    if (e < 0) return;  // past the last tile: the whole workgroup leaves before any barrier
    mb = (lo & ~(int64_t)15) + j * kBM;
    row_lo = lo > mb ? lo : mb;
    row_hi = hi < mb + kBM ? hi : mb + kBM;
    const int64_t G = (int64_t)kBK * GK;
    qweight += (int64_t)e * I * W;
    qzeros += (int64_t)e * (I / G) * W;
    scales += (int64_t)e * (I / G) * O;
    if (bias) bias += (int64_t)e * O;
  } else {
    mb = (int64_t)__builtin_amdgcn_readfirstlane(tm) * kBM;
  }
  // GK k-steps per quantization group (G = 32 * GK); I is a multiple of 128
  const int nsteps = (int)(I / kBK), ngroups = (int)(I / (kBK * GK));

  // A row tiles of this workgroup: 16 from mb/16, of which `tiles` exist in
  // the (16-row padded) tiled buffer; later ones read as zeros.
  const int64_t rtiles = (row_hi + 15) / 16 - mb / 16;
  const int tiles = (int)(rtiles < kBM / 16 ? rtiles : kBM / 16);
  const uint32_t tile_bytes = (uint32_t)nsteps * 1024u;  // one row tile over all of k
  const uint32_t a_bytes = (uint32_t)tiles * tile_bytes;
  const char *a_base = reinterpret_cast<const char *>(xt + (mb / 16) * (I / 32) * 512);
  auto a_rsrc = [&](int step) {
    const int st = step < nsteps ? step : nsteps - 1;  // past the end: any in-bounds step, unused
    const uint32_t kb = (uint32_t)st * 1024u;
    return raw_rsrc(a_base + kb, a_bytes - kb);
  };

  if (wave >= 4) {
    // ------------------------------ producer ------------------------------
    const int tp = threadIdx.x - 256;
    const int dw = tp & 15, drp = tp >> 4;  // word dw of the tile's 16, rows 2drp, 2drp+1 of a step
    const int64_t dword = n0 / 8 + dw;
    const uint32_t dwc = (uint32_t)(dword < W ? dword : W - 1);  // tail tile: any in-bounds word
    const uint32_t w_off = (uint32_t)((2 * drp) * W + dwc) * 4u;
    const uint32_t w_step_bytes = (uint32_t)(kBK * W * 4);

    struct Words {
      uint32_t ra, rb;
    };
    auto load_words = [&](int step, Words &wd) {
      const int st = step < nsteps ? step : nsteps - 1;
      const __amdgpu_buffer_rsrc_t r = raw_rsrc(qweight + (int64_t)st * kBK * W, w_step_bytes);
      wd.ra = __builtin_amdgcn_raw_buffer_load_b32(r, w_off, 0, 0);
      wd.rb = __builtin_amdgcn_raw_buffer_load_b32(r, w_off + (uint32_t)(W * 4), 0, 0);
    };
    struct GroupRaw {
      u32x4 sw;
      uint32_t zw;
    };
    auto load_group = [&](int g, GroupRaw &gr) {
      const int gg = g < ngroups ? g : ngroups - 1;
      const __amdgpu_buffer_rsrc_t rs = raw_rsrc(scales + (int64_t)gg * O, (uint32_t)(O * 2));
      gr.sw = __builtin_amdgcn_raw_buffer_load_b128(rs, dwc * 16u, 0, 0);
      const __amdgpu_buffer_rsrc_t rz = raw_rsrc(qzeros + (int64_t)gg * W, (uint32_t)(W * 4));
      gr.zw = __builtin_amdgcn_raw_buffer_load_b32(rz, dwc * 4u, 0, 0);
    };

    // Scales and zeros: a ring of NSLOT groups.  Group q sits in slot
    // q % NSLOT; it is decoded just before the first k-step of the group is
    // expanded, and the slot is refilled at once with group q + NSLOT.  Every
    // slot index below is a compile-time constant: the step's value mod 8 is.
    constexpr int NSLOT = GK == 1 ? 4 : 2;
    GroupConsts<DT> gc;
    const NibbleMasks nm;
    GroupRaw graw[NSLOT];
    Words wd[kWordRing];
#pragma unroll
    for (int q = 0; q < NSLOT; ++q) load_group(q, graw[q]);
#pragma unroll
    for (int k = 0; k < kWordRing; ++k) load_words(k, wd[k]);
    // step st (st % 8 == sm): enter its group if it is the group's first step
    auto enter_group = [&](int sm, int st) {
      if (sm % GK == 0) {
        GroupRaw &gr = graw[(sm / GK) % NSLOT];
        gc.decode(gr.sw, gr.zw);
        load_group(st / GK + NSLOT, gr);
      }
    };
    // tiles 0..4 before the first barrier: the consumers' first super-step
    // computes steps 0..3 and reads the fragments of steps 1..4
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      enter_group(k, k);
      expand_pair_to_lds<DT>(wd[k].ra, wd[k].rb, gc, nm, bl[k], dw, drp);
      load_words(k + kWordRing, wd[k]);
      __builtin_amdgcn_sched_barrier(0);  // one expansion's temporaries live at a time
    }
    __syncthreads();

    // Super-step S (the consumers' steps 4S..4S+3): expand steps 4S+5..4S+8
    // into tiles (4S+5..4S+8) % 8.  Their first reader runs in super-step
    // S+1, after the barrier that ends S.  Their slots' previous tiles
    // (4S-3..4S) were last read in super-step S-1, and the consumers wait for
    // their own LDS reads before each barrier.  Each word slot is refilled
    // kWordRing steps ahead.  Past the end everything runs on clamped,
    // in-bounds addresses into tiles no consumer uses.  kk: parity of S in a
    // two-super-step iteration, so that the ring slots (4kk+5+u) % 8 are
    // constants.
    auto psuper = [&](int S, int kk) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int slot = (4 * kk + 5 + u) % kTiles;  // == (4S+5+u) % 8
        enter_group(slot, 4 * S + 5 + u);
        Words &w = wd[slot];
        expand_pair_to_lds<DT>(w.ra, w.rb, gc, nm, bl[slot], dw, drp);
        load_words(4 * S + 5 + u + kWordRing, w);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
    };
    const int nsuper = nsteps / 4;  // I % 128 == 0
    for (int S0 = 0; S0 < nsuper; S0 += 2) {
      psuper(S0, 0);
      if (S0 + 1 < nsuper) psuper(S0 + 1, 1);
    }
    return;
  }

  // ------------------------------ consumer ------------------------------
  const int fr = lane & 15, fk = (lane >> 4) * 8;  // lane row / k block of each 16 x 32 fragment
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_off[i] = (uint32_t)(wave * 4 + i) * tile_bytes + (uint32_t)lane * 16u;
  auto load_a = [&](int step, u32x4 af[4]) {
    const __amdgpu_buffer_rsrc_t r = a_rsrc(step);
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = __builtin_amdgcn_raw_buffer_load_b128(r, a_off[i], 0, 0);
  };
  // B fragment of column tile j of one k step: column 16j + fr, k
  // block fk (physical block (fk/8) ^ (j&3)), one 16-byte LDS read.
  // Only the four lane offsets for j&3 live in registers; the tile and j>=4
  // are constant offsets folded into the LDS instructions.
  uint32_t fcol[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) fcol[jj] = (uint32_t)((jj * 16 + fr) * kBStride + 8 * ((fk >> 3) ^ jj));
  auto read_frag = [&](int tile, int j, u32x4 &b) {
    const uint16_t *col = &bl[0][0] + tile * (kBN * kBStride) + fcol[j & 3] + (j >> 2) * 64 * kBStride;
    b = *reinterpret_cast<const u32x4 *>(col);
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 ab[kASlots][4], bf[8];
#pragma unroll
  for (int k = 0; k < kASlots; ++k) load_a(k, ab[k]);
  __syncthreads();
  // When both waves of a SIMD are ready, issue the consumer's MFMAs first;
  // the producer's VALU work fills the cycles in between.
  __builtin_amdgcn_s_setprio(2);
#pragma unroll
  for (int j = 0; j < 8; ++j) read_frag(0, j, bf[j]);

  // Step s: for each column tile j, its four MFMAs on A slot s%4, then the
  // refill of fragment j with that of step s+1 (tile (s+1)%8, expanded at
  // least one barrier earlier), which has the other seven tiles' MFMAs to
  // arrive in; then the refill of the A slot with step s+4, and after every
  // fourth step a barrier, once this wave's LDS reads have landed (the
  // producer rewrites the slot of the last tile read in the next
  // super-step).  Halving the barriers of a two-step super-step measured
  // 202 -> 197.5 us at 2048 x 14336 -> 4096.  The scheduling barriers keep each refill after the
  // MFMAs that read the old fragment (an MFMA reads its sources when issued).
  auto cstep = [&](int step, u32x4(&A)[4], bool barrier) {
    const int next = (step + 1) % kTiles;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) mfma_acc<DT>(A[i], bf[j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      read_frag(next, j, bf[j]);
    }
    load_a(step + kASlots, A);
    if (barrier) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // (unrolled by kASlots: the A slots need constant indices; nsteps is a
  // positive multiple of 4.  A do-while has no zero-trip path, whose join
  // would let the compiler copy accumulators out before the drain below.)
  int step = 0;
  do {
#pragma unroll
    for (int k = 0; k < kASlots; ++k) cstep(step + k, ab[k], k == 3);
    step += kASlots;
  } while (step < nsteps);
  __builtin_amdgcn_s_setprio(0);
  mfma_drain();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc_fence(acc[i][j]);

  // Epilogue.  Each consumer wave stages its 64 x 128 fp32 tile through its
  // own LDS region, 32 rows at a time; a lane then holds 4 consecutive columns
  // of one row: bias added in fp32, one rounding, one 8-byte store (16 bytes
  // for fp32 output), so every row's 128 columns leave as whole cache lines.
  float *stg = stage[wave];
  const int64_t m0 = mb + wave * 64;
  const int sc = (lane & 31) * 4, srow = lane >> 5;  // quad column, row parity of this lane
  const int64_t n = n0 + sc;
  const bool n_ok = n < O;  // O % 8 == 0: a quad is wholly in or out
  f32x4 bias4{0.f, 0.f, 0.f, 0.f};
  if (bias && n_ok) {
    const u32x2 bb = *reinterpret_cast<const u32x2 *>(bias + n);
    bias4 = f32x4{f16_bits_to_f32(bb[0] & 0xffffu), f16_bits_to_f32(bb[0] >> 16), f16_bits_to_f32(bb[1] & 0xffffu),
                  f16_bits_to_f32(bb[1] >> 16)};
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    // D of tile (i, j): row 16i + 4(lane/16) + r, column 16j + lane%16
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          stg[(16 * ii + (lane >> 4) * 4 + r) * kStageRS + 16 * j + fr] = acc[2 * p + ii][j][r];
    wave_lds_sync();
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int lr = 2 * rr + srow;
      const f32x4 v = *reinterpret_cast<const f32x4 *>(stg + lr * kStageRS + sc) + bias4;
      const int64_t row = m0 + 32 * p + lr;
      if (row >= row_lo && row < row_hi && n_ok) {
        if (a.y_dt == kF32) {
          *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.y) + row * O + n) = v;
        } else {
          const u32x2 o = a.y_dt == kF16 ? u32x2{pack2<kF16>(v[0], v[1]), pack2<kF16>(v[2], v[3])}
                                         : u32x2{pack2<kBF16>(v[0], v[1]), pack2<kBF16>(v[2], v[3])};
          *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.y) + row * O + n) = o;
        }
      }
    }
    wave_lds_sync();  // this pass's reads are done before the next pass's writes
  }
}

template <int GK, bool MOE>
static void launch_prefill_gk(const LinearArgs &a, const uint16_t *x, dim3 grid, hipStream_t st) {
  if (a.x_dt == kF16)
    hipLaunchKernelGGL((prefill_gemm_kernel<kF16, GK, MOE>), grid, dim3(kThreads), 0, st, a, x);
  else
    hipLaunchKernelGGL((prefill_gemm_kernel<kBF16, GK, MOE>), grid, dim3(kThreads), 0, st, a, x);
}

template <bool MOE>
static void launch_prefill_moe(const LinearArgs &a, const uint16_t *x, dim3 grid, hipStream_t st) {
  if (a.group == 32) launch_prefill_gk<1, MOE>(a, x, grid, st);
  else if (a.group == 64) launch_prefill_gk<2, MOE>(a, x, grid, st);
  else launch_prefill_gk<4, MOE>(a, x, grid, st);
}

int64_t moe_work_tiles(int64_t tokens, int experts) {
  // sum over experts of ceil((rows + up to 15 rows of the first 16-row tile) / 256)
  return (tokens + 15 * (int64_t)experts + kBM - 1) / kBM + experts;
}

hipError_t launch_prefill_gemm(const LinearArgs &a, const uint16_t *x, hipStream_t st) {
  const int64_t n_tiles = (a.O + kBN - 1) / kBN;
  if (a.experts > 0) {
    launch_prefill_moe<true>(a, x, dim3((unsigned)(n_tiles * moe_work_tiles(a.tokens, a.experts))), st);
  } else {
    launch_prefill_moe<false>(a, x, dim3((unsigned)(n_tiles * ((a.tokens + kBM - 1) / kBM))), st);
  }
  return hipGetLastError();
}

}  // namespace paro
