// decode.hip - small-batch (tokens <= 16) rotated W4A16 linear: split-K MFMA
// GEMV, optionally with the activation rotation fused into the prologue.
//
//   y[m][n] = sum_g s[g][n] * sum_{k in g} x_r[m][k] * (q[k][n] - z[g][n]) + b[n]
//
// ("ParoQuant" wiki, Activation and weight transforms: Y = X_r Q(W_r)^T + b;
// Triton plans and tuning: unpack, subtract zero points, multiply by group
// scales, fp32 accumulation.)
//
// Work split.  A k-step is 32 rows of the weight.  A workgroup (NW waves)
// owns a tile of 128*WPL output columns and NW*KSW consecutive k-steps; wave
// w takes KSW consecutive k-steps of them.  The tile's row segments (64*WPL
// contiguous bytes per weight row) go straight from HBM into LDS: at entry
// every wave issues 1 KB buffer-to-LDS loads for all its k-steps, after its
// few register loads, so the weight stream holds no VGPRs and each k-step
// waits only for its own loads (vmcnt counts them in order).  A lane then
// reads the 8 rows of its 8-row block (lane>>4) of its WPL packed words
// (lane&15) from LDS.  Each packed word turns into eight MFMA
// B fragments (one per nibble slot = one output column each), so no
// transpose is needed: v_perm_b32 gathers the bytes of a row pair and one
// v_and_or_b32 with an exponent-bias constant turns a nibble into a
// half-precision number
// (fp16: 0x6400|q = 1024+q, 0x6400|(q<<4) = 1024+16q; bf16: 0x4300|q =
// 128+q).  The offset and the zero point are removed with the row sums of the
// rounded activations, which one extra MFMA against a fragment of ones
// produces in the output layout:
//   sum_k x (off + c*q) = off*xsum + c*sum_k x q
//   =>  sum_k x (q - z) = (acc - (off + c*z) * xsum) / c,
// folded into the running sum with the group scale at the end of every
// 128-row block and of the wave's k-steps (the fold is linear, so folding a
// group in pieces gives the same sum).  v_mfma_f32_16x16x32_{f16,bf16}: lane
// l holds A row l&15 and B column l&15 of its 8-element k block; the 16x16
// fp32 result has row 4*(l>>4)+r, column l&15 in register r.
//
// Workgroups are numbered tile-fastest (all column tiles of split 0, then of
// split 1, ...) and that order is dealt out to the XCDs in contiguous runs
// (xcd_local_order), so the tiles sharing the same weight rows run on one XCD
// at the same time and their row segments merge in its L2 into long DRAM
// bursts.
//
// Reduction.  The NW waves' tiles are summed in LDS in wave order, in
// "slots" of 4 consecutive outputs laid out so that stores and loads are
// consecutive 16-byte chunks (see the kernel).  With one K split the
// workgroup adds the bias and stores y.  Otherwise it stores its fp32 partial
// with 16-byte device-coherent stores (SC1: coherent across the XCDs' L2
// caches without whole-cache write-backs), waits for them, and bumps a
// device-scope counter; the last workgroup of the column tile to arrive
// loads every split's slots with 16-byte device-coherent loads, all in flight
// together, sums them in split order, adds the bias, stores y and resets the
// counter.  The result is independent of arrival order (bitwise
// deterministic).
#include <stdlib.h>

#include <type_traits>

#include "launch.hpp"
#include "mfma.hpp"

namespace paro {

// Optional per-wave timeline, compiled in only with PARO_DECODE_TIMELINE
// (csrc/decode_timeline.hip): lane 0 of every wave stores the 100 MHz
// realtime counter at fixed points of the kernel into
// decode_timeline_buf[workgroup][wave][16].  Marks: 0 entry, 1 weight loads
// issued, 2-5 k-steps 0-3 landed, 6 k-steps done, 7 reduction start (first
// barrier), 8 reduction stores done, 9 second barrier, 10 slots summed,
// 11 partial stores issued, 12 partial stores complete, 13 counter returned,
// 14 gather done (finishing workgroup), 15 outputs stored.
#ifdef PARO_DECODE_TIMELINE
__device__ unsigned long long *decode_timeline_buf;
#define DECODE_MARK(i)                                                                                  \
  do {                                                                                                  \
    if ((threadIdx.x & 63) == 0)                                                                        \
      decode_timeline_buf[((size_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)) * 16 + (i)] =   \
          __builtin_amdgcn_s_memrealtime();                                                             \
  } while (0)
#else
#define DECODE_MARK(i) \
  do {                 \
  } while (0)
#endif

constexpr int kDecodeRS = kG + 4;  // fused-rotation LDS row stride (floats)
constexpr int kCounterStride = 32; // uint32 per split-K counter: one 128-byte line each
// Cache policy of the raw buffer loads/stores that exchange split-K partials:
// SC1, the device-scope coherent form (the one relaxed device-scope atomics use).
constexpr int kDeviceCoherent = 16;

template <int DT>
struct MfmaTypes;
template <>
struct MfmaTypes<kF16> {
  typedef f16x8 v8;
  static constexpr uint32_t kMagic = 0x64006400u;  // 1024.0 in both halves
  static constexpr uint32_t kOnes = 0x3c003c00u;   // 1.0
  static constexpr float kOff = 1024.0f;
};
template <>
struct MfmaTypes<kBF16> {
  typedef bf16x8 v8;
  static constexpr uint32_t kMagic = 0x43004300u;  // 128.0 in both halves
  static constexpr uint32_t kOnes = 0x3f803f80u;   // 1.0
  static constexpr float kOff = 128.0f;
};

template <int DT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  typedef typename MfmaTypes<DT>::v8 v8;
  if constexpr (DT == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0,
                                                   0, 0);
}

// The nibble masks and the exponent pattern, held in VGPRs: each fragment
// word is then one v_and_or_b32 (with literal operands the compiler emits an
// AND and an OR, since the three-operand form takes no literal here).
struct NibbleMasks {
  uint32_t lo, hi, magic;
};
template <int DT>
__device__ __forceinline__ NibbleMasks nibble_masks() {
  NibbleMasks m{0x000f000fu, 0x00f000f0u, MfmaTypes<DT>::kMagic};
  asm volatile("" : "+v"(m.lo), "+v"(m.hi), "+v"(m.magic));
  return m;
}

// B fragment of nibble slot `s` from the 8 row words r[0..7] (rows k0..k0+7)
// of one packed column word.  Element e of the fragment is row k0+e.
// fp16: even slots give 1024+q, odd slots 1024+16q; bf16: 128+q everywhere.
template <int DT>
__device__ __forceinline__ void build_b_frags(const uint32_t r[8], u32x4 out[8], const NibbleMasks &m) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // P = [ra.b0, ra.b2, rb.b0, rb.b2], Q = [ra.b1, ra.b3, rb.b1, rb.b3]
    const uint32_t P = __builtin_amdgcn_perm(r[2 * i], r[2 * i + 1], 0x02000604u);
    const uint32_t Q = __builtin_amdgcn_perm(r[2 * i], r[2 * i + 1], 0x03010705u);
    const uint32_t P8 = P >> 8, Q8 = Q >> 8;
    if constexpr (DT == kF16) {
      out[0][i] = (P & m.lo) | m.magic;
      out[1][i] = (P & m.hi) | m.magic;
      out[2][i] = (Q & m.lo) | m.magic;
      out[3][i] = (Q & m.hi) | m.magic;
      out[4][i] = (P8 & m.lo) | m.magic;
      out[5][i] = (P8 & m.hi) | m.magic;
      out[6][i] = (Q8 & m.lo) | m.magic;
      out[7][i] = (Q8 & m.hi) | m.magic;
    } else {
      out[0][i] = (P & m.lo) | m.magic;
      out[1][i] = ((P >> 4) & m.lo) | m.magic;
      out[2][i] = (Q & m.lo) | m.magic;
      out[3][i] = ((Q >> 4) & m.lo) | m.magic;
      out[4][i] = (P8 & m.lo) | m.magic;
      out[5][i] = ((P >> 12) & m.lo) | m.magic;
      out[6][i] = (Q8 & m.lo) | m.magic;
      out[7][i] = ((Q >> 12) & m.lo) | m.magic;
    }
  }
}

// Scale factor c of slot s in the fragment encoding (see build_b_frags).
template <int DT>
__device__ __forceinline__ constexpr float slot_mult(int s) {
  return (DT == kF16 && (s & 1)) ? 16.0f : 1.0f;
}

// Bytes of weight rows one wave holds in LDS: KSW k-steps of 32 rows of the
// tile's 64*WPL-byte row segment.
constexpr int decode_wave_lds(int wpl, int ksw) { return ksw * 32 * 64 * wpl; }

// s_waitcnt immediate for "at most n vector-memory loads outstanding", the
// other counters left open (gfx9-family encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// One 1 KB global -> LDS load: lane l's 16 bytes at `voff` land at lds + 16l.
// (A plain device function: inside a kernel template the builtin would keep
// the host pass from emitting the kernel's launch stub.)
__device__ __forceinline__ void dma_1k(__amdgpu_buffer_rsrc_t r, unsigned char *lds, uint32_t voff) {
  typedef __attribute__((address_space(3))) void *lds_ptr;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, 0, 0, 0);
}

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// MT: token rows carried per wave (1, 2, 4, 8 or 16; M <= MT, rows >= M are
// zero).  FR = min(MT, 4) accumulator registers can hold real rows.
template <int DT, int WPL, int KSW, int NW, bool FUSED, int MT>
__global__ void __launch_bounds__(64 * NW)
decode_kernel(LinearArgs a, const uint16_t *__restrict__ xr, int splits, float *__restrict__ partial,
              uint32_t *__restrict__ counters) {
  constexpr int FR = MT < 4 ? MT : 4;
  constexpr int NT = 8 * WPL;                 // MFMA column tiles per wave
  constexpr int NG = KSW < 4 ? 1 : KSW / 4;   // groups a wave touches (its k-steps are aligned)
  constexpr int NTH = 64 * NW;
  constexpr int NTILE = 128 * WPL;
  constexpr int KBV = (MT + 3) / 4;                     // lane groups (kb) holding real rows
  constexpr int QUADS = MT * NTILE / 4;                 // output slots of the tile (16 bytes each)
  constexpr int QPT = (QUADS + NTH - 1) / NTH;          // slots per thread
  static_assert(QUADS == 2 * WPL * FR * 16 * KBV, "slot numbering covers the tile");
  constexpr int RB = 64 * WPL;                          // bytes of one weight row of the tile
  constexpr int LPR = 4 * WPL;                          // 16-byte lanes per row in one DMA load
  constexpr int RPI = 64 / LPR;                         // rows per DMA load (1 KB)
  constexpr int NI = 32 / RPI;                          // DMA loads per k-step
  constexpr int WLDS = decode_wave_lds(WPL, KSW);
  static_assert(KSW * NI <= 63, "the k-step waits count at most 63 loads");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  // Every argument the kernel reads, named in one empty asm at the top, so
  // that their scalar loads go out together: otherwise the compiler loads
  // some of them only after the first batch has returned, a second
  // dependent round trip before the weight stream can start.
  asm volatile("" ::"s"(a.I), "s"(a.O), "s"(a.tokens), "s"(a.krot), "s"(a.group), "s"(a.pairs), "s"(a.theta),
               "s"(a.cs), "s"(a.qweight), "s"(a.qzeros), "s"(a.scales), "s"(a.bias), "s"(a.x), "s"(a.y),
               "s"(a.y_dt), "s"(xr), "s"(splits), "s"(partial), "s"(counters));
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(wave_id());
  DECODE_MARK(0);
  const int cl = lane & 15, kb = lane >> 4;
  const int n_tiles = (int)((a.O + NTILE - 1) / NTILE);
  const int lwg = xcd_local_order((int)blockIdx.x, n_tiles * splits);
  const int tile = lwg % n_tiles, split = lwg / n_tiles;
  const int64_t I = a.I, O = a.O, W = O / 8;
  const int M = (int)a.tokens;
  const int64_t nks = I / 32;
  const int64_t ks0 = ((int64_t)split * NW + wave) * KSW;  // first k-step of this wave
  const int nk = (int)((ks0 >= nks) ? 0 : ((nks - ks0) < KSW ? (nks - ks0) : KSW));
  const uint16_t *__restrict__ x = reinterpret_cast<const uint16_t *>(a.x);
  const int64_t n0 = (int64_t)tile * NTILE;

  // ---- output slots ----
  // A slot is a 16-byte chunk of 4 consecutive columns of one row of the
  // tile: the chunk that lane (kb, cl) holds for its store number instr in
  // the reduction below,
  //   s = instr * 16 * KBV + kb * 16 + cl,   instr = (w * FR + i) * 2 + h,
  //   row = 4 * kb + i,   column = (cl * WPL + w) * 8 + 4 * h,
  // where KBV = ceil(MT / 4) lane groups hold real rows.  The LDS reduction
  // tiles and the split-K partials are slot-major, so every wave's stores and
  // every thread's loads there are consecutive 16-byte chunks (no LDS bank
  // conflicts); thread t owns slots t, t + NTH, ...
  auto slot_pos = [](int sl, int &row, int &col) {
    const int instr = sl / (16 * KBV), r = sl % (16 * KBV);
    const int h = instr % 2, i = (instr / 2) % FR, w = instr / (2 * FR);
    row = 4 * (r / 16) + i;
    col = ((r % 16) * WPL + w) * 8 + 4 * h;
  };

  // ---- small early loads: this thread's bias values ----
  // Branch-free: every load reads a valid address (a stand-in tensor when
  // there is no bias, a clamped column past O) and the value is selected
  // afterwards.  A slot is entirely inside or entirely past O (O % 8 == 0).
  float bias_v[QPT][4];
  const uint16_t *bias_src = a.bias ? a.bias : a.scales;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int sl = threadIdx.x + j * NTH;
    int row, col;
    slot_pos(sl, row, col);
    const int64_t n = n0 + col;
    const bool use = a.bias && sl < QUADS && row < M && n < O;
    const u32x2 b = *reinterpret_cast<const u32x2 *>(bias_src + (n < O ? n : O - 4));
#pragma unroll
    for (int c = 0; c < 4; ++c) bias_v[j][c] = use ? f16_bits_to_f32((b[c >> 1] >> (16 * (c & 1))) & 0xffffu) : 0.0f;
  }

  // Columns past O (last tile only) get zero scales, so whatever weight bits
  // they read contribute nothing; their outputs are never stored.  WPL words
  // never straddle O (O % 16 == 0 for WPL == 2, O % 32 == 0 for WPL == 4).
  const int64_t wbase = (int64_t)tile * 16 * WPL + cl * WPL;
  const bool wok = wbase < W;
  const int64_t wcl = wok ? wbase : W - WPL;

  float tot[NT][FR];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < FR; ++i) tot[j][i] = 0.0f;

  if (nk > 0) {
    // 128-channel rotation blocks hold 4 k-steps; quantization groups hold
    // G/32 = 1 << gsh (with G < 128 the plan gives each wave one k-step).  One
    // group over the whole row (G = I > 128, any multiple of 128): a shift
    // past every k-step, so all fall in group 0 (its rotation ran in a
    // separate pass).
    const bool row_group = a.group == I && a.group > kG;
    const int gsh = row_group ? 30 : __builtin_ctz((unsigned)a.group) - 5, gmask = kG - a.group;
    const int64_t g_first = ks0 / 4, q_first = ks0 >> gsh, nq = I / a.group;
    float *xs = reinterpret_cast<float *>(smem + NW * WLDS) + wave * (MT * kDecodeRS);  // fused rotation rows
    // ---- fused: the first group's rotation inputs ----
    RotParams rp;
    float xin[MT][2];
    float cs0 = 0.f, cs1 = 0.f;
    auto load_rot_inputs = [&](int64_t g) {
      const int64_t c0 = g * kG + 2 * lane;
      rp.load(a.pairs + g * kG, I, a.theta + g * kPairs, I / 2, a.krot, lane, gmask);
      cs0 = a.cs[c0];
      cs1 = a.cs[c0 + 1];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint32_t wv = *reinterpret_cast<const uint32_t *>(x + (int64_t)(m < M ? m : 0) * I + c0);
        xin[m][0] = act_to_f32<DT>(wv & 0xffffu);
        xin[m][1] = act_to_f32<DT>(wv >> 16);
      }
    };
    if constexpr (FUSED) load_rot_inputs(g_first);

    // ---- A fragments (non-fused), group scales and zeros ----
    u32x4 af[KSW];
    const int arow = cl < M ? cl : 0;
    if constexpr (!FUSED) {
#pragma unroll
      for (int k = 0; k < KSW; ++k) {
        const int64_t ks = ks0 + (k < nk ? k : 0);
        af[k] = *reinterpret_cast<const u32x4 *>(xr + (int64_t)arow * I + ks * 32 + kb * 8);
      }
    }
    u32x4 sv[NG][WPL];
    uint32_t zv[NG][WPL];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int64_t g0 = q_first + gi;
      const int64_t g = g0 < nq ? g0 : nq - 1;
#pragma unroll
      for (int w = 0; w < WPL; ++w) {
        sv[gi][w] = *reinterpret_cast<const u32x4 *>(a.scales + g * O + 8 * (wcl + w));  // wcl is in bounds
        zv[gi][w] = (uint32_t)a.qzeros[g * W + wcl + w];
      }
    }

    // ---- the weight rows of every k-step, straight into LDS ----
    // Issued after every other load of the prologue, so the per-k-step waits
    // below count only these.  One DMA load moves 1 KB: lane l's 16 bytes
    // land at slot l, i.e. LDS row position pos = j*RPI + l/LPR, chunk l%LPR.
    // Position pos holds k-step row (pos%4)*8 + pos/4, so the rows that the
    // four 8-row blocks read together sit in different LDS banks.  The raw
    // buffer covers this wave's rows only: offsets past them (columns past O
    // in the last row) read zeros instead of memory.
    const uint32_t W4 = (uint32_t)(W * 4);
    const __amdgpu_buffer_rsrc_t rw =
        raw_rsrc(a.qweight + ks0 * 32 * W, (uint32_t)nk * 32u * W4);
    unsigned char *wl = smem + wave * WLDS;
    uint32_t voff[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int pos = j * RPI + lane / LPR;
      const int row = (pos & 3) * 8 + (pos >> 2);
      voff[j] = (uint32_t)row * W4 + (uint32_t)tile * RB + (uint32_t)(lane % LPR) * 16u;
    }
    // Every wave issues all KSW k-steps (those past nk fall outside the
    // buffer and move zeros), so each k-step below waits for a fixed count.
#pragma unroll
    for (int k = 0; k < KSW; ++k)
#pragma unroll
      for (int j = 0; j < NI; ++j)
        dma_1k(rw, wl + k * 32 * RB + j * 1024, voff[j] + (uint32_t)k * 32u * W4);
    DECODE_MARK(1);

    // Nothing above may wait for a load: the weight stream starts first.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int w = 0; w < WPL; ++w)
        if (!wok) sv[gi][w] = u32x4{0u, 0u, 0u, 0u};
    if constexpr (!FUSED) {  // rows past M multiply as zeros
#pragma unroll
      for (int k = 0; k < KSW; ++k)
        if (cl >= M) af[k] = u32x4{0u, 0u, 0u, 0u};
    }
    const NibbleMasks nm = nibble_masks<DT>();
    const u32x4 ones = {MfmaTypes<DT>::kOnes, MfmaTypes<DT>::kOnes, MfmaTypes<DT>::kOnes,
                        MfmaTypes<DT>::kOnes};
    f32x4 acc[NT];
    f32x4 xsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    static_for<0, KSW>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if (k < nk) {
        const int64_t ks = ks0 + k;
        const int64_t g = ks / 4;  // rotation block
        // quantization group of this wave: k-step k of a wave lies in its
        // group k/4 (G = 128: the wave's first k-step starts a group when it
        // owns more than two; G < 128: one k-step; one group over the row:
        // every entry holds group 0)
        constexpr int gi = k / 4;
        if constexpr (FUSED) {
          if (k == 0 || (ks % 4) == 0) {  // entering a group: rotate it into LDS
            if (k != 0) load_rot_inputs(g);
            wave_lds_sync();
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              xs[m * kDecodeRS + 2 * lane] = m < M ? xin[m][0] * cs0 : 0.0f;
              xs[m * kDecodeRS + 2 * lane + 1] = m < M ? xin[m][1] * cs1 : 0.0f;
            }
            wave_lds_sync();
            rotate_rows_lds<MT>(xs, kDecodeRS, rp, a.pairs + g * kG, I, a.theta + g * kPairs, I / 2, a.krot,
                                lane, gmask);
          }
          const float *src = xs + (cl < MT ? cl : 0) * kDecodeRS + (ks % 4) * 32 + kb * 8;
          const float4 lo = *reinterpret_cast<const float4 *>(src);
          const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
          af[k] = u32x4{pack2<DT>(lo.x, lo.y), pack2<DT>(lo.z, lo.w), pack2<DT>(hi.x, hi.y),
                        pack2<DT>(hi.z, hi.w)};
          if (cl >= M) af[k] = u32x4{0u, 0u, 0u, 0u};
        }
        // this k-step's rows have landed in LDS (later k-steps may still be in flight)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((KSW - 1 - k) * NI));
        if (k < 4) DECODE_MARK(2 + k);
        const unsigned char *wk = wl + k * 32 * RB + cl * WPL * 4;
        uint32_t rw8[WPL][8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const unsigned char *p = wk + (r * 4 + kb) * RB;
          if constexpr (WPL == 4) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
            rw8[0][r] = v[0]; rw8[1][r] = v[1]; rw8[2][r] = v[2]; rw8[3][r] = v[3];
          } else if constexpr (WPL == 2) {
            const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
            rw8[0][r] = v[0]; rw8[1][r] = v[1];
          } else {
            rw8[0][r] = *reinterpret_cast<const uint32_t *>(p);
          }
        }
        xsum = mfma16<DT>(af[k], ones, xsum);
#pragma unroll
        for (int w = 0; w < WPL; ++w) {
          u32x4 bf[8];
          build_b_frags<DT>(rw8[w], bf, nm);
#pragma unroll
          for (int s = 0; s < 8; ++s) acc[w * 8 + s] = mfma16<DT>(af[k], bf[s], acc[w * 8 + s]);
        }
        // fold at the end of a 128-row block or of this wave's k-steps (a
        // whole-row group folds once per block, the fold being linear):
        //   tot += s/c * (acc - (off + c*z) * xsum)
        if (k % 4 == 3 || k == nk - 1) {
#pragma unroll
          for (int w = 0; w < WPL; ++w) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const int col = awq_col(s);
              const uint32_t sb = (sv[gi][w][col >> 1] >> (16 * (col & 1))) & 0xffffu;
              const float c = slot_mult<DT>(s);
              const float sc = f16_bits_to_f32(sb) * (1.0f / c);
              const float zz = MfmaTypes<DT>::kOff + c * (float)((zv[gi][w] >> (4 * s)) & 0xfu);
#pragma unroll
              for (int i = 0; i < FR; ++i) tot[w * 8 + s][i] += sc * (acc[w * 8 + s][i] - zz * xsum[i]);
              if (k + 1 < KSW) acc[w * 8 + s] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
          if (k + 1 < KSW) xsum = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    });
  }

  // ---- reduce the NW waves' tiles in LDS (wave order), slot-major ----
  DECODE_MARK(6);
  __syncthreads();  // every wave is done with its weight and rotation rows
  DECODE_MARK(7);
  f32x4 *red = reinterpret_cast<f32x4 *>(smem);  // [NW][QUADS]
  if (kb < KBV) {
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        // column c of the word is nibble slot 4 * (c & 1) + c / 2
        f32x4 *dst = red + wave * QUADS + ((w * FR + i) * 2) * 16 * KBV + kb * 16 + cl;
        dst[0] = f32x4{tot[w * 8 + 0][i], tot[w * 8 + 4][i], tot[w * 8 + 1][i], tot[w * 8 + 5][i]};
        dst[16 * KBV] = f32x4{tot[w * 8 + 2][i], tot[w * 8 + 6][i], tot[w * 8 + 3][i], tot[w * 8 + 7][i]};
      }
    }
  }
  DECODE_MARK(8);
  __syncthreads();
  DECODE_MARK(9);

  // this thread's slots: sum over the waves in wave order
  f32x4 v[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int sl = threadIdx.x + j * NTH;
    v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (sl < QUADS) {
#pragma unroll
      for (int w = 0; w < NW; ++w) v[j] += red[w * QUADS + sl];
    }
  }
  DECODE_MARK(10);
  // slot j of this thread: its row and output column, and whether it is stored
  auto slot_out = [&](int j, int &row, int64_t &n) {
    const int sl = threadIdx.x + j * NTH;
    int col;
    slot_pos(sl, row, col);
    n = n0 + col;
    return sl < QUADS && row < M && n < O;
  };
  auto store_slots = [&](const f32x4 *val) {
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      int row;
      int64_t n;
      if (slot_out(j, row, n)) {
        const float o0 = val[j][0] + bias_v[j][0], o1 = val[j][1] + bias_v[j][1];
        const float o2 = val[j][2] + bias_v[j][2], o3 = val[j][3] + bias_v[j][3];
        if (a.y_dt == kF32) {
          *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.y) + row * O + n) = f32x4{o0, o1, o2, o3};
        } else {
          u32x2 h;
          if (a.y_dt == kF16) h = u32x2{pack2<kF16>(o0, o1), pack2<kF16>(o2, o3)};
          else h = u32x2{pack2<kBF16>(o0, o1), pack2<kBF16>(o2, o3)};
          *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.y) + row * O + n) = h;
        }
      }
    }
  };
  if (splits == 1) {
    store_slots(v);
    DECODE_MARK(15);
    return;
  }

  // ---- split-K handoff (see the header) ----
  // partial: [tile][split][QUADS] 16-byte slots.  One raw buffer per tile:
  // its splits * QUADS * 16 bytes (at most 2^14 * 2048 * 16 = 2^29) keep every
  // offset in 32 bits.
  constexpr uint32_t sstride = (uint32_t)QUADS * 16u;  // bytes per split
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<char *>(partial) + (int64_t)tile * splits * sstride, (short)0,
      (int)((uint32_t)splits * sstride), 0x00020000);
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    int row;
    int64_t n;
    if (slot_out(j, row, n))
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[j]), prs,
                                             (uint32_t)split * sstride + 16u * (uint32_t)(threadIdx.x + j * NTH),
                                             0, kDeviceCoherent);
  }
  DECODE_MARK(11);
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  DECODE_MARK(12);
  uint32_t *cnt = counters + (int64_t)tile * kCounterStride;
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == (uint32_t)(splits - 1));
  }
  __syncthreads();
  DECODE_MARK(13);
  if (!s_last) return;
  // Gather every split's slots, all loads of a batch in flight together (the
  // addresses of splits past the last are clamped and their values dropped,
  // unstored slots are read and not used), summing in split order.
  constexpr int SB = QPT >= 16 ? 1 : 16 / QPT;  // splits per batch
  f32x4 sum[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) sum[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < splits; sp += SB) {
    f32x4 t[QPT][SB];
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const uint32_t sl = (uint32_t)(threadIdx.x + j * NTH);
      const uint32_t off = 16u * (sl < (uint32_t)QUADS ? sl : 0u);
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const uint32_t spc = (uint32_t)(sp + u < splits ? sp + u : splits - 1);
        t[j][u] = __builtin_bit_cast(f32x4,
                                     __builtin_amdgcn_raw_buffer_load_b128(prs, off + spc * sstride, 0, kDeviceCoherent));
      }
    }
#pragma unroll
    for (int j = 0; j < QPT; ++j)
#pragma unroll
      for (int u = 0; u < SB; ++u)
        if (sp + u < splits) sum[j] += t[j][u];
  }
  DECODE_MARK(14);
  store_slots(sum);
  DECODE_MARK(15);
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

static int token_rows(int64_t tokens) {
  return tokens <= 1 ? 1 : tokens <= 2 ? 2 : tokens <= 4 ? 4 : tokens <= 8 ? 8 : 16;
}

// LDS of one workgroup: the waves' weight rows (and, fused, their rotation
// rows) during the k-steps, then the NW slot-major fp32 reduction tiles
// (MT * NTILE floats each) in the same space.
static size_t decode_lds_bytes(int wpl, int ksw, int nw, int mt, bool fused) {
  const size_t stream = (size_t)nw * decode_wave_lds(wpl, ksw) + (fused ? (size_t)nw * mt * kDecodeRS * 4 : 0);
  const size_t red = (size_t)nw * mt * 128 * wpl * 4;
  return stream > red ? stream : red;
}
constexpr size_t kDecodeMaxLds = 160 * 1024 - 256;  // the static s_last flag takes a little

DecodePlan plan_decode(int64_t I, int64_t O, int64_t tokens, bool fused, int group) {
  DecodePlan p;
  const int64_t nks = I / 32;
  if (tokens <= 4) {
    // Few rows: the fold is nearly free (one register row), so a workgroup
    // owns eight k-steps of 128-byte row segments (four waves of two: one
    // wave per SIMD measured a little faster than eight waves of one),
    // keeping the K splits (whose partials the last workgroup gathers) at
    // nks / 8 while filling the chip.
    p.wpl = (O % 16 == 0) ? 2 : 1;
    p.ksw = 2;
    p.nw = 4;
    while (p.ksw > 1 && (int64_t)p.nw * (p.ksw / 2) >= nks) p.ksw /= 2;
  } else {
    // Up to 16 rows: the partial sums cost splits * tokens * O * 8 bytes, so
    // an eight-wave workgroup covers long K ranges (several k-steps per wave,
    // folded once per group).  256-column tiles with four k-steps per wave
    // measured fastest on 4096 -> 14336 at 16 tokens (one 128-byte segment
    // per weight row and lane group, four splits).
    p.wpl = (O % 16 == 0) ? 2 : 1;
    p.nw = 8;
    p.ksw = p.wpl == 2 ? 4 : 8;
    while (p.ksw > 1 && (int64_t)p.nw * (p.ksw / 2) >= nks) p.ksw /= 2;
  }
  // Tuning overrides, read once per process: PARO_DECODE_WPL / _KSW / _NW.
  static const int fw = env_int("PARO_DECODE_WPL", 0);
  static const int fk = env_int("PARO_DECODE_KSW", 0);
  static const int fn = env_int("PARO_DECODE_NW", 0);
  if (fw == 1 || (fw == 2 && O % 16 == 0)) p.wpl = fw;
  if (fk == 1 || fk == 2 || fk == 4 || fk == 8) p.ksw = fk;
  if (fn == 2 || fn == 4 || fn == 8 || fn == 16) p.nw = fn;
  // groups of 32 or 64 rows: one k-step per wave (the kernel keeps one
  // group's scales and zeros per wave and folds every k-step)
  if (group < kG) p.ksw = 1;
  // the k-steps' weight rows (and fused rotation rows), and then the
  // reduction tiles, must fit in LDS
  while ((p.ksw > 1 || p.wpl > 1) &&
         decode_lds_bytes(p.wpl, p.ksw, p.nw, token_rows(tokens), fused) > kDecodeMaxLds) {
    if (p.ksw > 1) p.ksw /= 2;
    else p.wpl /= 2;
  }
  p.ntile = 128 * p.wpl;
  p.n_tiles = (int)((O + p.ntile - 1) / p.ntile);
  p.splits = (int)((nks + p.nw * p.ksw - 1) / (p.nw * p.ksw));
  return p;
}

size_t decode_partial_bytes(const DecodePlan &p, int64_t tokens, int64_t O) {
  (void)O;
  if (p.splits <= 1) return 0;
  // [tile][split][slots]: token_rows(tokens) rows of ntile fp32 each
  return (size_t)p.n_tiles * (size_t)p.splits * (size_t)token_rows(tokens) * (size_t)p.ntile * 4;
}

template <int DT, int WPL, int KSW, int NW, bool FUSED>
static hipError_t launch_decode_t(const LinearArgs &a, const DecodePlan &p, const void *xr, uint32_t *counters,
                                  float *partial, hipStream_t st) {
  dim3 grid((unsigned)(p.n_tiles * p.splits));
  const int M = (int)a.tokens;
  const int mt = token_rows(M);
  const size_t shmem = decode_lds_bytes(WPL, KSW, NW, mt, FUSED);
  const uint16_t *xrp = reinterpret_cast<const uint16_t *>(xr);
#define PARO_DECODE_LAUNCH(MT)                                                                                \
  hipLaunchKernelGGL((decode_kernel<DT, WPL, KSW, NW, FUSED, MT>), grid, dim3(64 * NW), shmem, st, a, xrp, p.splits, \
                     partial, counters)
  switch (mt) {
    case 1: PARO_DECODE_LAUNCH(1); break;
    case 2: PARO_DECODE_LAUNCH(2); break;
    case 4: PARO_DECODE_LAUNCH(4); break;
    case 8: PARO_DECODE_LAUNCH(8); break;
    default: PARO_DECODE_LAUNCH(16); break;
  }
#undef PARO_DECODE_LAUNCH
  return hipGetLastError();
}

template <int DT, bool FUSED>
static hipError_t launch_decode_dt(const LinearArgs &a, const DecodePlan &p, const void *xr, uint32_t *counters,
                                   float *partials, hipStream_t st) {
  // every (wpl, ksw, nw) the planner produces is instantiated; other
  // combinations (tuning overrides only) are rejected
#define PARO_DECODE_CFG(WPL, KSW, NW) \
  if (p.wpl == WPL && p.ksw == KSW && p.nw == NW) return launch_decode_t<DT, WPL, KSW, NW, FUSED>(a, p, xr, counters, partials, st)
  PARO_DECODE_CFG(2, 2, 4);
  PARO_DECODE_CFG(2, 1, 4);
  PARO_DECODE_CFG(1, 2, 4);
  PARO_DECODE_CFG(1, 1, 4);
  PARO_DECODE_CFG(2, 1, 8);
  PARO_DECODE_CFG(2, 2, 8);
  PARO_DECODE_CFG(2, 4, 8);
  PARO_DECODE_CFG(1, 1, 8);
  PARO_DECODE_CFG(1, 2, 8);
  PARO_DECODE_CFG(1, 4, 8);
  PARO_DECODE_CFG(1, 8, 8);
#undef PARO_DECODE_CFG
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const LinearArgs &a, const DecodePlan &p, const void *xr, uint32_t *counters,
                         float *partials, hipStream_t st) {
  const bool fused = (xr == nullptr);
  if (a.x_dt == kF16)
    return fused ? launch_decode_dt<kF16, true>(a, p, xr, counters, partials, st)
                 : launch_decode_dt<kF16, false>(a, p, xr, counters, partials, st);
  return fused ? launch_decode_dt<kBF16, true>(a, p, xr, counters, partials, st)
               : launch_decode_dt<kBF16, false>(a, p, xr, counters, partials, st);
}

}  // namespace paro
