// decode_timeline.hip - per-wave timeline of the decode kernel (a diagnostic
// tool, not part of libparo).  Built with
//     python -m rotation_int4_weight_amd.build --decode-timeline
// it compiles decode.hip with PARO_DECODE_TIMELINE, so that lane 0 of every
// wave records the 100 MHz realtime counter at the marks listed in
// decode.hip, and runs one linear shape on synthetic weights:
//     decode_timeline I O tokens fused [sets] [launches]
// `sets` distinct weight copies are cycled so that the weights come from HBM
// (at least 256 MB of them, more than the last-level cache holds).  For each
// mark it prints, over the last launches, the median across waves of the
// time since the earliest entry of the launch (microseconds), averaged over
// launches, and the spread (p10, p90) of the last launch.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "decode.hip"

#define TL_CHECK(x)                                                                          \
  do {                                                                                       \
    hipError_t e_ = (x);                                                                     \
    if (e_ != hipSuccess) {                                                                  \
      fprintf(stderr, "%s failed: %s (line %d)\n", #x, hipGetErrorString(e_), __LINE__);    \
      exit(1);                                                                               \
    }                                                                                        \
  } while (0)

static const char *kMarkNames[16] = {
    "entry", "weight loads issued", "k-step 0 landed", "k-step 1 landed", "k-step 2 landed",
    "k-step 3 landed", "k-steps done", "reduction start", "reduction stores done", "second barrier",
    "slots summed", "partial stores issued", "partial stores complete", "counter returned",
    "gather done (finisher)", "outputs stored"};

int main(int argc, char **argv) {
  if (argc < 5) {
    fprintf(stderr, "usage: %s I O tokens fused [sets] [launches]\n", argv[0]);
    return 2;
  }
  const int64_t I = atoll(argv[1]), O = atoll(argv[2]), M = atoll(argv[3]);
  const bool fused = atoi(argv[4]) != 0;
  const int64_t G = 128, W = O / 8;
  const int krot = 8;
  if (I <= 0 || O <= 0 || I % 128 || O % 16 || M < 1 || M > 16) {
    fprintf(stderr, "need I %% 128 == 0, O %% 16 == 0, 1 <= tokens <= 16\n");
    return 2;
  }
  const size_t qbytes = (size_t)I * W * 4;
  const int sets = argc > 5 ? atoi(argv[5]) : (int)std::max<size_t>(2, ((size_t)256 << 20) / qbytes + 1);
  const int launches = argc > 6 ? atoi(argv[6]) : 200;
  std::vector<int32_t *> qw(sets);
  for (int i = 0; i < sets; ++i) {
    TL_CHECK(hipMalloc(&qw[i], qbytes));
    TL_CHECK(hipMemset(qw[i], 0x5a, qbytes));
  }
  int32_t *qz;
  uint16_t *sc, *bias, *x, *xr, *y;
  int16_t *pairs;
  float *theta, *cs;
  TL_CHECK(hipMalloc(&qz, (I / G) * W * 4));
  TL_CHECK(hipMemset(qz, 0x33, (I / G) * W * 4));
  TL_CHECK(hipMalloc(&sc, (I / G) * O * 2));
  TL_CHECK(hipMemset(sc, 0x20, (I / G) * O * 2));  // fp16 0x2020 ~ 0.008
  TL_CHECK(hipMalloc(&bias, O * 2));
  TL_CHECK(hipMemset(bias, 0, O * 2));
  TL_CHECK(hipMalloc(&x, M * I * 2));
  TL_CHECK(hipMemset(x, 0x30, M * I * 2));
  TL_CHECK(hipMalloc(&xr, M * I * 2));
  TL_CHECK(hipMemset(xr, 0x30, M * I * 2));
  TL_CHECK(hipMalloc(&y, M * O * 4));
  // identity pairing (2p, 2p+1) at every stage, zero angles, unit scales
  std::vector<int16_t> hp((size_t)krot * I);
  for (int t = 0; t < krot; ++t)
    for (int64_t c = 0; c < I; ++c) hp[(size_t)t * I + c] = (int16_t)(c % 128);
  std::vector<float> ones(I, 1.0f);
  TL_CHECK(hipMalloc(&pairs, (size_t)krot * I * 2));
  TL_CHECK(hipMemcpy(pairs, hp.data(), (size_t)krot * I * 2, hipMemcpyHostToDevice));
  TL_CHECK(hipMalloc(&theta, (size_t)krot * I / 2 * 4));
  TL_CHECK(hipMemset(theta, 0, (size_t)krot * I / 2 * 4));
  TL_CHECK(hipMalloc(&cs, I * 4));
  TL_CHECK(hipMemcpy(cs, ones.data(), I * 4, hipMemcpyHostToDevice));

  const paro::DecodePlan p = paro::plan_decode(I, O, M, fused, (int)G);
  printf("I=%lld O=%lld tokens=%lld %s: wpl=%d ksw=%d nw=%d ntile=%d tiles=%d splits=%d, %d weight sets\n",
         (long long)I, (long long)O, (long long)M, fused ? "fused" : "split", p.wpl, p.ksw, p.nw, p.ntile,
         p.n_tiles, p.splits, sets);
  uint32_t *counters;
  float *partials;
  TL_CHECK(hipMalloc(&counters, (size_t)p.n_tiles * 128 + 256));
  TL_CHECK(hipMemset(counters, 0, (size_t)p.n_tiles * 128 + 256));
  TL_CHECK(hipMalloc(&partials, paro::decode_partial_bytes(p, M, O) + 256));
  paro::LinearArgs a{};
  a.I = I;
  a.O = O;
  a.tokens = M;
  a.krot = krot;
  a.group = (int)G;
  a.pairs = pairs;
  a.theta = theta;
  a.cs = cs;
  a.qzeros = qz;
  a.scales = sc;
  a.bias = bias;
  a.x = x;
  a.x_dt = paro::kF16;
  a.y = y;
  a.y_dt = paro::kF16;

  const size_t waves = (size_t)p.n_tiles * p.splits * p.nw;
  unsigned long long *tl;
  TL_CHECK(hipMalloc(&tl, waves * 16 * 8));
  TL_CHECK(hipMemcpyToSymbol(HIP_SYMBOL(paro::decode_timeline_buf), &tl, sizeof(tl)));
  std::vector<unsigned long long> h(waves * 16);
  double avg[16] = {0};
  int cnt[16] = {0};
  std::vector<double> last[16];
  const int skip = launches / 10;
  for (int i = 0; i < launches; ++i) {
    a.qweight = qw[i % sets];
    TL_CHECK(hipMemset(tl, 0, waves * 16 * 8));
    TL_CHECK(paro::launch_decode(a, p, fused ? nullptr : xr, counters, partials, 0));
    TL_CHECK(hipDeviceSynchronize());
    if (i < skip) continue;
    TL_CHECK(hipMemcpy(h.data(), tl, h.size() * 8, hipMemcpyDeviceToHost));
    unsigned long long t0 = ~0ull;
    for (size_t w = 0; w < waves; ++w)
      if (h[w * 16] && h[w * 16] < t0) t0 = h[w * 16];
    for (int e = 0; e < 16; ++e) {
      std::vector<double> v;
      for (size_t w = 0; w < waves; ++w)
        if (h[w * 16 + e]) v.push_back((double)(h[w * 16 + e] - t0) * 0.01);
      if (v.empty()) continue;
      std::sort(v.begin(), v.end());
      avg[e] += v[v.size() / 2];
      cnt[e]++;
      if (i == launches - 1) last[e] = v;
    }
  }
  printf("%-2s %-26s %7s   %s\n", "", "mark", "median", "last launch: waves, p10 / p90 (us)");
  for (int e = 0; e < 16; ++e) {
    if (!cnt[e]) continue;
    const std::vector<double> &v = last[e];
    if (v.empty()) continue;
    printf("%2d %-26s %7.2f   %6zu, %6.2f / %6.2f\n", e, kMarkNames[e], avg[e] / cnt[e], v.size(),
           v[v.size() / 10], v[9 * v.size() / 10]);
  }
  return 0;
}
