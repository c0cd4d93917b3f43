// prefill_timeline.hip - per-wave timeline of the prefill GEMM (a diagnostic
// tool, not part of libparo).  Built with
//     python -m rotation_int4_weight_amd.build --prefill-timeline
// it compiles prefill.hip with PARO_PREFILL_TIMELINE, so that lane 0 of every
// wave records the 100 MHz realtime counter at the marks listed in
// prefill.hip, and runs one dense bf16 GEMM shape (group 128) on synthetic
// data through the library's launcher:
//     prefill_timeline I O tokens [sets] [launches]
// `sets` distinct weight copies are cycled (at least 512 MB of them).  It
// prints, per mark, the median across consumer (or producer) waves of the
// time since the earliest entry of the launch, averaged over the launches
// after the first tenth, and for every tile of a persistent workgroup its
// main-loop time per k step.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "prefill.hip"

#define TL_CHECK(x)                                                                          \
  do {                                                                                       \
    hipError_t e_ = (x);                                                                     \
    if (e_ != hipSuccess) {                                                                  \
      fprintf(stderr, "%s failed: %s (line %d)\n", #x, hipGetErrorString(e_), __LINE__);    \
      exit(1);                                                                               \
    }                                                                                        \
  } while (0)

int main(int argc, char **argv) {
  if (argc < 4) {
    fprintf(stderr, "usage: %s I O tokens [sets] [launches]\n", argv[0]);
    return 2;
  }
  const int64_t I = atoll(argv[1]), O = atoll(argv[2]), M = atoll(argv[3]);
  const int64_t G = 128, W = O / 8;
  if (I <= 0 || O <= 0 || I % 128 || O % 128 || M < 1) {
    fprintf(stderr, "need I %% 128 == 0, O %% 128 == 0, tokens >= 1\n");
    return 2;
  }
  const size_t qbytes = (size_t)I * W * 4;
  const int sets = argc > 4 ? atoi(argv[4]) : (int)std::max<size_t>(2, ((size_t)512 << 20) / qbytes + 1);
  const int launches = argc > 5 ? atoi(argv[5]) : 50;
  std::vector<int32_t *> qw(sets);
  for (int i = 0; i < sets; ++i) {
    TL_CHECK(hipMalloc(&qw[i], qbytes));
    TL_CHECK(hipMemset(qw[i], 0x5a, qbytes));
  }
  int32_t *qz;
  uint16_t *sc, *bias, *xt, *y;
  TL_CHECK(hipMalloc(&qz, (I / G) * W * 4));
  TL_CHECK(hipMemset(qz, 0x33, (I / G) * W * 4));
  TL_CHECK(hipMalloc(&sc, (I / G) * O * 2));
  TL_CHECK(hipMemset(sc, 0x20, (I / G) * O * 2));  // fp16 0x2020 ~ 0.008
  TL_CHECK(hipMalloc(&bias, O * 2));
  TL_CHECK(hipMemset(bias, 0, O * 2));
  const size_t xbytes = (size_t)paro::tiled_rows(M) * I * 2;
  TL_CHECK(hipMalloc(&xt, xbytes));
  TL_CHECK(hipMemset(xt, 0x3c, xbytes));  // bf16 0x3c3c ~ 0.011
  TL_CHECK(hipMalloc(&y, (size_t)M * O * 2));

  paro::LinearArgs a{};
  a.I = I;
  a.O = O;
  a.tokens = M;
  a.krot = 8;
  a.group = (int)G;
  a.qzeros = qz;
  a.scales = sc;
  a.bias = bias;
  a.x_dt = paro::kBF16;
  a.y = y;
  a.y_dt = paro::kBF16;

  // the launcher's own tile plan
  const int64_t n_tiles = (O + paro::kBN - 1) / paro::kBN;
  const int bm = paro::dense_tile_rows(M, n_tiles);
  const int64_t tiles = n_tiles * ((M + bm - 1) / bm);
  const int64_t grid = paro::persistent_grid(tiles);
  const int per_wg = (int)((tiles + grid - 1) / grid);
  printf("I=%lld O=%lld tokens=%lld: %d-row tiles, %lld tiles, %lld workgroups, up to %d tiles each, %lld k steps "
         "per tile, %d weight sets\n",
         (long long)I, (long long)O, (long long)M, bm, (long long)tiles, (long long)grid, per_wg,
         (long long)(I / 32), sets);

  const size_t waves = (size_t)grid * paro::kWaves;
  unsigned long long *tl;
  TL_CHECK(hipMalloc(&tl, waves * 48 * 8));
  TL_CHECK(hipMemcpyToSymbol(HIP_SYMBOL(paro::prefill_timeline_buf), &tl, sizeof(tl)));
  std::vector<unsigned long long> h(waves * 48);
  double avg[48] = {0};
  int cnt[48] = {0};
  const int skip = launches / 10;
  for (int i = 0; i < launches; ++i) {
    a.qweight = qw[i % sets];
    TL_CHECK(hipMemset(tl, 0, waves * 48 * 8));
    TL_CHECK(paro::launch_prefill_gemm(a, xt, 0));
    TL_CHECK(hipDeviceSynchronize());
    if (i < skip) continue;
    TL_CHECK(hipMemcpy(h.data(), tl, h.size() * 8, hipMemcpyDeviceToHost));
    unsigned long long t0 = ~0ull;
    for (size_t w = 0; w < waves; ++w)
      if (h[w * 48] && h[w * 48] < t0) t0 = h[w * 48];
    for (int e = 0; e < 48; ++e) {
      std::vector<double> v;
      for (size_t w = 0; w < waves; ++w) {
        const bool consumer = (w % paro::kWaves) < 4;
        const bool want = (e == 0 || e == 1) ? consumer : (e == 46 ? !consumer : consumer);
        if (want && h[w * 48 + e]) v.push_back((double)(h[w * 48 + e] - t0) * 0.01);
      }
      if (v.empty()) continue;
      std::sort(v.begin(), v.end());
      avg[e] += v[v.size() / 2];
      cnt[e]++;
    }
  }
  auto at = [&](int e) { return cnt[e] ? avg[e] / cnt[e] : -1.0; };
  printf("consumer waves (medians, us since the launch's first entry):\n");
  printf("  entry %.2f, pipeline primed %.2f; producers done %.2f\n", at(0), at(1), at(46));
  const int ksteps = (int)(I / 32);
  for (int it = 0; it < per_wg && it < 8; ++it) {
    const double s = at(2 + 4 * it), md = at(3 + 4 * it), dr = at(4 + 4 * it), ep = at(5 + 4 * it);
    if (s < 0) break;
    printf("  tile %d: start %.2f, main loop done %.2f (%.3f us per k step over %d), drained %.2f, "
           "epilogue stores issued %.2f\n",
           it, s, md, (md - s) / (ksteps - 4), ksteps - 4, dr, ep);
    if (it + 1 < per_wg && it + 1 < 8 && at(2 + 4 * (it + 1)) >= 0)
      printf("          -> next tile starts %.2f (%.2f us after this tile's main loop)\n", at(2 + 4 * (it + 1)),
             at(2 + 4 * (it + 1)) - md);
  }
  return 0;
}
