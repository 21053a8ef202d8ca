// Drives every host-side path of libtq (codebooks, rotations, sketch, tables,
// sizes, argument validation of every entry point) in a build instrumented
// with AddressSanitizer and UndefinedBehaviorSanitizer.  Device pointers are
// fake addresses: validation never dereferences them and the stub launches
// never run.  Exit status 0 and the line "host sanitizer driver ok" mean no
// check failed and no sanitizer report was raised (reports abort).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "tq.h"

static int g_fail = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
  // codebooks
  for (int d : {3, 8, 128, 1000}) {
    for (int bits = 1; bits <= 8; ++bits) {
      std::vector<double> c(1u << bits), t((1u << bits) - 1);
      CHECK(tq_codebook_build(d, bits, c.data(), t.data()) == TQ_OK);
      for (size_t i = 1; i < c.size(); ++i) CHECK(c[i] > c[i - 1]);
      for (size_t i = 0; i < t.size(); ++i) CHECK(std::fabs(t[i] - 0.5 * (c[i] + c[i + 1])) < 1e-15);
      CHECK(std::fabs(c.front() + c.back()) < 1e-12);
    }
  }
  CHECK(tq_codebook_build(2, 4, nullptr, nullptr) != TQ_OK);
  CHECK(tq_codebook_build(128, 9, nullptr, nullptr) != TQ_OK);
  CHECK(std::strlen(tq_last_error()) > 0);
  // rotations and sketch
  std::vector<double> pi(128 * 128), s(128 * 128);
  for (uint64_t seed : {0ull, 1ull, 12345ull}) {
    CHECK(tq_rotation_build(128, seed, pi.data()) == TQ_OK);
    double e = 0.0;
    for (int i = 0; i < 128; ++i)
      for (int j = 0; j < 128; ++j) {
        double a = 0.0;
        for (int k = 0; k < 128; ++k) a += pi[i * 128 + k] * pi[j * 128 + k];
        e = std::fmax(e, std::fabs(a - (i == j)));
      }
    CHECK(e < 1e-12);
    CHECK(tq_hadamard_rotation_build(128, seed, pi.data()) == TQ_OK);
    CHECK(tq_sketch_build(128, 128, seed, s.data()) == TQ_OK);
  }
  CHECK(tq_rotation_build(0, 0, pi.data()) != TQ_OK);
  CHECK(tq_hadamard_rotation_build(100, 0, pi.data()) != TQ_OK);
  CHECK(tq_sketch_build(0, 128, 0, s.data()) != TQ_OK);
  // tables for every spec the kernels take
  const size_t tb = tq_tables_bytes();
  CHECK(tb > 0);
  void* tab = std::aligned_alloc(256, (tb + 255) / 256 * 256);
  struct W { int lo, hi, split; } widths[] = {{2, 2, 128}, {3, 3, 128}, {4, 4, 128}, {4, 3, 64}, {3, 2, 64}, {8, 8, 128}};
  int n_ok = 0;
  for (const W& w : widths)
    for (int layout : {TQ_LAYOUT_RECORD, TQ_LAYOUT_TILED})
      for (int qjl : {0, TQ_QJL_M})
        for (int rot : {TQ_ROT_HAAR, TQ_ROT_HADAMARD, TQ_ROT_HADAMARD_FWHT})
          for (int nf : {0, 1}) {
            tq_spec sp{TQ_DIM, w.lo, w.hi, w.split, qjl, layout, 0, 1, rot, nf};
            const tq_status st = tq_tables_build(&sp, tab, tb);
            if (st == TQ_OK) {
              ++n_ok;
              CHECK(tq_code_bytes(&sp) == static_cast<size_t>(8 * (w.lo + w.hi)));
              CHECK(tq_cache_code_bytes(&sp, 96) > 0);
            } else {
              CHECK(std::strlen(tq_last_error()) > 0);
            }
          }
  CHECK(n_ok >= 60);
  tq_spec bad{TQ_DIM, 5, 5, 128, 0, 0, 0, 1, 0, 0};
  CHECK(tq_tables_build(&bad, tab, tb) != TQ_OK);
  CHECK(tq_tables_build(nullptr, tab, tb) != TQ_OK);

  // quantize entry points: validation, then a stub launch (TQ_E_HIP)
  tq_spec k4{TQ_DIM, 4, 4, 128, 0, TQ_LAYOUT_RECORD, 0, 1, 0, 0};
  CHECK(tq_tables_build(&k4, tab, tb) == TQ_OK);
  tq_cache kc{static_cast<uint8_t*>(fake(0x100000)), static_cast<float*>(fake(0x200000)), nullptr, nullptr, 128};
  CHECK(tq_quantize_kv(&k4, tab, TQ_BF16, fake(0x300000), 2, 100, 128 * 128, 128, 0, &kc, nullptr) == TQ_E_HIP);
  CHECK(tq_quantize_kv(&k4, tab, TQ_BF16, fake(0x300000), 2, 100, 128 * 128, 128, 40, &kc, nullptr) == TQ_E_ARG);
  CHECK(tq_quantize_kv(&k4, tab, 7, fake(0x300000), 2, 10, 128 * 128, 128, 0, &kc, nullptr) != TQ_OK);
  CHECK(tq_quantize_kv(&k4, tab, TQ_BF16, fake(0x300000), 0, 10, 0, 128, 0, &kc, nullptr) == TQ_OK);
  std::vector<int64_t> xo = {0, 128 * 128 * 64}, t0 = {0, 5}, nt = {100, 20};
  CHECK(tq_quantize_kv_ragged(&k4, tab, TQ_BF16, fake(0x300000), 2, 4, xo.data(), t0.data(), nt.data(), 128 * 128,
                              128, &kc, nullptr) == TQ_E_HIP);
  nt[1] = 200;
  CHECK(tq_quantize_kv_ragged(&k4, tab, TQ_BF16, fake(0x300000), 2, 4, xo.data(), t0.data(), nt.data(), 128 * 128,
                              128, &kc, nullptr) == TQ_E_ARG);
  tq_cache pool{static_cast<uint8_t*>(fake(0x100000)), static_cast<float*>(fake(0x200000)), nullptr, nullptr,
                TQ_PAGE_TOKENS};
  nt[1] = 20;
  CHECK(tq_quantize_kv_paged(&k4, tab, TQ_BF16, fake(0x300000), 2, 4, xo.data(), t0.data(), nt.data(), 128 * 128,
                             128, static_cast<const int32_t*>(fake(0x400000)), 4, 16, &pool, nullptr) == TQ_E_HIP);
  CHECK(tq_quantize_kv_paged(&k4, tab, TQ_BF16, fake(0x300000), 2, 4, xo.data(), t0.data(), nt.data(), 128 * 128,
                             128, nullptr, 4, 16, &pool, nullptr) == TQ_E_ARG);

  // decode: validation, plan, stub launch
  tq_spec v3{TQ_DIM, 3, 3, 128, 0, TQ_LAYOUT_TILED, 0, 1, 0, 0};
  void* vtab = std::aligned_alloc(256, (tb + 255) / 256 * 256);
  CHECK(tq_tables_build(&v3, vtab, tb) == TQ_OK);
  tq_cache vc{static_cast<uint8_t*>(fake(0x500000)), static_cast<float*>(fake(0x600000)), nullptr, nullptr, 128};
  for (int sink : {0, 16}) {
    tq_attn a{2, 32, 8, sink, 0.0883883f, sink ? 1e-6f : 0.0f, 128 + sink};
    const size_t ws = tq_attend_workspace_bytes(&a);
    CHECK(ws > 0);
    CHECK(tq_attend_decode(&k4, tab, &kc, &v3, vtab, &vc, &a, static_cast<const float*>(fake(0x700000)),
                           static_cast<const uint16_t*>(fake(0x710000)), static_cast<const uint16_t*>(fake(0x720000)),
                           static_cast<const int32_t*>(fake(0x730000)), static_cast<float*>(fake(0x740000)),
                           fake(0x800000), ws, nullptr) == TQ_E_HIP);
    CHECK(tq_attend_decode(&k4, tab, &kc, &v3, vtab, &vc, &a, static_cast<const float*>(fake(0x700000)),
                           static_cast<const uint16_t*>(fake(0x710000)), static_cast<const uint16_t*>(fake(0x720000)),
                           static_cast<const int32_t*>(fake(0x730000)), static_cast<float*>(fake(0x740000)),
                           fake(0x800000), ws - 4, nullptr) == TQ_E_WORKSPACE);
  }
  for (int64_t max_len : {0ll, 31ll, 32ll, 4096ll}) {
    tq_attn a{64, 32, 8, 0, 0.1f, 0.0f, max_len};
    CHECK(tq_attend_workspace_bytes(&a) > 0 || max_len == 0);
  }
  tq_attn bad_a{1, 6, 4, 0, 0.1f, 0.0f, 64};
  CHECK(tq_attend_decode(&k4, tab, &kc, &v3, vtab, &vc, &bad_a, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         0, nullptr) == TQ_E_ARG);
  tq_attn pa{2, 32, 8, 0, 0.1f, 0.0f, 256};
  CHECK(tq_attend_decode_paged(&k4, tab, &pool, &v3, vtab, &pool, &pa, static_cast<const float*>(fake(0x700000)),
                               nullptr, nullptr, static_cast<const int32_t*>(fake(0x730000)),
                               static_cast<const int32_t*>(fake(0x400000)), 4, 16,
                               static_cast<float*>(fake(0x740000)), fake(0x800000), 1 << 24, nullptr) == TQ_E_HIP);

  // search
  tq_spec s2{TQ_DIM, 2, 2, 128, TQ_QJL_M, TQ_LAYOUT_RECORD, 0, 1, 0, 0};
  CHECK(tq_tables_build(&s2, tab, tb) == TQ_OK);
  tq_cache db{static_cast<uint8_t*>(fake(0x100000)), static_cast<float*>(fake(0x200000)),
              static_cast<uint8_t*>(fake(0x900000)), static_cast<float*>(fake(0xA00000)), 256};
  const size_t iw = tq_ip_workspace_bytes();
  CHECK(tq_ip_scores(&s2, tab, &db, 4, 256, static_cast<const float*>(fake(0x700000)), 37,
                     static_cast<float*>(fake(0xB00000)), 4 * 256, fake(0x800000), iw, nullptr) == TQ_E_HIP);
  CHECK(tq_ip_scores(&s2, tab, &db, 4, 256, static_cast<const float*>(fake(0x700000)), 65,
                     static_cast<float*>(fake(0xB00000)), 4 * 256, fake(0x800000), iw, nullptr) != TQ_OK);
  CHECK(tq_format_version() == TQ_FORMAT_VERSION);

  std::free(tab);
  std::free(vtab);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host sanitizer driver ok\n");
  return 0;
}
