// Host-logic driver for the sanitizer build: drives every entry point of tgemm.h with
// directed and pseudo-random arguments (fake device addresses, never dereferenced) and
// checks, for each call, the return code against the argument rules the header states and
// each recorded launch against the arguments (sizes, strides, tile counts, config fitness,
// split-K workspace). Any out-of-bounds access, overflow or other undefined behaviour in
// the host logic stops the run under the sanitizers. Prints the config tables first (the
// test compares them with the library's) and "host logic ok" at the end.
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "stubs.h"
#include "tgemm.h"

namespace {

long checks = 0;

#define CHECK(cond, ...)                                                        \
  do {                                                                          \
    ++checks;                                                                   \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond);     \
      std::fprintf(stderr, __VA_ARGS__);                                        \
      std::fprintf(stderr, "\n");                                               \
      std::exit(1);                                                             \
    }                                                                           \
  } while (0)

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}
int64_t pick(const int64_t* v, int n) { return v[next() % (uint64_t)n]; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
const int64_t kMaxDim = (int64_t)1 << 31;

struct Cfg {
  tgemm_config_info info;
};
Cfg cfgs[64];
int ncfg = 0;
Cfg fp8cfgs[16];
int nfp8 = 0;

void load_tables() {
  ncfg = tgemm_num_configs();
  CHECK(ncfg > 1 && ncfg <= 64, "ncfg %d", ncfg);
  for (int i = 0; i < ncfg; ++i) CHECK(tgemm_config_desc(i, &cfgs[i].info) == TGEMM_OK, "desc %d", i);
  nfp8 = tgemm_fp8_num_configs();
  CHECK(nfp8 > 0 && nfp8 <= 16, "nfp8 %d", nfp8);
  for (int i = 0; i < nfp8; ++i) CHECK(tgemm_fp8_config_desc(i, &fp8cfgs[i].info) == TGEMM_OK, "fp8 desc %d", i);
  for (int i = 0; i < ncfg; ++i) {
    const tgemm_config_info& c = cfgs[i].info;
    std::printf("cfg %d %d %d %d %d %d %d %d %d %d %d %d %d %s\n", i, c.block_m, c.block_n, c.block_k, c.stages,
                c.waves_m, c.waves_n, c.panel, c.xcd_remap, c.generic, c.layouts, c.built, c.lds_bytes, c.name);
  }
  for (int i = 0; i < nfp8; ++i) {
    const tgemm_config_info& c = fp8cfgs[i].info;
    std::printf("fp8 %d %d %d %d %d %d %d %d %d %d %s\n", i, c.block_m, c.block_n, c.block_k, c.stages, c.waves_m,
                c.waves_n, c.panel, c.xcd_remap, c.built, c.name);
  }
}

// ------------------------------------------------------------------ the header's rules
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// gemm_f16_ex's argument checks, in the order the header lists the codes.
int expect_args(int ta, int tb, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                int64_t ldb, const void* C, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return TGEMM_EINVAL_DIM;
  const int64_t one = 1;
  const int64_t amin = std::max(one, ta ? M : K), bmin = std::max(one, tb ? K : N), cmin = std::max(one, N);
  if (lda < amin || ldb < bmin || ldc < cmin) return TGEMM_EINVAL_LD;
  if (M > 0 && N > 0 && C == nullptr) return TGEMM_ENULL;
  if (M > 0 && N > 0 && K > 0 && (A == nullptr || B == nullptr)) return TGEMM_ENULL;
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 1u) return TGEMM_EALIGN;
  return TGEMM_OK;
}

bool fast_ok(int ta, int tb, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
             int64_t ldb, const void* C, int64_t ldc) {
  return al16(A) && al16(B) && al16(C) && lda % 8 == 0 && ldb % 8 == 0 && ldc % 8 == 0 && (ta ? M : K) % 8 == 0 &&
         (tb ? K : N) % 8 == 0 && N % 8 == 0 && lda <= TGEMM_FAST_MAX_LD && ldb <= TGEMM_FAST_MAX_LD;
}

// One recorded GEMM launch against the call's arguments.
void check_gemm_launch(const stub::Launch& l, int ta, int tb, int64_t M, int64_t N, int64_t K, const void* A,
                       int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc, int relu) {
  CHECK(l.kind == stub::kGemm, "kind %d", l.kind);
  CHECK(l.cfg >= 0 && l.cfg < ncfg, "cfg %d", l.cfg);
  const tgemm_config_info& c = cfgs[l.cfg].info;
  const tgemm::GemmArgs& g = l.gemm;
  const int layout = 2 * ta + tb;
  CHECK(c.built == 1, "launch of a config this build does not compile: %d", l.cfg);
  CHECK((c.layouts >> layout) & 1, "cfg %d does not take layout %d", l.cfg, layout);
  CHECK(g.A == A && g.B == B && g.C == C && g.lda == lda && g.ldb == ldb && g.ldc == ldc, "pointers/strides");
  CHECK(g.M == M && g.N == N && g.K == K && g.layout == layout && g.relu == (relu != 0), "sizes");
  CHECK(g.tiles_m == cdiv(M, c.block_m) && g.tiles_n == cdiv(N, c.block_n), "tiles %d %d", g.tiles_m, g.tiles_n);
  CHECK(g.splits >= 1 && g.splits <= 8, "splits %d", g.splits);
  CHECK((int64_t)g.tiles_m * g.tiles_n * g.splits < kMaxDim, "grid");
  if (!c.generic) CHECK(fast_ok(ta, tb, M, N, K, A, lda, B, ldb, C, ldc), "fast config on ineligible arguments");
  if (g.splits > 1) {
    CHECK(!c.generic && c.layouts == 0xF, "split on cfg %d", l.cfg);
    CHECK(g.ws != nullptr && ((uintptr_t)g.ws & 255u) == 0 && g.ws_parts == 4096, "workspace");
    CHECK(g.splits <= cdiv(K, c.block_k), "more splits than k-tiles");
    CHECK((int64_t)g.tiles_m * g.tiles_n <= 1024, "split tiles");
  }
}

// ------------------------------------------------------------------ argument generators
const int64_t kDims[] = {0, 1, 7, 8, 15, 16, 17, 64, 127, 128, 129, 200, 255, 256, 257, 1000, 1024, 3000, 4095,
                         4096, 8192, 16384, 32768, 65536, 1 << 20, (int64_t)1 << 30, kMaxDim - 1, kMaxDim, -1};
const int64_t kSmallDims[] = {0, 1, 8, 16, 17, 24, 64, 65, 128, 136, 200, 256, 264, 520, 1000, 1024, 4096};

int64_t gen_dim(bool small) {
  if (small) return pick(kSmallDims, sizeof kSmallDims / sizeof kSmallDims[0]);
  return pick(kDims, sizeof kDims / sizeof kDims[0]);
}
// A leading dimension near the minimum, padded, at the fast limit, or far beyond it.
int64_t gen_ld(int64_t min) {
  const int64_t m = min < 1 ? 1 : min;
  switch (next() % 9) {
    case 0: return m;
    case 1: return m + 8;
    case 2: return (m + 7) / 8 * 8;
    case 3: return m - 1;
    case 4: return TGEMM_FAST_MAX_LD;
    case 5: return TGEMM_FAST_MAX_LD + 8;
    case 6: return (int64_t)1 << 40;
    case 7: return m + (int64_t)(next() % 64);
    default: return (m + 255) / 256 * 256;
  }
}
const void* gen_ptr(int which) {
  const uintptr_t base = (uintptr_t)0x100000000ull * (uintptr_t)(which + 1);
  switch (next() % 12) {
    case 0: return nullptr;
    case 1: return (const void*)(base + 2);
    case 2: return (const void*)(base + 8);
    case 3: return (const void*)(base + 1);
    case 4: return (const void*)(base + 4);
    default: return (const void*)base;
  }
}

// A forced config may refuse arguments its kernel does not take, or a grid of 2^31 or
// more of its own (smaller) tiles.
bool want_forced_ok(int rc, int want) {
  return (want == TGEMM_OK || want == TGEMM_EINVAL_DIM) && (rc == TGEMM_EINVAL_CFG || rc == TGEMM_EINVAL_DIM);
}

// ------------------------------------------------------------------ fp16 entry points
void fuzz_f16(int iters) {
  for (int it = 0; it < iters; ++it) {
    const bool small = next() % 3 != 0;
    const int ta = (int)(next() % 2), tb = (int)(next() % 2);
    const int64_t M = gen_dim(small), N = gen_dim(small), K = gen_dim(small);
    const int64_t lda = gen_ld(ta ? M : K), ldb = gen_ld(tb ? K : N), ldc = gen_ld(N);
    const void* A = gen_ptr(0);
    const void* B = gen_ptr(1);
    void* C = const_cast<void*>(gen_ptr(2));
    const int relu = (int)(next() % 2);
    int want = expect_args(ta, tb, M, N, K, A, lda, B, ldb, C, ldc);
    const bool nonempty = M > 0 && N > 0;
    if (want == TGEMM_OK && nonempty && K > 0) {  // one launch holds fewer than 2^31 workgroups
      const int sel = tgemm_select_config_ex(ta, tb, M, N, K, A, lda, B, ldb, C, ldc);
      CHECK(sel >= 0 && sel < ncfg, "select %d", sel);
      if (tgemm_num_workgroups(sel, M, N) >= kMaxDim) want = TGEMM_EINVAL_DIM;
    }

    // gemm_f16_ex
    stub::launches.clear();
    int rc = gemm_f16_ex(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, nullptr);
    CHECK(rc == want, "gemm_f16_ex rc %d want %d (%d%d %" PRId64 "x%" PRId64 "x%" PRId64 ")", rc, want, ta, tb, M,
          N, K);
    if (rc != TGEMM_OK || !nonempty) {
      CHECK(stub::launches.empty(), "launch after an error or for an empty output");
    } else if (K == 0) {
      CHECK(stub::launches.size() == 1 && stub::launches[0].kind == stub::kZeroFill, "zero fill");
      CHECK(stub::launches[0].zf_M == M && stub::launches[0].zf_N == N && stub::launches[0].zf_ldc == ldc, "zf");
    } else {
      CHECK(stub::launches.size() == 1, "one launch");
      check_gemm_launch(stub::launches[0], ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu);
      const int sel = tgemm_select_config_ex(ta, tb, M, N, K, A, lda, B, ldb, C, ldc);
      CHECK(sel == stub::launches[0].cfg, "select %d launched %d", sel, stub::launches[0].cfg);
      CHECK(cfgs[sel].info.generic == !fast_ok(ta, tb, M, N, K, A, lda, B, ldb, C, ldc), "generic iff ineligible");
    }

    // gemm_f16_ex_cfg on a random row
    const int idx = (int)(next() % (uint64_t)(ncfg + 2)) - 1;
    stub::launches.clear();
    rc = gemm_f16_ex_cfg(idx, ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, nullptr);
    if (idx < 0 || idx >= ncfg) {
      CHECK(rc == TGEMM_EINVAL_CFG, "cfg out of range rc %d", rc);
    } else if (rc == TGEMM_OK && nonempty && K > 0) {
      CHECK(stub::launches.size() == 1 && stub::launches[0].cfg == idx, "forced cfg");
      check_gemm_launch(stub::launches[0], ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu);
    } else if (rc != TGEMM_OK) {
      CHECK(stub::launches.empty(), "launch after an error");
      CHECK(rc == want || (want_forced_ok(rc, want)), "forced cfg rc %d want %d", rc, want);
    }

    // split-K: plan, workspace size, the managed-workspace and static-scratch entry points
    int pcfg = -1, psplits = -1;
    int64_t pws = -1;
    rc = tgemm_split_plan(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, &pcfg, &psplits, &pws);
    const int want_args = expect_args(ta, tb, M, N, K, A, lda, B, ldb, C, ldc);
    CHECK(rc == want_args, "split_plan rc %d want %d", rc, want_args);
    if (rc == TGEMM_OK && want == TGEMM_OK && nonempty && K > 0) {
      CHECK(pcfg >= 0 && pcfg < ncfg && psplits >= 1 && psplits <= 8 && pws >= 0, "plan");
      CHECK((psplits == 1) == (pws == 0), "workspace iff split");
      if (psplits > 1) {
        const int64_t w = tgemm_workspace_bytes_cfg(pcfg, psplits, M, N);
        CHECK(w == pws, "workspace_bytes_cfg %" PRId64 " plan %" PRId64, w, pws);
      }
      const uintptr_t ws = (uintptr_t)0x7e0000000000ull;
      stub::launches.clear();
      rc = gemm_f16_ws(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, (void*)ws, pws, nullptr);
      CHECK(rc == TGEMM_OK, "gemm_f16_ws rc %d", rc);
      CHECK(stub::launches.size() == 1, "ws launch");
      check_gemm_launch(stub::launches[0], ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu);
      CHECK(stub::launches[0].gemm.splits == psplits && stub::launches[0].cfg == pcfg, "ws follows the plan");
      if (psplits > 1) {
        CHECK(stub::launches[0].gemm.ws == (void*)ws, "ws pointer");
        CHECK(gemm_f16_ws(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, (void*)ws, pws - 1, nullptr) ==
                  TGEMM_EWORKSPACE, "short workspace");
        CHECK(gemm_f16_ws(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, nullptr, pws, nullptr) == TGEMM_ENULL,
              "null workspace");
        CHECK(gemm_f16_ws(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, (void*)(ws + 128), pws, nullptr) ==
                  TGEMM_EALIGN, "workspace alignment");
      }
      stub::launches.clear();
      rc = gemm_f16_ws_static(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, nullptr);
      if (pws <= TGEMM_STATIC_SCRATCH_BYTES) {
        CHECK(rc == TGEMM_OK && stub::launches.size() == 1, "static rc %d", rc);
        check_gemm_launch(stub::launches[0], ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu);
        CHECK(stub::launches[0].gemm.splits == psplits, "static follows the plan");
      } else {
        CHECK(rc == TGEMM_EWORKSPACE && stub::launches.empty(), "static over the limit rc %d", rc);
      }
    }

    // forced split counts
    const int sidx = (int)(next() % (uint64_t)ncfg), ssp = 1 + (int)(next() % 9);
    const int64_t need = tgemm_workspace_bytes_cfg(sidx, ssp, M, N);
    stub::launches.clear();
    rc = gemm_f16_ws_cfg(sidx, ssp, ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, (void*)0x7e0000000000ull,
                         need > 0 ? need : 0, nullptr);
    if (rc == TGEMM_OK && nonempty && K > 0) {
      CHECK(stub::launches.size() == 1 && stub::launches[0].cfg == sidx, "ws_cfg launch");
      check_gemm_launch(stub::launches[0], ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu);
      CHECK(stub::launches[0].gemm.splits == ssp, "forced splits");
    } else if (rc != TGEMM_OK) {
      CHECK(stub::launches.empty(), "launch after an error");
    }

    // tile map of the selected config covers the grid once
    if (rc == TGEMM_OK && M > 0 && N > 0 && M <= 4096 && N <= 4096) {
      const int c0 = (int)(next() % (uint64_t)ncfg);
      const int64_t nwg = tgemm_num_workgroups(c0, M, N);
      CHECK(nwg == cdiv(M, cfgs[c0].info.block_m) * cdiv(N, cfgs[c0].info.block_n), "num_workgroups");
      if (nwg <= 4096) {
        static uint8_t seen[4096];
        std::memset(seen, 0, sizeof seen);
        const int64_t tn = cdiv(N, cfgs[c0].info.block_n);
        for (int64_t wg = 0; wg < nwg; ++wg) {
          int64_t a = -1, b = -1;
          CHECK(tgemm_tile_of(c0, M, N, wg, &a, &b) == TGEMM_OK, "tile_of");
          CHECK(a >= 0 && b >= 0 && a * tn + b < nwg && !seen[a * tn + b], "tile map not a bijection");
          seen[a * tn + b] = 1;
        }
        int64_t a, b;
        CHECK(tgemm_tile_of(c0, M, N, nwg, &a, &b) == TGEMM_EINVAL_DIM, "tile_of past the grid");
      }
      // the split-K map covers every (tile, split) once; splits = 1 is tile_of's map
      const int sp = 1 + (int)(next() % 8);
      int64_t a0, b0;
      int s0;
      const int src = tgemm_split_tile_of(c0, M, N, sp, 0, &a0, &b0, &s0);
      CHECK(src == TGEMM_OK || (sp > 1 && src == TGEMM_EINVAL_CFG), "split_tile_of rc");
      if (src == TGEMM_OK && nwg * sp <= 4096) {
        static uint8_t seen[4096];
        std::memset(seen, 0, sizeof seen);
        const int64_t tn = cdiv(N, cfgs[c0].info.block_n);
        for (int64_t wg = 0; wg < nwg * sp; ++wg) {
          int64_t a = -1, b = -1, a1 = -1, b1 = -1;
          int s = -1;
          CHECK(tgemm_split_tile_of(c0, M, N, sp, wg, &a, &b, &s) == TGEMM_OK, "split_tile_of");
          const int64_t cell = (a * tn + b) * sp + s;
          CHECK(a >= 0 && b >= 0 && s >= 0 && s < sp && cell < nwg * sp && !seen[cell], "split map not a bijection");
          seen[cell] = 1;
          if (sp == 1) {
            CHECK(tgemm_tile_of(c0, M, N, wg, &a1, &b1) == TGEMM_OK && a1 == a && b1 == b, "split map at 1 split");
          }
        }
        CHECK(tgemm_split_tile_of(c0, M, N, sp, nwg * sp, &a0, &b0, &s0) == TGEMM_EINVAL_DIM, "split map past the grid");
      }
      CHECK(tgemm_split_tile_of(c0, M, N, 9, 0, &a0, &b0, &s0) == TGEMM_EINVAL_CFG, "split_tile_of splits > 8");
      CHECK(tgemm_split_tile_of(c0, M, N, 1, 0, &a0, &b0, nullptr) == TGEMM_ENULL, "split_tile_of null");
    }
  }
}

void fuzz_grouped(int iters) {
  for (int it = 0; it < iters; ++it) {
    const int ta = (int)(next() % 2), tb = (int)(next() % 2);
    const int count = (int)(next() % 40);
    tgemm_gemm_desc d[40];
    int want = TGEMM_OK;
    for (int i = 0; i < count; ++i) {
      d[i].M = gen_dim(true);
      d[i].N = gen_dim(true);
      d[i].K = gen_dim(true);
      d[i].A = gen_ptr(0);
      d[i].B = gen_ptr(1);
      d[i].C = const_cast<void*>(gen_ptr(2));
      d[i].lda = gen_ld(ta ? d[i].M : d[i].K);
      d[i].ldb = gen_ld(tb ? d[i].K : d[i].N);
      d[i].ldc = gen_ld(d[i].N);
      const int e = expect_args(ta, tb, d[i].M, d[i].N, d[i].K, d[i].A, d[i].lda, d[i].B, d[i].ldb, d[i].C,
                                d[i].ldc);
      if (want == TGEMM_OK) want = e;
    }
    stub::launches.clear();
    const int rc = gemm_f16_grouped(ta, tb, count, count ? d : nullptr, 1, nullptr);
    CHECK(rc == want, "grouped rc %d want %d", rc, want);
    if (rc != TGEMM_OK) {
      CHECK(stub::launches.empty(), "grouped launch after an error");
      continue;
    }
    // every non-empty member is computed exactly once: in a grouped launch or on its own
    int covered[40] = {0};
    for (const stub::Launch& l : stub::launches) {
      if (l.kind == stub::kGrouped) {
        const tgemm::GroupedArgs& ga = l.grouped;
        CHECK(ga.count >= 1 && ga.count <= tgemm::kMaxGroups, "group count %d", ga.count);
        CHECK(ga.wg_start[0] == 0 && ga.wg_start[ga.count] == l.nwg && l.nwg < kMaxDim, "group span");
        for (int g = 0; g < ga.count; ++g) {
          const tgemm::GroupEntry& e = ga.e[g];
          CHECK(e.tiles_m == cdiv(e.M, l.cfg) && e.tiles_n == cdiv(e.N, l.cfg), "group tiles");
          CHECK(ga.wg_start[g + 1] - ga.wg_start[g] == e.tiles_m * e.tiles_n, "group ranges");
          int hit = -1;
          for (int i = 0; i < count && hit < 0; ++i)
            if (!covered[i] && d[i].A == e.A && d[i].B == e.B && d[i].C == e.C && d[i].M == e.M && d[i].N == e.N &&
                d[i].K == e.K && d[i].lda == e.lda && d[i].ldb == e.ldb && d[i].ldc == e.ldc)
              hit = i;
          CHECK(hit >= 0, "group entry matches no member");
          CHECK(fast_ok(ta, tb, e.M, e.N, e.K, e.A, e.lda, e.B, e.ldb, e.C, e.ldc) && e.K > 0, "group fitness");
          covered[hit] = 1;
        }
      } else {
        int hit = -1;
        for (int i = 0; i < count && hit < 0; ++i) {
          if (covered[i]) continue;
          if (l.kind == stub::kZeroFill && d[i].C == l.zf_C && d[i].M == l.zf_M && d[i].N == l.zf_N && d[i].K == 0)
            hit = i;
          if (l.kind == stub::kGemm && d[i].C == l.gemm.C && d[i].M == l.gemm.M && d[i].N == l.gemm.N &&
              d[i].K == l.gemm.K && d[i].A == l.gemm.A)
            hit = i;
        }
        CHECK(hit >= 0, "single launch matches no member");
        if (l.kind == stub::kGemm)
          check_gemm_launch(l, ta, tb, d[hit].M, d[hit].N, d[hit].K, d[hit].A, d[hit].lda, d[hit].B, d[hit].ldb,
                            d[hit].C, d[hit].ldc, 1);
        covered[hit] = 1;
      }
    }
    for (int i = 0; i < count; ++i)
      CHECK(covered[i] == (d[i].M > 0 && d[i].N > 0), "member %d computed %d times", i, covered[i]);
  }
}

// ------------------------------------------------------------------ fp8
int expect_fp8(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const float* SA, const void* B,
               int64_t ldb, const float* SB, const void* C, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return TGEMM_EINVAL_DIM;
  const int64_t one = 1;
  if (lda < std::max(one, K) || ldb < std::max(one, K) || ldc < std::max(one, N)) return TGEMM_EINVAL_LD;
  if (M > 0 && N > 0 && C == nullptr) return TGEMM_ENULL;
  if (M > 0 && N > 0 && K > 0 && (!A || !B || !SA || !SB)) return TGEMM_ENULL;
  if (((uintptr_t)C & 1u) || (((uintptr_t)SA | (uintptr_t)SB) & 3u)) return TGEMM_EALIGN;
  return TGEMM_OK;
}

void fuzz_fp8(int iters) {
  for (int it = 0; it < iters; ++it) {
    const bool small = next() % 3 != 0;
    const int64_t M = gen_dim(small), N = gen_dim(small), K = gen_dim(small);
    const int64_t lda = gen_ld(K), ldb = gen_ld(K), ldc = gen_ld(N);
    const void* A = gen_ptr(0);
    const void* B = gen_ptr(1);
    void* C = const_cast<void*>(gen_ptr(2));
    const float* SA = (const float*)gen_ptr(3);
    const float* SB = (const float*)gen_ptr(4);
    const int want = expect_fp8(M, N, K, A, lda, SA, B, ldb, SB, C, ldc);
    stub::launches.clear();
    const int rc = gemm_fp8_block(M, N, K, A, lda, SA, B, ldb, SB, C, ldc, 0, nullptr);
    const bool big_generic = want == TGEMM_OK && M > 0 && N > 0 && K > 0 && cdiv(M, 16) * cdiv(N, 16) >= ((int64_t)1 << 32);
    CHECK(rc == want || (big_generic && rc == TGEMM_EINVAL_DIM), "fp8 rc %d want %d", rc, want);
    if (rc != TGEMM_OK || M == 0 || N == 0) {
      CHECK(stub::launches.empty(), "fp8 launch after an error");
      continue;
    }
    CHECK(stub::launches.size() == 1, "fp8 one launch");
    const stub::Launch& l = stub::launches[0];
    if (K == 0) {
      CHECK(l.kind == stub::kZeroFill, "fp8 zero fill");
      continue;
    }
    CHECK(l.kind == stub::kFp8, "fp8 kind");
    const tgemm::Fp8Args& g = l.fp8;
    CHECK(g.M == M && g.N == N && g.K == K && g.KB == cdiv(K, 128) && g.lda == lda && g.ldb == ldb && g.ldc == ldc,
          "fp8 args");
    if (l.cfg >= 0) {
      const tgemm_config_info& c = fp8cfgs[l.cfg].info;
      CHECK(c.built == 1, "fp8 launch of an unbuilt config");
      CHECK(g.tiles_m == cdiv(M, c.block_m) && g.tiles_n == cdiv(N, c.block_n), "fp8 tiles");
      CHECK(al16(A) && al16(B) && al16(C) && lda % 16 == 0 && ldb % 16 == 0 && K % 16 == 0 && ldc % 8 == 0 &&
                N % 8 == 0 && lda <= 2 * TGEMM_FAST_MAX_LD && ldb <= 2 * TGEMM_FAST_MAX_LD,
            "fp8 fast config on ineligible arguments");
    }
  }
}

void fuzz_quant(int iters) {
  for (int it = 0; it < iters; ++it) {
    const int64_t R = gen_dim(next() % 2), K = gen_dim(next() % 2);
    const int block_rows = (int)pick((const int64_t[]){1, 128, 64, 0}, 4);
    const int64_t ldx = gen_ld(K), ldq = gen_ld(K);
    const void* X = gen_ptr(0);
    void* Q = const_cast<void*>(gen_ptr(1));
    float* S = (float*)const_cast<void*>(gen_ptr(2));
    stub::launches.clear();
    const int rc = quant_fp8_block(R, K, X, ldx, block_rows, Q, ldq, S, nullptr);
    if (rc != TGEMM_OK || R == 0 || K == 0) {
      CHECK(stub::launches.empty(), "quant launch after an error or when empty");
      continue;
    }
    CHECK(R > 0 && K > 0 && R < kMaxDim && K < kMaxDim && (block_rows == 1 || block_rows == 128), "quant dims");
    CHECK(ldx >= K && ldq >= K && X && Q && S && !((uintptr_t)X & 1u) && !((uintptr_t)S & 3u), "quant args");
    CHECK(stub::launches.size() == 1 && stub::launches[0].kind == stub::kQuant, "quant launch");
    const tgemm::QuantArgs& q = stub::launches[0].quant;
    CHECK(q.R == R && q.K == K && q.KB == cdiv(K, 128) && q.ldx == ldx && q.ldq == ldq, "quant args");
    if (stub::launches[0].vec) CHECK(al16(X) && ((uintptr_t)Q & 7u) == 0 && ldx % 8 == 0 && ldq % 8 == 0 && K % 8 == 0, "vec");
  }
}

void directed() {
  const void* P = (const void*)0x100000;
  void* Cp = (void*)0x200000;
  // a launch the runtime rejects is reported as TGEMM_ELAUNCH
  stub::fail_next_launch = 1;
  CHECK(gemm_f16(256, 256, 256, P, 256, P, 256, Cp, 256, 1, nullptr) == TGEMM_ELAUNCH, "launch failure");
  stub::fail_next_launch = 1;
  CHECK(gemm_fp8_block(256, 256, 256, P, 256, (const float*)P, P, 256, (const float*)P, Cp, 256, 0, nullptr) ==
            TGEMM_ELAUNCH, "fp8 launch failure");
  stub::fail_next_launch = 0;
  // a row this build does not compile is refused before anything is enqueued
  for (int i = 0; i < ncfg; ++i) {
    stub::launches.clear();
    const int rc = gemm_f16_cfg(i, 256, 256, 256, P, 256, P, 256, Cp, 256, 1, nullptr);
    CHECK(cfgs[i].info.built ? rc == TGEMM_OK : rc == TGEMM_EINVAL_CFG, "cfg %d built %d rc %d", i,
          cfgs[i].info.built, rc);
    CHECK(stub::launches.size() == (size_t)(rc == TGEMM_OK), "cfg %d launches", i);
  }
  for (int i = 0; i < nfp8; ++i) {
    const int rc = gemm_fp8_block_cfg(i, 256, 256, 256, P, 256, (const float*)P, P, 256, (const float*)P, Cp, 256, 0,
                                      nullptr);
    CHECK(fp8cfgs[i].info.built ? rc == TGEMM_OK : rc == TGEMM_EINVAL_CFG, "fp8 cfg %d rc %d", i, rc);
  }
  // grouped: negative count, NULL list
  CHECK(gemm_f16_grouped(0, 0, -1, nullptr, 1, nullptr) == TGEMM_EINVAL_DIM, "grouped count");
  CHECK(gemm_f16_grouped(0, 0, 3, nullptr, 1, nullptr) == TGEMM_ENULL, "grouped null");
  CHECK(gemm_f16_grouped(0, 0, 0, nullptr, 1, nullptr) == TGEMM_OK, "grouped empty");
  // descriptor queries
  tgemm_config_info info;
  CHECK(tgemm_config_desc(ncfg, &info) == TGEMM_EINVAL_CFG && tgemm_config_desc(0, nullptr) == TGEMM_ENULL, "desc");
  CHECK(tgemm_workspace_bytes_cfg(-1, 1, 8, 8) == TGEMM_EINVAL_CFG && tgemm_workspace_bytes_cfg(0, 9, 8, 8) ==
            TGEMM_EINVAL_CFG && tgemm_workspace_bytes_cfg(0, 1, -1, 8) == TGEMM_EINVAL_DIM, "ws cfg");
  CHECK(tgemm_workspace_bytes(0, 0, kMaxDim - 1, kMaxDim - 1, kMaxDim - 1) >= 0, "ws bytes at the limits");
  for (int e = -9; e <= 1; ++e) CHECK(tgemm_strerror(e) != nullptr, "strerror");
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 4000;
  load_tables();
  directed();
  fuzz_f16(iters);
  fuzz_grouped(iters / 8);
  fuzz_fp8(iters);
  fuzz_quant(iters / 2);
  std::printf("host logic ok: %ld checks, %ld launches recorded\n", checks, stub::total_launches);
  return 0;
}
