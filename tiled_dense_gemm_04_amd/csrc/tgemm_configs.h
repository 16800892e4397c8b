// tgemm_configs.h -- the kernel-configuration lists of libtgemm, as X-macros.
//
// One list per kernel family. Every row is one entry of the config table (the row order
// is the index order, which tools and sweep results refer to) and, in a build that
// compiles it, one kernel instantiation. The last column, PROD, says which build compiles
// the row:
//   1  the product library: a config the selector can pick (its choice table,
//      tgemm_choice.inc, only names these);
//   0  only the tooling build (compiled with -DTGEMM_SWEEP_CONFIGS, which also carries the
//      stamps): variants kept so the offline sweep can keep comparing them. The product
//      library still lists the row, marked not built, so every index means the same
//      config in both builds.
// The lists hold numbers only, so host code (the selector, tests of the host logic) can
// read them without the kernels.
#pragma once

#ifdef TGEMM_SWEEP_CONFIGS
#define TGEMM_BUILT(PROD) 1
#else
#define TGEMM_BUILT(PROD) PROD
#endif
// TGEMM_IF_BUILT(PROD, x, y): x when the row is compiled into this build, else y.
#define TGEMM_IF_BUILT(PROD, x, y) TGEMM_IF_BUILT_I(TGEMM_BUILT(PROD), x, y)
#define TGEMM_IF_BUILT_I(b, x, y) TGEMM_IF_BUILT_II(b, x, y)
#define TGEMM_IF_BUILT_II(b, x, y) TGEMM_IF_BUILT_##b(x, y)
#define TGEMM_IF_BUILT_1(x, y) x
#define TGEMM_IF_BUILT_0(x, y) y

// Barrier-synchronous kernel (the first version, the sweep's baseline):
//   X(BM, BN, BK, WAVES_M, WAVES_N, STAGES, PANEL, XCD_REMAP, PROD)            rows 1-2
#define TGEMM_FAST_CONFIGS(X)         \
  X(256, 256, 64, 2, 4, 2, 4, 1, 0)   \
  X(128, 128, 64, 2, 2, 2, 4, 1, 0)

// Single-group pipelined kernel, A and B as given; row 7 (128 x 128, 64-deep k-tiles) is
// the smallest grids' default:
//   X(BM, BN, BK, WAVES_M, WAVES_N, STAGES, PANEL, XCD_REMAP, PROD)            rows 3-7
#define TGEMM_PIPE_CONFIGS(X)         \
  X(256, 256, 32, 2, 4, 4, 4, 1, 0)   \
  X(256, 256, 32, 2, 2, 4, 4, 1, 0)   \
  X(128, 128, 32, 2, 2, 4, 4, 1, 0)   \
  X(256, 128, 32, 2, 2, 4, 4, 1, 0)   \
  X(128, 128, 64, 2, 2, 2, 4, 1, 1)

// Ping-pong kernel with 32x32x16 MFMAs:
//   X(BM, BN, BK, WAVES_M, WAVES_N, STAGES, PANEL, XCD_REMAP, PROD)            row 8
#define TGEMM_PP_CONFIGS(X)           \
  X(256, 256, 32, 2, 4, 4, 4, 1, 0)

// Ping-pong kernel with 16x16x32 MFMAs, the default for everything but the smallest grids.
// ALL = 1: instantiated for all four operand layouts (else A and B as given only).
//   X(BM, BN, BK, WAVES_M, WAVES_N, STAGES, PANEL, XCD_REMAP, ALL, PROD)       rows 9-18
#define TGEMM_PP1_CONFIGS(X)             \
  X(256, 256, 32, 2, 4, 4, 4, 1, 1, 1)   \
  X(256, 256, 32, 4, 2, 4, 4, 1, 0, 0)   \
  X(256, 256, 32, 2, 4, 5, 4, 1, 0, 0)   \
  X(256, 256, 32, 2, 4, 4, 8, 1, 0, 0)   \
  X(256, 256, 32, 2, 4, 4, 2, 1, 0, 0)   \
  X(256, 256, 32, 2, 4, 4, 4, 0, 0, 1)   \
  X(128, 128, 32, 2, 4, 4, 4, 1, 1, 1)   \
  X(256, 128, 32, 2, 4, 4, 4, 1, 1, 0)   \
  X(128, 256, 32, 2, 4, 4, 4, 1, 1, 1)   \
  X(256, 192, 32, 2, 4, 4, 4, 1, 1, 1)

// Quad kernel (4 waves of 128 x 128):
//   X(BM, BN, BK, WAVES_M, WAVES_N, STAGES, PANEL, XCD_REMAP, ALL, PROD)       rows 19-20
#define TGEMM_QUAD_CONFIGS(X)            \
  X(256, 256, 32, 2, 2, 4, 4, 0, 0, 0)   \
  X(256, 256, 32, 2, 2, 4, 4, 1, 0, 0)

// Single-group pipelined kernel on 64 x 128 tiles, for small output grids with long K
// (twice the workgroups of 128 x 128 tiles). Listed after the quad rows so that every
// earlier index keeps its meaning:
//   X(BM, BN, BK, WAVES_M, WAVES_N, STAGES, PANEL, XCD_REMAP, PROD)            rows 21-22
#define TGEMM_PIPE2_CONFIGS(X)        \
  X(64, 128, 64, 2, 2, 3, 4, 1, 1)    \
  X(64, 128, 32, 2, 2, 4, 4, 1, 1)

// fp8 block-scaled kernels: X(BM, BN, WAVES_M, WAVES_N, STAGES, PANEL, XCD_REMAP, MODE, PROD)
// MODE 0: one group, single-buffered fragments (name suffix _db0); 1: one group,
// double-buffered fragments (_db1); 2: two wave groups in ping-pong (_pp).  fp8 rows 0-4
#define TGEMM_FP8_CONFIGS(X)             \
  X(256, 256, 2, 4, 2, 4, 1, 0, 1)       \
  X(128, 128, 2, 2, 3, 4, 1, 0, 1)       \
  X(256, 128, 4, 2, 3, 4, 1, 0, 0)       \
  X(256, 128, 4, 2, 3, 4, 1, 1, 1)       \
  X(256, 256, 2, 4, 2, 4, 1, 2, 1)
#define TGEMM_FP8_MODE_NAME_0 "_db0"
#define TGEMM_FP8_MODE_NAME_1 "_db1"
#define TGEMM_FP8_MODE_NAME_2 "_pp"
