// tgemm_internal.h -- shared between the HIP kernels and the host API of libtgemm.
//
// Holds the kernel-configuration table and the workgroup -> output-tile map. The map is
// one inline function compiled for both the device (the kernels call it) and the host
// (tgemm_tile_of exports it for tests), so the tested map is the executed map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {

// Number of XCDs on MI355X; the hardware dispatcher hands consecutive workgroup ids to
// XCDs round robin, and each XCD has its own L2.
constexpr int kNumXcd = 8;

// Work-group tile configuration (one compiled kernel instantiation per entry).
struct Config {
  int bm, bn, bk;       // workgroup tile
  int stages;           // LDS ring depth
  int waves_m, waves_n; // wavefront grid
  int panel;            // tile-rows per panel in the workgroup order
  int xcd_remap;        // keep consecutive logical tiles on one XCD
  int generic;          // unaligned-capable generic kernel
  int layouts;          // bit (2 * trans_a + trans_b) set: the config takes that layout
  int built;            // 1 = this build compiles the kernel (see tgemm_configs.h)
  const char* name;
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroup id -> output tile (tile_m, tile_n).
//
// Step 1 (XCD remap): hardware workgroup id `wg` runs on XCD wg % 8. Renumber so that each
// XCD receives a contiguous range of logical ids: XCD x takes logical ids
// [x*q + min(x, r), ...) where total = 8q + r. A bijection for every total.
// Step 2 (panel order): logical ids walk the tile grid in panels of `panel` tile-rows;
// inside a panel the tile-row index moves fastest, then the tile-column. Consecutive
// logical ids therefore share B columns and a small set of A rows, so the tiles one XCD
// runs at the same time re-use each other's operands from that XCD's L2. This is the
// panel-ordered block swizzle of "Writing High-Performance Kernels in TileLang, from
// GEMM to MLA" (atlascloud.ai), section "Let's write a GEMM" (use_swizzle with a panel
// size and column order), made XCD-aware for MI355X.
__host__ __device__ inline int64_t xcd_logical_id(int64_t wg, int64_t total, int xcd_remap) {
  if (!xcd_remap || total < kNumXcd) return wg;
  const int64_t q = total / kNumXcd, r = total % kNumXcd;
  const int64_t x = wg % kNumXcd, j = wg / kNumXcd;
  return (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

__host__ __device__ inline void panel_tile(int64_t t, int64_t tiles_m, int64_t tiles_n, int panel, int64_t* tm,
                                           int64_t* tn) {
  if (panel < 1) panel = 1;
  const int64_t per_panel = (int64_t)panel * tiles_n;
  const int64_t p = t / per_panel;
  const int64_t within = t - p * per_panel;
  int64_t rows = tiles_m - p * panel;
  if (rows > panel) rows = panel;
  *tm = p * panel + within % rows;
  *tn = within / rows;
}

__host__ __device__ inline void tile_of(int64_t wg, int64_t tiles_m, int64_t tiles_n, int panel,
                                        int xcd_remap, int64_t* tm, int64_t* tn) {
  panel_tile(xcd_logical_id(wg, tiles_m * tiles_n, xcd_remap), tiles_m, tiles_n, panel, tm, tn);
}

// Split-K launches run tiles * splits workgroups. Step 1 runs over all of them; logical id
// t then names split t / tiles of the tile with panel index t % tiles (step 2). An XCD's
// contiguous range of logical ids is thus, for the most part, one split (one k range) of a
// compact block of panel-neighbouring tiles: its L2 holds the A rows and B columns those
// tiles share over k / splits only, about sqrt(splits) times fewer bytes per XCD than
// whole tiles with all their splits would need. The tile's linear index *tile_id numbers
// its fixup counter and partial tiles. With splits = 1 this is tile_of.
__host__ __device__ inline void split_tile_of(int64_t wg, int64_t tiles_m, int64_t tiles_n, int splits, int panel,
                                              int xcd_remap, int64_t* tm, int64_t* tn, int64_t* tile_id,
                                              int* split) {
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t t = xcd_logical_id(wg, tiles * splits, xcd_remap);
  *split = (int)(t / tiles);
  *tile_id = t - *split * tiles;
  panel_tile(*tile_id, tiles_m, tiles_n, panel, tm, tn);
}

// Kernel arguments (passed by value).
struct GemmArgs {
  const _Float16* A;
  const _Float16* B;
  _Float16* C;
  int64_t lda, ldb, ldc;  // elements
  int M, N, K;
  int relu;
  int tiles_m, tiles_n;
  int layout;  // 2 * trans_a + trans_b: A given as K x M, B given as N x K
  int splits;  // split-K factor (1 = none); > 1 only for split-capable configs
  void* ws;    // split-K workspace: tile counters at 0, partial tiles at byte ws_parts
  int64_t ws_parts;
};

// The table (host only). Index order is part of the tooling ABI (gemm_f16_cfg, sweep
// results); *count receives the number of rows.
const Config* config_table(int* count);

// Launcher of table row idx (defined next to the kernels). Returns the hipError_t of the
// launch. `device` is the current HIP device ordinal (the device the launch goes to).
typedef hipError_t (*Launcher)(const GemmArgs&, hipStream_t, int device);
Launcher launcher(int idx);

// Grouped launch: independent GEMMs sharing operand layout and ReLU flag. GEMM i owns
// workgroups [wg_start[i], wg_start[i+1]) of the launch (tiles_m * tiles_n each).
constexpr int kMaxGroups = 32;
struct GroupEntry {
  const _Float16* A;
  const _Float16* B;
  _Float16* C;
  int64_t lda, ldb, ldc;
  int M, N, K;
  int tiles_m, tiles_n;
};
struct GroupedArgs {
  int count, relu, layout;
  int wg_start[kMaxGroups + 1];
  GroupEntry e[kMaxGroups];
};
typedef hipError_t (*GroupedLauncher)(const GroupedArgs&, int64_t nwg, hipStream_t, int device);
// The grouped launcher of table row idx, or nullptr if that config has none.
GroupedLauncher grouped_launcher(int idx);

// fp8 (E4M3) block-scaled GEMM: C = ReLU?(sum_kb SA[i,kb] SB[j/128,kb] sum_k a[i,k] b[j,k]),
// A M x K and B N x K codes (k contiguous), SA M x KB and SB ceil(N/128) x KB float32.
constexpr int kFp8Block = 128;
struct Fp8Args {
  const uint8_t* A;
  const uint8_t* B;
  const float* SA;
  const float* SB;
  _Float16* C;
  int64_t lda, ldb, ldc;  // bytes (A, B) and elements (C)
  int M, N, K, KB;        // KB = ceil(K / 128)
  int relu;
  int tiles_m, tiles_n;
  unsigned long long* stamps;  // instrumented build: the stamp table (else nullptr)
};
// fp8 tile configs (index order is tooling ABI: gemm_fp8_block_cfg, sweeps).
struct Fp8Config {
  int bm, bn, waves_m, waves_n, stages, panel, xcd_remap;
  int lds_bytes;  // dynamic LDS of one workgroup
  int built;      // 1 = this build compiles the kernel (see tgemm_configs.h)
  const char* name;
};
const Fp8Config* fp8_config_table(int* count);
// Launch fast config idx (A, B 16-byte aligned, lda, ldb, K multiples of 16, C 16-byte
// aligned, ldc and N multiples of 8), or the generic kernel (any arguments).
hipError_t launch_fp8(int idx, const Fp8Args& g, hipStream_t s, int device);
hipError_t launch_fp8_generic(const Fp8Args& g, hipStream_t s);

// Block quantizer binary16 -> E4M3 with float32 block scales (blocks of block_rows x 128).
struct QuantArgs {
  const _Float16* X;
  uint8_t* Q;
  float* S;
  int64_t ldx, ldq;  // elements (X), bytes (Q)
  int R, K, KB, block_rows;
};
// vec: X 16-byte aligned, Q 8-byte aligned, ldx, ldq and K multiples of 8.
hipError_t launch_quant_fp8(const QuantArgs& q, bool vec, hipStream_t s);

// Split-K scratch of the allocation-free entry point: a static device array of
// kStaticScratchBytes per device (tile counters first, then partial tiles). Writes its
// device address on the current device to *out (looked up once per device, then cached).
constexpr int64_t kStaticScratchBytes = 4096 + ((int64_t)64 << 20);
hipError_t static_scratch(int device, void** out);

// Zero-fill of an M x N block with row stride ldc (the K == 0 case).
hipError_t launch_zero_fill(_Float16* C, int M, int N, int64_t ldc, hipStream_t s);

// MFMA throughput probe (tooling build only): `blocks` workgroups of 8 waves, each wave
// issuing iters rounds of 16 x 16384 FLOP of independent fp16 MFMAs; one float per thread
// goes to out (blocks * 512 floats). Modes: 0 synthetic operands, 1 operands from ops
// (512 x 64 binary16 values), 2 as 1 with 32x32x16 MFMAs, 3 as 1 plus LDS fragment reads.
constexpr int kProbeThreads = 512, kProbeMfmaPerIter = 16, kProbeModes = 4;
#ifdef TGEMM_STAMPS
hipError_t launch_mfma_probe(int mode, int blocks, int iters, const _Float16* ops, float* out, hipStream_t s);
#endif

// LDS access probe (tooling build only): instruction kinds (ds_read_b32, ds_read_b64,
// ds_read_b128, ds_write_b32, ds_write_b64, ds_write_b128, ds_read_b64_tr_b16), up to
// kLdsProbeSlots instructions per round, byte addresses inside a kLdsProbeBytes block.
constexpr int kLdsProbeOps = 7, kLdsProbeSlots = 8, kLdsProbeBytes = 65536;
struct LdsProbeArgs {
  int32_t addr[kLdsProbeSlots][64];
  uint64_t active[kLdsProbeSlots];  // lanes that issue instruction j
  int ni, iters;
  float* out;
};
#ifdef TGEMM_STAMPS
hipError_t launch_lds_probe(int op, int blocks, const LdsProbeArgs& p, hipStream_t s);
#endif

// Workgroup timestamps of the instrumented build (TGEMM_STAMPS): kStampWords words per
// workgroup for the first kStampWorkgroups workgroups of every launch (later launches
// overwrite earlier ones).
constexpr int kStampWorkgroups = 4096, kStampWords = 8;
#ifdef TGEMM_STAMPS
hipError_t stamps_read(unsigned long long* host, int64_t words);
hipError_t stamps_clear();
unsigned long long* stamps_table();  // device address of the table on the current device
#endif

}  // namespace tgemm
