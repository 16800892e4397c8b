// tgemm_kernels.hip -- gfx950 kernels of libtgemm: C = ReLU?(A @ B), fp16 in, fp32
// accumulate, fp16 out, all row-major.
//
// The computation follows "Writing High-Performance Kernels in TileLang, from GEMM to
// MLA" (atlascloud.ai), section "Let's write a GEMM": a workgroup owns a block_M x
// block_N tile of C, clears a float32 accumulator, walks K in block_K steps through a
// multi-stage shared-memory pipeline (global -> shared copies of the A and B tiles, then a
// tile-level matrix multiply), applies max(x, 0) and writes the tile back as fp16.
// What is MI355X-specific here (and not on the pages):
//   * global -> LDS copies are buffer loads that write LDS directly (no VGPR staging);
//     the buffer descriptor's range check turns every out-of-matrix chunk into zeros,
//     which is how edge tiles are predicated;
//   * LDS tiles are XOR-swizzled for the 64 LDS banks of gfx950;
//   * B (row-major, N contiguous) is read from LDS with ds_read_b64_tr_b16, which
//     transposes 4x4 blocks of 16-bit values across lanes, so no transpose pass is needed;
//   * 32x32x16 fp16 MFMAs accumulate in fp32; operands are fed as (B^T, A^T) so that each
//     lane ends up holding four consecutive output columns, stored as one 8-byte write;
//   * the workgroup order is XCD-aware and panel-ordered (tile_of in tgemm_internal.h).
#include "tgemm_configs.h"
#include "tgemm_device.h"

#include <atomic>
#include <type_traits>
#include <utility>

namespace tgemm {

// Split-K scratch for callers that cannot allocate (gemm_f16_ws_static): the tile
// counters (zero when the library is loaded on a device; every split launch leaves the
// counters it used at zero) and the fp32 partial tiles. Host code must not pass this
// name to a kernel (on the host it is only a stand-in for the device symbol): it uses
// the device address static_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(int device, void** out) {
  constexpr int kMaxDev = 64;
  static std::atomic<void*> addr[kMaxDev];
  if (device < 0 || device >= kMaxDev) return hipErrorInvalidDevice;
  void* p = addr[device].load(std::memory_order_acquire);
  if (p == nullptr) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[device].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

namespace {

#ifdef TGEMM_STAMPS
__device__ unsigned long long g_stamps[kStampWorkgroups * kStampWords];
#define TG_STAMP_TABLE g_stamps
#else
#define TG_STAMP_TABLE nullptr
#endif


// ------------------------------------------------------------------------------------
// Fast kernel: BM x BN x BK tile, WM x WN waves, STAGES-deep LDS ring fed by buffer->LDS
// loads. Requirements (checked by the host): A, B, C 16-byte aligned; lda, ldb, ldc,
// K and N multiples of 8; K > 0.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD>
__global__ __launch_bounds__(64 * WM * WN) void gemm_fast(GemmArgs g) {
  WgClock clk;
  clk.start();
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_CH_ROW = BK / 8, B_CH_ROW = BN / 8;
  constexpr int A_UNITS = BM * A_CH_ROW, B_UNITS = BK * B_CH_ROW;
  constexpr int A_LD = A_UNITS / NT, B_LD = B_UNITS / NT;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert(A_UNITS % NT == 0 && B_UNITS % NT == 0, "loads must split evenly");
  static_assert(BK % 16 == 0 && BK >= 32 && BK <= 128, "block_k");
  static_assert(BN >= 128 && (BN * 2) % 256 == 0, "B rows must span the bank window");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  static_assert(A_LD + B_LD <= 16, "vmcnt budget");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const a_lds = smem;
  char* const b_lds = smem + STAGES * A_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int64_t tm64, tn64;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, PANEL, XCD, &tm64, &tn64);
  const int row0 = (int)tm64 * BM, col0 = (int)tn64 * BN;
  const int mvalid = min(BM, g.M - row0), nvalid = min(BN, g.N - col0);
  const int K = g.K;

  // Per-thread buffer offsets (bytes) of each chunk this thread copies, relative to the
  // tile's base at k0 = 0. Load i of wave w fills LDS bytes [(i*NW + w) * 1024, +1024):
  // lane u writes chunk slot (i*NW + w)*64 + u.
  uint32_t a_off[A_LD];
  int a_kc[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int u = (i * NW + wave) * 64 + lane;
    const int r = u / A_CH_ROW;
    const int c = (u % A_CH_ROW) ^ swz_a<BK>(r);
    a_kc[i] = 8 * c;
    a_off[i] = (r < mvalid) ? (uint32_t)(((int64_t)r * g.lda + 8 * c) * 2) : kOob;
  }
  uint32_t b_off[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int u = (i * NW + wave) * 64 + lane;
    const int k = u / B_CH_ROW;
    const int c = (u % B_CH_ROW) ^ swz_b(k);
    b_off[i] = (8 * c < nvalid) ? (uint32_t)(((int64_t)k * g.ldb + 8 * c) * 2) : kOob;
  }
  const _Float16* const a_tile = g.A + (int64_t)row0 * g.lda;
  const _Float16* const b_tile = g.B + col0;
  const int nk = (K + BK - 1) / BK;

  // Issue the buffer->LDS copies of k-tile kt into ring slot `slot`.
  auto issue = [&](int kt, int slot) {
    const int k0 = kt * BK;
    const int krem = K - k0;  // > 0
    const int kin = krem < BK ? krem : BK;
    // A: rows < mvalid, columns < kin are in range. The last row's range ends at kin;
    // columns >= kin of the other rows are masked below (only in a K-tail tile).
    const int64_t a_range = ((int64_t)(mvalid - 1) * g.lda + kin) * 2;
    const int4v ra = make_rsrc(a_tile + k0, (uint32_t)(a_range < kMaxRange ? a_range : kMaxRange));
    // B: rows < kin, columns < nvalid; rows >= kin fall past the range and read as zero.
    const int64_t b_range = ((int64_t)(kin - 1) * g.ldb + nvalid) * 2;
    const int4v rb = make_rsrc(b_tile + (int64_t)k0 * g.ldb,
                               (uint32_t)(b_range < kMaxRange ? b_range : kMaxRange));
    const uint32_t a_dst = lds_addr(a_lds) + slot * A_BYTES + wave * 1024;
    const uint32_t b_dst = lds_addr(b_lds) + slot * B_BYTES + wave * 1024;
    if (kin == BK) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) dma_to_lds(ra, a_dst + i * NW * 1024, a_off[i]);
    } else {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) dma_to_lds(ra, a_dst + i * NW * 1024, a_kc[i] < kin ? a_off[i] : kOob);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) dma_to_lds(rb, b_dst + i * NW * 1024, b_off[i]);
  };

  // Wave position and per-lane LDS read offsets.
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, lhi = lane >> 5;
  // A fragment (32 rows x 16 k): lane reads row wm*WTM + fm*32 + l32, k chunk 2*ks + lhi.
  const int a_row_off = (wm * WTM + l32) * BK * 2;
  const int a_sw = swz_a<BK>(l32);  // fm*32 and wm*WTM are multiples of the swizzle period
  // B fragment (16 k x 32 n) via two transposed reads; lane = 16g + 4j + q.
  const int bg = lane >> 4, bj = (lane >> 2) & 3, bq = lane & 3;
  const int b_krow = 8 * (bg >> 1) + bj;                         // + 16*ks + 4*h
  const int b_chunk = (wn * WTN) / 8 + 2 * (bg & 1) + (bq >> 1);  // + 4*fn
  const int b_half = (bq & 1) * 8;

  float16v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // LDS -> VGPR fragments of k-substep ks (16 k values) of ring slot `slot`.
  auto load_frags = [&](int slot, int ks, half8 (&af)[FM], half8 (&bf)[FN]) {
    const char* const As = a_lds + slot * A_BYTES;
    const char* const Bs = b_lds + slot * B_BYTES;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int off = a_row_off + fm * 32 * BK * 2 + (((2 * ks + lhi) ^ a_sw) << 4);
      af[fm] = *(const TG_LDS half8*)(As + off);
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      short4v part[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 16 * ks + 4 * h + b_krow;
        const int off = k * BN * 2 + (((b_chunk + 4 * fn) ^ swz_b(k)) << 4) + b_half;
        part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS short4v*)(Bs + off));
      }
      const short8v s8 = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
      bf[fn] = __builtin_bit_cast(half8, s8);
    }
  };
  auto mma = [&](const half8 (&af)[FM], const half8 (&bf)[FN]) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[fn], af[fm], acc[fm][fn], 0, 0, 0);
  };
  // One k-tile: fragments of substep ks+1 are read while the MFMAs of substep ks run.
  auto compute = [&](int slot) {
    half8 af[2][FM];
    half8 bf[2][FN];
    load_frags(slot, 0, af[0], bf[0]);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) load_frags(slot, ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mma(af[ks & 1], bf[ks & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Pipeline: STAGES-1 tiles in flight ahead of the one being multiplied.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s, s);
  constexpr int PER_TILE = A_LD + B_LD;
  clk.loop_begin();
  for (int kt = 0; kt < nk; ++kt) {
    // Tile kt has landed once at most min(STAGES-2, nk-1-kt) later tiles are in flight.
    const int ahead = nk - 1 - kt;
    if (STAGES >= 4 && ahead >= 2)
      wait_vmcnt<(STAGES >= 4 ? 2 : 0) * PER_TILE>();
    else if (STAGES >= 3 && ahead >= 1)
      wait_vmcnt<(STAGES >= 3 ? 1 : 0) * PER_TILE>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    compute(kt % STAGES);
  }

  clk.loop_end();

  // Epilogue: ReLU in fp32, round to fp16 (nearest even), 8-byte stores. Lane holds, for
  // tile (fm, fn) and group g4, row m = ... + l32 and columns n = ... + 8*g4 + 4*lhi + 0..3.
  const bool relu = g.relu != 0;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = wm * WTM + fm * 32 + l32;
    if (m >= mvalid) continue;
    _Float16* const crow = g.C + (int64_t)(row0 + m) * g.ldc + col0;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int n = wn * WTN + fn * 32 + 8 * g4 + 4 * lhi;
        if (n >= nvalid) continue;
        float v0 = acc[fm][fn][4 * g4 + 0], v1 = acc[fm][fn][4 * g4 + 1];
        float v2 = acc[fm][fn][4 * g4 + 2], v3 = acc[fm][fn][4 * g4 + 3];
        if (relu) {
          v0 = relu_f(v0);
          v1 = relu_f(v1);
          v2 = relu_f(v2);
          v3 = relu_f(v3);
        }
        half4 h = {(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
        store_c(crow + n, h);
      }
    }
  }
  clk.finish(nk, TG_STAMP_TABLE);
}

// ------------------------------------------------------------------------------------
// Pipelined kernel: same tiles, LDS layouts and edge handling as gemm_fast, scheduled so
// that the MFMA pipe never waits on memory instructions:
//   * the fragments of k-tile kt+1 are read from LDS into a second register set while the
//     MFMAs of k-tile kt run, interleaved instruction by instruction, so after each
//     workgroup barrier a wave issues MFMAs at once;
//   * the LDS ring has STAGES slots; tile t lives in slot t % STAGES and is copied
//     STAGES-1 iterations before it is read;
//   * every iteration issues exactly PER_TILE buffer->LDS copies, one between each group
//     of MFMAs (copies for tiles past the end use an empty buffer range and only write
//     zeros into a slot no later read needs), so the number of copies in flight is the
//     same at every wait and one constant s_waitcnt suffices;
//   * descriptors advance by a constant stride; only the last k-tile has its own range.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD>
__global__ __launch_bounds__(64 * WM * WN) void gemm_pipe(GemmArgs g) {
  WgClock clk;
  clk.start();
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KS = BK / 16;
  constexpr int A_CH_ROW = BK / 8, B_CH_ROW = BN / 8;
  constexpr int A_UNITS = BM * A_CH_ROW, B_UNITS = BK * B_CH_ROW;
  constexpr int A_LD = A_UNITS / NT, B_LD = B_UNITS / NT;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
  constexpr int PER_TILE = A_LD + B_LD;
  constexpr int N_MFMA = KS * FM * FN;
  constexpr int N_READ = KS * (FM + 2 * FN);
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert(A_UNITS % NT == 0 && B_UNITS % NT == 0, "loads must split evenly");
  static_assert(BK % 16 == 0 && BK >= 16 && BK <= 128, "block_k");
  static_assert(BN >= 128 && (BN * 2) % 256 == 0, "B rows must span the bank window");
  static_assert(STAGES >= 2, "stages");
  static_assert(PER_TILE * STAGES < 64, "vmcnt budget");
  static_assert(N_MFMA >= PER_TILE, "at least one MFMA between copies");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const a_lds = smem;
  char* const b_lds = smem + STAGES * A_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int64_t tm64, tn64;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, PANEL, XCD, &tm64, &tn64);
  const int row0 = (int)tm64 * BM, col0 = (int)tn64 * BN;
  const int mvalid = min(BM, g.M - row0), nvalid = min(BN, g.N - col0);
  const int K = g.K;
  const int nk = (K + BK - 1) / BK;
  const int kin_last = K - (nk - 1) * BK;  // 1 .. BK

  // Per-thread copy offsets (bytes from the descriptor base of a k-tile). A rows at or
  // past mvalid fall outside the A range and read as zero; B columns at or past nvalid
  // are masked here; A columns past K exist only in the last k-tile (masked there).
  uint32_t a_off[A_LD], a_off_last[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int u = (i * NW + wave) * 64 + lane;
    const int r = u / A_CH_ROW;
    const int c = (u % A_CH_ROW) ^ swz_a<BK>(r);
    a_off[i] = (uint32_t)(((int64_t)r * g.lda + 8 * c) * 2);
    a_off_last[i] = 8 * c < kin_last ? a_off[i] : kOob;
  }
  uint32_t b_off[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int u = (i * NW + wave) * 64 + lane;
    const int k = u / B_CH_ROW;
    const int c = (u % B_CH_ROW) ^ swz_b(k);
    b_off[i] = (8 * c < nvalid) ? (uint32_t)(((int64_t)k * g.ldb + 8 * c) * 2) : kOob;
  }
  // Descriptor ranges (bytes) for a full k-tile and for the last one.
  const int64_t a_rng_full64 = ((int64_t)(mvalid - 1) * g.lda + BK) * 2;
  const int64_t a_rng_last64 = ((int64_t)(mvalid - 1) * g.lda + kin_last) * 2;
  const int64_t b_rng_full64 = ((int64_t)(BK - 1) * g.ldb + nvalid) * 2;
  const int64_t b_rng_last64 = ((int64_t)(kin_last - 1) * g.ldb + nvalid) * 2;
  const uint32_t a_rng_full = (uint32_t)(a_rng_full64 < kMaxRange ? a_rng_full64 : kMaxRange);
  const uint32_t a_rng_last = (uint32_t)(a_rng_last64 < kMaxRange ? a_rng_last64 : kMaxRange);
  const uint32_t b_rng_full = (uint32_t)(b_rng_full64 < kMaxRange ? b_rng_full64 : kMaxRange);
  const uint32_t b_rng_last = (uint32_t)(b_rng_last64 < kMaxRange ? b_rng_last64 : kMaxRange);
  const char* const a_base = (const char*)(g.A + (int64_t)row0 * g.lda);
  const char* const b_base = (const char*)(g.B + col0);
  const int64_t a_step = (int64_t)BK * 2, b_step = (int64_t)BK * g.ldb * 2;
  const uint32_t a_lds0 = lds_addr(a_lds) + wave * 1024;
  const uint32_t b_lds0 = lds_addr(b_lds) + wave * 1024;

  // Copy j (0 .. PER_TILE-1) of k-tile t into its slot. Tiles past the end get range 0.
  struct Dma {
    int4v ra, rb;
    uint32_t a_dst, b_dst;
    bool last;
  };
  auto dma_setup = [&](int t) {
    Dma d;
    const uint32_t ar = t < nk - 1 ? a_rng_full : (t == nk - 1 ? a_rng_last : 0u);
    const uint32_t br = t < nk - 1 ? b_rng_full : (t == nk - 1 ? b_rng_last : 0u);
    const int tt = t < nk ? t : nk - 1;  // keep the base inside the matrix
    d.ra = make_rsrc(a_base + tt * a_step, ar);
    d.rb = make_rsrc(b_base + tt * b_step, br);
    const int slot = t % STAGES;
    d.a_dst = a_lds0 + slot * A_BYTES;
    d.b_dst = b_lds0 + slot * B_BYTES;
    d.last = t == nk - 1;
    return d;
  };
  auto dma_one = [&](const Dma& d, int j) {
    if (j < A_LD)
      dma_to_lds(d.ra, d.a_dst + j * NW * 1024, d.last ? a_off_last[j] : a_off[j]);
    else
      dma_to_lds(d.rb, d.b_dst + (j - A_LD) * NW * 1024, b_off[j - A_LD]);
  };

  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, lhi = lane >> 5;
  const int a_row_off = (wm * WTM + l32) * BK * 2;
  const int a_sw = swz_a<BK>(l32);
  const int bg = lane >> 4, bj = (lane >> 2) & 3, bq = lane & 3;
  const int b_krow = 8 * (bg >> 1) + bj;
  const int b_chunk = (wn * WTN) / 8 + 2 * (bg & 1) + (bq >> 1);
  const int b_half = (bq & 1) * 8;

  struct Frags {
    half8 a[KS][FM];
    short4v b[KS][FN][2];
  };
  // Read number r (0 .. N_READ-1) of a k-tile: per substep FM A reads, then 2*FN B reads.
  auto read_one = [&](int slot, Frags& f, int r) {
    const int ks = r / (FM + 2 * FN), q = r % (FM + 2 * FN);
    if (q < FM) {
      const char* const As = a_lds + slot * A_BYTES;
      const int off = a_row_off + q * 32 * BK * 2 + (((2 * ks + lhi) ^ a_sw) << 4);
      f.a[ks][q] = *(const TG_LDS half8*)(As + off);
    } else {
      const int fn = (q - FM) / 2, h = (q - FM) % 2;
      const char* const Bs = b_lds + slot * B_BYTES;
      const int k = 16 * ks + 4 * h + b_krow;
      const int off = k * BN * 2 + (((b_chunk + 4 * fn) ^ swz_b(k)) << 4) + b_half;
      f.b[ks][fn][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS short4v*)(Bs + off));
    }
  };

  float16v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto mfma_one = [&](const Frags& f, int m) {
    const int ks = m / (FM * FN), fm = (m / FN) % FM, fn = m % FN;
    const short8v b8 = __builtin_shufflevector(f.b[ks][fn][0], f.b[ks][fn][1], 0, 1, 2, 3, 4, 5, 6, 7);
    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, b8), f.a[ks][fm],
                                                         acc[fm][fn], 0, 0, 0);
  };

  // One k-tile: MFMAs from `cur`, the reads of the next tile (slot nslot) into `nxt`, and
  // the PER_TILE copies of tile kt+STAGES, in PER_TILE groups: the group's MFMAs with its
  // share of the reads interleaved (RPM reads after each MFMA), then one copy.
  constexpr int RPM = (N_READ + N_MFMA - 1) / N_MFMA;
  auto step = [&](const Frags& cur, Frags& nxt, int nslot, const Dma& d) {
#pragma unroll
    for (int grp = 0; grp < PER_TILE; ++grp) {
      const int mb = grp * N_MFMA / PER_TILE, me = (grp + 1) * N_MFMA / PER_TILE;
      const int rb = grp * N_READ / PER_TILE, re = (grp + 1) * N_READ / PER_TILE;
#pragma unroll
      for (int m = mb; m < me; ++m) mfma_one(cur, m);
#pragma unroll
      for (int r = rb; r < re; ++r) read_one(nslot, nxt, r);
#pragma unroll
      for (int m = mb; m < me; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      dma_one(d, grp);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: tiles 0 .. STAGES-1 in flight (PER_TILE copies each), tile 0 into registers.
#pragma unroll
  for (int t = 0; t < STAGES; ++t) {
    const Dma d = dma_setup(t);
#pragma unroll
    for (int j = 0; j < PER_TILE; ++j) dma_one(d, j);
  }
  Frags f0, f1;
  wait_vmcnt<PER_TILE * (STAGES - 1)>();
  lds_barrier();
#pragma unroll
  for (int r = 0; r < N_READ; ++r) read_one(0, f0, r);

  // Iteration kt: wait for this thread's copies of tile kt+1 (the tiles issued after it,
  // kt+2 .. kt+STAGES-1, may still fly), then the barrier (every wave's copies of tile
  // kt+1 have landed and every wave has finished reading tile kt, so slot kt % STAGES is
  // free), then MFMAs of tile kt + reads of tile kt+1 + copies of tile kt+STAGES.
  auto iteration = [&](int kt, const Frags& cur, Frags& nxt) {
    const Dma d = dma_setup(kt + STAGES);
    wait_vmcnt<PER_TILE * (STAGES - 2)>();
    lds_barrier();
    step(cur, nxt, (kt + 1) % STAGES, d);
  };
  clk.loop_begin();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    iteration(kt, f0, f1);
    iteration(kt + 1, f1, f0);
  }
  if (kt < nk) iteration(kt, f0, f1);
  // Drain: no copy may still be writing LDS when the workgroup exits.
  wait_vmcnt<0>();
  clk.loop_end();

  // Epilogue: ReLU and RNE in registers, then each wave's sub-tile through its own LDS
  // region (the ring is free once every wave passes the barrier) and out as 16-byte row
  // segments (StagedTile32).
  using ST = StagedTile32<WTM, WTN>;
  static_assert(NW * ST::BYTES <= STAGES * (A_BYTES + B_BYTES), "the staged tile fits in the ring");
  __syncthreads();
  char* const stage = smem + wave * ST::BYTES;
  if (g.relu != 0)
    ST::template stage<true>(stage, acc, lane);
  else
    ST::template stage<false>(stage, acc, lane);
  ST::wave_fence();
  ST::store(stage, lane, g.C + (int64_t)(row0 + wm * WTM) * g.ldc + col0 + wn * WTN, g.ldc, mvalid - wm * WTM,
            nvalid - wn * WTN);
  clk.finish(nk, TG_STAMP_TABLE);
}

// ------------------------------------------------------------------------------------
// Ping-pong kernel: 8 waves in two groups of 4 (waves 0-3 and 4-7), one wave of each
// group per SIMD. Every iteration (one k-tile) has two phases; in each phase one group
// only issues MFMAs (from registers) while the other only moves data (LDS -> its fragment
// registers, and its share of the buffer->LDS copies), then they swap. Each SIMD's MFMA
// pipe is fed by a wave that never waits on a memory instruction, and LDS/TA stalls land
// on the partner wave.
//
// Schedule (tile t lives in ring slot t % STAGES; PT0 / PT1 copies per thread per tile in
// group 0 / 1):
//   prologue: group 0 copies tiles 0 .. STAGES-1, group 1 tiles 0 .. STAGES-2; both wait
//             for tile 0; barrier; group 0 reads tile 0.
//   iteration kt: group 0: MFMAs of tile kt; wait (tile kt+1 landed for this thread);
//                          barrier; reads tile kt+1; copies tile kt+STAGES.
//                 group 1: reads tile kt; copies tile kt+STAGES-1; wait (tile kt+1
//                          landed for this thread); barrier; MFMAs of tile kt.
// Between two barriers group 0 reads then runs MFMAs while group 1 runs MFMAs then reads:
// the opposite order keeps the phases alternating without a barrier between them.
// Slot safety: in iteration kt group 0 copies tile kt+STAGES after barrier kt, into the
// slot of tile kt, whose last reads (group 1's, and group 0's in iteration kt-1) all come
// before barrier kt; group 1 copies tile kt+STAGES-1 before barrier kt, into the slot of
// tile kt-1, whose reads all come before barrier kt-1. Copies past the last tile use an
// empty range, so every thread issues exactly its PT copies per iteration and at each
// barrier exactly STAGES-2 later tiles may still be in flight for every thread.
// MF selects the MFMA: 32 = v_mfma_f32_32x32x16_f16, 16 = v_mfma_f32_16x16x32_f16 (half
// the accumulator traffic per FLOP, twice the instructions). TA / TB: A given transposed
// (K x M, lda >= M) / B given transposed (N x K, ldb >= K).
// The body works on workgroup `wg` of one GEMM's launch (blockIdx.x for a single GEMM,
// the index inside its GEMM for a grouped launch).
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD, int MF, bool TA,
          bool TB>
__device__ __forceinline__ void pingpong_body(const GemmArgs& g, const int wg) {
  WgClock clk;
  clk.start();
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int KS = BK / (512 / MF);  // MFMA k-substeps per k-tile
  static_assert(MF == 32 || MF == 16, "MFMA shape");
  using OpA = PpOperand<pp_lds_extent(BM), BK, MF, !TA, NW>;
  using OpB = PpOperand<pp_lds_extent(BN), BK, MF, TB, NW>;
  constexpr int A_BYTES = OpA::BYTES, B_BYTES = OpB::BYTES;
  // copies per thread and k-tile of wave group 0 and 1 (they differ when an operand's
  // copies do not split evenly over the threads, as for 192-wide tiles)
  constexpr int PT0 = OpA::LD_OF(0) + OpB::LD_OF(0), PT1 = OpA::LD_OF(1) + OpB::LD_OF(1);
  constexpr int PT = PT0;  // the larger
  static_assert(NW == 8, "two groups of four waves");
  static_assert(WTM % MF == 0 && WTN % MF == 0 && KS >= 1, "wave tile must be a multiple of the MFMA");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tiles start on swizzle periods");
  static_assert(BK % 16 == 0 && BK >= 16 && BK <= 128, "block_k");
  static_assert(STAGES >= 3, "the ring needs a slot being read, one in flight and one free");
  static_assert(PT * STAGES < 64, "vmcnt budget");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const a_lds = smem;
  char* const b_lds = smem + STAGES * A_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // waves w and w+4 share SIMD w % 4

  // Split-K (g.splits > 1): split s of a tile covers k-tiles [s * nk / splits,
  // (s + 1) * nk / splits); an XCD runs mostly one split of a block of neighbouring tiles.
  const int splits = g.splits;
  int64_t tm64, tn64, tile64;
  int split;
  split_tile_of(wg, g.tiles_m, g.tiles_n, splits, PANEL, XCD, &tm64, &tn64, &tile64, &split);
  const int tile_id = (int)tile64;
  const int row0 = (int)tm64 * BM, col0 = (int)tn64 * BN;
  const int mvalid = min(BM, g.M - row0), nvalid = min(BN, g.N - col0);
  const int K = g.K;
  const int nk = (K + BK - 1) / BK;
  const int kin_last = K - (nk - 1) * BK;
  const int kt0 = (int)((int64_t)split * nk / splits);
  const int nloc = (int)((int64_t)(split + 1) * nk / splits) - kt0;  // k-tiles of this workgroup

  OpA opa;
  OpB opb;
  opa.init_copies(g.A, g.lda, row0, mvalid, kin_last, wave, lane);
  opb.init_copies(g.B, g.ldb, col0, nvalid, kin_last, wave, lane);
  const uint32_t a_lds0 = lds_addr(a_lds) + wave * 1024;
  const uint32_t b_lds0 = lds_addr(b_lds) + wave * 1024;

  // This thread's PT copies of this workgroup's k-tile t (global k-tile kt0 + t; an empty
  // range from t = nloc on).
  struct Dma {
    int4v ra, rb;
    uint32_t a_dst, b_dst;
    bool last;
  };
  auto dma_setup = [&](int t) {
    Dma d;
    const int kt = kt0 + t, kt_end = kt0 + nloc;
    d.ra = opa.rsrc(kt, kt_end, nk);
    d.rb = opb.rsrc(kt, kt_end, nk);
    const int slot = t % STAGES;
    d.a_dst = a_lds0 + slot * A_BYTES;
    d.b_dst = b_lds0 + slot * B_BYTES;
    d.last = kt == nk - 1;
    return d;
  };
  // Copies of wave group G (a compile-time constant in each group's code).
  // (always inlined: an out-of-line copy would take the operands' addresses and move their
  // offset arrays to scratch memory)
  // Copies [LO, HI) of this thread's PT of tile t (A rows first, then B rows).
  auto copy_part = [&](int t, auto group, auto lo_c, auto hi_c) __attribute__((always_inline)) {
    constexpr int G = decltype(group)::value, LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
    constexpr int LA = OpA::LD_OF(G);
    const Dma d = dma_setup(t);
#pragma unroll
    for (int j = LO; j < (HI < LA ? HI : LA); ++j)
      dma_to_lds(d.ra, d.a_dst + j * NW * 1024, d.last ? opa.off_last[j] : opa.off[j]);
#pragma unroll
    for (int j = (LO > LA ? LO : LA); j < HI; ++j)
      dma_to_lds(d.rb, d.b_dst + (j - LA) * NW * 1024, d.last ? opb.off_last[j - LA] : opb.off[j - LA]);
  };
  using G0 = std::integral_constant<int, 0>;
  using G1 = std::integral_constant<int, 1>;
  // CM of each thread's PT copies per k-tile go out from its MFMA phase, spread between
  // the MFMAs, the rest from its memory phase. A copy holds the issuing wave ~60 clocks, so
  // where the memory phase outlasts the other wave's MFMAs a copy can move: on 128 x 128
  // tiles (8 MFMAs, ~130 clocks per MFMA phase) both copies move (512 x 4096 x 4096:
  // 36.7 -> 34.6 us, 1536^2 x 1024: 12.3 -> 11.8 us, 2048^2 x 4096: 40.8 -> 39.7 us; one
  // moved copy: no change; 1024^2 x 32768 with A transposed: 315.9 -> 273.2 us). Not with
  // both operands k-contiguous, whose plain 16-byte fragment reads keep the memory phase
  // short (1024^2 x 8192: 56.6 -> 60.8 us). On 256 x 128 and 256 x 192 tiles moving one or
  // two measured 3-11 % slower, and 256 x 256 tiles are balanced as they are. Each tile's copies stay
  // contiguous in issue order (group 0: memory part after barrier kt, MFMA part in the next
  // MFMA phase; group 1: MFMA part after barrier kt-1, memory part before barrier kt), so
  // the constant waits hold; only the prologue's waits change.
  constexpr int CM = BM == 128 && BN == 128 && !(OpA::KMAJOR && OpB::KMAJOR) ? (PT0 < PT1 ? PT0 : PT1) : 0;
  auto copy_tile = [&](int t, auto group) __attribute__((always_inline)) {
    constexpr int G = decltype(group)::value, P = G == 0 ? PT0 : PT1;
    copy_part(t, group, std::integral_constant<int, 0>{}, std::integral_constant<int, P - CM>{});
  };

  const int wm = wave / WN, wn = wave % WN;
  opa.init_frags(wm * WTM, lane);
  opb.init_frags(wn * WTN, lane);

  half8 fa[KS][FM], fb[KS][FN];
  auto read_tile = [&](int slot) {
    const char* const As = a_lds + slot * A_BYTES;
    const char* const Bs = b_lds + slot * B_BYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) fa[ks][fm] = opa.frag(As, fm, ks);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) fb[ks][fn] = opb.frag(Bs, fn, ks);
    }
  };

  constexpr int NACC = MF * MF / 64;  // accumulator floats per lane per MFMA tile
  typedef float accv __attribute__((ext_vector_type(NACC)));
  accv acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < NACC; ++r) acc[i][j][r] = 0.0f;

  // Operands go in as (B fragment, A fragment): D^T = B^T A^T, so a lane's accumulator
  // holds consecutive output columns of one row.
  auto mma_one = [&](int m) {
    const int ks = m / (FM * FN), fm = (m / FN) % FM, fn = m % FN;
    if constexpr (MF == 32)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[ks][fn], fa[ks][fm], acc[fm][fn], 0, 0, 0);
    else
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[ks][fn], fa[ks][fm], acc[fm][fn], 0, 0, 0);
  };
  constexpr int N_MFMA = KS * FM * FN;
  // The MFMAs of a tile with the CM MFMA-phase copies of tile t spread between them.
  auto mma_tile_copy = [&](int t, auto group) __attribute__((always_inline)) {
    constexpr int G = decltype(group)::value, P = G == 0 ? PT0 : PT1;
    static_for<N_MFMA>([&](auto m_c) {
      constexpr int m = decltype(m_c)::value;
      mma_one(m);
      static_for<CM>([&](auto c_c) {
        constexpr int c = decltype(c_c)::value;
        if constexpr ((c + 1) * N_MFMA / (CM + 1) == m + 1) {
          __builtin_amdgcn_sched_barrier(0);
          copy_part(t, group, std::integral_constant<int, P - CM + c>{}, std::integral_constant<int, P - CM + c + 1>{});
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    });
  };

  // Prologue: group 0 starts one copy ahead of group 1 (its next copy is in phase 2).
  if (grp == 0) {
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t) copy_part(t, G0{}, std::integral_constant<int, 0>{}, std::integral_constant<int, PT0>{});
    copy_tile(STAGES - 1, G0{});  // (its MFMA-phase copies go out in the first iteration)
    wait_vmcnt<PT0 * (STAGES - 1) - CM>();
  } else {
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t) copy_part(t, G1{}, std::integral_constant<int, 0>{}, std::integral_constant<int, PT1>{});
    // tile STAGES-1's MFMA-phase copies (those of the MFMAs of tile -1)
    copy_part(STAGES - 1, G1{}, std::integral_constant<int, PT1 - CM>{}, std::integral_constant<int, PT1>{});
    wait_vmcnt<PT1 * (STAGES - 2) + CM>();
  }
  lds_barrier();
  if (grp == 0) read_tile(0);

  clk.loop_begin();
  // One barrier per k-tile. Between barrier kt-1 and barrier kt, group 0 reads tile kt and
  // copies its share of tile kt-1+STAGES, then issues the MFMAs of tile kt; group 1 issues
  // the MFMAs of tile kt-1, then reads tile kt and copies its share of the same tile. The
  // opposite order keeps the phases alternating on every SIMD (one wave reads while the
  // other runs MFMAs) without a second barrier, and the barrier covers every LDS hazard:
  // before it, each wave waits for its own copies of tile kt+1 (two tiles' copies may stay
  // in flight), so after it tile kt+1 is complete for everyone; every read of the slot a
  // copy refills (tile kt's, refilled with tile kt+STAGES after barrier kt) happens before
  // barrier kt. sched_barrier(0) pins every phase: the compiler may not move MFMAs
  // (register-only, so not ordered by s_barrier) across a phase boundary.
  // Measured exception: 256 x 256 tiles with both operands k-contiguous run faster with a
  // second barrier per k-tile, between the two phases (4096^3: 104.4 against 110.9 us,
  // 8192^3: 793 against 859 us, one box). With either operand m- or n-contiguous the single
  // barrier is as fast or up to 6 % faster, and so it is for smaller tiles in every layout
  // (128 x 128 on 1024 x 1024 x 8192: 56.5 against 69.9 us). The extra barrier only adds
  // ordering, so the slot argument above holds unchanged.
  constexpr bool kMidBarrier = OpA::KMAJOR && OpB::KMAJOR && BM == 256 && BN == 256;
  if (grp == 0) {
    for (int kt = 0; kt < nloc; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
      mma_tile_copy(kt + STAGES - 1, G0{});  // MFMAs of tile kt (fragments read before the barrier)
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<PT0 * (STAGES - 2)>();
      lds_barrier();                 // tile kt+1 landed everywhere; reads of tile kt done
      __builtin_amdgcn_sched_barrier(0);
      read_tile((kt + 1) % STAGES);  // (past the last tile: a settled slot, unused)
      copy_tile(kt + STAGES, G0{});
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kMidBarrier) lds_barrier();
    }
  } else {
    for (int kt = 0; kt < nloc; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
      read_tile(kt % STAGES);
      copy_tile(kt + STAGES - 1, G1{});
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<PT1 * (STAGES - 2)>();
      lds_barrier();                 // tile kt+1 landed everywhere; reads of tile kt done
      __builtin_amdgcn_sched_barrier(0);
      mma_tile_copy(kt + STAGES, G1{});  // MFMAs of tile kt
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kMidBarrier) lds_barrier();
    }
  }
  wait_vmcnt<0>();
  clk.loop_end();

  // Split-K fixup. Every split stores its fp32 partial tile to the workspace in register
  // order (thread tid's j-th group of 4 accumulators at float4 index j * NT + tid:
  // coalesced, and the reader needs no reshuffle) and counts itself in with one atomic on
  // the tile's counter. The split that brings the count to `splits` is the last: it
  // resets the counter for the next call, adds the partial tiles in split order 0, 1, ...
  // (the same order whichever split finishes last, so results are deterministic) and runs
  // the epilogue; the others are done. The partial tiles cross XCDs, whose L2s are not
  // coherent with each other: they are stored and loaded with the device-coherence cache
  // policy (sc1, what device-scope atomic accesses use), which goes to the coherence
  // point, so no L2 write-back or invalidation is needed; every wave waits for its stores
  // to complete before the barrier that precedes the counter update.
  if (splits > 1) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int NT = 64 * NW, Q = NACC / 4, TILE_BYTES = BM * BN * 4;
    constexpr int kDeviceCoherent = 16;  // cache policy bit sc1
    unsigned int* const counter = (unsigned int*)g.ws + tile_id;
    char* const parts = (char*)g.ws + g.ws_parts + (size_t)tile_id * splits * TILE_BYTES;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(parts, 0, splits * TILE_BYTES, kBufWord3);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          const f4 v = {acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]};
          const int off = split * TILE_BYTES + (((fm * FN + fn) * Q + q) * NT + tid) * 16;
          __builtin_amdgcn_raw_buffer_store_b128(v, prs, off, 0, kDeviceCoherent);
        }
    wait_vmcnt<0>();
    __syncthreads();  // (also: every copy into the ring has landed, so smem is free)
    if (tid == 0) {
      const unsigned int before = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = before == (unsigned int)(splits - 1);
      if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *(TG_LDS int*)smem = last;
    }
    __syncthreads();
    const int last = *(const TG_LDS int*)smem;
    if (!last) {
      clk.finish(nloc, TG_STAMP_TABLE);
      return;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          const int off = (((fm * FN + fn) * Q + q) * NT + tid) * 16;
          f4 sum = __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, kDeviceCoherent);
          for (int sp = 1; sp < splits; ++sp)
            sum += __builtin_amdgcn_raw_buffer_load_b128(prs, sp * TILE_BYTES + off, 0, kDeviceCoherent);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[fm][fn][4 * q + e] = sum[e];
        }
    __syncthreads();  // the flag in smem is overwritten by the staging below
  }

  // Epilogue. Lane holds, for tile (fm, fn), row fm*MF + lane % MF of the wave tile and
  // columns fn*MF + 8*g4 + 4*(lane / MF) .. +3 (32x32) or fn*16 + 4*(lane / 16) .. +3
  // (16x16). ReLU in fp32 and rounding to fp16 (nearest even) happen in registers; then
  // every wave stages its WTM x WTN fp16 sub-tile in its own LDS region (the ring is free:
  // every copy, including the empty-range ones past the last tile, has landed once all
  // waves pass the barrier below) and writes it back row by row, 16 bytes per lane and
  // WTN / 8 lanes per row, so each store covers whole 16-byte-aligned row segments instead
  // of 8-byte pieces of MF rows. The 16x16 layout uses StagedTile (conflict-free 16-byte
  // staging writes after a lane swap); the 32x32 one (a sweep-only config) uses
  // StagedTile32 (the same after a 32-lane swap). N and ldc are multiples of 8 on this path, so a
  // chunk is either wholly inside the matrix or wholly outside.
  if constexpr (MF == 16) {
    using ST = StagedTile<WTM, WTN>;
    static_assert(NW * ST::BYTES == staged_bytes(NW, WTM, WTN) &&
                      NW * ST::BYTES <= pp_launch_lds_bytes<BM, BN, BK, WM, WN, STAGES>(),
                  "the staged tiles fit in the launch's LDS");
    __syncthreads();
    char* const stage = smem + wave * ST::BYTES;
    if (g.relu != 0)
      ST::template stage<true>(stage, acc, lane);
    else
      ST::template stage<false>(stage, acc, lane);
    ST::wave_fence();
    ST::store(stage, lane, g.C + (int64_t)(row0 + wm * WTM) * g.ldc + col0 + wn * WTN, g.ldc, mvalid - wm * WTM,
              nvalid - wn * WTN);
  } else {
    using ST = StagedTile32<WTM, WTN>;
    static_assert(NW * ST::BYTES <= STAGES * (A_BYTES + B_BYTES), "the staged tile fits in the ring");
    __syncthreads();
    char* const stage = smem + wave * ST::BYTES;
    if (g.relu != 0)
      ST::template stage<true>(stage, acc, lane);
    else
      ST::template stage<false>(stage, acc, lane);
    ST::wave_fence();
    ST::store(stage, lane, g.C + (int64_t)(row0 + wm * WTM) * g.ldc + col0 + wn * WTN, g.ldc, mvalid - wm * WTM,
              nvalid - wn * WTN);
  }
  clk.finish(nloc, TG_STAMP_TABLE);
}


template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD, int MF, bool TA,
          bool TB>
__global__ __launch_bounds__(64 * WM * WN) void gemm_pingpong(GemmArgs g) {
  pingpong_body<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, TA, TB>(g, (int)blockIdx.x);
}

// Grouped GEMM: up to kMaxGroups independent GEMMs (same operand layout and ReLU flag, any
// sizes) in one launch. GEMM i owns workgroups [wg_start[i], wg_start[i+1]); a workgroup
// finds its GEMM by a scalar search over the (uniform) table in the kernel arguments.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD, int MF, bool TA,
          bool TB>
__global__ __launch_bounds__(64 * WM * WN) void gemm_pingpong_grouped(GroupedArgs ga) {
  const int b = (int)blockIdx.x;
  int gi = 0;
  while (gi + 1 < ga.count && b >= ga.wg_start[gi + 1]) ++gi;
  const GroupEntry& e = ga.e[gi];
  GemmArgs g;
  g.A = e.A;
  g.B = e.B;
  g.C = e.C;
  g.lda = e.lda;
  g.ldb = e.ldb;
  g.ldc = e.ldc;
  g.M = e.M;
  g.N = e.N;
  g.K = e.K;
  g.relu = ga.relu;
  g.tiles_m = e.tiles_m;
  g.tiles_n = e.tiles_n;
  g.layout = ga.layout;
  g.splits = 1;
  g.ws = nullptr;
  g.ws_parts = 0;
  pingpong_body<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, TA, TB>(g, b - ga.wg_start[gi]);
}

// ------------------------------------------------------------------------------------
// Quad kernel: 4 waves, one per SIMD, each owning a (BM / WM) x (BN / WN) sub-tile (128 x
// 128 for 256 x 256 tiles): 256 fp32 accumulators per lane and 16x16x32 MFMAs. Against the
// ping-pong's eight 128 x 64 wave tiles it reads a third fewer bytes from LDS per FLOP
// (every wave reads the A rows and B columns of its sub-tile once per k-tile), and LDS ->
// register traffic is what costs this power-limited part its clock under load.
//
// One wave per SIMD keeps its own MFMA pipe busy, so the k-tile's NS = FM * FN MFMAs run
// in a fixed order and every memory instruction has a fixed MFMA slot (QuadSchedule): the
// MFMAs go in 8 blocks, (A half h, B quarter q) for h = 0, 1 and q = 0 .. 3, each block
// FM/2 x FN/4 MFMAs with the A fragment changing slowest. Each fragment register is
// reloaded with the next k-tile's data two slots after its last use in this one, which
// leaves every read at least NS/2 - FM/2 - 2 slots (24 of 64 MFMAs, ~380 clocks for the
// 128 x 128 wave tile) before its first use, with one register set and no unrolling. Reads
// whose slot falls past the end of the k-tile are issued in slot 0 of the next one (they
// belong to that k-tile). The one barrier per k-tile sits right before the first read of
// the next tile: there every wave has finished reading this tile (its slot-0 reads have
// long completed) and this wave's copies of the next tile have landed, so after it the next
// tile may be read and this tile's ring slot takes the copies of tile t+STAGES, which go
// out one every NS/PT slots until the next barrier (so the copy stream of one tile straddles
// two iterations). Every iteration issues exactly PT copies (empty ranges past the last
// tile), so one constant s_waitcnt vmcnt(PT * (STAGES - 2)) finds the next tile landed.
// Fragment reads of the quad kernel with their per-lane offsets precomputed (what
// PpOperand::frag computes for k substep 0, hoisted out of the loop).
template <typename Op, int NF>
struct QuadFrags {
  static constexpr bool KMAJ = Op::KMAJOR;
  static constexpr int MF = Op::MFRAG, BKV = Op::BKV, RV = Op::RV;
  uint32_t off[KMAJ ? 1 : NF][2];
  __device__ void init(const Op& op) {
    if constexpr (KMAJ) {
      off[0][0] = op.fr_base + ((op.fr_k ^ op.fr_x) << 4);
    } else {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int k = 4 * i + op.fr_k;
          off[f][i] = k * RV * 2 + (((op.fr_x + (MF / 8) * f) ^ Op::swz(k)) << 4) + op.fr_half;
        }
    }
  }
  __device__ half8 read(const char* S, int f) const {
    if constexpr (KMAJ) {
      return *(const TG_LDS half8*)(S + off[0][0] + f * MF * BKV * 2);
    } else {
      const short4v h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS short4v*)(S + off[f][0]));
      const short4v h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS short4v*)(S + off[f][1]));
      return __builtin_bit_cast(half8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
};

template <int FM, int FN>
struct QuadSchedule {
  static constexpr int HM = FM / 2, QN = FN / 4, BLK = HM * QN, NS = FM * FN;
  static_assert(FM % 2 == 0 && FN % 4 == 0, "A in halves, B in quarters");
  // MFMA slot s -> (fm, fn)
  __host__ __device__ static constexpr int fm_of(int s) { return (s / BLK / 4) * HM + (s % BLK) / QN; }
  __host__ __device__ static constexpr int fn_of(int s) { return (s / BLK % 4) * QN + (s % BLK) % QN; }
  // last slot reading A fragment j / B fragment f
  __host__ __device__ static constexpr int last_a(int j) { return (4 * (j / HM) + 3) * BLK + (j % HM) * QN + QN - 1; }
  __host__ __device__ static constexpr int last_b(int f) { return (4 + f / QN) * BLK + (HM - 1) * QN + f % QN; }
  // slot after whose MFMA the reload is issued (>= NS: slot - NS of the next k-tile): GAP
  // slots after the last use, so the load never overwrites a register an MFMA still in
  // flight reads (which would cost hazard wait states)
  static constexpr int GAP = 2;
  __host__ __device__ static constexpr int read_a(int j) { return last_a(j) + GAP; }
  __host__ __device__ static constexpr int read_b(int f) { return last_b(f) + GAP; }
  // the barrier follows slot BAR: the last slot before the first read of the next tile
  __host__ __device__ static constexpr int first_next_read() {
    int m = 2 * NS;
    for (int j = 0; j < FM; ++j) m = read_a(j) < m ? read_a(j) : m;
    for (int f = 0; f < FN; ++f) m = read_b(f) < m ? read_b(f) : m;
    return m;
  }
  static constexpr int BAR = first_next_read() - 1;
  // LDS instructions issued after slot s's MFMA (reads of fragments reloaded there;
  // IA / IB instructions per A / B fragment)
  template <int IA, int IB>
  __host__ __device__ static constexpr int reads_at(int s) {
    int n = 0;
    for (int j = 0; j < FM; ++j) n += (read_a(j) % NS == s) ? IA : 0;
    for (int f = 0; f < FN; ++f) n += (read_b(f) % NS == s) ? IB : 0;
    return n;
  }
  // The first MFMA of a k-tile needs fragments reloaded late in the previous one. An
  // explicit wait after slot RETIRE, for all but the LDS instructions issued after the
  // later of those two reloads, tells the compiler they have completed (it cannot track
  // that many loads across the loop edge and would otherwise wait for every load issued
  // at the end of the k-tile): RETIRE is a few slots before the end, and RETIRE_N counts
  // the instructions issued after the later reload up to RETIRE.
  __host__ __device__ static constexpr int first_reload() {
    const int ra = read_a(fm_of(0)), rb = read_b(fn_of(0));
    return ra > rb ? ra : rb;
  }
  static constexpr int RETIRE = NS - 9;
  template <int IA, int IB>
  __host__ __device__ static constexpr int retire_n() {
    int n = 0;
    for (int s = first_reload() + 1; s <= RETIRE; ++s) n += reads_at<IA, IB>(s);
    return n;
  }
};

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD, bool TA, bool TB>
__global__ __launch_bounds__(64 * WM * WN) void gemm_quad(GemmArgs g) {
  WgClock clk;
  clk.start();
  constexpr int NW = WM * WN, MF = 16;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  using Q = QuadSchedule<FM, FN>;
  constexpr int NS = Q::NS;
  using OpA = PpOperand<pp_lds_extent(BM), BK, MF, !TA, NW>;
  using OpB = PpOperand<pp_lds_extent(BN), BK, MF, TB, NW>;
  constexpr int A_BYTES = OpA::BYTES, B_BYTES = OpB::BYTES;
  constexpr int PT = OpA::LD + OpB::LD;
  constexpr int CSTEP = NS / PT;               // slots between copies
  static_assert(NW == 4, "one wave per SIMD");
  static_assert(BK == 32, "one 16x16x32 MFMA step per k-tile");
  static_assert(NS % PT == 0 && Q::BAR >= 0 && Q::BAR < NS, "copy spacing and barrier slot");
  static_assert(STAGES >= 3 && PT * (STAGES - 1) < 64, "ring depth and vmcnt budget");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const a_lds = smem;
  char* const b_lds = smem + STAGES * A_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int64_t tm64, tn64;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, PANEL, XCD, &tm64, &tn64);
  const int row0 = (int)tm64 * BM, col0 = (int)tn64 * BN;
  const int mvalid = min(BM, g.M - row0), nvalid = min(BN, g.N - col0);
  const int nk = (g.K + BK - 1) / BK;
  const int kin_last = g.K - (nk - 1) * BK;

  OpA opa;
  OpB opb;
  opa.init_copies(g.A, g.lda, row0, mvalid, kin_last, wave, lane);
  opb.init_copies(g.B, g.ldb, col0, nvalid, kin_last, wave, lane);
  const uint32_t a_lds0 = lds_addr(a_lds) + wave * 1024;
  const uint32_t b_lds0 = lds_addr(b_lds) + wave * 1024;

  struct Dma {
    int4v ra, rb;
    uint32_t a_dst, b_dst;
    bool last;
  };
  auto dma_setup = [&](int t) {
    Dma d;
    d.ra = opa.rsrc(t, nk, nk);
    d.rb = opb.rsrc(t, nk, nk);
    const int slot = t % STAGES;
    d.a_dst = a_lds0 + slot * A_BYTES;
    d.b_dst = b_lds0 + slot * B_BYTES;
    d.last = t == nk - 1;
    return d;
  };
  // The descriptors of tile u >= STAGES from running source pointers (no 64-bit multiply
  // per k-tile); past the last tile the range is empty and the pointer is never used.
  const char* pa_next = opa.base + (int64_t)STAGES * opa.step;
  const char* pb_next = opb.base + (int64_t)STAGES * opb.step;
  auto dma_next = [&](int u) {
    Dma d;
    d.ra = make_rsrc(pa_next, u < nk - 1 ? opa.rng_full : (u == nk - 1 ? opa.rng_last : 0u));
    d.rb = make_rsrc(pb_next, u < nk - 1 ? opb.rng_full : (u == nk - 1 ? opb.rng_last : 0u));
    pa_next += opa.step;
    pb_next += opb.step;
    const int slot = u % STAGES;
    d.a_dst = a_lds0 + slot * A_BYTES;
    d.b_dst = b_lds0 + slot * B_BYTES;
    d.last = u == nk - 1;
    return d;
  };
  auto dma_one = [&](const Dma& d, int j) {
    if (j < OpA::LD)
      dma_to_lds(d.ra, d.a_dst + j * NW * 1024, d.last ? opa.off_last[j] : opa.off[j]);
    else
      dma_to_lds(d.rb, d.b_dst + (j - OpA::LD) * NW * 1024, opb.off[j - OpA::LD]);
  };

  const int wm = wave / WN, wn = wave % WN;
  opa.init_frags(wm * WTM, lane);
  opb.init_frags(wn * WTN, lane);

  half8 fa[FM], fb[FN];  // the wave's fragments: one set, each reloaded after its last use
  // Per-lane byte offsets of every fragment inside a ring slot, computed once: a K-major
  // operand needs one (fragment f sits f * MF rows further: an immediate offset), an
  // MN-major one two per fragment (the transposed reads' swizzled chunks).
  QuadFrags<OpA, FM> qa;
  QuadFrags<OpB, FN> qb;
  qa.init(opa);
  qb.init(opb);
  auto read_a = [&](int slot, int f) { fa[f] = qa.read(a_lds + slot * A_BYTES, f); };
  auto read_b = [&](int slot, int f) { fb[f] = qb.read(b_lds + slot * B_BYTES, f); };

  typedef float f4 __attribute__((ext_vector_type(4)));
  f4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  // Copies: copy c of tile t+STAGES goes out after slot BAR + 1 + c * CSTEP of iteration t
  // (past NS: in the next iteration). The prologue issues tiles 0 .. STAGES-2 and the
  // copies of tile STAGES-1 that iteration 0 would have issued in iteration -1.
  constexpr int C_WRAP = (NS - (Q::BAR + 1) + CSTEP - 1) / CSTEP;  // copies before the wrap
  static_assert(C_WRAP >= 1 && C_WRAP <= PT, "copy stream");
#pragma unroll
  for (int t = 0; t < STAGES; ++t) {
    const Dma d = dma_setup(t);
#pragma unroll
    for (int j = 0; j < (t < STAGES - 1 ? PT : C_WRAP); ++j) dma_one(d, j);
  }
  wait_vmcnt<PT * (STAGES - 2) + C_WRAP>();
  lds_barrier();
#pragma unroll
  for (int f = 0; f < FM; ++f) read_a(0, f);
#pragma unroll
  for (int f = 0; f < FN; ++f) read_b(0, f);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the loop starts with no load in flight

  // Slots [LO, HI) of iteration t. `dc` holds the copies' descriptor: tile t-1+STAGES before
  // the barrier, tile t+STAGES after it (set there).
  Dma dc = dma_setup(STAGES - 1);
  auto run_slots = [&](auto lo_c, auto hi_c, int t) {
    constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
    const int slot = t % STAGES, nslot = (t + 1) % STAGES;
    static_for_range<LO, HI>([&](auto sl_c) {
      constexpr int sl = decltype(sl_c)::value;
      constexpr int fm = Q::fm_of(sl), fn = Q::fn_of(sl);
      __builtin_amdgcn_sched_barrier(0);
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[fn], fa[fm], acc[fm][fn], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      // reloads: those past the end of the previous k-tile (this tile's data), and this
      // slot's reloads with the next tile's data
      static_for<FM>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        if constexpr (Q::read_a(j) >= NS && Q::read_a(j) - NS == sl) read_a(slot, j);
        if constexpr (Q::read_a(j) == sl) read_a(nslot, j);
      });
      static_for<FN>([&](auto f_c) {
        constexpr int f = decltype(f_c)::value;
        if constexpr (Q::read_b(f) >= NS && Q::read_b(f) - NS == sl) read_b(slot, f);
        if constexpr (Q::read_b(f) == sl) read_b(nslot, f);
      });
      static_for<PT>([&](auto c_c) {
        constexpr int c = decltype(c_c)::value;
        constexpr int at = Q::BAR + 1 + c * CSTEP;
        if constexpr ((at >= NS && at - NS == sl) || at == sl) dma_one(dc, c);
      });
      if constexpr (sl == Q::RETIRE) {
        constexpr int IA = QuadFrags<OpA, FM>::KMAJ ? 1 : 2, IB = QuadFrags<OpB, FN>::KMAJ ? 1 : 2;
        constexpr int N = Q::template retire_n<IA, IB>();
        static_assert(N >= 0 && N < 16, "lgkmcnt range");
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));  // lgkmcnt(N) only
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (sl == Q::BAR) {
        __builtin_amdgcn_sched_barrier(0);
        // this tile fully read by every wave; this wave's copies of the next tile landed
        wait_vmcnt<PT * (STAGES - 2)>();
        lds_barrier();
        dc = dma_next(t + STAGES);
      }
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  using Zero = std::integral_constant<int, 0>;
  using End = std::integral_constant<int, NS>;
  clk.loop_begin();
  for (int t = 0; t < nk; ++t) run_slots(Zero{}, End{}, t);
  wait_vmcnt<0>();  // the copies past the last tile write zeros: drained before LDS is reused
  clk.loop_end();

  // Epilogue: ReLU and RNE in registers, each wave's WTM x WTN fp16 sub-tile staged in its
  // own LDS region and written back in 16-byte row segments (StagedTile).
  using ST = StagedTile<WTM, WTN>;
  static_assert(NW * ST::BYTES <= STAGES * (A_BYTES + B_BYTES), "the staged tile fits in the ring");
  __syncthreads();
  char* const stage = smem + wave * ST::BYTES;
  // The ReLU choice is made once for the whole tile (a per-value branch on the runtime
  // flag costs registers at 256 accumulators).
  if (g.relu != 0)
    ST::template stage<true>(stage, acc, lane);
  else
    ST::template stage<false>(stage, acc, lane);
  ST::wave_fence();
  ST::store(stage, lane, g.C + (int64_t)(row0 + wm * WTM) * g.ldc + col0 + wn * WTN, g.ldc, mvalid - wm * WTM,
            nvalid - wn * WTN);
  clk.finish(nk, TG_STAMP_TABLE);
}

// ------------------------------------------------------------------------------------
// Generic kernel: 64 x 64 x 32 tile, 4 waves (2 x 2 of 32 x 32), element-wise predicated
// loads (any 2-byte-aligned pointers, any strides and sizes, any operand layout). A is
// staged as [m][k] and B transposed to [n][k] in LDS so both fragments are plain 16-byte
// reads.
constexpr int GB_M = 64, GB_N = 64, GB_K = 32, G_PAD = 8;

__global__ __launch_bounds__(256) void gemm_generic(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) _Float16 As[GB_M][GB_K + G_PAD];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[GB_N][GB_K + G_PAD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, 1, 0, &tm, &tn);
  const int row0 = (int)tm * GB_M, col0 = (int)tn * GB_N;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lhi = lane >> 5;

  float16v acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  for (int k0 = 0; k0 < g.K; k0 += GB_K) {
#pragma unroll
    for (int e = 0; e < (GB_M * GB_K) / 256; ++e) {
      const int idx = tid + 256 * e;
      const int r = idx / GB_K, kk = idx % GB_K;
      const int gr = row0 + r, gk = k0 + kk;
      const int64_t ia = (g.layout & 2) ? (int64_t)gk * g.lda + gr : (int64_t)gr * g.lda + gk;
      As[r][kk] = (gr < g.M && gk < g.K) ? g.A[ia] : (_Float16)0.0f;
    }
#pragma unroll
    for (int e = 0; e < (GB_K * GB_N) / 256; ++e) {
      const int idx = tid + 256 * e;
      const int kk = idx / GB_N, n = idx % GB_N;
      const int gk = k0 + kk, gc = col0 + n;
      const int64_t ib = (g.layout & 1) ? (int64_t)gc * g.ldb + gk : (int64_t)gk * g.ldb + gc;
      Bs[n][kk] = (gk < g.K && gc < g.N) ? g.B[ib] : (_Float16)0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < GB_K / 16; ++ks) {
      const half8 a = *(const half8*)&As[wm * 32 + l32][16 * ks + 8 * lhi];
      const half8 b = *(const half8*)&Bs[wn * 32 + l32][16 * ks + 8 * lhi];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  const int m = row0 + wm * 32 + l32;
  if (m >= g.M) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int n = col0 + wn * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
    if (n < g.N) {
      const float v = g.relu ? relu_f(acc[r]) : acc[r];
      g.C[(int64_t)m * g.ldc + n] = (_Float16)v;
    }
  }
}

#ifdef TGEMM_STAMPS
// MFMA throughput probe (tooling, not part of the GEMM): every wave keeps independent
// accumulators and issues MFMAs on them back to back, `iters` rounds of kProbeMfmaPerIter x
// 16384 FLOP, with no memory traffic to speak of. Each thread then stores the sum of its
// accumulators so the work stays live. Measures the MFMA rate this board sustains at its
// power limit. The operands decide how much the multipliers toggle, and so the power:
//   MODE 0: register operands filled with pseudo-random binary16 values (random sign and
//           mantissa, magnitudes 2^-2 to 2^1), 16x16x32 MFMAs, 16 accumulators;
//   MODE 1: operands loaded once from `ops` (64 binary16 values per thread, for instance
//           samples of the workloads' N(0,1) inputs), 16x16x32 MFMAs;
//   MODE 2: as MODE 1 with 32x32x16 MFMAs (8 accumulators of 16 floats: the same FLOP per
//           round);
//   MODE 3: as MODE 1 plus the LDS read rate of the 256 x 256 ping-pong kernel (per wave,
//           6 ds_read_b128 per 16 MFMAs) from a 64 KiB block holding the same values; each
//           round's reads are the next round's operands, so they stay live.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe(int iters, const _Float16* ops, float* out) {
  WgClock clk;
  clk.start();
  const uint32_t tid = blockIdx.x * kProbeThreads + threadIdx.x;
  half8 a[4], b[4];
  if constexpr (MODE == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t ha = mix32(tid * 64u + 8u * i + e), hb = mix32(~(tid * 64u + 8u * i + e));
        const uint16_t ba = (uint16_t)(((ha >> 31) << 15) | ((13u + ((ha >> 10) & 3u)) << 10) | (ha & 0x3FFu));
        const uint16_t bb = (uint16_t)(((hb >> 31) << 15) | ((13u + ((hb >> 10) & 3u)) << 10) | (hb & 0x3FFu));
        a[i][e] = __builtin_bit_cast(_Float16, ba);
        b[i][e] = __builtin_bit_cast(_Float16, bb);
      }
  } else {
    const half8* const src = reinterpret_cast<const half8*>(ops) + threadIdx.x * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = src[i];
      b[i] = src[4 + i];
    }
  }
  typedef float float4v __attribute__((ext_vector_type(4)));
  float sum = 0.0f;
  if constexpr (MODE == 2) {
    constexpr int NACC = kProbeMfmaPerIter / 2;
    float16v acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    clk.loop_begin();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < NACC; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j & 3], a[j >> 1 & 3], acc[j], 0, 0, 0);
    }
    clk.loop_end();
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[j][r];
  } else {
    float4v acc[kProbeMfmaPerIter];
#pragma unroll
    for (int j = 0; j < kProbeMfmaPerIter; ++j) acc[j] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (MODE == 3) {
      // 64 KiB block: thread t's 64 values at bytes [128 t, 128 t + 128). Read j of a round
      // takes one contiguous KiB (conflict-free), at an offset that moves every round.
      __shared__ __attribute__((aligned(16))) char blk[kProbeThreads * 128];
      half8* const mine = reinterpret_cast<half8*>(blk + threadIdx.x * 128);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mine[i] = a[i];
        mine[4 + i] = b[i];
      }
      __syncthreads();
      const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
      clk.loop_begin();
      for (int it = 0; it < iters; ++it) {
        half8 na[3], nb[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const uint32_t base = ((wave * 6u + 2u * j + (uint32_t)it * 48u) & 63u) * 1024u + lane * 16u;
          na[j] = *reinterpret_cast<const half8*>(blk + base);
          nb[j] = *reinterpret_cast<const half8*>(blk + ((base + 1024u) & 0xFFFFu));
        }
#pragma unroll
        for (int j = 0; j < kProbeMfmaPerIter; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j & 3], a[j >> 2], acc[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          a[j] = na[j];
          b[j] = nb[j];
        }
      }
      clk.loop_end();
    } else {
      clk.loop_begin();
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kProbeMfmaPerIter; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j & 3], a[j >> 2], acc[j], 0, 0, 0);
      }
      clk.loop_end();
    }
#pragma unroll
    for (int j = 0; j < kProbeMfmaPerIter; ++j) sum += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  }
  out[tid] = sum;
  clk.finish(iters, TG_STAMP_TABLE);
}

// LDS access probe (tooling): one wave per workgroup issues `iters` rounds of p.ni LDS
// instructions of kind OP, instruction j of a round at byte address p.addr[j][lane] of a
// 64 KiB dynamic LDS block by the lanes set in p.active[j], then waits for them. Run under
// the SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS counters, it gives the bank-conflict cycles of
// any lane address pattern (the calibration of the host-side bank model). The block is
// not initialised (only the access pattern matters). The host checks every address
// against the block and the access width before launching.
typedef int int2v __attribute__((ext_vector_type(2)));

template <int OP>
__global__ __launch_bounds__(64) void lds_probe(LdsProbeArgs p) {
  extern __shared__ __attribute__((aligned(16))) char lds_block[];
  const int lane = threadIdx.x;
  const uint32_t base = lds_addr(lds_block);
  uint32_t a[kLdsProbeSlots];
#pragma unroll
  for (int j = 0; j < kLdsProbeSlots; ++j) a[j] = base + (uint32_t)p.addr[j][lane];
  const int4v w4 = {lane, lane + 1, lane + 2, lane + 3};
  for (int it = 0; it < p.iters; ++it) {
#pragma unroll
    for (int j = 0; j < kLdsProbeSlots; ++j) {
      if (j >= p.ni) break;
      if (!((p.active[j] >> lane) & 1)) continue;
      if (OP == 0) {
        int v;
        asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(a[j]) : "memory");
        asm volatile("" : : "v"(v));
      } else if (OP == 1) {
        int2v v;
        asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(a[j]) : "memory");
        asm volatile("" : : "v"(v));
      } else if (OP == 2) {
        int4v v;
        asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a[j]) : "memory");
        asm volatile("" : : "v"(v));
      } else if (OP == 3) {
        asm volatile("ds_write_b32 %0, %1" : : "v"(a[j]), "v"(w4[0]) : "memory");
      } else if (OP == 4) {
        const int2v w2 = {w4[0], w4[1]};
        asm volatile("ds_write_b64 %0, %1" : : "v"(a[j]), "v"(w2) : "memory");
      } else if (OP == 5) {
        asm volatile("ds_write_b128 %0, %1" : : "v"(a[j]), "v"(w4) : "memory");
      } else {
        int2v v;
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a[j]) : "memory");
        asm volatile("" : : "v"(v));
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  }
  if (lane == 0) p.out[blockIdx.x] = (float)p.iters;
}

#endif  // TGEMM_STAMPS

// C[i, j] = +0 for i < M, j < N (the empty sum when K == 0).
__global__ __launch_bounds__(256) void zero_fill(_Float16* C, int M, int N, int64_t ldc) {
  const int64_t total = (int64_t)M * N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = t / N, j = t - i * N;
    C[i * ldc + j] = (_Float16)0.0f;
  }
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD>
hipError_t launch_fast(const GemmArgs& g, hipStream_t s, int device) {
  constexpr int lds = STAGES * (BM * BK + BK * BN) * 2;
  auto kern = gemm_fast<BM, BN, BK, WM, WN, STAGES, PANEL, XCD>;
  // Opt in to more than 64 KiB of dynamic LDS, once per device.
  static std::atomic<uint64_t> ready{0};
  const uint64_t bit = 1ull << (device & 63);
  if (!(ready.load(std::memory_order_acquire) & bit)) {
    const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    ready.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int64_t nwg = (int64_t)g.tiles_m * g.tiles_n;
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * WM * WN), lds, s, g);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD, int MF, bool TA, bool TB>
hipError_t launch_pp_layout(const GemmArgs& g, hipStream_t s, int device) {
  constexpr int lds = pp_launch_lds_bytes<BM, BN, BK, WM, WN, STAGES>();
  auto kern = gemm_pingpong<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, TA, TB>;
  static std::atomic<uint64_t> ready{0};
  const uint64_t bit = 1ull << (device & 63);
  if (!(ready.load(std::memory_order_acquire) & bit)) {
    const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    ready.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int64_t nwg = (int64_t)g.tiles_m * g.tiles_n * g.splits;  // splits per tile
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * WM * WN), lds, s, g);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD, int MF, bool TA, bool TB>
hipError_t launch_pp_grouped_layout(const GroupedArgs& ga, int64_t nwg, hipStream_t s, int device) {
  constexpr int lds = pp_launch_lds_bytes<BM, BN, BK, WM, WN, STAGES>();
  auto kern = gemm_pingpong_grouped<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, TA, TB>;
  static std::atomic<uint64_t> ready{0};
  const uint64_t bit = 1ull << (device & 63);
  if (!(ready.load(std::memory_order_acquire) & bit)) {
    const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    ready.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * WM * WN), lds, s, ga);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD, int MF>
hipError_t launch_pp_grouped(const GroupedArgs& ga, int64_t nwg, hipStream_t s, int device) {
  switch (ga.layout) {
    case 1: return launch_pp_grouped_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, false, true>(ga, nwg, s, device);
    case 2: return launch_pp_grouped_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, true, false>(ga, nwg, s, device);
    case 3: return launch_pp_grouped_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, true, true>(ga, nwg, s, device);
    default: return launch_pp_grouped_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, false, false>(ga, nwg, s, device);
  }
}

// ALL: the config is instantiated for every operand layout (g.layout = 2 * trans_a +
// trans_b); otherwise only for A and B as given (the host never sends it another layout).
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD, int MF, bool ALL>
hipError_t launch_pp(const GemmArgs& g, hipStream_t s, int device) {
  if constexpr (ALL) {
    switch (g.layout) {
      case 1: return launch_pp_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, false, true>(g, s, device);
      case 2: return launch_pp_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, true, false>(g, s, device);
      case 3: return launch_pp_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, true, true>(g, s, device);
      default: break;
    }
  } else {
    if (g.layout != 0) return hipErrorInvalidValue;
  }
  return launch_pp_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, MF, false, false>(g, s, device);
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD, bool TA, bool TB>
hipError_t launch_quad_layout(const GemmArgs& g, hipStream_t s, int device) {
  constexpr int lds = pp_lds_bytes<BM, BN, BK, STAGES>();
  auto kern = gemm_quad<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, TA, TB>;
  static std::atomic<uint64_t> ready{0};
  const uint64_t bit = 1ull << (device & 63);
  if (!(ready.load(std::memory_order_acquire) & bit)) {
    const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    ready.fetch_or(bit, std::memory_order_acq_rel);
  }
  if (g.splits != 1) return hipErrorInvalidValue;
  const int64_t nwg = (int64_t)g.tiles_m * g.tiles_n;
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * WM * WN), lds, s, g);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD, bool ALL>
hipError_t launch_quad(const GemmArgs& g, hipStream_t s, int device) {
  if constexpr (ALL) {
    switch (g.layout) {
      case 1: return launch_quad_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, false, true>(g, s, device);
      case 2: return launch_quad_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, true, false>(g, s, device);
      case 3: return launch_quad_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, true, true>(g, s, device);
      default: break;
    }
  } else {
    if (g.layout != 0) return hipErrorInvalidValue;
  }
  return launch_quad_layout<BM, BN, BK, WM, WN, STAGES, PANEL, XCD, false, false>(g, s, device);
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int PANEL, int XCD>
hipError_t launch_pipe(const GemmArgs& g, hipStream_t s, int device) {
  constexpr int lds = STAGES * (BM * BK + BK * BN) * 2;
  auto kern = gemm_pipe<BM, BN, BK, WM, WN, STAGES, PANEL, XCD>;
  static std::atomic<uint64_t> ready{0};
  const uint64_t bit = 1ull << (device & 63);
  if (!(ready.load(std::memory_order_acquire) & bit)) {
    const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    ready.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int64_t nwg = (int64_t)g.tiles_m * g.tiles_n;
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * WM * WN), lds, s, g);
  return hipGetLastError();
}

hipError_t launch_generic(const GemmArgs& g, hipStream_t s, int) {
  const int64_t nwg = (int64_t)g.tiles_m * g.tiles_n;
  hipLaunchKernelGGL(gemm_generic, dim3((unsigned)nwg), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

#ifdef TGEMM_STAMPS
hipError_t launch_lds_probe(int op, int blocks, const LdsProbeArgs& p, hipStream_t s) {
  typedef void (*K)(LdsProbeArgs);
  static const K kernels[kLdsProbeOps] = {lds_probe<0>, lds_probe<1>, lds_probe<2>, lds_probe<3>,
                                          lds_probe<4>, lds_probe<5>, lds_probe<6>};
  if (op < 0 || op >= kLdsProbeOps) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernels[op], dim3((unsigned)blocks), dim3(64), kLdsProbeBytes, s, p);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int mode, int blocks, int iters, const _Float16* ops, float* out, hipStream_t s) {
  static void (*const kernels[kProbeModes])(int, const _Float16*, float*) = {mfma_probe<0>, mfma_probe<1>,
                                                                             mfma_probe<2>, mfma_probe<3>};
  if (mode < 0 || mode >= kProbeModes) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernels[mode], dim3((unsigned)blocks), dim3(kProbeThreads), 0, s, iters, ops, out);
  return hipGetLastError();
}

hipError_t stamps_read(unsigned long long* host, int64_t words) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_stamps), (size_t)words * sizeof(unsigned long long), 0,
                             hipMemcpyDeviceToHost);
}
unsigned long long* stamps_table() {
  void* p = nullptr;
  return hipGetSymbolAddress(&p, HIP_SYMBOL(g_stamps)) == hipSuccess ? static_cast<unsigned long long*>(p) : nullptr;
}

hipError_t stamps_clear() {
  static const unsigned long long zeros[kStampWorkgroups * kStampWords] = {};
  return hipMemcpyToSymbol(HIP_SYMBOL(g_stamps), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice);
}
#endif

hipError_t launch_zero_fill(_Float16* C, int M, int N, int64_t ldc, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_fill, dim3((unsigned)blocks), dim3(256), 0, s, C, M, N, ldc);
  return hipGetLastError();
}

// The config table: the X-macro lists of tgemm_configs.h drive both the table rows and the
// kernel instantiations, so a row always describes the kernel it launches. Rows this build
// does not compile keep their place in the table, marked not built, with a launcher that
// refuses (the host never calls it: it checks `built` first).
static hipError_t launch_unbuilt(const GemmArgs&, hipStream_t, int) { return hipErrorNotSupported; }

#define TGEMM_ROW(BM, BN, BK, WM, WN, S, P, X, PROD) \
  {BM, BN, BK, S, WM, WN, P, X, 0, 1, TGEMM_BUILT(PROD), "t" #BM "x" #BN "x" #BK "_s" #S "_w" #WM "x" #WN "_p" #P "_x" #X},
#define TGEMM_LAUNCHER(BM, BN, BK, WM, WN, S, P, X, PROD) \
  TGEMM_IF_BUILT(PROD, (launch_fast<BM, BN, BK, WM, WN, S, P, X>), launch_unbuilt),
#define TGEMM_COUNT(...) 0,
#define TGEMM_PIPE_ROW(BM, BN, BK, WM, WN, S, P, X, PROD) \
  {BM, BN, BK, S, WM, WN, P, X, 0, 1, TGEMM_BUILT(PROD), "p" #BM "x" #BN "x" #BK "_s" #S "_w" #WM "x" #WN "_p" #P "_x" #X},
#define TGEMM_PIPE_LAUNCHER(BM, BN, BK, WM, WN, S, P, X, PROD) \
  TGEMM_IF_BUILT(PROD, (launch_pipe<BM, BN, BK, WM, WN, S, P, X>), launch_unbuilt),
#define TGEMM_PP_ROW(BM, BN, BK, WM, WN, S, P, X, PROD) \
  {BM, BN, BK, S, WM, WN, P, X, 0, 1, TGEMM_BUILT(PROD), "q" #BM "x" #BN "x" #BK "_s" #S "_w" #WM "x" #WN "_p" #P "_x" #X},
#define TGEMM_PP_LAUNCHER(BM, BN, BK, WM, WN, S, P, X, PROD) \
  TGEMM_IF_BUILT(PROD, (launch_pp<BM, BN, BK, WM, WN, S, P, X, 32, false>), launch_unbuilt),
#define TGEMM_PP1_ROW(BM, BN, BK, WM, WN, S, P, X, ALL, PROD)                                                 \
  {BM, BN, BK, S, WM, WN, P, X, 0, ALL ? 0xF : 1, TGEMM_BUILT(PROD),                                        \
   "m" #BM "x" #BN "x" #BK "_s" #S "_w" #WM "x" #WN "_p" #P "_x" #X},
#define TGEMM_PP1_LAUNCHER(BM, BN, BK, WM, WN, S, P, X, ALL, PROD) \
  TGEMM_IF_BUILT(PROD, (launch_pp<BM, BN, BK, WM, WN, S, P, X, 16, ALL>), launch_unbuilt),
#define TGEMM_QUAD_ROW(BM, BN, BK, WM, WN, S, P, X, ALL, PROD)                                                \
  {BM, BN, BK, S, WM, WN, P, X, 0, ALL ? 0xF : 1, TGEMM_BUILT(PROD),                                        \
   "u" #BM "x" #BN "x" #BK "_s" #S "_w" #WM "x" #WN "_p" #P "_x" #X},
#define TGEMM_QUAD_LAUNCHER(BM, BN, BK, WM, WN, S, P, X, ALL, PROD) \
  TGEMM_IF_BUILT(PROD, (launch_quad<BM, BN, BK, WM, WN, S, P, X, ALL>), launch_unbuilt),

// Function-local statics: host-only tables (the device pass parses these bodies, which
// instantiates every kernel, but emits no host data).
const Config* config_table(int* count) {
  static const Config table[] = {
      {GB_M, GB_N, GB_K, 1, 2, 2, 1, 0, 1, 0xF, 1, "generic_64x64x32"},
      TGEMM_FAST_CONFIGS(TGEMM_ROW) TGEMM_PIPE_CONFIGS(TGEMM_PIPE_ROW) TGEMM_PP_CONFIGS(TGEMM_PP_ROW)
          TGEMM_PP1_CONFIGS(TGEMM_PP1_ROW) TGEMM_QUAD_CONFIGS(TGEMM_QUAD_ROW)
              TGEMM_PIPE2_CONFIGS(TGEMM_PIPE_ROW)};
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

// Grouped launchers exist for the two ping-pong configs the grouped entry point uses
// (9: 256 x 256, 15: 128 x 128); the table rows are checked against these shapes.
GroupedLauncher grouped_launcher(int idx) {
  int n = 0;
  const Config* t = config_table(&n);
  if (idx < 0 || idx >= n) return nullptr;
  const Config& c = t[idx];
  if (c.generic || c.layouts != 0xF || c.bk != 32 || c.stages != 4 || c.waves_m != 2 || c.waves_n != 4 ||
      c.panel != 4 || c.xcd_remap != 1)
    return nullptr;
  if (c.bm == 256 && c.bn == 256) return launch_pp_grouped<256, 256, 32, 2, 4, 4, 4, 1, 16>;
  if (c.bm == 128 && c.bn == 128) return launch_pp_grouped<128, 128, 32, 2, 4, 4, 4, 1, 16>;
  return nullptr;
}

Launcher launcher(int idx) {
  static const Launcher table[] = {launch_generic, TGEMM_FAST_CONFIGS(TGEMM_LAUNCHER)
                                       TGEMM_PIPE_CONFIGS(TGEMM_PIPE_LAUNCHER)
                                           TGEMM_PP_CONFIGS(TGEMM_PP_LAUNCHER)
                                               TGEMM_PP1_CONFIGS(TGEMM_PP1_LAUNCHER)
                                                   TGEMM_QUAD_CONFIGS(TGEMM_QUAD_LAUNCHER)
                                                       TGEMM_PIPE2_CONFIGS(TGEMM_PIPE_LAUNCHER)};
  static_assert(sizeof(table) / sizeof(table[0]) ==
                    1 + sizeof((int[]){TGEMM_FAST_CONFIGS(TGEMM_COUNT) TGEMM_PIPE_CONFIGS(TGEMM_COUNT)
                                           TGEMM_PP_CONFIGS(TGEMM_COUNT) TGEMM_PP1_CONFIGS(TGEMM_COUNT)
                                               TGEMM_QUAD_CONFIGS(TGEMM_COUNT) TGEMM_PIPE2_CONFIGS(TGEMM_COUNT)}) /
                            sizeof(int),
                "one launcher per config");
  return table[idx];
}

}  // namespace tgemm
