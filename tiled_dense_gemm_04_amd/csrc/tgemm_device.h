// tgemm_device.h -- device-side building blocks shared by the gfx950 kernels of libtgemm
// (fp16 kernels in tgemm_kernels.hip, fp8 block-scaled kernels in tgemm_fp8.hip): vector
// types, raw buffer descriptors, buffer->LDS copies, wait/barrier helpers, the LDS
// swizzles and the operand staging of the ping-pong kernels. Everything has internal
// linkage: each kernel source gets its own copy.
#pragma once

#include "tgemm_internal.h"

namespace tgemm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
#define TG_LDS __attribute__((address_space(3)))

// Buffer offset that lies beyond every descriptor range used here (all ranges are kept
// below 2^31 bytes), so a load at this offset returns zeros.
constexpr uint32_t kOob = 0x80000000u;
constexpr uint32_t kMaxRange = 0x7FFFFFF0u;
// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format, no swizzle).
constexpr int kBufWord3 = 0x00020000;

// s_waitcnt with only the vector-memory counter constrained (expcnt and lgkmcnt at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS reads/writes, then
// s_barrier. Outstanding buffer->LDS loads of later stages stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1, expanded at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// The same for I = LO .. HI-1.
template <int LO, int HI, typename F>
__device__ __forceinline__ void static_for_range(F&& f) {
  static_for<HI - LO>([&](auto i) { f(std::integral_constant<int, LO + decltype(i)::value>{}); });
}

__device__ __forceinline__ float relu_f(float x) { return x > 0.0f ? x : 0.0f; }

// Stores of the output tile are non-temporal 16-byte chunks: C is written once and not read
// back by the kernel, so it streams out instead of leaving dirty lines in L2 and the
// Infinity Cache to be written back later (4096^3 + ReLU: 105.6 against 107.2 us with
// ordinary stores, 8192^3: 810 against 823 us). Ordinary stores look faster where rows
// straddle 128-byte lines (4095 x 3000 x 1000: 28.3 against 31.0 us) only while every call
// rewrites the same C: with the buffers rotated past the caches the deferred write-backs
// of the partial lines cost more (38.3 against 31.3 us). 8-byte pieces stream badly (the
// pipelined kernel's former direct epilogue, 1024^3: 11.4 us), so every product kernel
// stages its tile and stores whole 16-byte chunks (1024^3: 9.9 us).
template <typename V>
__device__ __forceinline__ void store_c(_Float16* p, const V& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}

// Per-workgroup timestamps, compiled in only for the instrumented build (TGEMM_STAMPS) and
// empty otherwise; finish() writes them to the table it is given (the library's one table,
// defined next to the binary16 kernels and handed to the other kernels as an argument). Words per workgroup: wall clock (s_memrealtime, 100 MHz) at kernel
// start, main-loop start, main-loop end and after every wave's stores completed; shader
// clock ticks (s_memtime, which counts at the current shader clock) from kernel start to
// main-loop end; main-loop iterations; threads per workgroup; 1 (written). Ticks divided
// by wall time is the shader clock the workgroup ran at.
#ifdef TGEMM_STAMPS
struct WgClock {
  unsigned long long rt0, ct0, rt1, rt2, ct2;
  __device__ void start() {
    rt0 = __builtin_amdgcn_s_memrealtime();
    ct0 = __builtin_amdgcn_s_memtime();
  }
  __device__ void loop_begin() { rt1 = __builtin_amdgcn_s_memrealtime(); }
  __device__ void loop_end() {
    rt2 = __builtin_amdgcn_s_memrealtime();
    ct2 = __builtin_amdgcn_s_memtime();
  }
  // Called by every thread of the workgroup, at its very end.
  __device__ void finish(int iterations, unsigned long long* table) {
    wait_vmcnt<0>();
    __syncthreads();
    if (table != nullptr && threadIdx.x == 0 && blockIdx.x < (unsigned)kStampWorkgroups) {
      unsigned long long* o = &table[(size_t)blockIdx.x * kStampWords];
      o[0] = rt0;
      o[1] = rt1;
      o[2] = rt2;
      o[3] = __builtin_amdgcn_s_memrealtime();
      o[4] = ct2 - ct0;
      o[5] = (unsigned long long)iterations;
      o[6] = blockDim.x;
      o[7] = 1;
    }
  }
};
#else
struct WgClock {
  __device__ void start() {}
  __device__ void loop_begin() {}
  __device__ void loop_end() {}
  __device__ void finish(int, unsigned long long*) {}
};
#endif

typedef int int4v __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base address, stride 0, range in bytes, gfx9 word 3. All inputs
// are wave-uniform, so it lives in four SGPRs.
__device__ __forceinline__ int4v make_rsrc(const void* base, uint32_t range_bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  int4v r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)range_bytes);
  r[3] = kBufWord3;
  return r;
}

// One 16-byte buffer load per lane written straight to LDS: lane u's 16 bytes land at
// LDS byte lds_base + 16*u; a lane whose offset is outside the descriptor range writes
// zeros. Written as inline assembly so that the compiler does not treat the LDS write
// as pending before unrelated LDS reads (it cannot tell the ring slots apart and would
// wait for every copy in flight); completion is awaited explicitly with wait_vmcnt.
// M0 carries the LDS base; the kernels use M0 for nothing else (no indirect register
// indexing, no messages), so clobbering it is safe here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// TGEMM_DEBUG_FILL (a debugging build, never the product): every copy first overwrites its
// destination with all-ones bytes (a NaN as binary16, as an E4M3 code and as float32) and
// waits for that write, then issues the copy. A read of a slot before its copy has landed
// (a missing wait or barrier), or after the next copy into it was issued (a slot reused too
// early), then sees NaN, which reaches the output.
#ifdef TGEMM_DEBUG_FILL
__device__ __forceinline__ void debug_poison(uint32_t lds_base, int bytes_per_lane) {
  const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const uint32_t a = lds_base + lane * (uint32_t)bytes_per_lane;
  const int4v ones = {-1, -1, -1, -1};
  if (bytes_per_lane == 16)
    asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(a), "v"(ones) : "memory");
  else
    asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(a), "v"(-1) : "memory");
}
#endif

__device__ __forceinline__ void dma_to_lds(const int4v& rsrc, uint32_t lds_base, uint32_t voffset) {
#ifdef TGEMM_DEBUG_FILL
  debug_poison(lds_base, 16);
#endif
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const TG_LDS char*)p;
}

// ------------------------------------------------------------------------------------
// LDS layouts of the fast kernel.
//
// A stage: BM rows x BK halves, row r at byte r*BK*2, split in 16-byte chunks; logical
// chunk c of row r is stored at chunk c ^ swz_a(r). A fragment read (ds_read_b128) has 16
// lanes on 16 consecutive rows and the same logical chunk; with 64 banks x 4 bytes a
// 256-byte bank window holds 128/BK rows, and the XOR spreads the 16 rows over the 16
// chunk slots of the window.
template <int BK>
__host__ __device__ constexpr int swz_a(int r) {
  return (r / (128 / BK)) % (BK / 8);
}
// The same for 16x16x32 A fragments (16 lanes on 16 rows, four lane groups on the four
// 16-byte chunks of a 64-byte row, BK = 32). Measured with SQ_LDS_BANK_CONFLICT on gfx950:
// XOR by (r / 2) % 4 is conflict-free for this pattern, while (r / 4) % 4 (the 32x32x16
// choice above) conflicts 2-way. Rows of BK = 64 halves (the 128-byte rows of the fp8
// kernels) take (r / 2) % 8: two rows share a 256-byte bank window, and the XOR puts the
// 16 rows read by one instruction on 16 distinct 16-byte slots of it.
template <int BK, int MF>
__host__ __device__ constexpr int swz_a_mf(int r) {
  static_assert(MF == 32 || BK == 32 || BK == 64, "16x16 fragments are laid out for BK = 32 or 64");
  return MF == 16 ? (r >> 1) & (BK / 8 - 1) : swz_a<BK>(r);
}
// B stage: BK rows (k) x BN halves (n), row k at byte k*BN*2 (a multiple of 256 bytes);
// logical chunk c of row k is stored at chunk c ^ swz_b(k). A transposed read by 32 lanes
// touches either 4 consecutive k rows x 4 consecutive chunks (32x32x16 B fragments,
// c0 % 4 == 0, k < 8 within the group of 8) or rows k and k+8 for 4 consecutive k x 2
// chunks (16x16x32 fragments, c0 % 2 == 0). XOR by 4*(k%4) spreads the four rows of a
// group, XOR by 2*((k/8)%2) separates rows k and k+8: in both patterns the 16 (row,
// chunk) pairs land on 16 distinct 16-byte slots of the bank window.
__host__ __device__ constexpr int swz_b(int k) { return (4 * (k & 3)) ^ (2 * ((k >> 3) & 1)); }
// MN-major rows of 384 bytes (192 columns): row k starts 128 bytes further into the bank
// window than row k - 1, so the window position of a chunk depends on k % 2 as well. XOR by
// 2 ((k / 2) % 2) + 4 ((k / 8) % 2) spreads the 16 (row, chunk) pairs of a 16x16
// transposed read over 16 distinct 16-byte slots (checked with the host-side bank model)
// and keeps every chunk inside its row (only bits 1 and 2 of the chunk index change).
__host__ __device__ constexpr int swz_b384(int k) { return 2 * ((k >> 1) & 1) + 4 * ((k >> 3) & 1); }

// ------------------------------------------------------------------------------------
// Operand staging of the ping-pong kernel. An operand tile spans R output rows (A, R = BM)
// or columns (B, R = BN) and BK values of k. In memory the operand is either k-contiguous
// ("K-major": A as given, or B given transposed, N x K) or m/n-contiguous ("MN-major": B
// as given, or A given transposed, K x M). The LDS slot keeps the memory orientation:
//   K-major : R rows of BK halves; 16-byte chunk c of row r sits at chunk c ^ swz_a_mf(r);
//             a fragment (8 consecutive k of one m or n) is one ds_read_b128;
//   MN-major: BK rows of R halves (R*2 bytes, a multiple of the 256-byte bank window);
//             chunk c of row k sits at chunk c ^ swz_b(k); a fragment is two
//             ds_read_b64_tr_b16 (each gives a lane 4 k values of its m or n, gathered
//             from the rows of 4 lanes).
// Either way a lane ends up with the same fragment: 8 consecutive k (group lane / MF) of
// m or n index lane % MF, so the MFMA core does not depend on the layouts.
// Copies: 16-byte unit u of a k-tile lands at LDS byte 16u of the slot (the lane order of
// the LDS-DMA); the swizzle chooses which global chunk feeds it. Edges: rows past the
// matrix lie outside the descriptor range (K-major: m/n rows; MN-major: the k rows past K
// in the last tile) and read as zeros; chunks past the matrix along the contiguous
// dimension get an out-of-range offset (K-major: the k chunks past K in the last tile;
// MN-major: the m/n chunks past the edge). The contiguous dimension is a multiple of 8 on
// this path, so a chunk is wholly inside or wholly outside.
// LDS extent (rows or columns) used for an operand tile of R rows or columns: R itself
// when R is a multiple of 128 (MN-major rows then span whole 256-byte bank windows) or
// R = 192 (384-byte MN-major rows, swizzled by swz_b384), else R rounded up to 128 (the
// extra rows or columns are out-of-range copies that only write zeros, and no fragment
// reads them).
__host__ __device__ constexpr int pp_lds_extent(int R) { return R % 128 == 0 || R == 192 ? R : (R + 127) / 128 * 128; }

template <int BM, int BN, int BK, int STAGES>
__host__ __device__ constexpr int pp_lds_bytes() {
  return STAGES * (pp_lds_extent(BM) + pp_lds_extent(BN)) * BK * 2;
}

// Bytes of the epilogue's staged tiles (StagedTile: WTM rows of SCPR 16-byte chunks per wave)
// and the dynamic LDS of a ping-pong launch: the larger of the operand ring and the staging,
// which reuses the ring once the last k-tile is read.
__host__ __device__ constexpr int staged_bytes(int nw, int wtm, int wtn) {
  return nw * wtm * 16 * (wtn / 8 <= 4 ? 4 : wtn / 8 <= 8 ? 8 : wtn / 8 <= 16 ? 16 : 32);
}
template <int BM, int BN, int BK, int WM, int WN, int STAGES>
__host__ __device__ constexpr int pp_launch_lds_bytes() {
  return pp_lds_bytes<BM, BN, BK, STAGES>() > staged_bytes(WM * WN, BM / WM, BN / WN)
             ? pp_lds_bytes<BM, BN, BK, STAGES>()
             : staged_bytes(WM * WN, BM / WM, BN / WN);
}

// Copies: unit u = (i * NW + wave) * 64 + lane for copy i of a thread. When the units do
// not split evenly over the threads (R = 192: 768 units for 512 threads), every wave makes
// LD_ALL copies and the first half of the waves one more (LD in all); LD_OF(g) is the count
// of wave group g (waves [4g, 4g + 4) of an 8-wave workgroup), a compile-time constant in
// the code of each group, so the copy waits stay exact.
template <int R, int BK, int MF, bool KMAJ, int NW>
struct PpOperand {
  static constexpr int NT = 64 * NW;
  static constexpr int BYTES = R * BK * 2;
  static constexpr int CPR = KMAJ ? BK / 8 : R / 8;  // 16-byte chunks per LDS row
  static constexpr int UNITS = R * BK / 8;
  static constexpr int LD_ALL = UNITS / NT;          // copies every thread makes per k-tile
  static constexpr int REM = UNITS % NT;             // units of the extra copy (first half of the waves)
  static constexpr int LD = LD_ALL + (REM ? 1 : 0);  // copies of a thread of the first half
  static constexpr int KPM = 512 / MF;               // k per MFMA
  static constexpr bool KMAJOR = KMAJ;
  static constexpr int MFRAG = MF, BKV = BK, RV = R;
  static_assert(REM == 0 || REM * 2 == NT, "copies split evenly, or the extra copy over half the waves");
  static_assert(KMAJ || (R * 2) % 256 == 0 || R == 192, "MN-major rows: whole 256-byte bank windows, or 384 bytes");
  __host__ __device__ static constexpr int LD_OF(int group) { return LD_ALL + (REM && group == 0 ? 1 : 0); }

  const char* base;  // the tile's first element at k-tile 0
  int64_t step;      // bytes from one k-tile to the next
  uint32_t rng_full, rng_last;
  uint32_t off[LD], off_last[LD];
  int fr_base, fr_x, fr_k, fr_half;  // this lane's fragment-read constants

  __device__ static int swz(int row) {
    return KMAJ ? swz_a_mf<BK, MF>(row) : ((R * 2) % 256 == 0 ? swz_b(row) : swz_b384(row));
  }

  // X, ld: operand base and row stride (elements); r0: the tile's first m or n; rvalid:
  // its m or n extent inside the matrix; kin_last: k values in the last k-tile.
  __device__ void init_copies(const _Float16* X, int64_t ld, int r0, int rvalid, int kin_last, int wave,
                              int lane) {
    base = (const char*)(KMAJ ? X + (int64_t)r0 * ld : X + r0);
    step = KMAJ ? (int64_t)BK * 2 : (int64_t)BK * ld * 2;
    const int64_t full = KMAJ ? ((int64_t)(rvalid - 1) * ld + BK) * 2 : ((int64_t)(BK - 1) * ld + rvalid) * 2;
    const int64_t last =
        KMAJ ? ((int64_t)(rvalid - 1) * ld + kin_last) * 2 : ((int64_t)(kin_last - 1) * ld + rvalid) * 2;
    rng_full = (uint32_t)(full < kMaxRange ? full : kMaxRange);
    rng_last = (uint32_t)(last < kMaxRange ? last : kMaxRange);
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      // (for the extra copy of a wave of the second half u is past the tile: computed, never
      // issued)
      const int u = (i * NW + wave) * 64 + lane;
      const int row = u / CPR;
      const int c = (u % CPR) ^ swz(row);
      const uint32_t o = (uint32_t)(((int64_t)row * ld + 8 * c) * 2);
      if (KMAJ) {
        off[i] = o;
        off_last[i] = 8 * c < kin_last ? o : kOob;
      } else {
        off[i] = 8 * c < rvalid ? o : kOob;
        off_last[i] = off[i];
      }
    }
  }

  // Descriptor of k-tile t (of nk); an empty range from t_end on, so such a copy only
  // writes zeros into a slot no later read uses.
  __device__ int4v rsrc(int t, int t_end, int nk) const {
    const uint32_t r = t < t_end ? (t == nk - 1 ? rng_last : rng_full) : 0u;
    const int tt = t < nk ? t : nk - 1;
    return make_rsrc(base + tt * step, r);
  }

  // wbase: the wave's first m or n inside the tile (a multiple of the swizzle periods).
  __device__ void init_frags(int wbase, int lane) {
    const int lrow = lane % MF, lkg = lane / MF;
    if (KMAJ) {
      fr_base = (wbase + lrow) * BK * 2;
      fr_x = swz(lrow);
      fr_k = lkg;
      fr_half = 0;
    } else {
      // transposed reads: lane 16 g + 4 j + q reads row k0 + j of its group's 4-row block,
      // m/n 4q .. 4q+3 of its 16-wide block
      const int bg = lane >> 4, bj = (lane >> 2) & 3, bq = lane & 3;
      fr_k = (MF == 32 ? 8 * (bg >> 1) : 8 * bg) + bj;
      fr_x = wbase / 8 + (MF == 32 ? 2 * (bg & 1) : 0) + (bq >> 1);
      fr_half = (bq & 1) * 8;
      fr_base = 0;
    }
  }

  // Fragment f (the f-th MF block of the wave's range), k substep ks, from slot S.
  __device__ half8 frag(const char* S, int f, int ks) const {
    if (KMAJ) {
      const int chunk = (KPM / 8) * ks + fr_k;
      return *(const TG_LDS half8*)(S + fr_base + f * MF * BK * 2 + ((chunk ^ fr_x) << 4));
    } else {
      short4v h[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int k = KPM * ks + 4 * i + fr_k;
        const int off = k * R * 2 + (((fr_x + (MF / 8) * f) ^ swz(k)) << 4) + fr_half;
        h[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS short4v*)(S + off));
      }
      return __builtin_bit_cast(half8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
};


// ------------------------------------------------------------------------------------
// Epilogue of the 16x16 MFMA kernels: a wave's WTM x WTN tile of float32 accumulators
// (tile (fm, fn) holds, in lane l, row 16 fm + l % 16 and columns 16 fn + 4 (l / 16) .. +3)
// goes through the wave's own LDS region and out to C as 16-byte row segments.
//
// Staging: ReLU (optional) in float32 and rounding to fp16 in registers; then the tiles are
// taken in pairs (t0, t1) = (2q, 2q + 1) in (fm, fn) order, and v_permlane16_swap swaps
// lanes 16-31 of t0 with lanes 0-15 of t1 (and 48-63 with 32-47): afterwards the lanes with
// an even l / 16 hold 8 consecutive columns of one row of t0, the others 8 of t1, and each
// lane writes them with one ds_write_b128. Writes move 128 bytes per cycle in 8-lane passes
// (8 rows of one tile, one 16-byte chunk each); staged row r, 16-byte chunk c sits at chunk
// c ^ ((r / RPW) % SWZ), RPW rows per 128 bytes, so the 8 rows of a pass fall on 8
// distinct chunk slots: no bank conflicts (writing 8 bytes per lane straight from the
// accumulator layout takes 16-lane passes of 16 rows, at best 2-way conflicted, and twice
// the write cycles). Rows are padded to SCPR (a power of two) chunks.
// Store: lane i of read round j takes staged row (64 j + i) / SCPR, chunk (64 j + i) %
// SCPR (ds_read_b128; conflict-free: a 16-lane read pass covers 256 bytes of whole rows),
// skipping chunks past WTN / 8, and stores it unless it lies past M or N (N and ldc are
// multiples of 8 on these paths, so a chunk is wholly inside the matrix or outside).
template <int WTM, int WTN>
struct StagedTile {
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int CPR = WTN / 8;
  static constexpr int SCPR = CPR <= 4 ? 4 : (CPR <= 8 ? 8 : (CPR <= 16 ? 16 : 32));
  static constexpr int RB = SCPR * 16;  // bytes per staged row
  static constexpr int BYTES = WTM * RB;
  static constexpr int RPW = RB >= 128 ? 1 : 128 / RB;
  static constexpr int SWZ = SCPR < 8 ? SCPR : 8;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0 && (FM * FN) % 2 == 0, "pairs of 16 x 16 tiles");
  static_assert(64 % SCPR == 0 && (WTM * SCPR) % 64 == 0, "row-read shape");

  __device__ static int chunk_at(int r, int c) { return c ^ ((r / RPW) % SWZ); }

  template <bool RELU, typename Acc>
  __device__ static uint32_t pack2(const Acc& a, int e) {
    float x = a[e], y = a[e + 1];
    if (RELU) {
      x = relu_f(x);
      y = relu_f(y);
    }
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    const half2v h = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, h);
  }

  // acc: FM x FN accumulators of 4 floats (any indexable 4-vector type).
  template <bool RELU, typename Acc>
  __device__ static void stage(char* region, const Acc (&acc)[FM][FN], int lane) {
    const int lrow = lane & 15, lkg = lane >> 4;
    const bool second = (lkg & 1) != 0;
#pragma unroll
    for (int q = 0; q < FM * FN / 2; ++q) {
      const int t0 = 2 * q, t1 = 2 * q + 1;
      const auto s0 = __builtin_amdgcn_permlane16_swap(pack2<RELU>(acc[t0 / FN][t0 % FN], 0),
                                                       pack2<RELU>(acc[t1 / FN][t1 % FN], 0), false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(pack2<RELU>(acc[t0 / FN][t0 % FN], 2),
                                                       pack2<RELU>(acc[t1 / FN][t1 % FN], 2), false, false);
      const int4v v = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
      const int row = (second ? t1 / FN : t0 / FN) * 16 + lrow;
      const int c = (second ? t1 % FN : t0 % FN) * 2 + (lkg >> 1);
      *(TG_LDS int4v*)(region + row * RB + (chunk_at(row, c) << 4)) = v;
    }
  }

  // Rows past mvalid or chunks past nvalid (counted from the wave tile's origin) are not
  // stored; C points at the wave tile's first element.
  __device__ static void store(const char* region, int lane, _Float16* C, int64_t ldc, int mvalid, int nvalid) {
#pragma unroll
    for (int i = 0; i < WTM * SCPR / 64; ++i) {
      const int idx = i * 64 + lane;
      const int r = idx / SCPR, c = idx % SCPR;
      if (c >= CPR) continue;
      const half8 x = *(const TG_LDS half8*)(region + r * RB + (chunk_at(r, c) << 4));
      if (r < mvalid && 8 * c < nvalid) store_c(C + (int64_t)r * ldc + 8 * c, x);
    }
  }

  // The rows read back were written by other lanes of the same wave: keep the compiler
  // from moving the reads above the writes (LDS runs one wave's instructions in order).
  __device__ static void wave_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }
};

// Epilogue of the 32x32 MFMA kernels: a wave's WTM x WTN tile of float32 accumulators
// (tile (fm, fn) holds, in lane l, row 32 fm + l % 32 and columns 32 fn + 8 g + 4 (l / 32)
// .. +3 for g = 0 .. 3) goes through the wave's own LDS region and out to C as 16-byte row
// segments read back by consecutive lanes, like StagedTile.
// Staging: ReLU (optional) and rounding to fp16 in registers; then for each pair of column
// groups (g, g + 1) = (2q, 2q + 1) of a tile, v_permlane32_swap swaps lanes 32-63 of group
// 2q with lanes 0-31 of group 2q + 1. Afterwards lane l < 32 holds columns 16 q .. 16 q + 7
// of row l and lane l >= 32 columns 16 q + 8 .. 16 q + 15 of row l - 32, and each lane
// writes one 16-byte chunk (ds_write_b128). Staged row r, chunk c sits at chunk c ^ ((r /
// RPW) % SWZ), RPW rows per 128 bytes, as in StagedTile: the 8 rows of an 8-lane write pass
// fall on 8 distinct chunk slots, so the writes are conflict-free (8-byte writes straight
// from the accumulator layout were 2-way conflicted). Rows are padded to SCPR chunks (a
// power of two). Stores as in StagedTile::store (non-temporal).
template <int WTM, int WTN>
struct StagedTile32 {
  static constexpr int CPR = WTN / 8, SCPR = CPR <= 8 ? (CPR <= 4 ? 4 : 8) : (CPR <= 16 ? 16 : 32);
  static constexpr int RB = SCPR * 16, BYTES = WTM * RB;
  static constexpr int RPW = RB >= 128 ? 1 : 128 / RB;
  static constexpr int SWZ = SCPR < 8 ? SCPR : 8;
  static_assert(SCPR >= CPR && WTN % 32 == 0 && WTM % 32 == 0, "staged row shape");
  static_assert(64 % SCPR == 0 && (WTM * SCPR) % 64 == 0, "row-copy shape");

  __device__ static int chunk_at(int r, int c) { return c ^ ((r / RPW) % SWZ); }

  template <bool RELU, typename V>
  __device__ static uint32_t pack2(const V& a, int e) {
    float x = a[e], y = a[e + 1];
    if (RELU) {
      x = relu_f(x);
      y = relu_f(y);
    }
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    const half2v h = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, h);
  }

  template <bool RELU, typename Acc>
  __device__ static void stage(char* region, const Acc& acc, int lane) {
    constexpr int FM = WTM / 32, FN = WTN / 32;
    const int l32 = lane & 31, lhi = lane >> 5;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int r = fm * 32 + l32;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const auto s0 = __builtin_amdgcn_permlane32_swap(pack2<RELU>(acc[fm][fn], 8 * q),
                                                           pack2<RELU>(acc[fm][fn], 8 * q + 4), false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(pack2<RELU>(acc[fm][fn], 8 * q + 2),
                                                           pack2<RELU>(acc[fm][fn], 8 * q + 6), false, false);
          const int4v v = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
          const int c = fn * 4 + 2 * q + lhi;
          *(TG_LDS int4v*)(region + r * RB + (chunk_at(r, c) << 4)) = v;
        }
      }
    }
  }

  __device__ static void wave_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }

  __device__ static void store(const char* region, int lane, _Float16* C, int64_t ldc, int mvalid, int nvalid) {
#pragma unroll
    for (int i = 0; i < WTM * SCPR / 64; ++i) {
      const int idx = i * 64 + lane;
      const int r = idx / SCPR, c = idx % SCPR;
      if (c >= CPR) continue;
      const half8 x = *(const TG_LDS half8*)(region + r * RB + (chunk_at(r, c) << 4));
      if (r < mvalid && 8 * c < nvalid) store_c(C + (int64_t)r * ldc + 8 * c, x);
    }
  }
};

}  // namespace
}  // namespace tgemm
