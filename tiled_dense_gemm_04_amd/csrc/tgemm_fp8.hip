// tgemm_fp8.hip -- gfx950 kernels of the fp8 (E4M3) block-scaled GEMM and of the block
// quantizer that feeds it.
//
// Operation: fp8_block_scaled_linear(x, w_fp8, scale_w, block=128) in "TileLang-MUSA
// operator development" (7yue.com), section 8.2, with the per-block scaling named in the
// TileLang write-up measured on A100 (nxmr.cn 138173), section 7. The pages fix neither
// the encoding nor the block shapes; the reading taken (stated with the entry points in
// tgemm.h) is OCP E4M3 codes with float32 scales per 1 x 128 block of A and per 128 x 128
// block of B (N x K, a linear layer's weight):
//   C[i,j] = ReLU?( sum_kb SA[i,kb] * SB[j/128,kb] * sum_{k in block kb} a[i,k] * b[j,k] ).
// What is MI355X-specific:
//   * one v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3) covers exactly one 128-wide k-block of
//     a 16 x 16 output tile, so a k-tile is one scale block: each MFMA starts from zero and
//     its block sum is folded into the float32 accumulator by the VALU (acc += sa*sb * P)
//     while later MFMAs run. The fp8 MFMAs sum a block's 128 products with less than
//     float32 precision; promoting every block to float32 is what the block size bounds;
//   * operand tiles are K-major rows of 128 bytes. In LDS they are held exactly like the
//     binary16 ping-pong kernel's K-major tiles of 64 halves (the same bytes): the same
//     buffer->LDS copies, range-checked edges and swizzle. A lane's 32-byte fp8 fragment is
//     two 16-byte reads (k bytes 16g..16g+15 and 64+16g..64+16g+15 for lane group g); A
//     and B use the same k order, which is all the dot product needs;
//   * the per-row scales of A ride the same buffer->LDS copies, one dword per lane per
//     k-tile, so every wait counts copies exactly; each copy carries one slice of a group
//     of G k-tiles' scales, so that G consecutive lanes read G consecutive floats of one
//     row (a 1 x 128 block's scales sit KB floats apart in memory, one per row). B's block
//     scales, one per wave and k-tile, come through the scalar path;
//   * XCD-aware, panel-ordered tile order as in the binary16 kernels.
#include "tgemm_configs.h"
#include "tgemm_device.h"

#include <atomic>

namespace tgemm {
namespace {

typedef int int8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));

constexpr int kF8Kh = kFp8Block / 2;  // k-tile width in binary16 units (the LDS view)

// One 4-byte buffer load per lane written straight to LDS at lds_base + 4*lane (zeros for
// a lane outside the descriptor range). Inline assembly for the reason given at
// dma_to_lds; M0 is clobbered the same way.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_dword_to_lds(const int4v& rsrc, uint32_t lds_base, uint32_t voffset) {
#ifdef TGEMM_DEBUG_FILL
  debug_poison(lds_base, 4);
#endif
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ int8v cat_frag(const half8& lo, const half8& hi) {
  const int4v l = __builtin_bit_cast(int4v, lo), h = __builtin_bit_cast(int4v, hi);
  return __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7);
}

// E4M3 code -> float (exact): exponent field 0 is f * 2^-9, S.1111.111 is NaN, otherwise
// (1 + f/8) * 2^(e-7), i.e. float exponent field e + 120 and fraction f << 20.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15, f = c & 7;
  float v;
  if (e == 0)
    v = (float)f * 0x1p-9f;
  else if (e == 15 && f == 7)
    v = __builtin_nanf("");
  else
    v = __uint_as_float(((e + 120) << 23) | (f << 20));
  return (c & 0x80) ? -v : v;
}

// Two floats -> two E4M3 codes (bytes 0 and 1 of the result, the rest of `old` kept) with
// gfx950's conversion instruction (OCP E4M3, round to nearest even; HI selects bytes 2
// and 3 instead). The quantizer only converts x / s with |x| <= amax and s = amax / 448,
// so |x / s| <= 448 (1 + 2^-23) and no value ever needs saturation beyond rounding to 448.
// Checked bit for bit against the oracle, every rounding tie and subnormal included.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// ------------------------------------------------------------------------------------
// Block-scaled GEMM, fast path. BM x BN tile, WM x WN waves (wave tile WTM x WTN of 16 x 16
// MFMA tiles), k-tile = one 128-wide scale block, STAGES-deep LDS ring.
// Per k-tile every thread issues PT copies: its share of the A and B tiles (16 bytes each)
// and one dword of A row scales (a slice of a later scale group; waves with no lanes in a
// slice write zeros to a spare 256 bytes). The first scale group is fetched before any
// tile. Schedule (tile t in slot t % STAGES): copies of tiles 0 .. STAGES-1, wait for tile
// 0, barrier; then for each kt: MFMAs + folds of tile kt, wait for this thread's copies of
// tile kt+1, barrier (everyone's have landed, and every wave is done with tile kt's slot),
// copies of tile kt+STAGES into that slot (past the last tile: empty ranges, zeros, never
// read).
// DB (double-buffered fragments, STAGES >= 3): every fragment of a k-tile (A, B and the
// scales) is read into registers at once, one k-tile ahead: iteration kt waits for tile
// kt+1, passes one barrier (after which the slot of tile kt, read in the iteration
// before, is free), refills that slot with tile kt+STAGES, reads tile kt+1's fragments
// into the second register set and runs tile kt's MFMAs and folds from the first. Reads
// of the next tile then overlap the MFMAs of this one; this needs a wave tile small
// enough for two fragment sets (64 x 64).
// Requirements (checked by the host): A, B 16-byte aligned, lda, ldb, K multiples of 16;
// C 16-byte aligned, ldc and N multiples of 8; (BM - 1) * KB * 4 < 2^31.
// k-tiles per group of A row scales (8 measured no faster on 256 x 256 tiles and slower
// on 128 x 128 ones).
constexpr int kScaleGroup = 4;
// Position of the scale of k-tile g (of its group) of tile row r in a [BM][G] group slot of
// LDS: a row's G floats stay together (one 16-byte run, so a copy's lanes still fetch 16
// contiguous bytes per row), swapped in pairs on rows whose bit 3 is set. The loop reads
// one scale per MFMA row with ds_read_b32, the 16 rows r0 .. r0 + 15 of a 16 x 16 tile (r0
// a multiple of 16), and such a read is served 32 banks per cycle: without the swap rows r
// and r + 8 fall on one bank (2 extra cycles per read), with it all 16 rows fall on
// distinct banks.
__host__ __device__ constexpr int scale_pos(int r, int g) { return r * kScaleGroup + (g ^ ((r >> 3) & 1)); }

template <int BM, int BN, int WM, int WN, int STAGES, int PANEL, int XCD, bool DB>
__global__ __launch_bounds__(64 * WM * WN) void gemm_fp8_block_kernel(Fp8Args g) {
  WgClock clk;
  clk.start();
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  using OpA = PpOperand<BM, kF8Kh, 16, true, NW>;
  using OpB = PpOperand<BN, kF8Kh, 16, true, NW>;
  constexpr int A_BYTES = OpA::BYTES, B_BYTES = OpB::BYTES;
  constexpr int G = kScaleGroup;                          // k-tiles per A-scale group
  constexpr int SG_BYTES = BM * G * 4;                   // one group: [BM rows][G]
  constexpr int NG0 = BM * G / (64 * NW);                // copies per wave for group 0
  constexpr int PT = OpA::LD + OpB::LD + 1;
  static_assert(BM % 128 == 0 && BN % 128 == 0, "operand tiles of whole 128-row LDS extents");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile of 16 x 16 MFMA tiles");
  static_assert(kFp8Block % WTN == 0, "a wave's columns lie in one scale block of B");
  static_assert(BM <= 64 * NW && (BM * G) % (64 * NW) == 0 && BM % G == 0, "scale copy shape");
  static_assert(G >= STAGES, "a group slot is refilled only after its last k-tile is read");
  static_assert(STAGES >= (DB ? 3 : 2) && PT * STAGES + NG0 < 64, "ring depth / vmcnt budget");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const a_lds = smem;
  char* const b_lds = smem + STAGES * A_BYTES;
  char* const s_lds = b_lds + STAGES * B_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int64_t tm64, tn64;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, PANEL, XCD, &tm64, &tn64);
  const int row0 = (int)tm64 * BM, col0 = (int)tn64 * BN;
  const int mvalid = min(BM, g.M - row0), nvalid = min(BN, g.N - col0);
  const int nk = g.KB;
  const int kin_last = g.K - (nk - 1) * kFp8Block;  // bytes of k in the last tile (16 | it)

  OpA opa;
  OpB opb;
  opa.init_copies((const _Float16*)g.A, g.lda / 2, row0, mvalid, kin_last / 2, wave, lane);
  opb.init_copies((const _Float16*)g.B, g.ldb / 2, col0, nvalid, kin_last / 2, wave, lane);

  // A row scales go to LDS in groups of G k-tiles, [BM rows][G] floats per group, in a
  // ring of three group slots. Group 0 is fetched before the loop; every k-tile copy t then
  // fetches slice t % G (BM / G rows) of group t / G + 1, so each copy is one dword per
  // lane, G consecutive lanes read G consecutive floats of one row, and the group is
  // complete (and its slot free) well before its first k-tile. Within a group slot the
  // scales sit at scale_pos (pairs swapped on every other 8 rows), so the loop's one-float
  // reads are conflict-free. (Two other conflict-free layouts measured slower: [16-row
  // block][G][16], whose copies touch 4 bytes per lane instead of 16, by 0.4 %, and aligned
  // ds_read_b64 pairs plus a select by 1.1-1.8 %.) Slices start on multiples of 16 rows, so
  // lane si of a slice fetches the scale that position si of the slice holds: row si / G of
  // the slice, k-tile (si % G) ^ ((si / G) >> 3 & 1).
  static_assert((BM / G) % 16 == 0, "scale slices start on 16-row boundaries");
  const float* const sa_base = g.SA + (int64_t)row0 * g.KB;
  const int si = wave * 64 + lane;  // this lane's element of a slice
  const uint32_t s_off =
      si < BM ? (uint32_t)(((si / G) * g.KB + ((si % G) ^ ((si / G) >> 3 & 1))) * 4) : kOob;
  // B block scales: one per wave per k-tile, read through the scalar path. (Waves whose
  // columns all lie past N read the last block row: their results are dropped.)
  const int sb_blk = min((col0 + (wave % WN) * WTN) / kFp8Block, (g.N - 1) / kFp8Block);
  const float* const sb_row = g.SB + (int64_t)sb_blk * g.KB;

  const uint32_t a_lds0 = lds_addr(a_lds) + wave * 1024;
  const uint32_t b_lds0 = lds_addr(b_lds) + wave * 1024;
  // Waves with no lanes in a slice write their (zero) copy to a spare 256 bytes.
  const bool s_real = wave * 64 < BM;
  const uint32_t s_lds0 = s_real ? lds_addr(s_lds) + wave * 256 : lds_addr(s_lds) + 3 * SG_BYTES;
  const uint32_t s_step = s_real ? 1u : 0u;  // branch-free in the loop
  auto copy_tile = [&](int t) {
    const int4v ra = opa.rsrc(t, nk, nk);
    const int4v rb = opb.rsrc(t, nk, nk);
    const int slot = t % STAGES;
    const bool last = t == nk - 1;
#pragma unroll
    for (int j = 0; j < OpA::LD; ++j)
      dma_to_lds(ra, a_lds0 + slot * A_BYTES + j * NW * 1024, last ? opa.off_last[j] : opa.off[j]);
#pragma unroll
    for (int j = 0; j < OpB::LD; ++j)
      dma_to_lds(rb, b_lds0 + slot * B_BYTES + j * NW * 1024, last ? opb.off_last[j] : opb.off[j]);
    {
      // Written without conditionals: a uniform branch here splits the loop body and
      // costs the register allocator dearly.
      const int grp = t / G + 1, part = t % G;
      const int r0 = part * (BM / G), k0 = grp * G;
      const int rl = max(mvalid - r0, 0), kl = max(g.KB - k0, 0);
      const uint32_t rng = (uint32_t)(max((rl - 1) * g.KB + kl, 0) * 4 * min(kl, 1));
      const int4v rs = make_rsrc(sa_base + (int64_t)r0 * g.KB + min(k0, nk - 1), rng);
      dma_dword_to_lds(rs, s_lds0 + s_step * ((grp % 3) * SG_BYTES + part * BM * 4), s_off);
    }
  };
  // A row scale of k-tile t for tile row r (scale_pos inside the group slot of t).
  auto sa_at = [&](int t, int r) { return ((const TG_LDS float*)(s_lds + ((t / G) % 3) * SG_BYTES))[scale_pos(r, t % G)]; };
  // Group 0, before the first operand copies: NG0 copies per wave over the whole group.
  {
    const int4v rs = make_rsrc(sa_base, (uint32_t)(((int64_t)(mvalid - 1) * g.KB + g.KB) * 4));
#pragma unroll
    for (int j = 0; j < NG0; ++j) {
      const int i = (wave * NG0 + j) * 64 + lane;  // position i of group 0's slot
      dma_dword_to_lds(rs, lds_addr(s_lds) + (wave * NG0 + j) * 256,
                       (uint32_t)(((i / G) * g.KB + ((i % G) ^ ((i / G) >> 3 & 1))) * 4));
    }
  }

  const int wm = wave / WN, wn = wave % WN;
  const int lrow = lane % 16;  // the MFMA row of this lane in a 16 x 16 tile
  opa.init_frags(wm * WTM, lane);
  opb.init_frags(wn * WTN, lane);

  float4v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  // Operands go in as (B fragment, A fragment): a lane's result holds four consecutive
  // output columns (16 * fn + 4 * (lane / 16) ..) of one row (16 * fm + lrow) of the wave tile.
  // MFMA t (t = fm * FN + fn) writes result register t % 3, and the block sum of MFMA t-2
  // (issued two MFMAs earlier, so complete) is folded into its accumulator right after,
  // so no MFMA waits for a result and the folds run on the VALU under later MFMAs.
  const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};

  if constexpr (!DB) {
    // The last D rows of MFMA tiles of k-tile kt are issued after the barrier that frees
    // its slot (their operands are already in registers): they keep the MFMA pipe busy
    // while the wave waits for k-tile kt+1 and reads its first fragments, and their folds
    // run after that barrier. The A fragment of row fm+PF is read at the start of row fm
    // (a ring of PF+1 fragments; PF >= D leaves the deferred rows' fragments in the ring).
    // sched_barrier(0) around each MFMA and each fold keeps exactly this order.
    constexpr int D = FM >= 4 ? 3 : FM - 1;
    constexpr int PF = D > 2 ? D : 2;
    constexpr int TM = (FM - D) * FN;
    int8v fb[FN];
    int8v fa[PF + 1];
    float sc[FM];
    float4v ptail[D > 0 ? D * FN : 1];
    float sctail[D > 0 ? D : 1];
    auto main_part = [&](int kt, float sb) {
      const int slot = kt % STAGES;
      const bool fold_prev = kt > 0;
      const char* const As = a_lds + slot * A_BYTES;
      const char* const Bs = b_lds + slot * B_BYTES;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) sc[fm] = sa_at(kt, wm * WTM + fm * 16 + lrow) * sb;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) fb[fn] = cat_frag(opb.frag(Bs, fn, 0), opb.frag(Bs, fn, 1));
#pragma unroll
      for (int r = 0; r < PF; ++r) fa[r] = cat_frag(opa.frag(As, r, 0), opa.frag(As, r, 1));
      if (D > 0 && fold_prev) {  // the previous k-tile's deferred rows
#pragma unroll
        for (int r = 0; r < D; ++r)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) acc[FM - D + r][fn] += sctail[r] * ptail[r * FN + fn];
      }
      __builtin_amdgcn_sched_barrier(0);
      float4v p[3];
#pragma unroll
      for (int t = 0; t < TM + 2; ++t) {
        if (t < TM) {
          const int fm = t / FN, fn = t % FN;
          if (fn == 0 && fm + PF < FM) fa[(fm + PF) % (PF + 1)] = cat_frag(opa.frag(As, fm + PF, 0), opa.frag(As, fm + PF, 1));
          __builtin_amdgcn_sched_barrier(0);
          p[t % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[fn], fa[fm % (PF + 1)], zero, 0, 0, 0, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (t >= 2) {
          const int u = t - 2;
          acc[u / FN][u % FN] += sc[u / FN] * p[u % 3];
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    auto tail_part = [&]() {
#pragma unroll
      for (int r = 0; r < D; ++r) {
        const int fm = FM - D + r;
        sctail[r] = sc[fm];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          ptail[r * FN + fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[fn], fa[fm % (PF + 1)], zero, 0, 0, 0, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // One barrier per k-tile: after tile kt's reads each wave waits for its own copies of
    // tile kt+1 (those of tiles kt+2 .. kt+STAGES-1 may still be in flight), and a single
    // barrier then both frees tile kt's slot for tile kt+STAGES and makes tile kt+1 visible
    // to every wave. (A barrier before the reads as well measured 3-9 % slower.)
#pragma unroll
    for (int t = 0; t < STAGES; ++t) copy_tile(t);
    clk.loop_begin();
    wait_vmcnt<PT * (STAGES - 1)>();
    lds_barrier();             // tile 0 landed everywhere
    for (int kt = 0; kt < nk; ++kt) {
      const float sb = sb_row[kt];
      main_part(kt, sb);
      wait_vmcnt<PT * (STAGES - 2)>();
      lds_barrier();           // tile kt+1 landed everywhere; every wave is done with tile kt
      copy_tile(kt + STAGES);  // refill tile kt's slot (past the end: empty ranges, zeros)
      if (D > 0) tail_part();
    }
    if (D > 0) {
#pragma unroll
      for (int r = 0; r < D; ++r)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[FM - D + r][fn] += sctail[r] * ptail[r * FN + fn];
    }
    wait_vmcnt<0>();
    clk.loop_end();
  } else {
    struct Frags {
      int8v a[FM], b[FN];
      float sa[FM], sb;
    };
    auto read_frags = [&](int kt, Frags& f) {
      const int slot = kt % STAGES;
      const char* const As = a_lds + slot * A_BYTES;
      const char* const Bs = b_lds + slot * B_BYTES;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) f.b[fn] = cat_frag(opb.frag(Bs, fn, 0), opb.frag(Bs, fn, 1));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) f.a[fm] = cat_frag(opa.frag(As, fm, 0), opa.frag(As, fm, 1));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) f.sa[fm] = sa_at(kt, wm * WTM + fm * 16 + lrow);
      f.sb = sb_row[min(kt, nk - 1)];
    };
    constexpr int T = FM * FN;
    auto mma_frags = [&](const Frags& f) {
      float4v p[3];
#pragma unroll
      for (int t = 0; t < T + 2; ++t) {
        if (t < T)
          p[t % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[t % FN], f.a[t / FN], zero, 0, 0, 0, 0, 0, 0);
        if (t >= 2) {
          const int u = t - 2;
          acc[u / FN][u % FN] += (f.sa[u / FN] * f.sb) * p[u % 3];
        }
      }
    };

#pragma unroll
    for (int t = 0; t < STAGES; ++t) copy_tile(t);
    wait_vmcnt<PT * (STAGES - 1)>();
    lds_barrier();
    Frags f0, f1;
    read_frags(0, f0);
    clk.loop_begin();
    auto iteration = [&](int kt, const Frags& cur, Frags& nxt) {
      wait_vmcnt<PT * (STAGES - 2)>();    // this thread's copies of tile kt+1 have landed
      lds_barrier();                      // everyone's have; every wave is done with tile kt
      copy_tile(kt + STAGES);             // into tile kt's slot (past the end: zeros)
      read_frags(kt + 1, nxt);            // past the last tile: a settled slot, unused
      mma_frags(cur);
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      iteration(kt, f0, f1);
      iteration(kt + 1, f1, f0);
    }
    if (kt < nk) iteration(kt, f0, f1);
    wait_vmcnt<0>();
    clk.loop_end();
  }

  // Epilogue: ReLU in float32, round to fp16, stage the wave's WTM x WTN sub-tile in its
  // own LDS region (the ring is free once every wave passes the barrier) and write it back
  // as 16-byte row segments (StagedTile).
  using ST = StagedTile<WTM, WTN>;
  static_assert(NW * ST::BYTES <= STAGES * (A_BYTES + B_BYTES), "staged tile fits in the ring");
  __syncthreads();
  char* const stage = smem + wave * ST::BYTES;
  if (g.relu != 0)
    ST::template stage<true>(stage, acc, lane);
  else
    ST::template stage<false>(stage, acc, lane);
  ST::wave_fence();
  ST::store(stage, lane, g.C + (int64_t)(row0 + wm * WTM) * g.ldc + col0 + wn * WTN, g.ldc, mvalid - wm * WTM,
            nvalid - wn * WTN);
  clk.finish(nk, g.stamps);
}

// ------------------------------------------------------------------------------------
// Block-scaled GEMM, ping-pong variant: the binary16 ping-pong's split of the 8 waves into
// two groups of 4 (one wave of each per SIMD), applied to the fp8 k-tile of one 128-wide
// scale block. In every interval between two barriers one group issues MFMAs and folds,
// from fragments already in its registers, while the other reads LDS.
// The ring has two slots ((BM + BN) x 128 bytes each: three would not fit in LDS), so a
// slot may only be refilled once both groups hold all of its fragments in registers: a
// wave reads every A and B fragment of its 128 x 64 sub-tile (and the row scales) for a
// k-tile in one go, 96 registers, and keeps them through its MFMAs.
// Schedule (tile t in slot t % 2). Interval kt (between barrier kt-1 and barrier kt):
//   group 0: reads tile kt; copies all of tile kt+1 (and a slice of a later scale group)
//            into the other slot; MFMAs + folds of tile kt; waits for its copies;
//   group 1: MFMAs + folds of tile kt-1; reads tile kt.
// Slot safety: tile kt+1's copies go to the slot of tile kt-1, which both groups finished
// reading before barrier kt-1 (group 1's MFMAs of tile kt-1 run from registers). Every
// group-0 thread waits for all its copies before barrier kt, so after it tile kt+1 is
// complete.
// What bounds it (measured, 4096^3): the fold after each MFMA (4 FMAs per lane) does not
// overlap the same wave's MFMAs, so a wave alone on its SIMD issues an MFMA + fold every
// ~48 clocks against 32 for MFMAs alone, while two waves interleaving MFMAs + folds on one
// SIMD reach ~35; and each 64-lane copy holds the issuing wave ~50 clocks, so group 0's
// 17 copies per k-tile delay its MFMAs by ~900 clocks. Copies issued from group 1's MFMA
// phase instead (one after every MFMA, every second, or only the B rows there) measured
// 3-6 % slower. Against the single-group kernel this schedule is ~5 % faster at 4096^3
// and 8192^3.
// Scale groups as in gemm_fp8_block_kernel (G k-tiles per group, three group slots): the
// copies of tile t carry slice t % G of group t / G + 1, one dword per group-0 lane.
template <int BM, int BN, int WM, int WN, int STAGES, int PANEL, int XCD>
__global__ __launch_bounds__(64 * WM * WN) void gemm_fp8_pp_kernel(Fp8Args g) {
  WgClock clk;
  clk.start();
  constexpr int NW = WM * WN, NC = NW / 2;  // NC waves (group 0) issue the copies
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  using OpA = PpOperand<BM, kF8Kh, 16, true, NC>;
  using OpB = PpOperand<BN, kF8Kh, 16, true, NC>;
  constexpr int A_BYTES = OpA::BYTES, B_BYTES = OpB::BYTES;
  constexpr int G = kScaleGroup;
  constexpr int SG_BYTES = BM * G * 4;
  constexpr int NG0 = BM * G / (64 * NC);     // copies per group-0 wave for scale group 0
  constexpr int NCOPY = OpA::LD + OpB::LD + 1;  // copies per group-0 thread per k-tile
  static_assert(NW == 8 && WM == 2 && STAGES == 2, "two groups of four waves (rows of wave tiles), two slots");
  static_assert(OpA::REM == 0 && OpB::REM == 0, "copies split evenly over group 0");
  static_assert(BM == 64 * NC, "one scale dword per group-0 lane per k-tile");
  static_assert(kFp8Block % WTN == 0 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  static_assert(G >= 2, "a scale group slot is refilled only after its last k-tile is read");
  static_assert(NCOPY + NG0 < 64, "vmcnt budget");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const a_lds = smem;
  char* const b_lds = smem + STAGES * A_BYTES;
  char* const s_lds = b_lds + STAGES * B_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / NC;
  const int cw = wave % NC;  // this wave's share of the copies (group 0 issues them)

  int64_t tm64, tn64;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, PANEL, XCD, &tm64, &tn64);
  const int row0 = (int)tm64 * BM, col0 = (int)tn64 * BN;
  const int mvalid = min(BM, g.M - row0), nvalid = min(BN, g.N - col0);
  const int nk = g.KB;
  const int kin_last = g.K - (nk - 1) * kFp8Block;

  OpA opa;
  OpB opb;
  opa.init_copies((const _Float16*)g.A, g.lda / 2, row0, mvalid, kin_last / 2, cw, lane);
  opb.init_copies((const _Float16*)g.B, g.ldb / 2, col0, nvalid, kin_last / 2, cw, lane);

  const float* const sa_base = g.SA + (int64_t)row0 * g.KB;
  const int si = cw * 64 + lane;  // this lane's element of a scale slice
  static_assert((BM / G) % 16 == 0, "scale slices start on 16-row boundaries");
  const uint32_t s_off = (uint32_t)(((si / G) * g.KB + ((si % G) ^ ((si / G) >> 3 & 1))) * 4);  // scale_pos
  const int sb_blk = min((col0 + (wave % WN) * WTN) / kFp8Block, (g.N - 1) / kFp8Block);
  const float* const sb_row = g.SB + (int64_t)sb_blk * g.KB;

  const uint32_t a_lds0 = lds_addr(a_lds) + cw * 1024;
  const uint32_t b_lds0 = lds_addr(b_lds) + cw * 1024;
  const uint32_t s_lds0 = lds_addr(s_lds) + cw * 256;
  // Copy j of a thread sits RSTEP rows after copy 0, a multiple of the swizzle period, so
  // its offset is copy 0's plus j * RSTEP rows. An out-of-range offset (kOob, a k chunk
  // past K) stays out of range and below 2^32: the fast path takes lda, ldb <= 2^23 bytes,
  // so (LD - 1) * RSTEP rows <= 7 * 2^28 bytes < 2^31. Two registers per operand instead
  // of 2 * LD keep the ping-pong's 96 fragment registers from spilling.
  constexpr int RSTEP = NC * 64 / OpA::CPR;
  static_assert(OpA::CPR == OpB::CPR && RSTEP % 16 == 0, "copy rows step by whole swizzle periods");
  static_assert((OpA::LD - 1) * RSTEP <= 8 * 32 && (OpB::LD - 1) * RSTEP <= 8 * 32, "offset headroom below 2^32");
  const uint32_t a_rstep = (uint32_t)RSTEP * (uint32_t)g.lda, b_rstep = (uint32_t)RSTEP * (uint32_t)g.ldb;
  const uint32_t a_off = opa.off[0], a_off_last = opa.off_last[0];
  const uint32_t b_off = opb.off[0], b_off_last = opb.off_last[0];
  auto copy_tile = [&](int t) {
    const int4v ra = opa.rsrc(t, nk, nk);
    const int4v rb = opb.rsrc(t, nk, nk);
    const int slot = t % STAGES;
    const bool last = t == nk - 1;
    const uint32_t ao = last ? a_off_last : a_off, bo = last ? b_off_last : b_off;
#pragma unroll
    for (int j = 0; j < OpA::LD; ++j) dma_to_lds(ra, a_lds0 + slot * A_BYTES + j * NC * 1024, ao + j * a_rstep);
#pragma unroll
    for (int j = 0; j < OpB::LD; ++j) dma_to_lds(rb, b_lds0 + slot * B_BYTES + j * NC * 1024, bo + j * b_rstep);
    const int sgrp = t / G + 1, part = t % G;
    const int r0 = part * (BM / G), k0 = sgrp * G;
    const int rl = max(mvalid - r0, 0), kl = max(g.KB - k0, 0);
    const uint32_t rng = (uint32_t)(max((rl - 1) * g.KB + kl, 0) * 4 * min(kl, 1));
    const int4v rs = make_rsrc(sa_base + (int64_t)r0 * g.KB + min(k0, nk - 1), rng);
    dma_dword_to_lds(rs, s_lds0 + (sgrp % 3) * SG_BYTES + part * BM * 4, s_off);
  };
  // A row scale of k-tile t for tile row r (scale_pos inside the group slot of t).
  auto sa_at = [&](int t, int r) { return ((const TG_LDS float*)(s_lds + ((t / G) % 3) * SG_BYTES))[scale_pos(r, t % G)]; };

  const int wm = wave / WN, wn = wave % WN;
  const int lrow = lane % 16;
  opa.init_frags(wm * WTM, lane);
  opb.init_frags(wn * WTN, lane);

  float4v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  int8v fa[FM], fb[FN];
  float sa[FM], sb = 0.0f;
  // B's block scales through the scalar path (read-only in this kernel): a uniform value
  // that an LDS-read wait covers, where a vector load would be waited on together with
  // the copies in flight.
  typedef __attribute__((address_space(4))) const float* ConstF32;
  const ConstF32 sbp = (ConstF32)sb_row;
  auto read_tile = [&](int kt) {
    const int slot = kt % STAGES;
    const char* const As = a_lds + slot * A_BYTES;
    const char* const Bs = b_lds + slot * B_BYTES;
    sb = sbp[kt];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) fb[fn] = cat_frag(opb.frag(Bs, fn, 0), opb.frag(Bs, fn, 1));
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) fa[fm] = cat_frag(opa.frag(As, fm, 0), opa.frag(As, fm, 1));
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) sa[fm] = sa_at(kt, wm * WTM + fm * 16 + lrow);
  };
  // MFMA t (t = fm * FN + fn) writes result register t % 2; the block sum of MFMA t-1 is
  // folded right after it (acc += sa * sb * P) while MFMA t runs. sched_barrier(0) keeps
  // that order (left alone, the compiler folds each result right behind its own MFMA and
  // waits for it).
  const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
  auto mma_tile = [&]() {
    float4v p[2];
#pragma unroll
    for (int t = 0; t < FM * FN + 1; ++t) {
      if (t < FM * FN) {
        p[t % 2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[t % FN], fa[t / FN], zero, 0, 0, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t >= 1) {
        const int u = t - 1;
        acc[u / FN][u % FN] += (sa[u / FN] * sb) * p[u % 2];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Prologue (group 0): scale group 0 and tile 0, waited for; then the first barrier.
  if (grp == 0) {
    const int4v rs = make_rsrc(sa_base, (uint32_t)(((int64_t)(mvalid - 1) * g.KB + g.KB) * 4));
#pragma unroll
    for (int j = 0; j < NG0; ++j) {
      const int i = (cw * NG0 + j) * 64 + lane;  // position i of group 0's slot
      dma_dword_to_lds(rs, lds_addr(s_lds) + (cw * NG0 + j) * 256,
                       (uint32_t)(((i / G) * g.KB + ((i % G) ^ ((i / G) >> 3 & 1))) * 4));
    }
    copy_tile(0);
    wait_vmcnt<0>();
  }
  lds_barrier();
  clk.loop_begin();
  // sched_barrier(0) pins every phase (the MFMAs are register-only, so s_barrier alone
  // would not keep the compiler from moving them across it).
  if (grp == 0) {
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
      read_tile(kt);
      copy_tile(kt + 1);  // into the slot of tile kt-1 (past the last tile: empty ranges)
      __builtin_amdgcn_sched_barrier(0);
      mma_tile();
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();
      lds_barrier();      // (barrier kt) tile kt+1 landed everywhere; both groups hold tile kt
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
      read_tile(kt);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();      // (barrier kt)
      __builtin_amdgcn_sched_barrier(0);
      mma_tile();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();
  clk.loop_end();

  using ST = StagedTile<WTM, WTN>;
  static_assert(NW * ST::BYTES <= STAGES * (A_BYTES + B_BYTES), "staged tile fits in the ring");
  __syncthreads();
  char* const stage = smem + wave * ST::BYTES;
  if (g.relu != 0)
    ST::template stage<true>(stage, acc, lane);
  else
    ST::template stage<false>(stage, acc, lane);
  ST::wave_fence();
  ST::store(stage, lane, g.C + (int64_t)(row0 + wm * WTM) * g.ldc + col0 + wn * WTN, g.ldc, mvalid - wm * WTM,
            nvalid - wn * WTN);
  clk.finish(nk, g.stamps);
}

template <int BM, int BN, int WM, int WN, int STAGES>
constexpr int fp8_lds_bytes() {
  return STAGES * (BM + BN) * kFp8Block + 3 * BM * kScaleGroup * 4 + 256;
}

// ------------------------------------------------------------------------------------
// Block-scaled GEMM, generic path (any alignment, stride or K): one output element per
// thread, products of decoded codes summed per block in float32, then scaled and
// accumulated in float32 like the fast path.
__global__ __launch_bounds__(256) void gemm_fp8_block_generic(Fp8Args g) {
  const int64_t tiles_n = (g.N + 15) / 16;
  const int64_t t = blockIdx.x;
  const int i = (int)(t / tiles_n) * 16 + (int)(threadIdx.x / 16);
  const int j = (int)(t % tiles_n) * 16 + (int)(threadIdx.x % 16);
  if (i >= g.M || j >= g.N) return;
  const uint8_t* const a = g.A + (int64_t)i * g.lda;
  const uint8_t* const b = g.B + (int64_t)j * g.ldb;
  const float* const sa = g.SA + (int64_t)i * g.KB;
  const float* const sb = g.SB + (int64_t)(j / kFp8Block) * g.KB;
  float acc = 0.0f;
  for (int kb = 0; kb < g.KB; ++kb) {
    const int k0 = kb * kFp8Block, k1 = min(g.K, k0 + kFp8Block);
    float p = 0.0f;
    for (int k = k0; k < k1; ++k) p += e4m3_to_f32(a[k]) * e4m3_to_f32(b[k]);
    acc += (sa[kb] * sb[kb]) * p;
  }
  g.C[(int64_t)i * g.ldc + j] = (_Float16)(g.relu ? relu_f(acc) : acc);
}

// x / s as the IEEE float32 division rounds it, from r = 1 / s (an IEEE division, once per
// block): the product x * r corrected once with its exact residual (Markstein's
// correction step), the sign of a zero x kept. Equal to x / s bit for bit for every
// binary16 x and every block maximum (amax / 448) with |x| <= amax: checked exhaustively
// on the CPU (about 10^9 pairs) by the test suite.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float y0 = x * r;
  const float e = __builtin_fmaf(-y0, s, x);
  return __builtin_copysignf(__builtin_fmaf(e, r, y0), x);
}

// A block's scale amax / 448 as the IEEE float32 division rounds it (1 for an all-zero
// block), from RN(1/448) and one corrected product (Markstein's step again): equal to the
// division for every binary16 amax, checked exhaustively on the CPU by the test suite.
__device__ __forceinline__ float block_scale(float amax) {
  constexpr float kInv448 = 1.0f / 448.0f;
  const float s0 = amax * kInv448;
  return amax > 0.0f ? __builtin_fmaf(__builtin_fmaf(-s0, 448.0f, amax), kInv448, s0) : 1.0f;
}

// ------------------------------------------------------------------------------------
// Block quantizer, 1 x 128 blocks (activations): a group of 16 lanes per block, 8
// elements per lane, NB blocks per group (group g of a workgroup takes blocks g, g + 16, ..
// of the workgroup's 16 * NB consecutive blocks, so every load covers 16 consecutive blocks
// across the workgroup, and all NB loads are issued before any arithmetic: more bytes in
// flight per lane). The workgroup's first block is decoded once (uniform: one division);
// a group's blocks are at most NB * 16 blocks further, which wraps past at most one row end
// when NB * 16 <= KB (the host picks NB = 2 only then) and is counted off in a short loop
// otherwise. Scale s = amax / 448 in float32 (1 for an all-zero block), codes E4M3(x / s)
// with x / s rounded as the IEEE float32 division. All 64 lanes of a wave take part in the
// shuffles; lanes of groups past the last block skip their loads and stores.
template <bool VEC, int NB>
__global__ __launch_bounds__(256) void quant_fp8_rows(QuantArgs q) {
  const int sub = threadIdx.x % 16;
  const uint32_t KB = (uint32_t)q.KB;
  const uint64_t nblk = (uint64_t)q.R * KB;
  const uint32_t wg0 = blockIdx.x * 16 * NB;  // < 2^32: the grid has ceil(nblk / (16 NB)) workgroups
  const uint32_t row0 = wg0 / KB, kb0 = wg0 - row0 * KB;
  const uint32_t g = threadIdx.x / 16;
  bool active[NB];
  int64_t row[NB];
  uint32_t kbs[NB];
  float x[NB][8];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    uint32_t kb = kb0 + g + 16 * i, rw = row0;
    if (NB * 16 <= (int)KB) {
      const bool wrap = kb >= KB;
      kb -= wrap ? KB : 0u;
      rw += wrap ? 1u : 0u;
    } else {
      while (kb >= KB) {
        kb -= KB;
        ++rw;
      }
    }
    active[i] = (uint64_t)wg0 + g + 16 * i < nblk;
    row[i] = active[i] ? rw : 0;
    kbs[i] = active[i] ? kb : 0;
    const int k = (int)kbs[i] * kFp8Block + 8 * sub;
    if (VEC) {
      half8 h = {0, 0, 0, 0, 0, 0, 0, 0};
      if (active[i] && k < q.K) h = *(const half8*)(q.X + row[i] * q.ldx + k);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = (float)h[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = (active[i] && k + e < q.K) ? (float)q.X[row[i] * q.ldx + k + e] : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[i][e]));
#pragma unroll
    for (int w = 1; w < 16; w <<= 1) m = fmaxf(m, __shfl_xor(m, w, 16));
    const float s = block_scale(m);
    const float r = 1.0f / s;
    if (!active[i]) continue;
    const int k = (int)kbs[i] * kFp8Block + 8 * sub;
    if (VEC) {
      if (k < q.K) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = div_by_scale(x[i][e], s, r);
        const uint32_t lo = e4m3_pack2<true>(y[2], y[3], e4m3_pack2<false>(y[0], y[1], 0u));
        const uint32_t hi = e4m3_pack2<true>(y[6], y[7], e4m3_pack2<false>(y[4], y[5], 0u));
        *(uint2v*)(q.Q + row[i] * q.ldq + k) = (uint2v){lo, hi};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k + e < q.K) q.Q[row[i] * q.ldq + k + e] = (uint8_t)e4m3_pack2<false>(div_by_scale(x[i][e], s, r), 0.0f, 0u);
    }
    if (sub == 0) q.S[row[i] * q.KB + kbs[i]] = s;
  }
}

// Block quantizer, 128 x 128 blocks (weights): one workgroup of 256 threads per block,
// thread t on rows t / 16 + 16 i (i < 8) and columns 8 (t % 16) .. +7; the block's
// maximum is reduced across the workgroup through LDS.
template <bool VEC>
__global__ __launch_bounds__(256) void quant_fp8_tiles(QuantArgs q) {
  __shared__ float wmax[4];
  const int kb = (int)(blockIdx.x % q.KB);
  const int64_t rb = blockIdx.x / q.KB;
  const int t = threadIdx.x;
  const int c8 = 8 * (t % 16), k = kb * kFp8Block + c8;
  const int64_t r0 = rb * 128 + t / 16;
  float x[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r0 + 16 * i;
    if (VEC) {
      half8 h = {0, 0, 0, 0, 0, 0, 0, 0};
      if (r < q.R && k < q.K) h = *(const half8*)(q.X + r * q.ldx + k);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = (float)h[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = (r < q.R && k + e < q.K) ? (float)q.X[r * q.ldx + k + e] : 0.0f;
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[i][e]));
#pragma unroll
  for (int w = 1; w < 64; w <<= 1) m = fmaxf(m, __shfl_xor(m, w, 64));
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = block_scale(m);
  const float rs = 1.0f / s;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r0 + 16 * i;
    if (r >= q.R) continue;
    if (VEC) {
      if (k < q.K) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = div_by_scale(x[i][e], s, rs);
        const uint32_t lo = e4m3_pack2<true>(y[2], y[3], e4m3_pack2<false>(y[0], y[1], 0u));
        const uint32_t hi = e4m3_pack2<true>(y[6], y[7], e4m3_pack2<false>(y[4], y[5], 0u));
        *(uint2v*)(q.Q + r * q.ldq + k) = (uint2v){lo, hi};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k + e < q.K) q.Q[r * q.ldq + k + e] = (uint8_t)e4m3_pack2<false>(div_by_scale(x[i][e], s, rs), 0.0f, 0u);
    }
  }
  if (t == 0) q.S[rb * q.KB + kb] = s;
}

// MODE: 0 single-buffered fragments, 1 double-buffered (DB), 2 ping-pong.
template <int BM, int BN, int WM, int WN, int STAGES, int PANEL, int XCD, int MODE>
hipError_t launch_fp8_cfg(const Fp8Args& g, hipStream_t s, int device) {
  constexpr int lds = fp8_lds_bytes<BM, BN, WM, WN, STAGES>();
  static_assert(lds <= 160 * 1024, "LDS");
  void (*kern)(Fp8Args);
  if constexpr (MODE == 2)
    kern = gemm_fp8_pp_kernel<BM, BN, WM, WN, STAGES, PANEL, XCD>;
  else
    kern = gemm_fp8_block_kernel<BM, BN, WM, WN, STAGES, PANEL, XCD, MODE == 1>;
  static std::atomic<uint64_t> ready{0};
  const uint64_t bit = 1ull << (device & 63);
  if (!(ready.load(std::memory_order_acquire) & bit)) {
    const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    ready.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)g.tiles_m * g.tiles_n)), dim3(64 * WM * WN), lds, s, g);
  return hipGetLastError();
}

}  // namespace

static hipError_t launch_fp8_unbuilt(const Fp8Args&, hipStream_t, int) { return hipErrorNotSupported; }

// The fp8 rows of tgemm_configs.h: X(BM, BN, WAVES_M, WAVES_N, STAGES, PANEL, XCD, MODE, PROD)
#define TGEMM_FP8_ROW(BM, BN, WM, WN, S, P, X, MODE, PROD)                                        \
  {BM, BN, WM, WN, S, P, X, fp8_lds_bytes<BM, BN, WM, WN, S>(), TGEMM_BUILT(PROD),               \
   "f" #BM "x" #BN "x128_s" #S "_w" #WM "x" #WN TGEMM_FP8_MODE_NAME_##MODE},
#define TGEMM_FP8_LAUNCHER(BM, BN, WM, WN, S, P, X, MODE, PROD) \
  TGEMM_IF_BUILT(PROD, (launch_fp8_cfg<BM, BN, WM, WN, S, P, X, MODE>), launch_fp8_unbuilt),

const Fp8Config* fp8_config_table(int* count) {
  static const Fp8Config table[] = {TGEMM_FP8_CONFIGS(TGEMM_FP8_ROW)};
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

hipError_t launch_fp8(int idx, const Fp8Args& g, hipStream_t s, int device) {
  typedef hipError_t (*L)(const Fp8Args&, hipStream_t, int);
  static const L table[] = {TGEMM_FP8_CONFIGS(TGEMM_FP8_LAUNCHER)};
  if (idx < 0 || idx >= (int)(sizeof(table) / sizeof(table[0]))) return hipErrorInvalidValue;
  return table[idx](g, s, device);
}

hipError_t launch_fp8_generic(const Fp8Args& g, hipStream_t s) {
  const int64_t tiles = (int64_t)((g.M + 15) / 16) * ((g.N + 15) / 16);
  hipLaunchKernelGGL(gemm_fp8_block_generic, dim3((unsigned)tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const QuantArgs& q, bool vec, hipStream_t s) {
  if (q.block_rows == 1) {
    // Two blocks per lane group where rows hold at least 32 blocks (measured 3-12 % faster
    // on large inputs), one otherwise (short rows would pay for the row wrap-around).
    const int64_t blocks = (int64_t)q.R * q.KB;
    const bool two = q.KB >= 32;
    const int64_t per_wg = two ? 32 : 16;
    const dim3 grid((unsigned)((blocks + per_wg - 1) / per_wg));
    void (*const kern)(QuantArgs) = two ? (vec ? quant_fp8_rows<true, 2> : quant_fp8_rows<false, 2>)
                                        : (vec ? quant_fp8_rows<true, 1> : quant_fp8_rows<false, 1>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, q);
  } else {
    const dim3 grid((unsigned)((int64_t)((q.R + 127) / 128) * q.KB));
    if (vec)
      hipLaunchKernelGGL(quant_fp8_tiles<true>, grid, dim3(256), 0, s, q);
    else
      hipLaunchKernelGGL(quant_fp8_tiles<false>, grid, dim3(256), 0, s, q);
  }
  return hipGetLastError();
}

}  // namespace tgemm
