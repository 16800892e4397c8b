// tgemm_api.cpp -- host side of the libtgemm C ABI (declared in include/tgemm.h):
// argument validation, the per-device architecture check, config selection and launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/tgemm.h"
#ifdef TGEMM_STAMPS
#include "../../include/tgemm_stamps.h"
#endif
#include "tgemm_internal.h"

static_assert(TGEMM_STATIC_SCRATCH_BYTES == tgemm::kStaticScratchBytes,
              "the header states the static scratch size the kernels' source defines");
static_assert(TGEMM_PROBE_THREADS == tgemm::kProbeThreads &&
                  TGEMM_PROBE_MFMA_PER_ITER == tgemm::kProbeMfmaPerIter,
              "probe shape in the header matches the kernel");

namespace {

using tgemm::Config;

int table_size() {
  int n = 0;
  tgemm::config_table(&n);
  return n;
}
const Config& cfg_row(int idx) {
  int n = 0;
  return tgemm::config_table(&n)[idx];
}

constexpr int kSelectNoop = -100;      // M == 0 or N == 0
constexpr int kSelectZeroFill = -101;  // K == 0
constexpr int kMaxDevices = 64;

// layout = 2 * trans_a + trans_b. A is M x K (lda >= K) or, transposed, K x M (lda >= M);
// B is K x N (ldb >= N) or, transposed, N x K (ldb >= K).
int validate(int layout, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
             int64_t ldb, const void* C, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0 || M >= TGEMM_MAX_DIM || N >= TGEMM_MAX_DIM || K >= TGEMM_MAX_DIM)
    return TGEMM_EINVAL_DIM;
  const int64_t kmin = K > 1 ? K : 1, nmin = N > 1 ? N : 1, mmin = M > 1 ? M : 1;
  const int64_t amin = (layout & 2) ? mmin : kmin, bmin = (layout & 1) ? kmin : nmin;
  if (lda < amin || ldb < bmin || ldc < nmin) return TGEMM_EINVAL_LD;
  const bool out_nonempty = M > 0 && N > 0;
  if (out_nonempty && C == nullptr) return TGEMM_ENULL;
  if (out_nonempty && K > 0 && (A == nullptr || B == nullptr)) return TGEMM_ENULL;
  if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) |
       reinterpret_cast<uintptr_t>(C)) & 1u)
    return TGEMM_EALIGN;
  return TGEMM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Can a fast (non-generic) config take these arguments? 16-byte chunks along each
// operand's contiguous dimension (K for A as given and for B transposed, M for A
// transposed, N for B as given) and along the rows of C, and operand strides whose
// 256-row tiles fit a 32-bit buffer range (the generic kernel indexes in 64 bits).
bool fast_eligible(int layout, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                   const void* B, int64_t ldb, const void* C, int64_t ldc) {
  const int64_t a_contig = (layout & 2) ? M : K, b_contig = (layout & 1) ? K : N;
  return aligned16(A) && aligned16(B) && aligned16(C) && (lda % 8) == 0 && (ldb % 8) == 0 &&
         (ldc % 8) == 0 && (a_contig % 8) == 0 && (b_contig % 8) == 0 && (N % 8) == 0 &&
         lda <= TGEMM_FAST_MAX_LD && ldb <= TGEMM_FAST_MAX_LD;
}

int64_t workgroups(const Config& c, int64_t M, int64_t N) {
  return tgemm::ceil_div(M, c.bm) * tgemm::ceil_div(N, c.bn);
}

// Config choice for a fast-eligible call (rows of the table in tgemm_kernels.hip:
// 9 = 16x16x32 ping-pong 256x256, 18 = the same with 256x192 tiles, 16 = 256x128,
// 15 = 128x128, 7 = 4-wave pipelined 128x128 with BK 64). Counted in rounds of 256
// workgroups (one per compute unit): when the grid fits one round, the smallest tile whose
// tiles still fit one round (smaller tiles finish sooner: 1536^2 x 4096 42.5 us with
// 128 x 128 against 53.1 us with 256 x 128; 3072^2 74.3 us with 256 x 192 against 102.8 us
// for 128 x 128 in three rounds); beyond one round, 256 x 192 tiles if they need no more
// rounds than 256 x 256 ones (6144^2 x 4096: 255 against 275 us), else 256 x 256.
// Transposed operands take the ping-pong kernels only (15 instead of 7). 14 = config 9
// without the XCD remap, for A and B as given when all 256 x 256 tiles fit one round: the
// hardware's round-robin dispatch then also gives each XCD a 4 x 8 block of tiles (one
// tile-row of each of four panels), and measured 0.6-1.5 % faster at 4096^3 on three boxes;
// over several rounds the remap keeps each XCD's tiles together and wins (8192^3: 1-1.5 %).
constexpr int kCfgBig = 9, kCfgSmall = 7, kCfgSmallT = 15, kCfgMid = 16, kCfg192 = 18, kCfgBigOneRound = 14;
constexpr int64_t kRound = 256;  // workgroups in flight at once: one per compute unit
int choose_fast(int layout, int64_t M, int64_t N, int64_t K) {
  (void)K;
  const int64_t tm = tgemm::ceil_div(M, 256);
  const int64_t t256 = tm * tgemm::ceil_div(N, 256), t192 = tm * tgemm::ceil_div(N, 192);
  const int64_t t256x128 = tm * tgemm::ceil_div(N, 128);
  const int64_t t128 = tgemm::ceil_div(M, 128) * tgemm::ceil_div(N, 128);
  if (t128 <= kRound) return layout == 0 ? kCfgSmall : kCfgSmallT;
  if (t256x128 <= kRound) return kCfgMid;
  if (t192 <= kRound) return kCfg192;
  if (t256 <= kRound) return layout == 0 ? kCfgBigOneRound : kCfgBig;
  return tgemm::ceil_div(t192, kRound) <= tgemm::ceil_div(t256, kRound) ? kCfg192 : kCfgBig;
}

int select(int layout, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
           int64_t ldb, const void* C, int64_t ldc) {
  const int v = validate(layout, M, N, K, A, lda, B, ldb, C, ldc);
  if (v != TGEMM_OK) return v;
  if (M == 0 || N == 0) return kSelectNoop;
  if (K == 0) return kSelectZeroFill;
  if (fast_eligible(layout, M, N, K, A, lda, B, ldb, C, ldc)) return choose_fast(layout, M, N, K);
  return 0;
}

int layout_of(int trans_a, int trans_b) { return (trans_a ? 2 : 0) | (trans_b ? 1 : 0); }

// Once per device: is it gfx950? 0 = unknown, 1 = yes, 2 = no.
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device(int* device_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TGEMM_EDEVICE;
  *device_out = dev;
  if (dev >= kMaxDevices) return TGEMM_EDEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TGEMM_EDEVICE;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? TGEMM_OK : TGEMM_EDEVICE;
}

// Split-K plan, for output grids too small to fill the GPU's 256 compute units when K is
// long. From a sweep on MI355X (split-K costs one round trip of fp32 partial tiles through
// the device-coherence point, so each split must keep a long run of k-tiles):
//   128 x 128 tiles if there are at most 128 of them: splits = min(8, 256 / tiles,
//     k-tiles / 64);
//   else 256 x 256 tiles if there are at most 128 of them: splits = min(8, 256 / tiles,
//     k-tiles / 256);
//   no split if that gives fewer than 2 (e.g. 1024^3, 16384 x 512 x 4096, 4096^3).
// Measured: 1024 x 1024 x 32768 299 -> 101 us, 512 x 512 x 16384 159 -> 44 us, 2048 x 2048
// x 16384 173 -> 162 us. Only the 16x16x32 ping-pong configs take splits.
constexpr int kMaxSplits = 8, kNumCu = 256;
struct SplitPlan {
  int cfg, splits;
};

SplitPlan split_plan(int layout, int64_t M, int64_t N, int64_t K, int base_cfg) {
  (void)layout;
  SplitPlan p{base_cfg, 1};
  if (cfg_row(base_cfg).generic) return p;
  const int64_t t256 = tgemm::ceil_div(M, 256) * tgemm::ceil_div(N, 256);
  const int64_t t128 = tgemm::ceil_div(M, 128) * tgemm::ceil_div(N, 128);
  if (t256 >= 160) return p;
  int cfg;
  int64_t s;
  if (t128 <= 128) {
    cfg = kCfgSmallT;
    s = kNumCu / t128;
    const int64_t by_k = tgemm::ceil_div(K, cfg_row(cfg).bk) / 64;
    if (s > by_k) s = by_k;
  } else if (t256 <= 128) {
    cfg = kCfgBig;
    s = kNumCu / t256;
    const int64_t by_k = tgemm::ceil_div(K, cfg_row(cfg).bk) / 256;
    if (s > by_k) s = by_k;
  } else {
    return p;
  }
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 2) return p;
  return SplitPlan{cfg, (int)s};
}

// Workspace layout of a split launch: a fixed region of kMaxSplitTiles tile counters (so
// calls of any shape on one workspace use the same counter bytes, which every call leaves
// at zero), then splits fp32 partial tiles per output tile.
constexpr int64_t kMaxSplitTiles = 1024, kWsParts = kMaxSplitTiles * 4;
int64_t ws_bytes(const Config& c, int splits, int64_t M, int64_t N) {
  if (splits <= 1) return 0;
  return kWsParts + workgroups(c, M, N) * splits * (int64_t)c.bm * c.bn * 4;
}

bool split_capable(const Config& c) { return !c.generic && c.layouts == 0xF; }

int run(int cfg, int layout, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
        const void* B, int64_t ldb, void* C, int64_t ldc, int relu, void* stream, int splits = 1,
        void* ws = nullptr) {
  int dev = -1;
  const int d = check_device(&dev);
  if (d != TGEMM_OK) return d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cfg == kSelectZeroFill) {
    return tgemm::launch_zero_fill(static_cast<_Float16*>(C), (int)M, (int)N, ldc, s) == hipSuccess
               ? TGEMM_OK
               : TGEMM_ELAUNCH;
  }
  const Config& c = cfg_row(cfg);
  const int64_t nwg = workgroups(c, M, N) * splits;
  if (nwg >= ((int64_t)1 << 31)) return TGEMM_EINVAL_DIM;
  tgemm::GemmArgs g;
  g.A = static_cast<const _Float16*>(A);
  g.B = static_cast<const _Float16*>(B);
  g.C = static_cast<_Float16*>(C);
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.relu = relu != 0;
  g.tiles_m = (int)tgemm::ceil_div(M, c.bm);
  g.tiles_n = (int)tgemm::ceil_div(N, c.bn);
  g.layout = layout;
  g.splits = splits;
  g.ws = ws;
  g.ws_parts = splits > 1 ? kWsParts : 0;
  return tgemm::launcher(cfg)(g, s, dev) == hipSuccess ? TGEMM_OK : TGEMM_ELAUNCH;
}

// ---------------------------------------------------------------- fp8 block-scaled path
int fp8_table_size() {
  int n = 0;
  tgemm::fp8_config_table(&n);
  return n;
}
const tgemm::Fp8Config& fp8_row(int idx) {
  int n = 0;
  return tgemm::fp8_config_table(&n)[idx];
}
constexpr int kFp8Generic = TGEMM_FP8_GENERIC;  // the generic kernel (-102)
// 0: 256 x 256; 1: 128 x 128; 2: 256 x 128 (single fragment set, kept for the sweep);
// 3: 256 x 128 with double-buffered fragments (92 us against 103 us for 2 at 4096^3).
constexpr int kFp8Cfg256 = 0, kFp8Cfg128 = 1, kFp8Cfg256x128 = 3;

int fp8_validate(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const float* SA,
                 const void* B, int64_t ldb, const float* SB, const void* C, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0 || M >= TGEMM_MAX_DIM || N >= TGEMM_MAX_DIM || K >= TGEMM_MAX_DIM)
    return TGEMM_EINVAL_DIM;
  const int64_t kmin = K > 1 ? K : 1, nmin = N > 1 ? N : 1;
  if (lda < kmin || ldb < kmin || ldc < nmin) return TGEMM_EINVAL_LD;
  const bool out_nonempty = M > 0 && N > 0;
  if (out_nonempty && C == nullptr) return TGEMM_ENULL;
  if (out_nonempty && K > 0 && (A == nullptr || B == nullptr || SA == nullptr || SB == nullptr))
    return TGEMM_ENULL;
  if ((reinterpret_cast<uintptr_t>(C) & 1u) ||
      ((reinterpret_cast<uintptr_t>(SA) | reinterpret_cast<uintptr_t>(SB)) & 3u))
    return TGEMM_EALIGN;
  return TGEMM_OK;
}

// Fast configs need 16-byte operand rows in k (A, B), 16-byte output row segments (C),
// 32-bit scale offsets inside a 256-row tile, and operand strides whose 256-row tiles fit
// a 32-bit buffer range (codes are one byte: twice the binary16 limit in elements).
bool fp8_fast_eligible(int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, int64_t ldc) {
  const int64_t KB = tgemm::ceil_div(K, tgemm::kFp8Block);
  return aligned16(A) && aligned16(B) && aligned16(C) && lda % 16 == 0 && ldb % 16 == 0 && K % 16 == 0 &&
         ldc % 8 == 0 && N % 8 == 0 && 256 * KB * 4 < ((int64_t)1 << 31) && lda <= 2 * TGEMM_FAST_MAX_LD &&
         ldb <= 2 * TGEMM_FAST_MAX_LD;
}

// Wave-quantized cost: one config's launch takes about ceil(tiles / 256) rounds of
// workgroups (one per compute unit), each round costing about as long as its tile's work.
// Relative round costs measured at K = 4096: 256 x 256 1, 256 x 128 0.75, 128 x 128 0.57
// (e.g. 3072 x 3072: 144 tiles of 256 x 256 in one round, 56 us, beat 288 of 256 x 128 in
// two, 76 us; 2048 x 4096: 256 tiles of 256 x 128 in one round, 42 us, beat 128 of
// 256 x 256, 56 us).
int fp8_choose(int64_t M, int64_t N) {
  const auto rounds = [](int64_t tiles) { return (double)tgemm::ceil_div(tiles, (int64_t)kNumCu); };
  const double c256 = 1.00 * rounds(tgemm::ceil_div(M, 256) * tgemm::ceil_div(N, 256));
  const double c256x128 = 0.75 * rounds(tgemm::ceil_div(M, 256) * tgemm::ceil_div(N, 128));
  const double c128 = 0.57 * rounds(tgemm::ceil_div(M, 128) * tgemm::ceil_div(N, 128));
  if (c128 < c256x128 && c128 < c256) return kFp8Cfg128;
  return c256x128 < c256 ? kFp8Cfg256x128 : kFp8Cfg256;
}

int fp8_select(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const float* SA, const void* B,
               int64_t ldb, const float* SB, const void* C, int64_t ldc) {
  const int v = fp8_validate(M, N, K, A, lda, SA, B, ldb, SB, C, ldc);
  if (v != TGEMM_OK) return v;
  if (M == 0 || N == 0) return kSelectNoop;
  if (K == 0) return kSelectZeroFill;
  return fp8_fast_eligible(N, K, A, lda, B, ldb, C, ldc) ? fp8_choose(M, N) : kFp8Generic;
}

int fp8_run(int cfg, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const float* SA,
            const void* B, int64_t ldb, const float* SB, void* C, int64_t ldc, int relu, void* stream) {
  int dev = -1;
  const int d = check_device(&dev);
  if (d != TGEMM_OK) return d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cfg == kSelectZeroFill)
    return tgemm::launch_zero_fill(static_cast<_Float16*>(C), (int)M, (int)N, ldc, s) == hipSuccess
               ? TGEMM_OK
               : TGEMM_ELAUNCH;
  tgemm::Fp8Args g;
  g.A = static_cast<const uint8_t*>(A);
  g.B = static_cast<const uint8_t*>(B);
  g.SA = SA;
  g.SB = SB;
  g.C = static_cast<_Float16*>(C);
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.KB = (int)tgemm::ceil_div(K, tgemm::kFp8Block);
  g.relu = relu != 0;
#ifdef TGEMM_STAMPS
  g.stamps = tgemm::stamps_table();
#else
  g.stamps = nullptr;
#endif
  if (cfg == kFp8Generic) {
    if (tgemm::ceil_div(M, 16) * tgemm::ceil_div(N, 16) >= ((int64_t)1 << 32)) return TGEMM_EINVAL_DIM;
    g.tiles_m = g.tiles_n = 0;
    return tgemm::launch_fp8_generic(g, s) == hipSuccess ? TGEMM_OK : TGEMM_ELAUNCH;
  }
  const tgemm::Fp8Config& c = fp8_row(cfg);
  const int64_t tm = tgemm::ceil_div(M, c.bm), tn = tgemm::ceil_div(N, c.bn);
  if (tm * tn >= ((int64_t)1 << 31)) return TGEMM_EINVAL_DIM;
  g.tiles_m = (int)tm;
  g.tiles_n = (int)tn;
  return tgemm::launch_fp8(cfg, g, s, dev) == hipSuccess ? TGEMM_OK : TGEMM_ELAUNCH;
}

}  // namespace

extern "C" {

int gemm_fp8_block(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const float* scale_a,
                   const void* B, int64_t ldb, const float* scale_b, void* C, int64_t ldc, int relu,
                   void* stream) {
  const int cfg = fp8_select(M, N, K, A, lda, scale_a, B, ldb, scale_b, C, ldc);
  if (cfg == kSelectNoop) return TGEMM_OK;
  if (cfg < 0 && cfg != kSelectZeroFill && cfg != kFp8Generic) return cfg;
  return fp8_run(cfg, M, N, K, A, lda, scale_a, B, ldb, scale_b, C, ldc, relu, stream);
}

int gemm_fp8_block_cfg(int idx, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                       const float* scale_a, const void* B, int64_t ldb, const float* scale_b, void* C,
                       int64_t ldc, int relu, void* stream) {
  if (idx != kFp8Generic && (idx < 0 || idx >= fp8_table_size())) return TGEMM_EINVAL_CFG;
  const int cfg = fp8_select(M, N, K, A, lda, scale_a, B, ldb, scale_b, C, ldc);
  if (cfg == kSelectNoop) return TGEMM_OK;
  if (cfg < 0 && cfg != kSelectZeroFill && cfg != kFp8Generic) return cfg;
  if (cfg == kSelectZeroFill) return fp8_run(cfg, M, N, K, A, lda, scale_a, B, ldb, scale_b, C, ldc, relu, stream);
  if (idx != kFp8Generic && cfg == kFp8Generic) return TGEMM_EINVAL_CFG;  // needs the generic kernel
  return fp8_run(idx, M, N, K, A, lda, scale_a, B, ldb, scale_b, C, ldc, relu, stream);
}

int tgemm_fp8_select_config(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                            int64_t ldb, const void* C, int64_t ldc) {
  static const float kScaleProbe[1] = {0.0f};  // only its alignment is looked at
  return fp8_select(M, N, K, A, lda, kScaleProbe, B, ldb, kScaleProbe, C, ldc);
}

int tgemm_fp8_num_configs(void) { return fp8_table_size(); }

int tgemm_fp8_config_desc(int idx, tgemm_config_info* out) {
  if (out == nullptr) return TGEMM_ENULL;
  if (idx < 0 || idx >= fp8_table_size()) return TGEMM_EINVAL_CFG;
  const tgemm::Fp8Config& c = fp8_row(idx);
  std::memset(out, 0, sizeof(*out));
  out->block_m = c.bm;
  out->block_n = c.bn;
  out->block_k = tgemm::kFp8Block;
  out->stages = c.stages;
  out->waves_m = c.waves_m;
  out->waves_n = c.waves_n;
  out->panel = c.panel;
  out->xcd_remap = c.xcd_remap;
  out->generic = 0;
  out->layouts = 1 << 1;  // A as given (M x K), B transposed (N x K)
  out->lds_bytes = c.lds_bytes;
  std::strncpy(out->name, c.name, sizeof(out->name) - 1);
  return TGEMM_OK;
}

int quant_fp8_block(int64_t R, int64_t K, const void* X, int64_t ldx, int block_rows, void* Q, int64_t ldq,
                    float* scale, void* stream) {
  if (R < 0 || K < 0 || R >= TGEMM_MAX_DIM || K >= TGEMM_MAX_DIM) return TGEMM_EINVAL_DIM;
  if (block_rows != 1 && block_rows != 128) return TGEMM_EINVAL_DIM;
  const int64_t kmin = K > 1 ? K : 1;
  if (ldx < kmin || ldq < kmin) return TGEMM_EINVAL_LD;
  if (R == 0 || K == 0) return TGEMM_OK;
  if (X == nullptr || Q == nullptr || scale == nullptr) return TGEMM_ENULL;
  if ((reinterpret_cast<uintptr_t>(X) & 1u) || (reinterpret_cast<uintptr_t>(scale) & 3u)) return TGEMM_EALIGN;
  const int64_t KB = tgemm::ceil_div(K, tgemm::kFp8Block);
  // 1 x 128 blocks are numbered in 32 bits (2^32 blocks would be 1 TiB of input)
  if (block_rows == 1 && R * KB >= ((int64_t)1 << 32)) return TGEMM_EINVAL_DIM;
  const int64_t groups = block_rows == 1 ? tgemm::ceil_div(R * KB, 16) : tgemm::ceil_div(R, 128) * KB;
  if (groups >= ((int64_t)1 << 31)) return TGEMM_EINVAL_DIM;
  int dev = -1;
  const int d = check_device(&dev);
  if (d != TGEMM_OK) return d;
  tgemm::QuantArgs q;
  q.X = static_cast<const _Float16*>(X);
  q.Q = static_cast<uint8_t*>(Q);
  q.S = scale;
  q.ldx = ldx;
  q.ldq = ldq;
  q.R = (int)R;
  q.K = (int)K;
  q.KB = (int)KB;
  q.block_rows = block_rows;
  const bool vec = aligned16(X) && (reinterpret_cast<uintptr_t>(Q) & 7u) == 0 && ldx % 8 == 0 && ldq % 8 == 0 &&
                   K % 8 == 0;
  return tgemm::launch_quant_fp8(q, vec, static_cast<hipStream_t>(stream)) == hipSuccess ? TGEMM_OK
                                                                                           : TGEMM_ELAUNCH;
}

int gemm_f16_ex(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void* A,
                int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int relu, void* stream) {
  const int layout = layout_of(trans_a, trans_b);
  const int cfg = select(layout, M, N, K, A, lda, B, ldb, C, ldc);
  if (cfg == kSelectNoop) return TGEMM_OK;
  if (cfg < 0 && cfg != kSelectZeroFill) return cfg;
  return run(cfg, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream);
}

int gemm_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
             int64_t ldb, void* C, int64_t ldc, int relu, void* stream) {
  return gemm_f16_ex(0, 0, M, N, K, A, lda, B, ldb, C, ldc, relu, stream);
}

int gemm_f16_ex_cfg(int idx, int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void* A,
                    int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int relu, void* stream) {
  if (idx < 0 || idx >= table_size()) return TGEMM_EINVAL_CFG;
  const int layout = layout_of(trans_a, trans_b);
  const int cfg = select(layout, M, N, K, A, lda, B, ldb, C, ldc);
  if (cfg == kSelectNoop) return TGEMM_OK;
  if (cfg < 0 && cfg != kSelectZeroFill) return cfg;
  if (cfg == kSelectZeroFill) return run(cfg, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream);
  const Config& c = cfg_row(idx);
  if (!(c.layouts & (1 << layout))) return TGEMM_EINVAL_CFG;
  if (!c.generic && !fast_eligible(layout, M, N, K, A, lda, B, ldb, C, ldc)) return TGEMM_EINVAL_CFG;
  return run(idx, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream);
}

int gemm_f16_cfg(int idx, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                 const void* B, int64_t ldb, void* C, int64_t ldc, int relu, void* stream) {
  return gemm_f16_ex_cfg(idx, 0, 0, M, N, K, A, lda, B, ldb, C, ldc, relu, stream);
}

int64_t tgemm_workspace_bytes(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K) {
  const int layout = layout_of(trans_a, trans_b);
  if (M <= 0 || N <= 0 || K <= 0 || M >= TGEMM_MAX_DIM || N >= TGEMM_MAX_DIM || K >= TGEMM_MAX_DIM)
    return 0;
  // the plan for 16-byte-aligned operands with tight leading dimensions (other arguments
  // either plan the same or take the generic kernel, which needs no workspace)
  const int64_t lda = (layout & 2) ? M : K, ldb = (layout & 1) ? K : N;
  const uintptr_t a16 = 256;
  const int cfg = select(layout, M, N, K, (const void*)a16, lda, (const void*)a16, ldb, (const void*)a16, N);
  if (cfg < 0) return 0;
  const SplitPlan p = split_plan(layout, M, N, K, cfg);
  return ws_bytes(cfg_row(p.cfg), p.splits, M, N);
}

int tgemm_split_plan(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                     const void* B, int64_t ldb, const void* C, int64_t ldc, int* cfg_out, int* splits_out,
                     int64_t* workspace_bytes_out) {
  if (cfg_out == nullptr || splits_out == nullptr || workspace_bytes_out == nullptr) return TGEMM_ENULL;
  const int layout = layout_of(trans_a, trans_b);
  const int cfg = select(layout, M, N, K, A, lda, B, ldb, C, ldc);
  if (cfg < 0 && cfg != kSelectNoop && cfg != kSelectZeroFill) return cfg;
  SplitPlan p{cfg, 1};
  if (cfg >= 0) p = split_plan(layout, M, N, K, cfg);
  *cfg_out = p.cfg;
  *splits_out = p.splits;
  *workspace_bytes_out = cfg >= 0 ? ws_bytes(cfg_row(p.cfg), p.splits, M, N) : 0;
  return TGEMM_OK;
}

int gemm_f16_ws_cfg(int idx, int splits, int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                    const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int relu,
                    void* workspace, int64_t workspace_bytes, void* stream) {
  if (idx < 0 || idx >= table_size()) return TGEMM_EINVAL_CFG;
  if (splits < 1 || splits > kMaxSplits) return TGEMM_EINVAL_CFG;
  const int layout = layout_of(trans_a, trans_b);
  const int cfg = select(layout, M, N, K, A, lda, B, ldb, C, ldc);
  if (cfg == kSelectNoop) return TGEMM_OK;
  if (cfg < 0 && cfg != kSelectZeroFill) return cfg;
  if (cfg == kSelectZeroFill) return run(cfg, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream);
  const Config& c = cfg_row(idx);
  if (!(c.layouts & (1 << layout))) return TGEMM_EINVAL_CFG;
  if (!c.generic && !fast_eligible(layout, M, N, K, A, lda, B, ldb, C, ldc)) return TGEMM_EINVAL_CFG;
  if (splits > 1) {
    if (!split_capable(c) || splits > tgemm::ceil_div(K, c.bk) || workgroups(c, M, N) > kMaxSplitTiles)
      return TGEMM_EINVAL_CFG;
    if (workspace == nullptr) return TGEMM_ENULL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return TGEMM_EALIGN;
    if (workspace_bytes < ws_bytes(c, splits, M, N)) return TGEMM_EWORKSPACE;
  }
  return run(idx, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream, splits, workspace);
}

int64_t tgemm_workspace_bytes_cfg(int idx, int splits, int64_t M, int64_t N) {
  if (idx < 0 || idx >= table_size() || splits < 1 || splits > kMaxSplits) return TGEMM_EINVAL_CFG;
  if (M < 0 || N < 0 || M >= TGEMM_MAX_DIM || N >= TGEMM_MAX_DIM) return TGEMM_EINVAL_DIM;
  const Config& c = cfg_row(idx);
  if (splits > 1 && (!split_capable(c) || workgroups(c, M, N) > kMaxSplitTiles)) return TGEMM_EINVAL_CFG;
  return ws_bytes(c, splits, M, N);
}

int gemm_f16_ws_static(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                       const void* B, int64_t ldb, void* C, int64_t ldc, int relu, void* stream) {
  const int layout = layout_of(trans_a, trans_b);
  const int cfg = select(layout, M, N, K, A, lda, B, ldb, C, ldc);
  if (cfg == kSelectNoop) return TGEMM_OK;
  if (cfg < 0 && cfg != kSelectZeroFill) return cfg;
  if (cfg == kSelectZeroFill) return run(cfg, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream);
  const SplitPlan p = split_plan(layout, M, N, K, cfg);
  if (p.splits == 1) return run(cfg, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream);
  if (ws_bytes(cfg_row(p.cfg), p.splits, M, N) > TGEMM_STATIC_SCRATCH_BYTES) return TGEMM_EWORKSPACE;
  int dev = -1;
  const int d = check_device(&dev);
  if (d != TGEMM_OK) return d;
  void* scratch = nullptr;
  if (tgemm::static_scratch(dev, &scratch) != hipSuccess) return TGEMM_EDEVICE;
  return run(p.cfg, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream, p.splits, scratch);
}

int gemm_f16_ws(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                const void* B, int64_t ldb, void* C, int64_t ldc, int relu, void* workspace,
                int64_t workspace_bytes, void* stream) {
  const int layout = layout_of(trans_a, trans_b);
  const int cfg = select(layout, M, N, K, A, lda, B, ldb, C, ldc);
  if (cfg == kSelectNoop) return TGEMM_OK;
  if (cfg < 0 && cfg != kSelectZeroFill) return cfg;
  if (cfg == kSelectZeroFill) return run(cfg, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream);
  const SplitPlan p = split_plan(layout, M, N, K, cfg);
  if (p.splits == 1) return run(cfg, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream);
  if (workspace == nullptr) return TGEMM_ENULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return TGEMM_EALIGN;
  if (workspace_bytes < ws_bytes(cfg_row(p.cfg), p.splits, M, N)) return TGEMM_EWORKSPACE;
  return run(p.cfg, layout, M, N, K, A, lda, B, ldb, C, ldc, relu, stream, p.splits, workspace);
}

int gemm_f16_grouped(int trans_a, int trans_b, int count, const tgemm_gemm_desc* gemms, int relu,
                     void* stream) {
  if (count < 0) return TGEMM_EINVAL_DIM;
  if (count == 0) return TGEMM_OK;
  if (gemms == nullptr) return TGEMM_ENULL;
  const int layout = layout_of(trans_a, trans_b);
  // validate everything before enqueueing anything
  int64_t t128 = 0;
  for (int i = 0; i < count; ++i) {
    const tgemm_gemm_desc& d = gemms[i];
    const int v = select(layout, d.M, d.N, d.K, d.A, d.lda, d.B, d.ldb, d.C, d.ldc);
    if (v < 0 && v != kSelectNoop && v != kSelectZeroFill) return v;
    if (v >= 0 && fast_eligible(layout, d.M, d.N, d.K, d.A, d.lda, d.B, d.ldb, d.C, d.ldc))
      t128 += tgemm::ceil_div(d.M, 128) * tgemm::ceil_div(d.N, 128);
  }
  int dev = -1;
  const int dc = check_device(&dev);
  if (dc != TGEMM_OK) return dc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // One tile config for the whole group, counted in rounds of 256 workgroups as in
  // choose_fast: 128 x 128 tiles when all of them fit one round, else 256 x 256 (a round of
  // 144 tiles of 256 x 256 beats 576 of 128 x 128 in three by about a third).
  const int cfg = t128 <= kRound ? kCfgSmallT : kCfgBig;
  const tgemm::GroupedLauncher gl = tgemm::grouped_launcher(cfg);
  const Config& c = cfg_row(cfg);
  if (gl == nullptr) return TGEMM_ELAUNCH;
  tgemm::GroupedArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.relu = relu != 0;
  ga.layout = layout;
  int64_t nwg = 0;
  auto flush = [&]() -> int {
    if (ga.count == 0) return TGEMM_OK;
    ga.wg_start[ga.count] = (int)nwg;
    const hipError_t e = gl(ga, nwg, s, dev);
    ga.count = 0;
    nwg = 0;
    return e == hipSuccess ? TGEMM_OK : TGEMM_ELAUNCH;
  };
  for (int i = 0; i < count; ++i) {
    const tgemm_gemm_desc& d = gemms[i];
    const int v = select(layout, d.M, d.N, d.K, d.A, d.lda, d.B, d.ldb, d.C, d.ldc);
    if (v == kSelectNoop) continue;
    if (v == kSelectZeroFill || !fast_eligible(layout, d.M, d.N, d.K, d.A, d.lda, d.B, d.ldb, d.C, d.ldc)) {
      // K == 0, or arguments only the generic kernel takes: a launch of its own
      const int r = run(v, layout, d.M, d.N, d.K, d.A, d.lda, d.B, d.ldb, d.C, d.ldc, relu, stream);
      if (r != TGEMM_OK) return r;
      continue;
    }
    const int64_t tm = tgemm::ceil_div(d.M, c.bm), tn = tgemm::ceil_div(d.N, c.bn);
    if (ga.count == tgemm::kMaxGroups || nwg + tm * tn >= ((int64_t)1 << 31)) {
      const int r = flush();
      if (r != TGEMM_OK) return r;
    }
    tgemm::GroupEntry& e = ga.e[ga.count];
    e.A = static_cast<const _Float16*>(d.A);
    e.B = static_cast<const _Float16*>(d.B);
    e.C = static_cast<_Float16*>(d.C);
    e.lda = d.lda;
    e.ldb = d.ldb;
    e.ldc = d.ldc;
    e.M = (int)d.M;
    e.N = (int)d.N;
    e.K = (int)d.K;
    e.tiles_m = (int)tm;
    e.tiles_n = (int)tn;
    ga.wg_start[ga.count] = (int)nwg;
    nwg += tm * tn;
    ++ga.count;
  }
  return flush();
}

int tgemm_select_config_ex(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void* A,
                           int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc) {
  return select(layout_of(trans_a, trans_b), M, N, K, A, lda, B, ldb, C, ldc);
}

int tgemm_select_config(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                        const void* B, int64_t ldb, const void* C, int64_t ldc) {
  return select(0, M, N, K, A, lda, B, ldb, C, ldc);
}

const char* tgemm_strerror(int code) {
  switch (code) {
    case TGEMM_OK: return "success";
    case TGEMM_EINVAL_DIM: return "invalid dimension (negative, >= 2^31, or too many tiles)";
    case TGEMM_EINVAL_LD: return "invalid leading dimension (below the stored row length)";
    case TGEMM_ENULL: return "null pointer for a non-empty operand";
    case TGEMM_EDEVICE: return "current HIP device is not gfx950 (MI355X) or is unavailable";
    case TGEMM_ELAUNCH: return "kernel launch failed";
    case TGEMM_EINVAL_CFG: return "invalid config index, or config cannot take these arguments";
    case TGEMM_EALIGN: return "operand pointer not aligned to 2 bytes, or workspace not aligned to 256 bytes";
    case TGEMM_EWORKSPACE: return "workspace smaller than tgemm_workspace_bytes for these sizes";
    default: return "unknown error code";
  }
}

const char* tgemm_version(void) { return "libtgemm 0.1.0 (gfx950)"; }

int tgemm_num_configs(void) { return table_size(); }

int tgemm_config_desc(int idx, tgemm_config_info* out) {
  if (out == nullptr) return TGEMM_ENULL;
  if (idx < 0 || idx >= table_size()) return TGEMM_EINVAL_CFG;
  const Config& c = cfg_row(idx);
  std::memset(out, 0, sizeof(*out));
  out->block_m = c.bm;
  out->block_n = c.bn;
  out->block_k = c.bk;
  out->stages = c.stages;
  out->waves_m = c.waves_m;
  out->waves_n = c.waves_n;
  out->panel = c.panel;
  out->xcd_remap = c.xcd_remap;
  out->generic = c.generic;
  out->layouts = c.layouts;
  // operand tiles are held in LDS at a multiple of 128 rows / columns
  out->lds_bytes = c.generic ? 0 : c.stages * ((c.bm + 127) / 128 * 128 + (c.bn + 127) / 128 * 128) * c.bk * 2;
  std::strncpy(out->name, c.name, sizeof(out->name) - 1);
  return TGEMM_OK;
}

int64_t tgemm_num_workgroups(int idx, int64_t M, int64_t N) {
  if (idx < 0 || idx >= table_size() || M < 0 || N < 0) return -1;
  return workgroups(cfg_row(idx), M, N);
}

int tgemm_tile_of(int idx, int64_t M, int64_t N, int64_t wg, int64_t* tile_m, int64_t* tile_n) {
  if (idx < 0 || idx >= table_size()) return TGEMM_EINVAL_CFG;
  if (tile_m == nullptr || tile_n == nullptr) return TGEMM_ENULL;
  const Config& c = cfg_row(idx);
  const int64_t tm = tgemm::ceil_div(M, c.bm), tn = tgemm::ceil_div(N, c.bn);
  if (M <= 0 || N <= 0 || wg < 0 || wg >= tm * tn) return TGEMM_EINVAL_DIM;
  // The generic kernel runs the plain row-panel order (panel 1, no XCD remap).
  const int panel = c.generic ? 1 : c.panel;
  const int xcd = c.generic ? 0 : c.xcd_remap;
  tgemm::tile_of(wg, tm, tn, panel, xcd, tile_m, tile_n);
  return TGEMM_OK;
}

int tgemm_mfma_probe(int blocks, int iters, void* out, void* stream) {
  if (out == nullptr) return TGEMM_ENULL;
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 24)) return TGEMM_EINVAL_DIM;
  int dev = -1;
  const int d = check_device(&dev);
  if (d != TGEMM_OK) return d;
  return tgemm::launch_mfma_probe(blocks, iters, static_cast<float*>(out),
                                  static_cast<hipStream_t>(stream)) == hipSuccess
             ? TGEMM_OK
             : TGEMM_ELAUNCH;
}

#ifdef TGEMM_STAMPS
static_assert(TGEMM_STAMP_WORKGROUPS == tgemm::kStampWorkgroups &&
                  TGEMM_STAMP_WORDS == tgemm::kStampWords,
              "stamp table shape in the header matches the kernels");

int tgemm_stamps_capacity(int* workgroups, int* words_per_workgroup) {
  if (workgroups == nullptr || words_per_workgroup == nullptr) return TGEMM_ENULL;
  *workgroups = tgemm::kStampWorkgroups;
  *words_per_workgroup = tgemm::kStampWords;
  return TGEMM_OK;
}

int tgemm_stamps_read(uint64_t* host, int64_t words) {
  if (host == nullptr) return TGEMM_ENULL;
  if (words < 0 || words > (int64_t)tgemm::kStampWorkgroups * tgemm::kStampWords) return TGEMM_EINVAL_DIM;
  if (words == 0) return TGEMM_OK;
  return tgemm::stamps_read(reinterpret_cast<unsigned long long*>(host), words) == hipSuccess
             ? TGEMM_OK
             : TGEMM_ELAUNCH;
}

int tgemm_stamps_clear(void) { return tgemm::stamps_clear() == hipSuccess ? TGEMM_OK : TGEMM_ELAUNCH; }
#endif

}  // extern "C"
