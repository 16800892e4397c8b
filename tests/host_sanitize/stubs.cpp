// Host-only stand-ins for everything tgemm_api.cpp calls outside itself: the config tables
// (rebuilt from the same X-macro lists as the kernels' tables), recording launchers in
// place of the kernels, and the two HIP runtime calls of the device check. Built with
// tgemm_api.cpp and driver.cpp into one executable under AddressSanitizer and
// UndefinedBehaviorSanitizer: no GPU, no HIP runtime library.
#include "stubs.h"

#include <cstdio>
#include <cstring>
#include <deque>
#include <string>
#include <vector>

#include "tgemm_configs.h"

namespace stub {
std::vector<Launch> launches;
int fail_next_launch = 0;
long total_launches = 0;

static hipError_t result() {
  ++total_launches;
  if (fail_next_launch) {
    fail_next_launch = 0;
    return hipErrorLaunchFailure;
  }
  return hipSuccess;
}
}  // namespace stub

namespace {

// Names as the kernels' tables spell them (a deque: the strings never move).
std::deque<std::string>& names() {
  static std::deque<std::string> n;
  return n;
}
const char* keep(const std::string& s) {
  names().push_back(s);
  return names().back().c_str();
}
std::string row_name(const char* kind, int bm, int bn, int bk, int s, int wm, int wn, int p, int x) {
  char buf[64];
  std::snprintf(buf, sizeof buf, "%s%dx%dx%d_s%d_w%dx%d_p%d_x%d", kind, bm, bn, bk, s, wm, wn, p, x);
  return buf;
}

std::vector<tgemm::Config> build_table() {
  std::vector<tgemm::Config> t;
  t.push_back({64, 64, 32, 1, 2, 2, 1, 0, 1, 0xF, 1, "generic_64x64x32"});
#define ROW9(KIND)                                                                                         \
  [&](int bm, int bn, int bk, int wm, int wn, int s, int p, int x, int prod) {                             \
    t.push_back({bm, bn, bk, s, wm, wn, p, x, 0, 1, TGEMM_BUILT(prod), keep(row_name(KIND, bm, bn, bk, s, wm, wn, p, x))}); \
  }
#define ROW10(KIND)                                                                                        \
  [&](int bm, int bn, int bk, int wm, int wn, int s, int p, int x, int all, int prod) {                    \
    t.push_back({bm, bn, bk, s, wm, wn, p, x, 0, all ? 0xF : 1, TGEMM_BUILT(prod),                        \
                 keep(row_name(KIND, bm, bn, bk, s, wm, wn, p, x))});                                      \
  }
  auto fast = ROW9("t");
  auto pipe = ROW9("p");
  auto pp = ROW9("q");
  auto pp1 = ROW10("m");
  auto quad = ROW10("u");
#define CALL_FAST(...) fast(__VA_ARGS__);
#define CALL_PIPE(...) pipe(__VA_ARGS__);
#define CALL_PP(...) pp(__VA_ARGS__);
#define CALL_PP1(...) pp1(__VA_ARGS__);
#define CALL_QUAD(...) quad(__VA_ARGS__);
  TGEMM_FAST_CONFIGS(CALL_FAST)
  TGEMM_PIPE_CONFIGS(CALL_PIPE)
  TGEMM_PP_CONFIGS(CALL_PP)
  TGEMM_PP1_CONFIGS(CALL_PP1)
  TGEMM_QUAD_CONFIGS(CALL_QUAD)
  TGEMM_PIPE2_CONFIGS(CALL_PIPE)
  return t;
}

std::vector<tgemm::Fp8Config> build_fp8_table() {
  std::vector<tgemm::Fp8Config> t;
  auto row = [&](int bm, int bn, int wm, int wn, int s, int p, int x, int mode, int prod) {
    char buf[64];
    std::snprintf(buf, sizeof buf, "f%dx%dx128_s%d_w%dx%d%s", bm, bn, s, wm, wn,
                  mode == 2 ? "_pp" : mode == 1 ? "_db1" : "_db0");
    t.push_back({bm, bn, wm, wn, s, p, x, 0, TGEMM_BUILT(prod), keep(buf)});
  };
#define CALL_FP8(...) row(__VA_ARGS__);
  TGEMM_FP8_CONFIGS(CALL_FP8)
  return t;
}

const std::vector<tgemm::Config>& table() {
  static const std::vector<tgemm::Config> t = build_table();
  return t;
}
const std::vector<tgemm::Fp8Config>& fp8_table() {
  static const std::vector<tgemm::Fp8Config> t = build_fp8_table();
  return t;
}

template <int I>
hipError_t record_gemm(const tgemm::GemmArgs& g, hipStream_t s, int device) {
  stub::Launch l{};
  l.kind = stub::kGemm;
  l.cfg = I;
  l.gemm = g;
  l.stream = s;
  l.device = device;
  stub::launches.push_back(l);
  return stub::result();
}

template <int... I>
struct GemmRecorders {
  static constexpr tgemm::Launcher table[] = {record_gemm<I>...};
};
template <int... I>
constexpr tgemm::Launcher GemmRecorders<I...>::table[];

using Recorders = GemmRecorders<0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21, 22,
                                23, 24, 25, 26, 27, 28, 29, 30, 31>;

template <int I>
hipError_t record_grouped(const tgemm::GroupedArgs& ga, int64_t nwg, hipStream_t s, int device) {
  stub::Launch l{};
  l.kind = stub::kGrouped;
  l.cfg = I;
  l.grouped = ga;
  l.nwg = nwg;
  l.stream = s;
  l.device = device;
  stub::launches.push_back(l);
  return stub::result();
}

}  // namespace

namespace tgemm {

const Config* config_table(int* count) {
  *count = (int)table().size();
  return table().data();
}

Launcher launcher(int idx) {
  static_assert(sizeof(Recorders::table) / sizeof(Recorders::table[0]) >= 32, "recorders");
  if (idx < 0 || idx >= (int)table().size()) return nullptr;
  return Recorders::table[idx];
}

// Like the kernels' version: only the 256 x 256 and 128 x 128 ping-pong rows with all four
// layouts, 4 stages, 2 x 4 waves, panel 4 and the XCD remap have grouped launchers.
GroupedLauncher grouped_launcher(int idx) {
  if (idx < 0 || idx >= (int)table().size()) return nullptr;
  const Config& c = table()[idx];
  if (c.generic || c.layouts != 0xF || c.bk != 32 || c.stages != 4 || c.waves_m != 2 || c.waves_n != 4 ||
      c.panel != 4 || c.xcd_remap != 1)
    return nullptr;
  if (c.bm == 256 && c.bn == 256) return record_grouped<256>;
  if (c.bm == 128 && c.bn == 128) return record_grouped<128>;
  return nullptr;
}

const Fp8Config* fp8_config_table(int* count) {
  *count = (int)fp8_table().size();
  return fp8_table().data();
}

hipError_t launch_fp8(int idx, const Fp8Args& g, hipStream_t s, int device) {
  if (idx < 0 || idx >= (int)fp8_table().size()) return hipErrorInvalidValue;
  stub::Launch l{};
  l.kind = stub::kFp8;
  l.cfg = idx;
  l.fp8 = g;
  l.stream = s;
  l.device = device;
  stub::launches.push_back(l);
  return stub::result();
}

hipError_t launch_fp8_generic(const Fp8Args& g, hipStream_t s) {
  stub::Launch l{};
  l.kind = stub::kFp8;
  l.cfg = -1;
  l.fp8 = g;
  l.stream = s;
  stub::launches.push_back(l);
  return stub::result();
}

hipError_t launch_quant_fp8(const QuantArgs& q, bool vec, hipStream_t s) {
  stub::Launch l{};
  l.kind = stub::kQuant;
  l.quant = q;
  l.vec = vec;
  l.stream = s;
  stub::launches.push_back(l);
  return stub::result();
}

hipError_t launch_zero_fill(_Float16* C, int M, int N, int64_t ldc, hipStream_t s) {
  stub::Launch l{};
  l.kind = stub::kZeroFill;
  l.zf_C = C;
  l.zf_M = M;
  l.zf_N = N;
  l.zf_ldc = ldc;
  l.stream = s;
  stub::launches.push_back(l);
  return stub::result();
}

// The static scratch array's device address: a fixed fake, 256-byte aligned.
hipError_t static_scratch(int device, void** out) {
  if (device < 0) return hipErrorInvalidDevice;
  *out = reinterpret_cast<void*>((uintptr_t)0x7f0000000000ull + (uintptr_t)device * 0x100000000ull);
  return hipSuccess;
}

}  // namespace tgemm

// The HIP runtime calls of the device check: device 0, a gfx950.
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}

hipError_t hipGetDeviceProperties(hipDeviceProp_t* prop, int device) {
  (void)device;
  std::memset(prop, 0, sizeof(*prop));
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}
