// Recorded launches of the host-only sanitizer build (see stubs.cpp).
#pragma once

#include <vector>

#include "tgemm_internal.h"

namespace stub {

enum Kind { kGemm, kGrouped, kFp8, kQuant, kZeroFill };

struct Launch {
  Kind kind;
  int cfg;  // table row (gemm, fp8; -1: fp8 generic) or tile size (grouped)
  tgemm::GemmArgs gemm;
  tgemm::GroupedArgs grouped;
  int64_t nwg;
  tgemm::Fp8Args fp8;
  tgemm::QuantArgs quant;
  bool vec;
  _Float16* zf_C;
  int zf_M, zf_N;
  int64_t zf_ldc;
  hipStream_t stream;
  int device;
};

extern std::vector<Launch> launches;
extern long total_launches;   // every launch recorded since the start
extern int fail_next_launch;  // the next recorded launch reports a launch failure

}  // namespace stub
