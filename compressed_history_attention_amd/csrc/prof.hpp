// Per-stage HIP-event timing of the tuned path (profiling aid).
#pragma once

#include "nkv_common.hpp"

namespace nkv {

bool prof_on();

// Records a start event on construction and a stop event on destruction
// (only while profiling is enabled).
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_;
};

}  // namespace nkv
