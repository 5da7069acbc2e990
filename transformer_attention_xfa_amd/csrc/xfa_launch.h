// Host-side launch interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xfa {

struct FwdArgs {
  const void* q; const void* k; const void* v; void* out; float* lse;
  int64_t BH, S, hd; float scale; int causal; bool bf16; hipStream_t stream;
};

struct PreArgs {
  const void* out; const void* dout; float* delta;
  int64_t BH, S, hd; bool bf16; hipStream_t stream;
};

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* dout;
  const float* lse; const float* delta;
  void* dq; void* dk; void* dv;
  int64_t BH, S, hd; float scale; int causal; bool bf16; hipStream_t stream;
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd_preprocess(const PreArgs& a);
hipError_t launch_bwd(const BwdArgs& a);

}  // namespace xfa
