// Host-side launch interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xfa {

// Attention-probabilities dropout: on iff thresh > 0; element index i of the
// [B*H, S, S] probabilities is kept iff the top 24 bits of the generator's
// output for (seed, i) are >= thresh = ceil(p 2^24); kept probabilities are
// scaled by inv_keep = 1 / (1 - p).
struct DropArgs {
  uint64_t seed = 0; uint32_t thresh = 0; float inv_keep = 1.f;
};

struct FwdArgs {
  const void* q; const void* k; const void* v; void* out; float* lse;
  int64_t BH, S, hd; float scale; int causal; bool bf16; hipStream_t stream;
  DropArgs drop;
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
  DropArgs drop;
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd_preprocess(const PreArgs& a);
hipError_t launch_bwd(const BwdArgs& a);

}  // namespace xfa
