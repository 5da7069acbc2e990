// Host-side launch interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xfa {

struct FwdArgs {
  const void* q; const void* k; const void* v; void* out; float* lse;
  int64_t BH, S, hd; float scale; int causal; bool bf16; hipStream_t stream;
};

// Backward workspace: an fp32 dQ accumulator [BH, S, hd] followed by one
// arrival counter per (head, backward query tile).
struct Workspace {
  float* dq_acc;
  unsigned* counters;
  int64_t n_counters;
};

struct PreArgs {
  const void* out; const void* dout; float* delta; Workspace ws;
  int64_t BH, S, hd; bool bf16; hipStream_t stream;
};

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* dout;
  const float* lse; const float* delta;
  void* dq; void* dk; void* dv; Workspace ws;
  int64_t BH, S, hd; float scale; int causal; bool bf16; hipStream_t stream;
};

// Query rows per backward query tile (the counter granularity).
int bwd_query_tile(bool is_bf16, int64_t hd);
// Workspace layout for these sizes; `base` may be null to only get the size.
size_t bwd_workspace(void* base, int64_t BH, int64_t S, int64_t hd, bool is_bf16, Workspace* ws);

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd_preprocess(const PreArgs& a);
hipError_t launch_bwd(const BwdArgs& a);

}  // namespace xfa
