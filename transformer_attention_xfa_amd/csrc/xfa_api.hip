// C-ABI layer of libxfa.so: argument checks, then kernel launches on the
// caller's stream.  Declarations and the full contract are in xfa.h.
#include <math.h>
#include <stdint.h>

#include "xfa.h"
#include "xfa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Shape {
  int64_t BH = 0, S = 0, hd = 0;
  bool empty = false;
  bool bf16 = false;
};

// Checks shared by every entry point; fills `sh` on success.
xfa_status_t check_common(int64_t B, int64_t H, int64_t S, int64_t hd, float scale, int causal,
                          int dtype, Shape* sh) {
  if (dtype != XFA_DTYPE_F32 && dtype != XFA_DTYPE_BF16) return XFA_ERR_INVALID_ARGUMENT;
  if (B < 0 || H < 0 || S < 0 || hd <= 0) return XFA_ERR_INVALID_ARGUMENT;
  if (!(isfinite(scale) && scale > 0.f)) return XFA_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return XFA_ERR_INVALID_ARGUMENT;
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128) return XFA_ERR_UNSUPPORTED;
  // the kernels index positions with int
  if (S > (int64_t(1) << 30)) return XFA_ERR_UNSUPPORTED;
  // one head of one fp32 tensor, plus the blocks the kernels stage past its
  // end (fewer than 256 rows), must stay below 2^31 bytes: the staging
  // offsets of out-of-range lanes start at 2^31 and must not wrap
  if ((S + 256) * hd * 4 > int64_t(INT32_MAX)) return XFA_ERR_UNSUPPORTED;
  if (B > 0 && H > INT64_MAX / B) return XFA_ERR_UNSUPPORTED;
  const int64_t BH = B * H;
  // each kernel of the three entry points but the preprocess launches one
  // 256-thread workgroup per (head, 128-row tile) on a 1-D grid, and a
  // dispatch counts its work-items in 32 bits
  if (BH > 0 && (S + 127) / 128 > ((int64_t(1) << 24) - 1) / BH) return XFA_ERR_UNSUPPORTED;
  sh->BH = BH;
  sh->S = S;
  sh->hd = hd;
  sh->empty = (BH == 0 || S == 0);
  sh->bf16 = dtype == XFA_DTYPE_BF16;
  return XFA_OK;
}

xfa_status_t check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr || !aligned16(p)) return XFA_ERR_INVALID_ARGUMENT;
  return XFA_OK;
}

xfa_status_t from_hip(hipError_t e) { return e == hipSuccess ? XFA_OK : XFA_ERR_HIP; }

// Dropout probability p in [0, 1) -> the kernels' threshold and scale
// (thresh = ceil(p 2^24): keep iff the generator's top 24 bits >= thresh,
// the same decision as (bits / 2^24) >= p in float32; thresh 0 = off).
xfa_status_t drop_args(float p, uint64_t seed, xfa::DropArgs* d) {
  if (!(p >= 0.f && p < 1.f)) return XFA_ERR_INVALID_ARGUMENT;   // also rejects NaN
  d->seed = seed;
  d->thresh = (uint32_t)ceil((double)p * 16777216.0);
  d->inv_keep = 1.f / (1.f - p);
  return XFA_OK;
}

}  // namespace

extern "C" {

xfa_status_t xfa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t B, int64_t H, int64_t S, int64_t hd, float scale, int causal,
                     int dtype, void* stream) {
  Shape sh;
  xfa_status_t st = check_common(B, H, S, hd, scale, causal, dtype, &sh);
  if (st != XFA_OK || sh.empty) return st;
  if ((st = check_ptrs({q, k, v, out, lse})) != XFA_OK) return st;
  xfa::FwdArgs a{q, k, v, out, lse, sh.BH, sh.S, sh.hd, scale, causal, sh.bf16, (hipStream_t)stream};
  return from_hip(xfa::launch_fwd(a));
}

xfa_status_t xfa_fwd_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t B, int64_t H, int64_t S, int64_t hd, float scale, int causal,
                             float dropout_p, uint64_t seed, int dtype, void* stream) {
  Shape sh;
  xfa::DropArgs d;
  xfa_status_t st = check_common(B, H, S, hd, scale, causal, dtype, &sh);
  if (st == XFA_OK) st = drop_args(dropout_p, seed, &d);
  if (st != XFA_OK || sh.empty) return st;
  st = check_ptrs({q, k, v, out, lse});
  if (st != XFA_OK) return st;
  xfa::FwdArgs a{q, k, v, out, lse, sh.BH, sh.S, sh.hd, scale, causal, sh.bf16, (hipStream_t)stream, d};
  return from_hip(xfa::launch_fwd(a));
}

xfa_status_t xfa_bwd_preprocess(const void* out, const void* dout, float* delta, int64_t B,
                                int64_t H, int64_t S, int64_t hd, float scale, int causal,
                                int dtype, void* stream) {
  Shape sh;
  xfa_status_t st = check_common(B, H, S, hd, scale, causal, dtype, &sh);
  if (st != XFA_OK || sh.empty) return st;
  if ((st = check_ptrs({out, dout, delta})) != XFA_OK) return st;
  xfa::PreArgs a{out, dout, delta, sh.BH, sh.S, sh.hd, sh.bf16, (hipStream_t)stream};
  return from_hip(xfa::launch_bwd_preprocess(a));
}

size_t xfa_bwd_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int) {
  // dQ is formed by its own query-outer kernel: nothing is accumulated
  // across workgroups, so no workspace
  return 0;
}

xfa_status_t xfa_bwd(const void* q, const void* k, const void* v, const void* dout,
                     const float* lse, const float* delta, void* dq, void* dk, void* dv,
                     void* /*workspace: size 0, unused*/, int64_t B, int64_t H, int64_t S, int64_t hd,
                     float scale, int causal, int dtype, void* stream) {
  Shape sh;
  xfa_status_t st = check_common(B, H, S, hd, scale, causal, dtype, &sh);
  if (st != XFA_OK || sh.empty) return st;
  if ((st = check_ptrs({q, k, v, dout, lse, delta, dq, dk, dv})) != XFA_OK) return st;
  xfa::BwdArgs a{q, k, v, dout, lse, delta, dq, dk, dv,
                 sh.BH, sh.S, sh.hd, scale, causal, sh.bf16, (hipStream_t)stream};
  return from_hip(xfa::launch_bwd(a));
}

xfa_status_t xfa_bwd_dropout(const void* q, const void* k, const void* v, const void* dout,
                             const float* lse, const float* delta, void* dq, void* dk, void* dv,
                             void* /*workspace: size 0, unused*/, int64_t B, int64_t H, int64_t S,
                             int64_t hd, float scale, int causal, float dropout_p, uint64_t seed,
                             int dtype, void* stream) {
  Shape sh;
  xfa::DropArgs d;
  xfa_status_t st = check_common(B, H, S, hd, scale, causal, dtype, &sh);
  if (st == XFA_OK) st = drop_args(dropout_p, seed, &d);
  if (st != XFA_OK || sh.empty) return st;
  st = check_ptrs({q, k, v, dout, lse, delta, dq, dk, dv});
  if (st != XFA_OK) return st;
  xfa::BwdArgs a{q, k, v, dout, lse, delta, dq, dk, dv,
                 sh.BH, sh.S, sh.hd, scale, causal, sh.bf16, (hipStream_t)stream, d};
  return from_hip(xfa::launch_bwd(a));
}

const char* xfa_status_string(xfa_status_t s) {
  switch (s) {
    case XFA_OK: return "xfa: ok";
    case XFA_ERR_INVALID_ARGUMENT: return "xfa: invalid argument";
    case XFA_ERR_UNSUPPORTED: return "xfa: unsupported size";
    case XFA_ERR_HIP: return "xfa: HIP launch failed";
  }
  return "xfa: unknown status";
}

}  // extern "C"
