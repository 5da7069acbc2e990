// The atomic traffic alone of the other way to sum dQ (T14 flash-attention
// design doc, "Key Design Decisions" 3 and the escape hatches: the page's
// backward adds across rows with fp32 atomics; its follow-up gives each key
// block its own dK/dV, which leaves dQ_i = sum_j ds_ij K_j to be summed
// across key blocks).  With key workgroups of 128 keys that keep dK and dV in
// registers, each workgroup contributes to every 32-query block it sweeps a
// [32, hd] fp32 partial of dQ; summed by atomics, the smallest traffic is one
// fp32 atomic add per dQ element per (key workgroup, query block) pair.  This
// kernel issues exactly that traffic and nothing else (no loads, no matrix
// work), adding 1.0 each time, so after one launch on a zeroed buffer
//   acc[bh][q][d] = number of key workgroups that see query q
//                 = q / 128 + 1 (causal) or ceil(S / 128) (full).
// Its time is a lower bound of what the atomic design would spend on atomics
// per backward.  Benchmark scaffolding, not part of libxfa.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kKeys = 128;     // keys per key workgroup
constexpr int kRows = 32;      // queries per query block
constexpr int kThreads = 256;

// consecutive workgroup ids go to the 8 XCDs in turn; give each XCD a
// contiguous range of logical ids (one head's workgroups share an L2)
__device__ inline int xcd_logical(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = bid & 7, slot = bid >> 3;
  return x * q + (x < r ? x : r) + slot;
}

__global__ __launch_bounds__(kThreads) void dq_atomic_floor_kernel(float* __restrict__ acc, int S, int hd,
                                                                  int nkt, int causal, int nwg) {
  const int lid = xcd_logical(blockIdx.x, nwg);
  const int bh = lid / nkt, kt = lid - bh * nkt;
  const int nb = (S + kRows - 1) / kRows;
  const int n0 = causal ? kt * (kKeys / kRows) : 0;
  float* head = acc + (size_t)bh * S * hd;
  const int per_block = kRows * hd;              // multiple of kThreads (hd >= 8)
  for (int n = n0; n < nb; ++n) {
    for (int e = threadIdx.x; e < per_block; e += kThreads) {
      const int row = n * kRows + e / hd;
      if (row < S) __hip_atomic_fetch_add(head + (size_t)row * hd + (e % hd), 1.0f, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

// acc: [BH, S, hd] fp32 device buffer (zeroed by the caller for a checkable
// result).  0 = enqueued on `stream`, 1 = bad arguments (nothing enqueued),
// 3 = launch failed.
extern "C" int xfa_comparator_dq_atomic_floor(float* acc, int64_t BH, int64_t S, int64_t hd, int causal,
                                              void* stream) {
  if (BH < 0 || S < 0 || (hd != 16 && hd != 32 && hd != 64 && hd != 128) || (causal != 0 && causal != 1))
    return 1;
  if (BH == 0 || S == 0) return 0;
  if (acc == nullptr || S > (int64_t(1) << 30)) return 1;
  const int64_t nkt = (S + kKeys - 1) / kKeys;
  if (BH > int64_t(INT32_MAX) / nkt) return 1;
  const int nwg = (int)(BH * nkt);
  hipLaunchKernelGGL(dq_atomic_floor_kernel, dim3(nwg), dim3(kThreads), 0, (hipStream_t)stream, acc, (int)S,
                     (int)hd, (int)nkt, causal, nwg);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
