// Backward preprocess: D = rowsum(dO * O).
//
// D_i = sum_d dO_i[d] * O_i[d]  (T14 flash-attention design doc, "What
// flash-attention is", backward part, and Key Design Decision 3: the softmax
// Jacobian's row term sum_j P_ij dP_ij equals this per-query dot product).
// One row of O / dO is spread over the lanes that hold its 16-byte chunks;
// each thread keeps several rows' loads in flight, sums its chunk in fp32 and
// the row is finished with a butterfly over those lanes.
#include "xfa_common.h"
#include "xfa_launch.h"

namespace xfa {

constexpr int kPreThreads = 256;
constexpr int kPreUnroll = 2;

// At most this many workgroups per launch (the dispatch counts work-items in
// 32 bits); a larger problem loops over its rows in strides of the grid.
constexpr int64_t kPreMaxGroups = int64_t(1) << 20;

template <typename T, int HD>
__global__ __launch_bounds__(kPreThreads) void bwd_pre_kernel(
    const T* __restrict__ O, const T* __restrict__ dO, float* __restrict__ Dl, int64_t nrows) {
  constexpr int VE = Vec16<T>::N;
  constexpr int LPR = HD / VE;                     // lanes per row (power of two, <= 32)
  constexpr int RPI = kPreThreads / LPR;           // rows per workgroup per unroll step
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  const int64_t stride = (int64_t)gridDim.x * RPI * kPreUnroll;
  // the lanes of a row share row0, so they take every branch together
  for (int64_t row0 = (int64_t)blockIdx.x * RPI * kPreUnroll + tid / LPR; row0 < nrows; row0 += stride) {
    typename Vec16<T>::type a[kPreUnroll], b[kPreUnroll];
#pragma unroll
    for (int u = 0; u < kPreUnroll; ++u) {
      const int64_t r = row0 + (int64_t)u * RPI;
      if (r < nrows) {
        a[u] = ld16(O + r * HD + sub * VE);
        b[u] = ld16(dO + r * HD + sub * VE);
      } else {
        a[u] = typename Vec16<T>::type{};
        b[u] = typename Vec16<T>::type{};
      }
    }
#pragma unroll
    for (int u = 0; u < kPreUnroll; ++u) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) s += (float)a[u][e] * (float)b[u][e];
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, LPR);
      const int64_t r = row0 + (int64_t)u * RPI;
      if (sub == 0 && r < nrows) Dl[r] = s;
    }
  }
}

template <typename T, int HD>
static hipError_t launch_pre_t(const PreArgs& a) {
  constexpr int LPR = HD / Vec16<T>::N;
  constexpr int rows_per_wg = (kPreThreads / LPR) * kPreUnroll;
  const int64_t nrows = a.BH * a.S;
  const int64_t nwg = min((nrows + rows_per_wg - 1) / rows_per_wg, kPreMaxGroups);
  hipLaunchKernelGGL((bwd_pre_kernel<T, HD>), dim3((unsigned)nwg), dim3(kPreThreads), 0, a.stream,
                     (const T*)a.out, (const T*)a.dout, a.delta, nrows);
  return hipGetLastError();
}

template <typename T>
static hipError_t pre_dispatch(const PreArgs& a) {
  switch (a.hd) {
    case 16: return launch_pre_t<T, 16>(a);
    case 32: return launch_pre_t<T, 32>(a);
    case 64: return launch_pre_t<T, 64>(a);
    case 128: return launch_pre_t<T, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_preprocess(const PreArgs& a) {
  return a.bf16 ? pre_dispatch<bf16>(a) : pre_dispatch<float>(a);
}

}  // namespace xfa
