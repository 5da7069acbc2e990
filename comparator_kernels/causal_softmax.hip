// Row softmax of attention scores for the composed-attention comparator
// (comparator.py): the step between the two library GEMMs of attention
// written out with its S x S probabilities (T14 flash-attention design doc,
// "What flash-attention is": the composed path the fused kernel replaces).
// This is benchmark scaffolding, not part of libxfa.so.
//
// scores [rows, S] (rows = B*H*S, row r is query r % S of its head) in T
// (bf16 or fp32) -> probs [rows, S] in T: p_ij = exp(s_ij * scale - m_i) /
// sum_j exp(...) over the keys query i sees (j <= i when causal), p_ij = 0 for
// the others.  One wave per row: a pass forms each lane's running maximum
// and sum (exp2 with scale * log2 e folded), the wave combines them, a second
// pass writes every element of the row.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline float to_f(bf16 x) { return (float)x; }
__device__ inline float to_f(float x) { return x; }
template <typename T> __device__ inline T from_f(float x);
template <> __device__ inline bf16 from_f<bf16>(float x) { return (bf16)x; }
template <> __device__ inline float from_f<float>(float x) { return x; }

// merge (m2, l2) into (m, l): sums of 2^(x - m) over two sets of values
__device__ inline void merge(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == -__builtin_huge_valf()) return;      // both empty
  l = l * __builtin_amdgcn_exp2f(m - mn) + l2 * __builtin_amdgcn_exp2f(m2 - mn);
  m = mn;
}

template <typename T>
__global__ __launch_bounds__(256) void causal_softmax_kernel(const T* __restrict__ s, T* __restrict__ p,
                                                             int64_t rows, int S, float c_log2, int causal) {
  constexpr int V = 16 / sizeof(T);               // elements per 16-byte chunk
  typedef T vec __attribute__((ext_vector_type(V)));
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int i = (int)(row % S);
  const int n = causal ? i + 1 : S;               // keys this query sees: [0, n)
  const T* src = s + row * S;
  T* dst = p + row * S;
  const bool vec_ok = (S % V) == 0;               // rows start 16-byte aligned

  float m = -__builtin_huge_valf(), l = 0.f;
  auto add = [&](float x) {
    x *= c_log2;
    if (x > m) {
      l = l * __builtin_amdgcn_exp2f(m - x) + 1.f;
      m = x;
    } else {
      l += __builtin_amdgcn_exp2f(x - m);
    }
  };
  if (vec_ok) {
    for (int j0 = V * lane; j0 < n; j0 += V * 64) {
      const vec x = *reinterpret_cast<const vec*>(src + j0);
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (j0 + e < n) add(to_f(x[e]));
    }
  } else {
    for (int j = lane; j < n; j += 64) add(to_f(src[j]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    merge(m, l, m2, l2);
  }
  const float inv = 1.f / l;                      // l >= 1: key 0 is always seen
  if (vec_ok) {
    for (int j0 = V * lane; j0 < S; j0 += V * 64) {
      vec y;
      if (j0 < n) {
        const vec x = *reinterpret_cast<const vec*>(src + j0);
#pragma unroll
        for (int e = 0; e < V; ++e)
          y[e] = from_f<T>(j0 + e < n ? __builtin_amdgcn_exp2f(to_f(x[e]) * c_log2 - m) * inv : 0.f);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) y[e] = from_f<T>(0.f);
      }
      *reinterpret_cast<vec*>(dst + j0) = y;
    }
  } else {
    for (int j = lane; j < S; j += 64)
      dst[j] = from_f<T>(j < n ? __builtin_amdgcn_exp2f(to_f(src[j]) * c_log2 - m) * inv : 0.f);
  }
}

}  // namespace

// dtype 0: fp32, 1: bf16.  Returns 0, or 1 for bad arguments, 3 for a failed
// launch.  Enqueued on `stream`; nothing is allocated.
extern "C" int xfa_comparator_causal_softmax(const void* scores, void* probs, int64_t BH, int64_t S,
                                             float scale, int causal, int dtype, void* stream) {
  if (BH < 0 || S < 0 || !(scale > 0.f) || (causal != 0 && causal != 1) || (dtype != 0 && dtype != 1)) return 1;
  if (BH == 0 || S == 0) return 0;
  if (!scores || !probs || S > (int64_t(1) << 30)) return 1;
  const int64_t rows = BH * S;
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > INT32_MAX) return 1;
  const float c = scale * 1.4426950408889634f;
  if (dtype == 1)
    hipLaunchKernelGGL(causal_softmax_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const bf16*)scores, (bf16*)probs, rows, (int)S, c, causal);
  else
    hipLaunchKernelGGL(causal_softmax_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const float*)scores, (float*)probs, rows, (int)S, c, causal);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
