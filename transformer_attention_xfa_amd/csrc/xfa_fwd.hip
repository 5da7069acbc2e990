// Forward pass: online-softmax attention over KV tiles (T14 flash-attention
// design doc, section "What flash-attention is": the running-max / running-sum
// recurrence, out = acc / l and L = m + log l, the inlined causal mask and the
// skip of tiles wholly above the diagonal).
//
// Work split (differs from the page's one-block-per-query-row kernel, which
// left the GPU underfilled): one workgroup per (head, tile of BQ = 32*NW
// queries); wave w owns 32 consecutive queries.  Each wave computes the
// transposed scores S^T = K . Q^T so that every lane owns one query: the
// row max / row sum of the online softmax are then in-lane reductions plus one
// exchange between the two lane halves, and the per-query rescale factor is a
// per-lane scalar.  O^T = V^T . P^T reuses the score tile straight from
// registers as the B operand; V^T is read from the row-major V tile with the
// LDS transpose read.  K and V tiles are staged in LDS, with the next tile's
// global loads in flight while the current one is processed.  The exponent is
// taken in base 2 with log2(e) folded into the score scale.
#include "xfa_common.h"
#include "xfa_launch.h"

namespace xfa {

template <typename T, int HD, int NW, int BK>
__global__ __launch_bounds__(NW * 64, 2) void fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, T* __restrict__ O,
    float* __restrict__ Lse, int S, float scale_log2, int causal, int nqt, int nwg) {
  using M = Mma<T>;
  constexpr int BQ = NW * 32;
  constexpr int NT = NW * 64;
  constexpr int HDP = HD < 32 ? 32 : HD;        // d padded to whole 32-row blocks
  constexpr int NDB = HDP / 32;                 // 32-row d blocks of O^T
  constexpr int NKB = BK / 32;                  // 32-key blocks per KV tile
  constexpr int NC = HD / M::KD;                // instructions along d for S^T
  constexpr int NU = 32 / M::KD;                // instructions per 32-key block for P.V
  constexpr int VE = Vec16<T>::N;               // elements per 16-byte transfer
  constexpr int CPR = HD / VE;                  // 16-byte chunks per row
  constexpr int KLD = HD + (sizeof(T) == 2 ? 8 : 4);    // padded LDS row strides
  constexpr int VLD = HDP + (sizeof(T) == 2 ? 16 : 4);
  constexpr int TILE_CHUNKS = BK * CPR;
  constexpr int PF = (TILE_CHUNKS + NT - 1) / NT;       // chunks per thread per tile
  static_assert(HD % M::KD == 0 && HD % VE == 0, "unsupported head dim");

  __shared__ __attribute__((aligned(16))) T Ks[BK * KLD];
  __shared__ __attribute__((aligned(16))) T Vs[BK * VLD];

  const int tid = threadIdx.x;
  const int l = lane();
  const int h = l >> 5;
  const int w = tid >> 6;

  // heaviest query tiles first, one head's tiles together per XCD
  const int lid = xcd_logical(blockIdx.x, nwg);
  const int bh = lid / nqt;
  const int qt = nqt - 1 - (lid - bh * nqt);

  const size_t hoff = (size_t)bh * S * HD;
  const T* Qh = Q + hoff;
  const T* Kh = K + hoff;
  const T* Vh = V + hoff;

  const int q0 = qt * BQ;
  const int qw0 = q0 + 32 * w;                   // first query of this wave
  const int qi = qw0 + (l & 31);                 // this lane's query
  const int q_last = min(q0 + BQ, S) - 1;        // last real query of the workgroup
  const int qw_last = min(qw0 + 31, S - 1);      // last real query of this wave
  const bool wave_live = qw0 < S;
  const int n_tiles = causal ? (q_last / BK + 1) : ((S + BK - 1) / BK);

  // padding columns of the V tile (d >= HD) stay zero for the whole kernel
  if constexpr (HDP != HD) {
    for (int e = tid; e < BK * (HDP - HD); e += NT) {
      const int r = e / (HDP - HD), c = HD + e % (HDP - HD);
      Vs[r * VLD + c] = (T)0.f;
    }
  }

  // Q fragments: B operand of S^T = K . Q^T (column = query, natural d order)
  typename M::frag qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (qi < S) qf[c] = ld_nat(Qh + (size_t)qi * HD + c * M::KD + M::KW * h);
    else qf[c] = M::zero();
  }

  typename Vec16<T>::type pk[PF], pv[PF];
  auto prefetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      const int r = e / CPR, c = (e - r * CPR) * VE;
      const int key = kt * BK + r;
      if (e < TILE_CHUNKS && key < S) {
        pk[i] = ld16(Kh + (size_t)key * HD + c);
        pv[i] = ld16(Vh + (size_t)key * HD + c);
      } else {
        pk[i] = typename Vec16<T>::type{};
        pv[i] = typename Vec16<T>::type{};
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      if (e < TILE_CHUNKS) {
        const int r = e / CPR, c = (e - r * CPR) * VE;
        st16(Ks + r * KLD + c, pk[i]);
        st16(Vs + r * VLD + c, pv[i]);
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) oacc[d] = zero16();
  float m_run = kNegInf;   // running max of this lane's query, log2 units
  float l_run = 0.f;       // running sum over the keys this lane half holds

  prefetch(0);
  for (int kt = 0; kt < n_tiles; ++kt) {
    __syncthreads();
    stage();
    __syncthreads();
    if (kt + 1 < n_tiles) prefetch(kt + 1);

    const int k0 = kt * BK;
    // the wave skips tiles wholly above its part of the diagonal
    if (!wave_live || (causal && k0 > qw_last)) continue;

    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = zero16();
      const T* krow = Ks + (kb * 32 + (l & 31)) * KLD + M::KW * h;
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc[kb] = M::mma(ld_nat(krow + c * M::KD), qf[c], sacc[kb]);
    }

    const bool need_mask = (k0 + BK > S) || (causal && k0 + BK - 1 > qw0);
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float s = sacc[kb][v] * scale_log2;
        if (need_mask) {
          const int key = k0 + kb * 32 + acc_row(v, h);
          if (key >= S || (causal && key > qi)) s = kNegInf;
        }
        sacc[kb][v] = s;
        mt = fmaxf(mt, s);
      }
    }
    mt = fmaxf(mt, swap_halves(mt));
    const float m_new = fmaxf(m_run, mt);   // finite: key 0 is visible to every query
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(sacc[kb][v] - m_new);
        sacc[kb][v] = p;
        ps += p;
      }
    }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int d = 0; d < NDB; ++d) oacc[d] *= alpha;

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const typename M::frag pf = frag_from_acc(sacc[kb], u, T{});
#pragma unroll
        for (int d = 0; d < NDB; ++d)
          oacc[d] = M::mma(ld_res(Vs, VLD, kb * 32, u, d * 32), pf, oacc[d]);
      }
    }
  }

  if (!wave_live) return;
  const float l_tot = l_run + swap_halves(l_run);
  const float inv_l = 1.f / l_tot;
  if (qi < S) {
    T* orow = O + hoff + (size_t)qi * HD;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = d * 32 + 8 * g + 4 * h;
        if (dd < HD) {
          if constexpr (sizeof(T) == 2) {
            bf16x4 o4{(bf16)(oacc[d][4 * g + 0] * inv_l), (bf16)(oacc[d][4 * g + 1] * inv_l),
                      (bf16)(oacc[d][4 * g + 2] * inv_l), (bf16)(oacc[d][4 * g + 3] * inv_l)};
            *reinterpret_cast<bf16x4*>(orow + dd) = o4;
          } else {
            f32x4 o4{oacc[d][4 * g + 0] * inv_l, oacc[d][4 * g + 1] * inv_l,
                     oacc[d][4 * g + 2] * inv_l, oacc[d][4 * g + 3] * inv_l};
            *reinterpret_cast<f32x4*>(orow + dd) = o4;
          }
        }
      }
    }
    if (h == 0) Lse[(size_t)bh * S + qi] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <typename T, int HD>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  constexpr int NW = 4;
  constexpr int BK = 64;
  constexpr int BQ = NW * 32;
  const int nqt = (int)((a.S + BQ - 1) / BQ);
  const long long nwg_ll = (long long)a.BH * nqt;
  const int nwg = (int)nwg_ll;
  const float scale_log2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_kernel<T, HD, NW, BK>), dim3(nwg), dim3(NW * 64), 0, a.stream,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.S,
                     scale_log2, a.causal, nqt, nwg);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_hd(const FwdArgs& a) {
  switch (a.hd) {
    case 16: return launch_fwd_t<T, 16>(a);
    case 32: return launch_fwd_t<T, 32>(a);
    case 64: return launch_fwd_t<T, 64>(a);
    case 128: return launch_fwd_t<T, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a) {
  return a.bf16 ? dispatch_hd<bf16>(a) : dispatch_hd<float>(a);
}

}  // namespace xfa
