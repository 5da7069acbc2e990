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
// taken in base 2: with c = scale * log2(e) and m the running maximum of the
// raw logits, p = 2^(x c - m c) is one fused multiply-add and one exp2.
// Only tiles that cross the diagonal or the sequence end evaluate the mask.
#include "xfa_common.h"
#include "xfa_launch.h"

namespace xfa {

template <typename T, int HD, int NW, int BK>
__global__ __launch_bounds__(NW * 64, 2) void fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, T* __restrict__ O,
    float* __restrict__ Lse, int S, float c_log2, int causal, int nqt, int nwg) {
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
  constexpr uint32_t ROWB = HD * sizeof(T);             // bytes per row in HBM
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
  const uint32_t head_bytes = (uint32_t)S * ROWB;
  const rsrc_t rQ = make_rsrc(Q + hoff, head_bytes);
  const rsrc_t rK = make_rsrc(K + hoff, head_bytes);
  const rsrc_t rV = make_rsrc(V + hoff, head_bytes);

  const int q0 = qt * BQ;
  const int qw0 = q0 + 32 * w;                   // first query of this wave
  const int qi = qw0 + (l & 31);                 // this lane's query
  const int q_last = min(q0 + BQ, S) - 1;        // last real query of the workgroup
  const int qw_last = min(qw0 + 31, S - 1);      // last real query of this wave
  const bool wave_live = qw0 < S;
  const int n_tiles = causal ? (q_last / BK + 1) : ((S + BK - 1) / BK);
  // last key this lane's query may see
  const int key_lim = causal ? min(qi, S - 1) : S - 1;

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
    const uint32_t off = (uint32_t)qi * ROWB + (c * M::KD + M::KW * h) * sizeof(T);
    if constexpr (sizeof(T) == 2) qf[c] = bload16<bf16>(rQ, off);
    else qf[c] = bload4(rQ, off);
  }

  typename Vec16<T>::type pk[PF], pv[PF];
  auto prefetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      const int r = e / CPR, c = (e - r * CPR) * VE;
      const uint32_t off = (uint32_t)(kt * BK + r) * ROWB + c * sizeof(T);
      if (TILE_CHUNKS % NT == 0 || e < TILE_CHUNKS) {
        pk[i] = bload16<T>(rK, off);   // rows past the end read as zeros
        pv[i] = bload16<T>(rV, off);
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      if (TILE_CHUNKS % NT == 0 || e < TILE_CHUNKS) {
        const int r = e / CPR, c = (e - r * CPR) * VE;
        st16(Ks + r * KLD + c, pk[i]);
        st16(Vs + r * VLD + c, pv[i]);
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) oacc[d] = zero16();
  float m_run = kNegInf;   // running max of this lane's raw logits
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

    // mask keys past this query (causal) or past the sequence end; only tiles
    // that reach the diagonal or the end need it
    if ((k0 + BK > S) || (causal && k0 + BK - 1 > qw0)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int rel = key_lim - (k0 + kb * 32 + 4 * h);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          sacc[kb][v] = (8 * (v >> 2) + (v & 3) > rel) ? kNegInf : sacc[kb][v];
      }
    }
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, sacc[kb][v]);
    mt = fmaxf(mt, swap_halves(mt));
    const float m_new = fmaxf(m_run, mt);   // finite: key 0 is visible to every query
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c_log2);
    m_run = m_new;
    const float mc = m_new * c_log2;

    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v], c_log2, -mc));
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
  // rows past the sequence end fall outside the buffer and are dropped
  const rsrc_t rO = make_rsrc(O + hoff, head_bytes);
  const uint32_t orow = (uint32_t)qi * ROWB;
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = d * 32 + 8 * g + 4 * h;
      if (HDP == HD || dd < HD)
        bstore_row4(rO, orow + dd * sizeof(T), oacc[d][4 * g] * inv_l, oacc[d][4 * g + 1] * inv_l,
                    oacc[d][4 * g + 2] * inv_l, oacc[d][4 * g + 3] * inv_l, T{});
    }
  }
  if (h == 0) {
    const rsrc_t rL = make_rsrc(Lse + (size_t)bh * S, (uint32_t)S * 4u);
    bstore4(rL, (uint32_t)qi * 4u, (m_run * c_log2 + __log2f(l_tot)) * kLn2);
  }
}

template <typename T, int HD>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  constexpr int NW = 4;
  constexpr int BK = 64;
  constexpr int BQ = NW * 32;
  const int nqt = (int)((a.S + BQ - 1) / BQ);
  const int nwg = (int)(a.BH * nqt);
  hipLaunchKernelGGL((fwd_kernel<T, HD, NW, BK>), dim3(nwg), dim3(NW * 64), 0, a.stream,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.S,
                     a.scale * kLog2e, a.causal, nqt, nwg);
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
