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
// registers as the B operand; for bf16 the V tile is staged into LDS already
// transposed (a swizzled [d][key] layout, see TTile), so each V^T fragment is
// one 16-byte read.  K and V tiles are staged in LDS, with the next tile's
// global loads in flight while the current one is processed.  The exponent is
// taken in base 2: with c = scale * log2(e) and a reference maximum m (log2
// units), p = 2^(x c - m) is one fused multiply-add and one exp2.  Only tiles
// that cross the diagonal or the sequence end evaluate the mask, and the row
// sum l is taken over the bf16-rounded weights that enter P.V.
#include <type_traits>

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

  constexpr bool TV = sizeof(T) == 2;           // bf16: V staged transposed
  using TT = TTile<BK>;
  constexpr int VUN = (BK / 4) * (HD / 2);      // 4-row x 2-column units of a V tile
  constexpr int PFV = TV ? (VUN + NT - 1) / NT : PF;
  constexpr int VS_ELEMS = TV ? HDP * BK : BK * VLD;

  __shared__ __attribute__((aligned(16))) T Ks[BK * KLD];
  __shared__ __attribute__((aligned(16))) T Vs[VS_ELEMS];

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

  // padding of the V tile (d >= HD) stays zero for the whole kernel
  if constexpr (HDP != HD) {
    if constexpr (TV) {
      for (int e = tid; e < (HDP - HD) * BK; e += NT) Vs[HD * BK + e] = (T)0.f;
    } else {
      for (int e = tid; e < BK * (HDP - HD); e += NT) {
        const int r = e / (HDP - HD), c = HD + e % (HDP - HD);
        Vs[r * VLD + c] = (T)0.f;
      }
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

  typename Vec16<T>::type pk[PF], pv[TV ? 1 : PF];
  unsigned pvt[TV ? PFV : 1][4];
  auto prefetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      const int r = e / CPR, c = (e - r * CPR) * VE;
      const uint32_t off = (uint32_t)(kt * BK + r) * ROWB + c * sizeof(T);
      if (TILE_CHUNKS % NT == 0 || e < TILE_CHUNKS) {
        pk[i] = bload16<T>(rK, off);   // rows past the end read as zeros
        if constexpr (!TV) pv[i] = bload16<T>(rV, off);
      }
    }
    if constexpr (TV) {
#pragma unroll
      for (int i = 0; i < PFV; ++i) {
        const int e = tid + i * NT;
        const int cp = e % (HD / 2), rg = e / (HD / 2);
        const uint32_t off = (uint32_t)(kt * BK + 4 * rg) * ROWB + cp * 4u;
        if (VUN % NT == 0 || e < VUN) {
#pragma unroll
          for (int k = 0; k < 4; ++k) pvt[i][k] = __float_as_uint(bload4(rV, off + k * ROWB));
        }
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
        if constexpr (!TV) st16(Vs + r * VLD + c, pv[i]);
      }
    }
    if constexpr (TV) {
      unsigned* vt = reinterpret_cast<unsigned*>(Vs);
#pragma unroll
      for (int i = 0; i < PFV; ++i) {
        const int e = tid + i * NT;
        if (VUN % NT == 0 || e < VUN) {
          const int cp = e % (HD / 2), rg = e / (HD / 2);
          const int p = swap23(4 * rg);
          u32x2 col0, col1;
          transpose_4x2(pvt[i], col0, col1);
          const bool odd_first = (l >> 3) & 1;
          const int c_first = 2 * cp + (odd_first ? 1 : 0);
          const int dw_half = 2 * ((p >> 2) & 1);
          *reinterpret_cast<u32x2*>(vt + TT::chunk_dw(c_first, p >> 3) + dw_half) = odd_first ? col1 : col0;
          *reinterpret_cast<u32x2*>(vt + TT::chunk_dw(c_first ^ 1, p >> 3) + dw_half) = odd_first ? col0 : col1;
        }
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) oacc[d] = zero16();
  // The reference maximum m_ref (log2 units) only moves when some lane's
  // tile maximum exceeds it by more than kRescale; until then p stays below
  // 2^kRescale and the accumulators need no rescaling.  out = acc / l does
  // not depend on the reference, so this changes no result beyond rounding.
  constexpr float kRescale = 8.f;
  float m_ref = kNegInf;
  float l_run = 0.f;       // running sum over the keys this lane half holds

  auto tile = [&](auto masked, int k0) {
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = zero16();
      const T* krow = Ks + (kb * 32 + (l & 31)) * KLD + M::KW * h;
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc[kb] = M::mma(ld_nat(krow + c * M::KD), qf[c], sacc[kb]);
    }
    if constexpr (decltype(masked)::value) {
      // keys past this query (causal) or past the sequence end
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
    mt = fmaxf(mt, swap_halves(mt)) * c_log2;   // row maximum, log2 units (scale > 0)
    if (__builtin_amdgcn_ballot_w64(mt > m_ref + kRescale)) {
      const float m_new = fmaxf(m_ref, mt);     // key 0 is visible to every query
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d) oacc[d] *= alpha;
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        sacc[kb][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v], c_log2, -m_ref));

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const typename M::frag pf = frag_from_acc(sacc[kb], u, T{});
        if constexpr (sizeof(T) == 2) {
          // row sum of the bf16 weights that enter P.V, two per dot2
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          const bf16x2 one2{(bf16)1.f, (bf16)1.f};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[2 * e], pf[2 * e + 1]}, one2, l_run, false);
        } else {
          l_run += pf;
        }
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          typename M::frag vf;
          if constexpr (TV) {
            const int c = d * 32 + (l & 31);
            vf = *reinterpret_cast<const bf16x8*>(Vs + 2 * TT::chunk_dw(c, 4 * kb + 2 * u + h));
          } else {
            vf = ld_res(Vs, VLD, kb * 32, u, d * 32);
          }
          oacc[d] = M::mma(vf, pf, oacc[d]);
        }
      }
    }
  };

  // Tiles before n_full are unmasked for every wave of the workgroup; the
  // rest (the diagonal and the sequence end) go through the masked variant.
  const int n_full = min(causal ? (q0 + 1) / BK : n_tiles, S / BK);
  auto step = [&](auto masked, int kt) {
    __syncthreads();
    stage();
    __syncthreads();
    if (kt + 1 < n_tiles) prefetch(kt + 1);
    const int k0 = kt * BK;
    // the wave skips tiles wholly above its part of the diagonal
    if (wave_live && !(causal && k0 > qw_last)) tile(masked, k0);
  };
  prefetch(0);
  for (int kt = 0; kt < n_full; ++kt) step(std::false_type{}, kt);
  for (int kt = n_full; kt < n_tiles; ++kt) step(std::true_type{}, kt);

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
    bstore4(rL, (uint32_t)qi * 4u, (m_ref + __log2f(l_tot)) * kLn2);
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
