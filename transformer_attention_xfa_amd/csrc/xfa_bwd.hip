// Backward pass by recomputation (T14 flash-attention design doc, "What
// flash-attention is", backward part): for every unmasked (query i, key j)
//   s_ij = Q_i . K_j * scale,  p_ij = exp(s_ij - L_i),  dp_ij = dO_i . V_j,
//   ds_ij = p_ij (dp_ij - D_i) scale,
//   dQ_i += ds_ij K_j,  dK_j += ds_ij Q_i,  dV_j += p_ij dO_i,
// without any S x S buffer.
//
// Work split (the page's kernel looped over query rows and added dK/dV with
// atomics, which it names as its bottleneck; its own follow-up is a key-block
// owned dK/dV pass, Key Design Decisions / escape hatches): one workgroup per
// (head, tile of 32*NW keys); wave w owns 32 keys and keeps their dK and dV in
// registers for the whole sweep over query tiles, starting at the first query
// tile that reaches the diagonal.  Per query tile each wave computes
// S = Q . K^T and dP = dO . V^T with the lane owning one key, so that
// dV^T += dO^T . P and dK^T += Q^T . dS take P and dS straight from registers
// (dO^T and Q^T come from the row-major LDS tiles by the transpose read).  dS
// is then passed through LDS so that the workgroup forms dQ = dS . K for the
// tile over all of its keys, and adds it into an fp32 dQ accumulator with
// atomics (one add per element per key tile, not per key).  When a workgroup
// is done it publishes its additions and counts itself in on every query tile
// it touched; the workgroup that completes a tile's count writes that tile of
// dq in the output type.  Nothing ever waits on another workgroup.
#include "xfa_common.h"
#include "xfa_launch.h"

namespace xfa {

__device__ inline void atomic_add_f32(float* p, float v) { unsafeAtomicAdd(p, v); }

template <typename T, int HD, int NW, int BQ>
__global__ __launch_bounds__(NW * 64, 1) void bwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ Dl,
    T* __restrict__ dQ, T* __restrict__ dK, T* __restrict__ dV, float* __restrict__ dQacc,
    unsigned* __restrict__ counters, int S, float scale, float scale_log2, int causal, int nkt,
    int nwg) {
  using M = Mma<T>;
  constexpr int BKV = NW * 32;                   // keys per workgroup
  constexpr int NT = NW * 64;
  constexpr int HDP = HD < 32 ? 32 : HD;
  constexpr int NDB = HDP / 32;                  // 32-row d blocks
  constexpr int NQB = BQ / 32;                   // 32-query blocks per query tile
  constexpr int NC = HD / M::KD;                 // instructions along d
  constexpr int NU = 32 / M::KD;                 // instructions per 32-wide k block
  constexpr int VE = Vec16<T>::N;
  constexpr int CPR = HD / VE;
  constexpr int PADN = sizeof(T) == 2 ? 16 : 4;
  constexpr int QLD = HDP + PADN;                // Q / dO / K tile row stride
  constexpr int SLD = BQ + PADN;                 // dS tile row stride
  constexpr int QCH = BQ * CPR;                  // 16-byte chunks per Q (or dO) tile
  constexpr int PF = (QCH + NT - 1) / NT;
  constexpr int NOB = NQB * NDB;                 // dQ output blocks per query tile
  constexpr int OBW = (NOB + NW - 1) / NW;       // dQ output blocks per wave
  static_assert(HD % M::KD == 0 && HD % VE == 0, "unsupported head dim");
  static_assert(BQ <= NT, "L/D staging assumes one thread per query");

  __shared__ __attribute__((aligned(16))) T Qs[BQ * QLD];
  __shared__ __attribute__((aligned(16))) T dOs[BQ * QLD];
  __shared__ __attribute__((aligned(16))) T Ks[BKV * QLD];
  __shared__ __attribute__((aligned(16))) T dSs[BKV * SLD];
  __shared__ __attribute__((aligned(16))) float Ls[BQ];
  __shared__ __attribute__((aligned(16))) float Ds[BQ];
  __shared__ int last_of[NT];

  const int tid = threadIdx.x;
  const int l = lane();
  const int h = l >> 5;
  const int w = tid >> 6;

  // heaviest key tiles (the earliest keys see the most queries) first,
  // one head's tiles together per XCD
  const int lid = xcd_logical(blockIdx.x, nwg);
  const int bh = lid / nkt;
  const int kt = lid - bh * nkt;

  const size_t hoff = (size_t)bh * S * HD;
  const T* Qh = Q + hoff;
  const T* dOh = dO + hoff;
  const float* Lh = Lse + (size_t)bh * S;
  const float* Dh = Dl + (size_t)bh * S;
  float* dQh = dQacc + hoff;

  const int j0 = kt * BKV;                       // first key of the workgroup
  const int jw0 = j0 + 32 * w;                   // first key of this wave
  const int kj = jw0 + (l & 31);                 // this lane's key
  const bool wave_live = jw0 < S;
  const int nqt = (S + BQ - 1) / BQ;
  const int qt_first = causal ? j0 / BQ : 0;

  // zero the padding columns once; stage the workgroup's K tile (B operand of dQ)
  if constexpr (HDP != HD) {
    for (int e = tid; e < BQ * (HDP - HD); e += NT) {
      const int r = e / (HDP - HD), c = HD + e % (HDP - HD);
      Qs[r * QLD + c] = (T)0.f;
      dOs[r * QLD + c] = (T)0.f;
    }
    for (int e = tid; e < BKV * (HDP - HD); e += NT) {
      const int r = e / (HDP - HD), c = HD + e % (HDP - HD);
      Ks[r * QLD + c] = (T)0.f;
    }
  }
  for (int e = tid; e < BKV * CPR; e += NT) {
    const int r = e / CPR, c = (e - r * CPR) * VE;
    const int key = j0 + r;
    typename Vec16<T>::type x{};
    if (key < S) x = ld16(K + hoff + (size_t)key * HD + c);
    st16(Ks + r * QLD + c, x);
  }

  // this lane's key row of K and V: B operands of S = Q.K^T and dP = dO.V^T
  typename M::frag kf[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (kj < S) {
      kf[c] = ld_nat(K + hoff + (size_t)kj * HD + c * M::KD + M::KW * h);
      vf[c] = ld_nat(V + hoff + (size_t)kj * HD + c * M::KD + M::KW * h);
    } else {
      kf[c] = M::zero();
      vf[c] = M::zero();
    }
  }

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    dkacc[d] = zero16();
    dvacc[d] = zero16();
  }

  typename Vec16<T>::type pq[PF], pd[PF];
  float pl = 0.f, pdl = 0.f;
  auto prefetch = [&](int qt) {
    const int q0 = qt * BQ;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      const int r = e / CPR, c = (e - r * CPR) * VE;
      const int q = q0 + r;
      if (e < QCH && q < S) {
        pq[i] = ld16(Qh + (size_t)q * HD + c);
        pd[i] = ld16(dOh + (size_t)q * HD + c);
      } else {
        pq[i] = typename Vec16<T>::type{};
        pd[i] = typename Vec16<T>::type{};
      }
    }
    if (tid < BQ) {
      const int q = q0 + tid;
      pl = q < S ? Lh[q] * kLog2e : 0.f;
      pdl = q < S ? Dh[q] : 0.f;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      if (e < QCH) {
        const int r = e / CPR, c = (e - r * CPR) * VE;
        st16(Qs + r * QLD + c, pq[i]);
        st16(dOs + r * QLD + c, pd[i]);
      }
    }
    if (tid < BQ) {
      Ls[tid] = pl;
      Ds[tid] = pdl;
    }
  };

  prefetch(qt_first);
  for (int qt = qt_first; qt < nqt; ++qt) {
    __syncthreads();
    stage();
    __syncthreads();
    if (qt + 1 < nqt) prefetch(qt + 1);

    const int q0 = qt * BQ;
    const int q_last = min(q0 + BQ, S) - 1;
    // keys of this wave all above the diagonal of this query tile: nothing to add
    const bool active = wave_live && !(causal && jw0 > q_last);

    if (active) {
      f32x16 sacc[NQB], pacc[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        sacc[qb] = zero16();
        pacc[qb] = zero16();
        const T* qrow = Qs + (qb * 32 + (l & 31)) * QLD + M::KW * h;
        const T* dorow = dOs + (qb * 32 + (l & 31)) * QLD + M::KW * h;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sacc[qb] = M::mma(ld_nat(qrow + c * M::KD), kf[c], sacc[qb]);
          pacc[qb] = M::mma(ld_nat(dorow + c * M::KD), vf[c], pacc[qb]);
        }
      }

      const bool need_mask = (q0 + BQ > S) || (jw0 + 32 > S) || (causal && jw0 + 31 > q0);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = qb * 32 + 8 * g + 4 * h;
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(Ls + r0);
          const f32x4 D4 = *reinterpret_cast<const f32x4*>(Ds + r0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * g + e;
            float p = __builtin_amdgcn_exp2f(sacc[qb][v] * scale_log2 - L4[e]);
            if (need_mask) {
              const int q = q0 + r0 + e;
              if (q >= S || kj >= S || (causal && kj > q)) p = 0.f;
            }
            sacc[qb][v] = p;
            pacc[qb][v] = p * (pacc[qb][v] - D4[e]) * scale;
          }
        }
      }

      // dV^T += dO^T . P,  dK^T += Q^T . dS   (k runs over the tile's queries)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const typename M::frag pf = frag_from_acc(sacc[qb], u, T{});
          const typename M::frag sf = frag_from_acc(pacc[qb], u, T{});
#pragma unroll
          for (int d = 0; d < NDB; ++d) {
            dvacc[d] = M::mma(ld_res(dOs, QLD, qb * 32, u, d * 32), pf, dvacc[d]);
            dkacc[d] = M::mma(ld_res(Qs, QLD, qb * 32, u, d * 32), sf, dkacc[d]);
          }
        }
      }

      // dS to LDS as [key][query]: 4 consecutive queries per store
      T* srow = dSs + (32 * w + (l & 31)) * SLD;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = qb * 32 + 8 * g + 4 * h;
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x4*>(srow + c0) =
                bf16x4{(bf16)pacc[qb][4 * g], (bf16)pacc[qb][4 * g + 1], (bf16)pacc[qb][4 * g + 2],
                       (bf16)pacc[qb][4 * g + 3]};
          } else {
            *reinterpret_cast<f32x4*>(srow + c0) =
                f32x4{pacc[qb][4 * g], pacc[qb][4 * g + 1], pacc[qb][4 * g + 2], pacc[qb][4 * g + 3]};
          }
        }
      }
    } else {
      T* srow = dSs + (32 * w + (l & 31)) * SLD;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = qb * 32 + 8 * g + 4 * h;
          if constexpr (sizeof(T) == 2) *reinterpret_cast<bf16x4*>(srow + c0) = bf16x4{};
          else *reinterpret_cast<f32x4*>(srow + c0) = f32x4{};
        }
      }
    }
    __syncthreads();

    // dQ tile = dS . K over the workgroup's keys; each wave takes some
    // (32 queries x 32 d) output blocks and adds them into the accumulator.
    const int nkb = causal ? min(NW, (q_last - j0) / 32 + 1) : NW;   // key blocks not wholly masked
#pragma unroll
    for (int ob = 0; ob < OBW; ++ob) {
      const int b = w + NW * ob;
      if (b < NOB) {
        const int qb = b / NDB, db = b - (b / NDB) * NDB;
        f32x16 acc = zero16();
        for (int kb = 0; kb < nkb; ++kb) {
#pragma unroll
          for (int u = 0; u < NU; ++u)
            acc = M::mma(ld_res(dSs, SLD, kb * 32, u, qb * 32), ld_res(Ks, QLD, kb * 32, u, db * 32), acc);
        }
        const int d = db * 32 + (l & 31);
        if (d < HD) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int q = q0 + qb * 32 + acc_row(v, h);
            if (q < S) atomic_add_f32(dQh + (size_t)q * HD + d, acc[v]);
          }
        }
      }
    }
  }

  // dK_j, dV_j for this lane's key: C tile column = key, rows = d
  if (kj < S) {
    T* dkrow = dK + hoff + (size_t)kj * HD;
    T* dvrow = dV + hoff + (size_t)kj * HD;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = d * 32 + 8 * g + 4 * h;
        if (dd < HD) {
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x4*>(dkrow + dd) =
                bf16x4{(bf16)dkacc[d][4 * g], (bf16)dkacc[d][4 * g + 1], (bf16)dkacc[d][4 * g + 2],
                       (bf16)dkacc[d][4 * g + 3]};
            *reinterpret_cast<bf16x4*>(dvrow + dd) =
                bf16x4{(bf16)dvacc[d][4 * g], (bf16)dvacc[d][4 * g + 1], (bf16)dvacc[d][4 * g + 2],
                       (bf16)dvacc[d][4 * g + 3]};
          } else {
            *reinterpret_cast<f32x4*>(dkrow + dd) =
                f32x4{dkacc[d][4 * g], dkacc[d][4 * g + 1], dkacc[d][4 * g + 2], dkacc[d][4 * g + 3]};
            *reinterpret_cast<f32x4*>(dvrow + dd) =
                f32x4{dvacc[d][4 * g], dvacc[d][4 * g + 1], dvacc[d][4 * g + 2], dvacc[d][4 * g + 3]};
          }
        }
      }
    }
  }

  // Publish this workgroup's dQ additions, then count it in on each query
  // tile it added to.  The arrival that completes a tile (every key tile that
  // reaches it has published) converts the tile's fp32 sums into dq.
  __threadfence();
  __syncthreads();
  unsigned* cnt = counters + (size_t)bh * nqt;
  for (int base = qt_first; base < nqt; base += NT) {
    const int qt = base + tid;
    int last = 0;
    if (qt < nqt) {
      const int q_last = min(qt * BQ + BQ, S) - 1;
      const unsigned expected = causal ? (unsigned)min(nkt, q_last / BKV + 1) : (unsigned)nkt;
      last = atomicAdd(cnt + qt, 1u) == expected - 1u;
    }
    last_of[tid] = last;
    __syncthreads();
    const int nbatch = min(NT, nqt - base);
    for (int t = 0; t < nbatch; ++t) {
      if (!last_of[t]) continue;
      __threadfence();
      const int r0 = (base + t) * BQ;
      const int nr = min(BQ, S - r0);
      const float* src = dQh + (size_t)r0 * HD;
      T* dst = dQ + hoff + (size_t)r0 * HD;
      for (int e = tid * 4; e < nr * HD; e += NT * 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(src + e);
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<bf16x4*>(dst + e) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
        } else {
          *reinterpret_cast<f32x4*>(dst + e) = x;
        }
      }
    }
    __syncthreads();
  }
}

template <typename T, int HD>
struct BwdCfg {
  static constexpr int NW = 4;
  // fp32 tiles at hd = 128 would not fit the 160 KiB of LDS with 64 queries
  static constexpr int BQ = (sizeof(T) == 4 && HD == 128) ? 32 : 64;
};

template <typename T, int HD>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  constexpr int NW = BwdCfg<T, HD>::NW;
  constexpr int BQ = BwdCfg<T, HD>::BQ;
  constexpr int BKV = NW * 32;
  const int nkt = (int)((a.S + BKV - 1) / BKV);
  const int nwg = (int)(a.BH * nkt);
  hipLaunchKernelGGL((bwd_kernel<T, HD, NW, BQ>), dim3(nwg), dim3(NW * 64), 0, a.stream,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout, a.lse, a.delta,
                     (T*)a.dq, (T*)a.dk, (T*)a.dv, a.ws.dq_acc, a.ws.counters, (int)a.S, a.scale,
                     a.scale * kLog2e, a.causal, nkt, nwg);
  return hipGetLastError();
}

int bwd_query_tile(bool is_bf16, int64_t hd) {
  if (is_bf16) return BwdCfg<bf16, 64>::BQ;
  return hd == 128 ? BwdCfg<float, 128>::BQ : BwdCfg<float, 64>::BQ;
}

size_t bwd_workspace(void* base, int64_t BH, int64_t S, int64_t hd, bool is_bf16, Workspace* ws) {
  const int64_t bq = bwd_query_tile(is_bf16, hd);
  const size_t acc_bytes = (size_t)(BH * S * hd) * sizeof(float);
  const int64_t n_counters = BH * ((S + bq - 1) / bq);
  const size_t cnt_bytes = ((size_t)n_counters * sizeof(unsigned) + 255) & ~(size_t)255;
  if (ws) {
    ws->dq_acc = static_cast<float*>(base);
    ws->counters = base ? reinterpret_cast<unsigned*>(static_cast<char*>(base) + acc_bytes) : nullptr;
    ws->n_counters = n_counters;
  }
  return acc_bytes + cnt_bytes;
}

template <typename T>
static hipError_t bwd_dispatch(const BwdArgs& a) {
  switch (a.hd) {
    case 16: return launch_bwd_t<T, 16>(a);
    case 32: return launch_bwd_t<T, 32>(a);
    case 64: return launch_bwd_t<T, 64>(a);
    case 128: return launch_bwd_t<T, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a) {
  return a.bf16 ? bwd_dispatch<bf16>(a) : bwd_dispatch<float>(a);
}

}  // namespace xfa
