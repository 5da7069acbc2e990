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
// tile that reaches the diagonal.  Per 32-query block each wave computes
// S = Q . K^T and dP = dO . V^T with the lane owning one key, so that
// dV^T += dO^T . P and dK^T += Q^T . dS take P and dS straight from registers
// (dO^T and Q^T come from the row-major LDS tiles by the transpose read).  dS
// is then passed through LDS so that the workgroup forms dQ = dS . K for the
// tile over all of its keys, and adds it into an fp32 dQ accumulator with
// atomics (one add per element per key tile, not per key).  Query tiles are
// double-buffered in LDS: the next tile is staged while dQ is formed, so an
// iteration has two barriers.
//
// The factor `scale` of ds is applied once at the end instead of per pair:
// dK is scaled when written, and the dQ accumulator when it is converted.
// When a workgroup is done it publishes its dQ additions and counts itself in
// on every query tile it touched; the workgroup that completes a tile's count
// writes that tile of dq in the output type.  Nothing waits on another
// workgroup.
#include "xfa_common.h"
#include "xfa_launch.h"

namespace xfa {

template <typename T, int HD, int NW, int BQ>
__global__ __launch_bounds__(NW * 64, 1) void bwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ Dl,
    T* __restrict__ dQ, T* __restrict__ dK, T* __restrict__ dV, float* __restrict__ dQacc,
    unsigned* __restrict__ counters, int S, float scale, float c_log2, int causal, int nkt,
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
  constexpr uint32_t ROWB = HD * sizeof(T);
  static_assert(HD % M::KD == 0 && HD % VE == 0, "unsupported head dim");
  static_assert(BQ <= NT, "L/D staging assumes one thread per query");

  __shared__ __attribute__((aligned(16))) T Qs[2][BQ * QLD];
  __shared__ __attribute__((aligned(16))) T dOs[2][BQ * QLD];
  __shared__ __attribute__((aligned(16))) T Ks[BKV * QLD];
  __shared__ __attribute__((aligned(16))) T dSs[BKV * SLD];
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][BQ];
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
  const uint32_t head_bytes = (uint32_t)S * ROWB;
  const rsrc_t rQ = make_rsrc(Q + hoff, head_bytes);
  const rsrc_t rK = make_rsrc(K + hoff, head_bytes);
  const rsrc_t rV = make_rsrc(V + hoff, head_bytes);
  const rsrc_t rdO = make_rsrc(dO + hoff, head_bytes);
  const rsrc_t rL = make_rsrc(Lse + (size_t)bh * S, (uint32_t)S * 4u);
  const rsrc_t rD = make_rsrc(Dl + (size_t)bh * S, (uint32_t)S * 4u);
  const rsrc_t rAcc = make_rsrc(dQacc + hoff, (uint32_t)S * HD * 4u);

  const int j0 = kt * BKV;                       // first key of the workgroup
  const int jw0 = j0 + 32 * w;                   // first key of this wave
  const int kj = jw0 + (l & 31);                 // this lane's key
  const bool wave_live = jw0 < S;
  const int nqt = (S + BQ - 1) / BQ;
  const int qt_first = causal ? j0 / BQ : 0;
  // queries that see this lane's key: [q_lo, q_hi)
  const int q_lo = causal ? kj : 0;
  const int q_hi = kj < S ? S : 0;

  // zero the padding columns once; stage the workgroup's K tile (B operand of dQ)
  if constexpr (HDP != HD) {
    for (int e = tid; e < BQ * (HDP - HD); e += NT) {
      const int r = e / (HDP - HD), c = HD + e % (HDP - HD);
      Qs[0][r * QLD + c] = Qs[1][r * QLD + c] = (T)0.f;
      dOs[0][r * QLD + c] = dOs[1][r * QLD + c] = (T)0.f;
    }
    for (int e = tid; e < BKV * (HDP - HD); e += NT) {
      const int r = e / (HDP - HD), c = HD + e % (HDP - HD);
      Ks[r * QLD + c] = (T)0.f;
    }
  }
  for (int e = tid; e < BKV * CPR; e += NT) {
    const int r = e / CPR, c = (e - r * CPR) * VE;
    st16(Ks + r * QLD + c, bload16<T>(rK, (uint32_t)(j0 + r) * ROWB + c * sizeof(T)));
  }

  // this lane's key row of K and V: B operands of S = Q.K^T and dP = dO.V^T
  typename M::frag kf[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t off = (uint32_t)kj * ROWB + (c * M::KD + M::KW * h) * sizeof(T);
    if constexpr (sizeof(T) == 2) {
      kf[c] = bload16<bf16>(rK, off);
      vf[c] = bload16<bf16>(rV, off);
    } else {
      kf[c] = bload4(rK, off);
      vf[c] = bload4(rV, off);
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
      const uint32_t off = (uint32_t)(q0 + r) * ROWB + c * sizeof(T);
      if (QCH % NT == 0 || e < QCH) {
        pq[i] = bload16<T>(rQ, off);   // rows past the end read as zeros
        pd[i] = bload16<T>(rdO, off);
      }
    }
    if (tid < BQ) {
      pl = bload4(rL, (uint32_t)(q0 + tid) * 4u) * kLog2e;
      pdl = bload4(rD, (uint32_t)(q0 + tid) * 4u);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      if (QCH % NT == 0 || e < QCH) {
        const int r = e / CPR, c = (e - r * CPR) * VE;
        st16(Qs[buf] + r * QLD + c, pq[i]);
        st16(dOs[buf] + r * QLD + c, pd[i]);
      }
    }
    if (tid < BQ) {
      Ls[buf][tid] = pl;
      Ds[buf][tid] = pdl;
    }
  };

  prefetch(qt_first);
  stage(0);
  __syncthreads();
  if (qt_first + 1 < nqt) prefetch(qt_first + 1);

  T* srow = dSs + (32 * w + (l & 31)) * SLD;   // this lane's key row of the dS tile
  for (int qt = qt_first; qt < nqt; ++qt) {
    const int buf = (qt - qt_first) & 1;
    const T* Qb = Qs[buf];
    const T* dOb = dOs[buf];
    const int q0 = qt * BQ;
    const int q_last = min(q0 + BQ, S) - 1;
    // keys of this wave all above the diagonal of this query tile: nothing to add
    const bool active = wave_live && !(causal && jw0 > q_last);
    const bool need_mask = (q0 + BQ > S) || (jw0 + 32 > S) || (causal && jw0 + 31 > q0);

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      if (active) {
        f32x16 sacc = zero16(), pacc = zero16();
        const T* qrow = Qb + (qb * 32 + (l & 31)) * QLD + M::KW * h;
        const T* dorow = dOb + (qb * 32 + (l & 31)) * QLD + M::KW * h;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sacc = M::mma(ld_nat(qrow + c * M::KD), kf[c], sacc);
          pacc = M::mma(ld_nat(dorow + c * M::KD), vf[c], pacc);
        }
        // p = 2^(s c - L log2 e), dS = p (dp - D); masked pairs give p = 0
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = qb * 32 + 8 * g + 4 * h;
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(Ls[buf] + r0);
          const f32x4 D4 = *reinterpret_cast<const f32x4*>(Ds[buf] + r0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * g + e;
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], c_log2, -L4[e]));
            sacc[v] = p;
            pacc[v] = p * (pacc[v] - D4[e]);
          }
        }
        if (need_mask) {
          const int base = q0 + qb * 32 + 4 * h;
          const int lo = q_lo - base, hi = q_hi - base;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rel = 8 * (v >> 2) + (v & 3);
            const bool keep = (rel >= lo) & (rel < hi);
            sacc[v] = keep ? sacc[v] : 0.f;
            pacc[v] = keep ? pacc[v] : 0.f;
          }
        }
        // dV^T += dO^T . P,  dK^T += Q^T . dS   (k runs over the block's queries)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const typename M::frag pf = frag_from_acc(sacc, u, T{});
          const typename M::frag sf = frag_from_acc(pacc, u, T{});
#pragma unroll
          for (int d = 0; d < NDB; ++d) {
            dvacc[d] = M::mma(ld_res(dOb, QLD, qb * 32, u, d * 32), pf, dvacc[d]);
            dkacc[d] = M::mma(ld_res(Qb, QLD, qb * 32, u, d * 32), sf, dkacc[d]);
          }
        }
        // dS to LDS as [key][query]: 4 consecutive queries per store
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = qb * 32 + 8 * g + 4 * h;
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x4*>(srow + c0) =
                bf16x4{(bf16)pacc[4 * g], (bf16)pacc[4 * g + 1], (bf16)pacc[4 * g + 2], (bf16)pacc[4 * g + 3]};
          } else {
            *reinterpret_cast<f32x4*>(srow + c0) =
                f32x4{pacc[4 * g], pacc[4 * g + 1], pacc[4 * g + 2], pacc[4 * g + 3]};
          }
        }
      } else {
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
      if (NOB % NW == 0 || b < NOB) {
        const int qb = b / NDB, db = b - (b / NDB) * NDB;
        f32x16 acc = zero16();
        for (int kb = 0; kb < nkb; ++kb) {
#pragma unroll
          for (int u = 0; u < NU; ++u)
            acc = M::mma(ld_res(dSs, SLD, kb * 32, u, qb * 32), ld_res(Ks, QLD, kb * 32, u, db * 32), acc);
        }
        const int d = db * 32 + (l & 31);
        if (HDP == HD || d < HD) {
          // rows past the sequence end fall outside the buffer and are dropped
          const uint32_t off0 = ((uint32_t)(q0 + qb * 32 + 4 * h) * HD + d) * 4u;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            batomic_add(rAcc, off0 + (uint32_t)(8 * (v >> 2) + (v & 3)) * HD * 4u, acc[v]);
        }
      }
    }

    // stage the next query tile into the other buffer while others finish dQ
    if (qt + 1 < nqt) {
      stage(buf ^ 1);
      if (qt + 2 < nqt) prefetch(qt + 2);
    }
    __syncthreads();
  }

  // dK_j (scaled here), dV_j for this lane's key: C tile column = key, rows = d
  {
    const rsrc_t rdK = make_rsrc(dK + hoff, head_bytes);
    const rsrc_t rdV = make_rsrc(dV + hoff, head_bytes);
    const uint32_t krow = (uint32_t)kj * ROWB;   // keys past the end are dropped
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = d * 32 + 8 * g + 4 * h;
        if (HDP == HD || dd < HD) {
          const uint32_t off = krow + dd * sizeof(T);
          bstore_row4(rdK, off, dkacc[d][4 * g] * scale, dkacc[d][4 * g + 1] * scale,
                      dkacc[d][4 * g + 2] * scale, dkacc[d][4 * g + 3] * scale, T{});
          bstore_row4(rdV, off, dvacc[d][4 * g], dvacc[d][4 * g + 1], dvacc[d][4 * g + 2],
                      dvacc[d][4 * g + 3], T{});
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
  const rsrc_t rdQ = make_rsrc(dQ + hoff, head_bytes);
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
      const uint32_t e0 = (uint32_t)(base + t) * BQ * HD;   // first element of the tile
      const int n = min(BQ, S - (base + t) * BQ) * HD;
      for (int e = tid * 4; e < n; e += NT * 4) {
        const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rAcc, (e0 + e) * 4u, 0, 0));
        bstore_row4(rdQ, (e0 + e) * sizeof(T), x[0] * scale, x[1] * scale, x[2] * scale, x[3] * scale, T{});
      }
    }
    __syncthreads();
  }
}

template <typename T, int HD>
struct BwdCfg {
  static constexpr int NW = 4;
  // fp32 tiles at hd >= 64 would not fit the 160 KiB of LDS with 64 queries
  static constexpr int BQ = (sizeof(T) == 4 && HD >= 64) ? 32 : 64;
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
  switch (hd) {
    case 16: return BwdCfg<float, 16>::BQ;
    case 32: return BwdCfg<float, 32>::BQ;
    case 64: return BwdCfg<float, 64>::BQ;
  }
  return BwdCfg<float, 128>::BQ;
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
