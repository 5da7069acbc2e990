// Backward pass by recomputation (T14 flash-attention design doc, "What
// flash-attention is", backward part): for every unmasked (query i, key j)
//   s_ij = Q_i . K_j * scale,  p_ij = exp(s_ij - L_i),  dp_ij = dO_i . V_j,
//   ds_ij = p_ij (dp_ij - D_i) scale,
//   dQ_i += ds_ij K_j,  dK_j += ds_ij Q_i,  dV_j += p_ij dO_i,
// without any S x S buffer.
//
// Work split.  The page's kernel looped over query rows and added dK/dV into
// global memory with atomics, which it names as its bottleneck; its own
// follow-up is a key-block-owned dK/dV pass (Key Design Decisions, escape
// hatches).  Here one launch holds two kinds of workgroups, each owning its
// outputs outright, so nothing is summed across workgroups:
//   * key workgroups, one per (head, tile of 32*NW keys): wave w keeps dK and
//     dV of its 32 keys in registers and sweeps the query tiles from the
//     diagonal on.  S = Q.K^T and dP = dO.V^T are formed with the lane owning
//     a key, so dV^T += dO^T.P and dK^T += Q^T.dS take P and dS straight from
//     registers;
//   * query workgroups, one per (head, tile of 32*NW queries): wave w keeps dQ
//     of its 32 queries in registers and sweeps the key tiles up to the
//     diagonal, forming S^T and dP^T with the lane owning a query, so that
//     dQ^T += K^T.dS^T takes dS^T straight from registers.
// The query workgroups recompute S and dP (two extra contractions per pair);
// in exchange there are no atomics, no cross-workgroup ordering and no
// workspace, and dQ is bitwise reproducible.
//
// For bf16 the operands whose contraction index runs along tile rows (dO^T,
// Q^T for the key workgroups, K^T for the query workgroups) are staged into
// LDS transposed (TTile), so every operand fragment is one 16-byte read.
// The factor `scale` of ds is applied once, to dK and dQ when they are
// written.  Only tiles at the diagonal or the sequence end evaluate the mask.
#include <type_traits>

#include "xfa_common.h"
#include "xfa_launch.h"

namespace xfa {

template <typename T>
struct BwdParams {
  const T* Q; const T* K; const T* V; const T* dO;
  const float* Lse; const float* Dl;
  T* dQ; T* dK; T* dV;
  int S; float scale; float c_log2; int causal;
};

// Tile geometry shared by both workgroup kinds.
template <typename T, int HD, int NW>
struct BwdGeo {
  using M = Mma<T>;
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int NT = NW * 64;
  static constexpr int HDP = HD < 32 ? 32 : HD;
  static constexpr int NDB = HDP / 32;           // 32-row d blocks
  static constexpr int NC = HD / M::KD;          // instructions along d
  static constexpr int NU = 32 / M::KD;          // instructions per 32-wide k block
  static constexpr int VE = Vec16<T>::N;
  static constexpr int CPR = HD / VE;            // 16-byte chunks per row
  // row-major tiles: a row stride of 4 (mod 8) dwords reads conflict-free
  static constexpr int LD = HDP + (BF ? 8 : 4);
  static constexpr uint32_t ROWB = HD * sizeof(T);
  static_assert(HD % M::KD == 0 && HD % VE == 0, "unsupported head dim");
};

// Four rows x two bf16 columns of a row-major tile -> a transposed tile.
template <typename TT>
__device__ inline void put_t(unsigned* t, int c, int r, const unsigned x[4]) {
  u32x2 col0, col1;
  transpose_4x2(x, col0, col1);
  const int p = swap23(r);
  const bool odd_first = (lane() >> 3) & 1;
  const int c_first = c + (odd_first ? 1 : 0);
  const int dw_half = 2 * ((p >> 2) & 1);
  *reinterpret_cast<u32x2*>(t + TT::chunk_dw(c_first, p >> 3) + dw_half) = odd_first ? col1 : col0;
  *reinterpret_cast<u32x2*>(t + TT::chunk_dw(c_first ^ 1, p >> 3) + dw_half) = odd_first ? col0 : col1;
}

// Four consecutive C-tile results, scaled, to one row of an output tensor.
template <typename T>
__device__ inline void store4(rsrc_t r, uint32_t off, const f32x16& a, int g, float s) {
  bstore_row4(r, off, a[4 * g] * s, a[4 * g + 1] * s, a[4 * g + 2] * s, a[4 * g + 3] * s, T{});
}

// ------------------------------------------------------------ key workgroups
template <typename T, int HD, int NW, int BQ>
struct KeyTiles {
  using G = BwdGeo<T, HD, NW>;
  static constexpr int QE = BQ * G::LD;                    // elements of a row-major Q / dO tile
  static constexpr int TE = G::BF ? G::HDP * BQ : 0;       // elements of a transposed tile
  static constexpr size_t BYTES = (2 * QE + 2 * TE) * sizeof(T) + 2 * BQ * sizeof(float);
};

template <typename T, int HD, int NW, int BQ>
__device__ __forceinline__ void key_role(const BwdParams<T>& p, int bh, int kt, char* smem) {
  using G = BwdGeo<T, HD, NW>;
  using M = typename G::M;
  using KT_ = KeyTiles<T, HD, NW, BQ>;
  using TQ = TTile<BQ>;
  constexpr bool BF = G::BF;
  constexpr int NT = G::NT, HDP = G::HDP, NDB = G::NDB, NC = G::NC, NU = G::NU;
  constexpr int VE = G::VE, CPR = G::CPR, LD = G::LD;
  constexpr uint32_t ROWB = G::ROWB;
  constexpr int BKV = NW * 32;
  constexpr int NQB = BQ / 32;
  constexpr int QCH = BQ * CPR;                  // 16-byte chunks of a Q tile
  constexpr int PF = (QCH + NT - 1) / NT;
  constexpr int QUN = (BQ / 4) * (HD / 2);       // 4-row x 2-column units of a Q tile
  constexpr int PFT = BF ? (QUN + NT - 1) / NT : 1;
  static_assert(BQ <= NT, "L/D staging assumes one thread per query");

  T* Qs = reinterpret_cast<T*>(smem);
  T* dOs = Qs + KT_::QE;
  T* QT = dOs + KT_::QE;
  T* dOT = QT + KT_::TE;
  float* Ls = reinterpret_cast<float*>(dOT + KT_::TE);
  float* Ds = Ls + BQ;

  const int S = p.S;
  const int tid = threadIdx.x, l = lane(), h = l >> 5, w = tid >> 6;
  const size_t hoff = (size_t)bh * S * HD;
  const uint32_t head_bytes = (uint32_t)S * ROWB;
  const rsrc_t rQ = make_rsrc(p.Q + hoff, head_bytes);
  const rsrc_t rK = make_rsrc(p.K + hoff, head_bytes);
  const rsrc_t rV = make_rsrc(p.V + hoff, head_bytes);
  const rsrc_t rdO = make_rsrc(p.dO + hoff, head_bytes);
  const rsrc_t rL = make_rsrc(p.Lse + (size_t)bh * S, (uint32_t)S * 4u);
  const rsrc_t rD = make_rsrc(p.Dl + (size_t)bh * S, (uint32_t)S * 4u);

  const int j0 = kt * BKV;                       // first key of the workgroup
  const int jw0 = j0 + 32 * w;                   // first key of this wave
  const int kj = jw0 + (l & 31);                 // this lane's key
  const bool wave_live = jw0 < S;
  const int nqt = (S + BQ - 1) / BQ;
  const int qt_first = p.causal ? j0 / BQ : 0;
  // queries that see this lane's key: [q_lo, q_hi)
  const int q_lo = p.causal ? kj : 0;
  const int q_hi = kj < S ? S : 0;

  if constexpr (HDP != HD) {   // padding (d >= HD) stays zero
    for (int e = tid; e < BQ * (HDP - HD); e += NT) {
      const int r = e / (HDP - HD), c = HD + e % (HDP - HD);
      Qs[r * LD + c] = (T)0.f;
      dOs[r * LD + c] = (T)0.f;
    }
    if constexpr (BF)
      for (int e = tid; e < (HDP - HD) * BQ; e += NT) QT[HD * BQ + e] = dOT[HD * BQ + e] = (T)0.f;
  }

  // this lane's key row of K and V: B operands of S = Q.K^T and dP = dO.V^T
  typename M::frag kf[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t off = (uint32_t)kj * ROWB + (c * M::KD + M::KW * h) * sizeof(T);
    if constexpr (BF) {
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

  // the next query tile in flight: row-major chunks and (bf16) 4x2 units
  typename Vec16<T>::type pq[PF], pd[PF];
  unsigned tq[PFT][4], td[PFT][4];
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
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < PFT; ++i) {
        const int e = tid + i * NT;
        const int cp = e % (HD / 2), rg = e / (HD / 2);
        const uint32_t off = (uint32_t)(q0 + 4 * rg) * ROWB + cp * 4u;
        if (QUN % NT == 0 || e < QUN) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            tq[i][k] = __float_as_uint(bload4(rQ, off + k * ROWB));
            td[i][k] = __float_as_uint(bload4(rdO, off + k * ROWB));
          }
        }
      }
    }
    if (tid < BQ) {
      pl = bload4(rL, (uint32_t)(q0 + tid) * 4u) * kLog2e;
      pdl = bload4(rD, (uint32_t)(q0 + tid) * 4u);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      if (QCH % NT == 0 || e < QCH) {
        const int r = e / CPR, c = (e - r * CPR) * VE;
        st16(Qs + r * LD + c, pq[i]);
        st16(dOs + r * LD + c, pd[i]);
      }
    }
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < PFT; ++i) {
        const int e = tid + i * NT;
        if (QUN % NT == 0 || e < QUN) {
          const int cp = e % (HD / 2), rg = e / (HD / 2);
          put_t<TQ>(reinterpret_cast<unsigned*>(QT), 2 * cp, 4 * rg, tq[i]);
          put_t<TQ>(reinterpret_cast<unsigned*>(dOT), 2 * cp, 4 * rg, td[i]);
        }
      }
    }
    if (tid < BQ) {
      Ls[tid] = pl;
      Ds[tid] = pdl;
    }
  };

  // one query tile: dV and dK updates of this wave's keys
  auto compute = [&](auto masked, int qt) {
    const int q0 = qt * BQ;
    const int q_last = min(q0 + BQ, S) - 1;
    // keys of this wave all above the diagonal of this query tile: nothing to add
    if (!wave_live || (p.causal && jw0 > q_last)) return;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      f32x16 sacc = zero16(), pacc = zero16();
      const T* qrow = Qs + (qb * 32 + (l & 31)) * LD + M::KW * h;
      const T* dorow = dOs + (qb * 32 + (l & 31)) * LD + M::KW * h;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        sacc = M::mma(ld_nat(qrow + c * M::KD), kf[c], sacc);
        pacc = M::mma(ld_nat(dorow + c * M::KD), vf[c], pacc);
      }
      // p = 2^(s c - L log2 e), dS = p (dp - D)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = qb * 32 + 8 * g + 4 * h;
        const f32x4 L4 = *reinterpret_cast<const f32x4*>(Ls + r0);
        const f32x4 D4 = *reinterpret_cast<const f32x4*>(Ds + r0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * g + e;
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], p.c_log2, -L4[e]));
          sacc[v] = pr;
          pacc[v] = pr * (pacc[v] - D4[e]);
        }
      }
      if constexpr (decltype(masked)::value) {
        // masked pairs give p = 0 and dS = 0
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
          typename M::frag af, bf;
          if constexpr (BF) {
            const int c = d * 32 + (l & 31);
            const int j = 4 * qb + 2 * u + h;
            af = *reinterpret_cast<const bf16x8*>(dOT + 2 * TQ::chunk_dw(c, j));
            bf = *reinterpret_cast<const bf16x8*>(QT + 2 * TQ::chunk_dw(c, j));
          } else {
            af = ld_res(dOs, LD, qb * 32, u, d * 32);
            bf = ld_res(Qs, LD, qb * 32, u, d * 32);
          }
          dvacc[d] = M::mma(af, pf, dvacc[d]);
          dkacc[d] = M::mma(bf, sf, dkacc[d]);
        }
      }
    }
  };

  auto step = [&](auto masked, int qt) {
    __syncthreads();          // all waves done with the previous tile
    stage();
    __syncthreads();
    if (qt + 1 < nqt) prefetch(qt + 1);
    compute(masked, qt);
  };

  // query tiles in [qt_mid0, qt_mid1) are unmasked for every key of the workgroup
  const int qt_mid0 = min(nqt, p.causal ? max(qt_first, (j0 + BKV - 1 + BQ - 1) / BQ) : qt_first);
  const int qt_mid1 = max(qt_mid0, (j0 + BKV <= S) ? S / BQ : qt_mid0);   // S / BQ <= nqt
  prefetch(qt_first);
  for (int qt = qt_first; qt < qt_mid0; ++qt) step(std::true_type{}, qt);
  for (int qt = qt_mid0; qt < qt_mid1; ++qt) step(std::false_type{}, qt);
  for (int qt = qt_mid1; qt < nqt; ++qt) step(std::true_type{}, qt);

  // dK_j (scaled), dV_j for this lane's key: C tile column = key, rows = d
  const rsrc_t rdK = make_rsrc(p.dK + hoff, head_bytes);
  const rsrc_t rdV = make_rsrc(p.dV + hoff, head_bytes);
  const uint32_t krow = (uint32_t)kj * ROWB;   // keys past the end are dropped
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = d * 32 + 8 * g + 4 * h;
      if (HDP == HD || dd < HD) {
        store4<T>(rdK, krow + dd * sizeof(T), dkacc[d], g, p.scale);
        store4<T>(rdV, krow + dd * sizeof(T), dvacc[d], g, 1.f);
      }
    }
  }
}

// ---------------------------------------------------------- query workgroups
template <typename T, int HD, int NW, int BK>
struct QueryTiles {
  using G = BwdGeo<T, HD, NW>;
  static constexpr int KE = BK * G::LD;                    // elements of a row-major K / V tile
  static constexpr int TE = G::BF ? G::HDP * BK : 0;       // elements of the transposed K tile
  static constexpr size_t BYTES = (2 * KE + TE) * sizeof(T);
};

template <typename T, int HD, int NW, int BK>
__device__ __forceinline__ void query_role(const BwdParams<T>& p, int bh, int qq, char* smem) {
  using G = BwdGeo<T, HD, NW>;
  using M = typename G::M;
  using QT_ = QueryTiles<T, HD, NW, BK>;
  using TK = TTile<BK>;
  constexpr bool BF = G::BF;
  constexpr int NT = G::NT, HDP = G::HDP, NDB = G::NDB, NC = G::NC, NU = G::NU;
  constexpr int VE = G::VE, CPR = G::CPR, LD = G::LD;
  constexpr uint32_t ROWB = G::ROWB;
  constexpr int BQ = NW * 32;
  constexpr int NKB = BK / 32;
  constexpr int KCH = BK * CPR;
  constexpr int PF = (KCH + NT - 1) / NT;
  constexpr int KUN = (BK / 4) * (HD / 2);
  constexpr int PFT = BF ? (KUN + NT - 1) / NT : 1;

  T* Ks = reinterpret_cast<T*>(smem);
  T* Vs = Ks + QT_::KE;
  T* KTs = Vs + QT_::KE;

  const int S = p.S;
  const int tid = threadIdx.x, l = lane(), h = l >> 5, w = tid >> 6;
  const size_t hoff = (size_t)bh * S * HD;
  const uint32_t head_bytes = (uint32_t)S * ROWB;
  const rsrc_t rQ = make_rsrc(p.Q + hoff, head_bytes);
  const rsrc_t rK = make_rsrc(p.K + hoff, head_bytes);
  const rsrc_t rV = make_rsrc(p.V + hoff, head_bytes);
  const rsrc_t rdO = make_rsrc(p.dO + hoff, head_bytes);
  const rsrc_t rL = make_rsrc(p.Lse + (size_t)bh * S, (uint32_t)S * 4u);
  const rsrc_t rD = make_rsrc(p.Dl + (size_t)bh * S, (uint32_t)S * 4u);

  const int q0 = qq * BQ;
  const int qw0 = q0 + 32 * w;                   // first query of this wave
  const int qi = qw0 + (l & 31);                 // this lane's query
  const int q_last = min(q0 + BQ, S) - 1;
  const int qw_last = min(qw0 + 31, S - 1);
  const bool wave_live = qw0 < S;
  const int n_tiles = p.causal ? (q_last / BK + 1) : ((S + BK - 1) / BK);
  const int key_lim = p.causal ? min(qi, S - 1) : S - 1;   // last key this query sees

  if constexpr (HDP != HD) {
    if constexpr (BF) {
      for (int e = tid; e < (HDP - HD) * BK; e += NT) KTs[HD * BK + e] = (T)0.f;
    } else {
      for (int e = tid; e < BK * (HDP - HD); e += NT) {
        const int r = e / (HDP - HD), c = HD + e % (HDP - HD);
        Ks[r * LD + c] = (T)0.f;
      }
    }
  }

  // this lane's query row of Q and dO: B operands of S^T = K.Q^T and dP^T = V.dO^T
  typename M::frag qf[NC], of[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t off = (uint32_t)qi * ROWB + (c * M::KD + M::KW * h) * sizeof(T);
    if constexpr (BF) {
      qf[c] = bload16<bf16>(rQ, off);
      of[c] = bload16<bf16>(rdO, off);
    } else {
      qf[c] = bload4(rQ, off);
      of[c] = bload4(rdO, off);
    }
  }
  const float L2 = bload4(rL, (uint32_t)qi * 4u) * kLog2e;
  const float Di = bload4(rD, (uint32_t)qi * 4u);

  f32x16 dqacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) dqacc[d] = zero16();

  typename Vec16<T>::type pk[PF], pv[PF];
  unsigned tk[PFT][4];
  auto prefetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      const int r = e / CPR, c = (e - r * CPR) * VE;
      const uint32_t off = (uint32_t)(kt * BK + r) * ROWB + c * sizeof(T);
      if (KCH % NT == 0 || e < KCH) {
        pk[i] = bload16<T>(rK, off);   // rows past the end read as zeros
        pv[i] = bload16<T>(rV, off);
      }
    }
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < PFT; ++i) {
        const int e = tid + i * NT;
        const int cp = e % (HD / 2), rg = e / (HD / 2);
        const uint32_t off = (uint32_t)(kt * BK + 4 * rg) * ROWB + cp * 4u;
        if (KUN % NT == 0 || e < KUN) {
#pragma unroll
          for (int k = 0; k < 4; ++k) tk[i][k] = __float_as_uint(bload4(rK, off + k * ROWB));
        }
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * NT;
      if (KCH % NT == 0 || e < KCH) {
        const int r = e / CPR, c = (e - r * CPR) * VE;
        st16(Ks + r * LD + c, pk[i]);
        st16(Vs + r * LD + c, pv[i]);
      }
    }
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < PFT; ++i) {
        const int e = tid + i * NT;
        if (KUN % NT == 0 || e < KUN) {
          const int cp = e % (HD / 2), rg = e / (HD / 2);
          put_t<TK>(reinterpret_cast<unsigned*>(KTs), 2 * cp, 4 * rg, tk[i]);
        }
      }
    }
  };

  // one key tile: dQ update of this wave's queries
  auto compute = [&](auto masked, int k0) {
    f32x16 sacc[NKB], pacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = zero16();
      pacc[kb] = zero16();
      const T* krow = Ks + (kb * 32 + (l & 31)) * LD + M::KW * h;
      const T* vrow = Vs + (kb * 32 + (l & 31)) * LD + M::KW * h;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        sacc[kb] = M::mma(ld_nat(krow + c * M::KD), qf[c], sacc[kb]);
        pacc[kb] = M::mma(ld_nat(vrow + c * M::KD), of[c], pacc[kb]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if constexpr (decltype(masked)::value) {
        const int rel = key_lim - (k0 + kb * 32 + 4 * h);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          sacc[kb][v] = (8 * (v >> 2) + (v & 3) > rel) ? kNegInf : sacc[kb][v];
      }
      // p = 2^(s c - L log2 e) (0 where masked), dS^T = p (dp - D)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v], p.c_log2, -L2));
        pacc[kb][v] = pr * (pacc[kb][v] - Di);
      }
    }
    // dQ^T += K^T . dS^T   (k runs over the tile's keys)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const typename M::frag sf = frag_from_acc(pacc[kb], u, T{});
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          typename M::frag af;
          if constexpr (BF)
            af = *reinterpret_cast<const bf16x8*>(KTs + 2 * TK::chunk_dw(d * 32 + (l & 31), 4 * kb + 2 * u + h));
          else
            af = ld_res(Ks, LD, kb * 32, u, d * 32);
          dqacc[d] = M::mma(af, sf, dqacc[d]);
        }
      }
    }
  };

  // tiles before n_full are unmasked for every wave of the workgroup
  const int n_full = min(p.causal ? (q0 + 1) / BK : n_tiles, S / BK);
  auto step = [&](auto masked, int kt) {
    __syncthreads();
    stage();
    __syncthreads();
    if (kt + 1 < n_tiles) prefetch(kt + 1);
    const int k0 = kt * BK;
    // the wave skips tiles wholly above its part of the diagonal
    if (wave_live && !(p.causal && k0 > qw_last)) compute(masked, k0);
  };
  prefetch(0);
  for (int kt = 0; kt < n_full; ++kt) step(std::false_type{}, kt);
  for (int kt = n_full; kt < n_tiles; ++kt) step(std::true_type{}, kt);

  // dQ_i (scaled): C tile column = query, rows = d
  const rsrc_t rdQ = make_rsrc(p.dQ + hoff, head_bytes);
  const uint32_t qrow = (uint32_t)qi * ROWB;   // queries past the end are dropped
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = d * 32 + 8 * g + 4 * h;
      if (HDP == HD || dd < HD) store4<T>(rdQ, qrow + dd * sizeof(T), dqacc[d], g, p.scale);
    }
  }
}

// ------------------------------------------------------------------ kernel
template <typename T, int HD>
struct BwdCfg {
  static constexpr int NW = 4;
  // query tile of the key workgroups (fp32 tiles at hd >= 64 are halved to fit LDS)
  static constexpr int BQ = (sizeof(T) == 4 && HD >= 64) ? 32 : 64;
  // key tile of the query workgroups
  static constexpr int BK = 64;
  static constexpr size_t SMEM = KeyTiles<T, HD, NW, BQ>::BYTES > QueryTiles<T, HD, NW, BK>::BYTES
                                     ? KeyTiles<T, HD, NW, BQ>::BYTES
                                     : QueryTiles<T, HD, NW, BK>::BYTES;
};

// Per head: nkt key workgroups (heaviest first: the earliest keys see the
// most queries), then nqq query workgroups (heaviest first: the last queries
// see the most keys).  One head's workgroups stay on one XCD.
template <typename T, int HD>
__global__ __launch_bounds__((BwdCfg<T, HD>::NW * 64), 1) void bwd_kernel(BwdParams<T> p, int nkt, int nqq,
                                                                         int nwg) {
  using C = BwdCfg<T, HD>;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  const int per_head = nkt + nqq;
  const int lid = xcd_logical(blockIdx.x, nwg);
  const int bh = lid / per_head;
  const int r = lid - bh * per_head;
  if (r < nkt) key_role<T, HD, C::NW, C::BQ>(p, bh, r, smem);
  else query_role<T, HD, C::NW, C::BK>(p, bh, nqq - 1 - (r - nkt), smem);
}

template <typename T, int HD>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  using C = BwdCfg<T, HD>;
  constexpr int BKV = C::NW * 32;                // keys per key workgroup
  constexpr int BQQ = C::NW * 32;                // queries per query workgroup
  const int nkt = (int)((a.S + BKV - 1) / BKV);
  const int nqq = (int)((a.S + BQQ - 1) / BQQ);
  const int nwg = (int)(a.BH * (nkt + nqq));
  BwdParams<T> p{(const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout, a.lse, a.delta,
                 (T*)a.dq, (T*)a.dk, (T*)a.dv, (int)a.S, a.scale, a.scale * kLog2e, a.causal};
  hipLaunchKernelGGL((bwd_kernel<T, HD>), dim3(nwg), dim3(C::NW * 64), 0, a.stream, p, nkt, nqq, nwg);
  return hipGetLastError();
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
