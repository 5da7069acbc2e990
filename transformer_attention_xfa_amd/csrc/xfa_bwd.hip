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
// hatches).  Here two kinds of workgroups (two launches) each own their
// outputs outright, so nothing is summed across workgroups:
//   * key workgroups, one per (head, 32*NW keys): wave w keeps dK and dV of
//     its 32 keys in registers and sweeps the 32-query blocks from the
//     diagonal on.  S = Q.K^T and dP = dO.V^T are formed with the lane owning
//     a key, so dV^T += dO^T.P and dK^T += Q^T.dS take P and dS straight from
//     registers;
//   * query workgroups, one per (head, 32*NW queries): wave w keeps dQ of its
//     32 queries in registers and sweeps the 32-key blocks up to the
//     diagonal, forming S^T and dP^T with the lane owning a query, so that
//     dQ^T += K^T.dS^T takes dS^T straight from registers.
// The query workgroups recompute S and dP (two extra contractions per pair);
// in exchange there are no atomics, no cross-workgroup ordering and no
// workspace, and dQ is bitwise reproducible.
//
// Pipeline.  The streamed 32-row blocks (Q, dO, L, D for a key workgroup;
// K, V for a query workgroup) rotate through four LDS buffers filled by DMA
// (buffer loads that write LDS, xfa_stage.h), so no registers hold staged
// data: block m+3 is fetched during iteration m into the buffer block m-1
// used, a block has more than an iteration to land, and one `s_waitcnt
// vmcnt` plus one workgroup barrier end each iteration.  A wave stalls on
// the issue of each 1 KiB strip of a fetch, so the strips go out one at a
// time between contractions, which keep the matrix core busy meanwhile.  In
// a key workgroup (one wave per SIMD), bf16 iteration n forms the two score
// contractions of block n+1 interleaved with the exponentials and dS of
// block n, then block n's u = 0 gradient contractions; its u = 1 gradient
// contractions run at the start of iteration n+1 from operands carried in
// registers across the barrier, with that iteration's fetch spread over
// them.  The score contractions of n+1 do not depend on block n's
// exponentials, so the matrix cores have work while the vector units
// evaluate them.  A query workgroup runs two waves per SIMD and interleaves
// the same way (scores of block n+1 between the exponentials and transposed
// K reads of block n, then block n's dQ contractions, with the fetch spread
// over those).
//
// The operands whose contraction index runs along block rows (dO^T and Q^T
// for the key workgroups, K^T for the query workgroups) are read from the
// row-major tiles with the LDS transpose read (ds_read_b64_tr_b16 for bf16),
// so every block is staged once, row-major.  A block is staged in units of 4
// rows x one 16-byte column chunk.  Rows past the sequence end load as zeros,
// and with zero Q / dO (or K / V) rows such pairs add nothing, so only blocks
// at the causal diagonal evaluate the mask.  The factor `scale` of ds is
// applied once, to dK and dQ when they are written.
#include <type_traits>

#include "xfa_common.h"
#include "xfa_launch.h"
#include "xfa_stage.h"

namespace xfa {

template <typename T>
struct BwdParams {
  const T* Q; const T* K; const T* V; const T* dO;
  const float* Lse; const float* Dl;
  T* dQ; T* dK; T* dV;
  int S; float scale; float c_log2; int causal;
  DropArgs drop;   // attention-probabilities dropout (used when DROP)
};

// ------------------------------------------------------------ key workgroups
// One LDS buffer: the images of the Q and dO blocks and the block's L and
// D, as Dma<..., 2, true> lays them out.
template <typename T, int HD, int NW>
struct KeyBuf {
  using DM = Dma<T, HD, NW, 2, true>;
  static constexpr size_t BYTES = DM::BYTES;
  static constexpr int NBUF = 4;   // rotating buffers (a fifth, fetched earlier, measured slower)
  T* q; T* dO; float* L; float* D;
  __device__ KeyBuf(char* base) {
    q = reinterpret_cast<T*>(base);
    dO = reinterpret_cast<T*>(base + DM::TILE);
    L = reinterpret_cast<float*>(base + 2 * DM::TILE);
    D = reinterpret_cast<float*>(base + 2 * DM::TILE + 1024);
  }
};

// DROP: the forward's dropout mask M (kept probabilities times 1 / (1 - p)),
// regenerated from the seed and each element's index: dV takes P o M and
// dS = P o (M o dP - D).
template <typename T, int HD, int NW, bool DROP>
__device__ __forceinline__ void key_role(const BwdParams<T>& p, int bh, int kt, char* smem) {
  using G = BlockGeo<T, HD, NW>;
  using M = typename G::M;
  using KB = KeyBuf<T, HD, NW>;
  constexpr bool BF = G::BF;
  constexpr int NB = G::NB, NDB = G::NDB, NC = G::NC, NU = G::NU;
  constexpr uint32_t ROWB = G::ROWB;
  constexpr int BKV = NW * 32;

  const int S = p.S;
  const int tid = threadIdx.x, l = lane(), h = l >> 5, w = tid >> 6;
  const size_t hoff = (size_t)bh * S * HD;
  const uint32_t head_bytes = (uint32_t)S * ROWB;
  const rsrc_t rK = make_rsrc(p.K + hoff, head_bytes);
  const rsrc_t rV = make_rsrc(p.V + hoff, head_bytes);

  const int j0 = kt * BKV;                       // first key of the workgroup
  const int kj = j0 + 32 * w + (l & 31);         // this lane's key
  const int nb = (S + NB - 1) / NB;              // query blocks
  const int n0 = p.causal ? j0 / NB : 0;         // first block that sees a key here
  // blocks [n0, nm) cross the diagonal of this workgroup's keys
  const int nm = p.causal ? min(nb, n0 + BKV / NB) : n0;
  const int nl = nb - 1;

  constexpr int NBUF = KB::NBUF;
  auto buf = [&](int n) { return KB(smem + (size_t)((unsigned)n % NBUF) * KB::BYTES); };
  const TileRead<T, HD, NW> rd;

  // dropout: element v of block n is query n NB + 8 (v / 4) + 4 h + v % 4 and
  // this lane's key, flat index (bh S + query) S + kj; igold = index * kGolden
  const uint64_t sg = (uint64_t)S * kGolden;
  const uint64_t lane_g = ((uint64_t)bh * (uint64_t)S * (uint64_t)S + (uint64_t)kj) * kGolden;
  auto block_g = [&](int n) { return lane_g + (uint64_t)(n * NB + 4 * h) * sg; };
  // M of element v of the block with base bg (1 without dropout)
  auto mask = [&](uint64_t bg, int v) {
    if constexpr (DROP) {
      const uint64_t ig = bg + (uint64_t)(8 * (v >> 2) + (v & 3)) * sg;
      return drop_keep(p.drop.seed, ig, p.drop.thresh) ? p.drop.inv_keep : 0.f;
    } else {
      return 1.f;
    }
  };

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

  // Blocks rotate through four LDS buffers filled by DMA: block m is fetched
  // two iterations before it is first read (see the loop body).
  using DM = typename KB::DM;
  constexpr int NPW = DM::NPW;
  DM dma;
  dma.init({make_desc(p.Q + hoff, head_bytes), make_desc(p.dO + hoff, head_bytes)},
           make_desc(p.Lse + (size_t)bh * S, (uint32_t)S * 4u), make_desc(p.Dl + (size_t)bh * S, (uint32_t)S * 4u));
  const uint32_t smem0 = lds_addr(smem);
  auto fetch = [&](int n) { dma.issue(smem0 + (uint32_t)((unsigned)n % NBUF) * KB::BYTES, n * NB); };
  constexpr int AHEAD = NBUF - 3;   // blocks still in flight when a block is waited for
  // S and dP of block n: C tiles with column = this lane's key, rows = queries
  auto sdp = [&](int n, f32x16& s, f32x16& dp) {
    KB b = buf(n);
    s = zero16();
    dp = zero16();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      s = M::mma(rd.nat(b.q, c), kf[c], s);
      dp = M::mma(rd.nat(b.dO, c), vf[c], dp);
    }
  };

  // p = 2^(s c - L log2 e), dS = p (dp - D); dV^T += dO^T.P, dK^T += Q^T.dS
  // (a block's L is read as -L log2 e, see prescale)
  auto finish = [&](auto masked, int n, f32x16 s, f32x16 dp) {
    KB b = buf(n);
    const uint64_t bg = block_g(n);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 L4 = *reinterpret_cast<const f32x4*>(b.L + 8 * g + 4 * h);
      const f32x4 D4 = *reinterpret_cast<const f32x4*>(b.D + 8 * g + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * g + e;
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], p.c_log2, L4[e]));
        const float m = mask(bg, v);
        s[v] = pr * m;
        dp[v] = pr * (dp[v] * m - D4[e]);
      }
    }
    if constexpr (decltype(masked)::value) {
      // query q sees key kj iff q >= kj
      const int lo = kj - (n * NB + 4 * h);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool keep = 8 * (v >> 2) + (v & 3) >= lo;
        s[v] = keep ? s[v] : 0.f;
        dp[v] = keep ? dp[v] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const typename M::frag pf = frag_from_acc(s, u, T{});
      const typename M::frag sf = frag_from_acc(dp, u, T{});
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        typename M::frag af, bf;
        af = rd.tr(b.dO, u, d);
        bf = rd.tr(b.q, u, d);
        dvacc[d] = M::mma(af, pf, dvacc[d]);
        dkacc[d] = M::mma(bf, sf, dkacc[d]);
      }
    }
  };

  // the compiler's own loads (kf, vf) land before the staging loads start
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    settle(kf[c]);
    settle(vf[c]);
  }
  // A block's L is rewritten in place as -L log2 e one iteration before its
  // exponentials (the block has landed by then and nothing else reads its L
  // in between): wave w takes rows 8w..8w+7, every lane of a group of eight
  // writing the same value.  Split in two so the read has time to land.
  const int lrow = 8 * w + (l & 7);
  auto prescale_read = [&](int n) { return buf(n).L[lrow]; };
  auto prescale_write = [&](int n, float x) { buf(n).L[lrow] = -x * kLog2e; };
  f32x16 sa, pa, sb, pb;
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) fetch(n0 + i);
  wait_vm<AHEAD * NPW>();      // blocks n0, n0+1 landed, the rest in flight
  __syncthreads();
  prescale_write(n0, prescale_read(n0));
  sdp(n0, sa, pa);
  __syncthreads();
  Pipe pipe(sa, pa, sb, pb);
  // bf16: the u = 1 gradient contractions of a block run at the start of the
  // next iteration, their operands carried in registers across the barrier,
  // so the matrix core has work while that iteration's first LDS reads land.
  // The carried operands start as zeros (contractions that add nothing).
  // Carried: the transposed dO and Q operands of u = 1 and the u = 1
  // fragments of P and dS.
  typename M::frag cta[NDB], ctb[NDB], cpf{}, csf{};
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    cta[d] = typename M::frag{};
    ctb[d] = typename M::frag{};
  }
  auto carried = [&]() {
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      dvacc[d] = M::mma(cta[d], cpf, dvacc[d]);
      dkacc[d] = M::mma(ctb[d], csf, dkacc[d]);
    }
  };
  // The same contractions with block nf's fetch spread between them: one
  // strip after each contraction, so the wave's stall on each strip's issue
  // overlaps a contraction instead of idling the matrix core.
  auto carried_fetch = [&](int nf) {
    const uint32_t fb = smem0 + (uint32_t)((unsigned)nf % NBUF) * KB::BYTES;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      __builtin_amdgcn_sched_barrier(0);
      dvacc[d] = M::mma(cta[d], cpf, dvacc[d]);
      if (2 * d < NPW) dma.issue_one(fb, nf * NB, 2 * d);
      __builtin_amdgcn_sched_barrier(0);
      dkacc[d] = M::mma(ctb[d], csf, dkacc[d]);
      if (2 * d + 1 < NPW) dma.issue_one(fb, nf * NB, 2 * d + 1);
    }
#pragma unroll
    for (int t = 2 * NDB; t < NPW; ++t) dma.issue_one(fb, nf * NB, t);
    __builtin_amdgcn_sched_barrier(0);
  };
  // bf16 iteration with the work interleaved by hand (sched_barrier fences
  // keep the order): the score contractions of block n+1 alternate with the
  // exponentials and dS of block n and the reads of block n's gradient
  // operands.  Same arithmetic as sdp() then finish().
  auto fused = [&](auto masked, auto par, int n) {
    if constexpr (BF) {
      static_assert(NU == 2, "bf16 contraction steps are 16 deep");
      const float lx = prescale_read(n + 1);
      KB bn = buf(n + 1), bc = buf(n);
      f32x16& sn = pipe.next(par).s;
      f32x16& dn = pipe.next(par).dp;
      // scores of block n (read in place) and its P and dS
      const f32x16& s = pipe.cur(par).s;
      const f32x16& dp = pipe.cur(par).dp;
      f32x16 ps, ds;
      const int lo = kj - (n * NB + 4 * h);      // masked: query row rel sees key kj iff rel >= lo
      const uint64_t bg = block_g(n);
      constexpr int NG = NU * NDB;               // gradient contraction pairs
      // LDS reads are spread over the contraction steps so that the matrix
      // core never waits behind a long queue of them: the score operands are
      // read PD steps ahead, L and D of block n one row group ahead of the
      // exponentials, and the transposed dO and Q operands of block n (the
      // gradient contractions' A operands) NGA pairs during the score steps
      // and the rest NGA pairs ahead during the gradient steps.
      constexpr int PD = 2;
      constexpr int NGA = NG / 2;
      typename M::frag qa[NC], oa[NC], ta[NDB], tb[NDB];
      f32x4 L4[4], D4[4];
      auto read_ld = [&](int g) {
        L4[g] = *reinterpret_cast<const f32x4*>(bc.L + 8 * g + 4 * h);
        D4[g] = *reinterpret_cast<const f32x4*>(bc.D + 8 * g + 4 * h);
      };
      auto read_sc = [&](int c) {
        qa[c] = rd.nat(bn.q, c);
        oa[c] = rd.nat(bn.dO, c);
      };
      // u = 0 operands into ta/tb, u = 1 operands straight into the carried set
      auto read_tr = [&](int g) {
        if (g < NDB) {
          ta[g] = rd.tr(bc.dO, 0, g);
          tb[g] = rd.tr(bc.q, 0, g);
        } else {
          cta[g - NDB] = rd.tr(bc.dO, 1, g - NDB);
          ctb[g - NDB] = rd.tr(bc.q, 1, g - NDB);
        }
      };
      // The exponentials are spread over all the contraction steps, since a
      // wave's vector instructions overlap its own matrix instructions only
      // up to a few per contraction: the elements of the u = 0 fragment
      // (0..7) during the score steps, the others during the u = 0 gradient
      // steps, so each fragment is complete when its contractions start.
      // Steps are numbered 0..NC-1 (score), NC..NC+NG-1 (gradient).
      constexpr int SPLIT = 8;
      constexpr int EA = (SPLIT + NC - 1) / NC;          // elements per score step
      constexpr int EB = (16 - SPLIT + NDB - 1) / NDB;   // elements per u = 0 gradient step
      auto fin_step = [](int v) { return v < SPLIT ? v / EA : NC + (v - SPLIT) / EB; };
      // row group g of L and D is read two steps before its first element
      // (one step ahead left the exponentials waiting on the read: +1 %)
      auto ld_step = [&](int g) { return fin_step(4 * g) - 2; };
      auto softmax = [&](int v) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], p.c_log2, L4[v >> 2][v & 3]));
        const float m = mask(bg, v);
        float pv = pr * m, dv = pr * (dp[v] * m - D4[v >> 2][v & 3]);
        if constexpr (decltype(masked)::value) {
          const bool keep = 8 * (v >> 2) + (v & 3) >= lo;
          pv = keep ? pv : 0.f;
          dv = keep ? dv : 0.f;
        }
        // pinned here: otherwise the compiler sinks the arithmetic to the
        // fragment conversion, bunching it where no contraction overlaps it
        settle(pv);
        settle(dv);
        ps[v] = pv;
        ds[v] = dv;
      };
      auto step_extras = [&](int st) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (ld_step(g) == st) read_ld(g);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (fin_step(v) == st) softmax(v);
      };
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (ld_step(g) < 0) read_ld(g);
#pragma unroll
      for (int c = 0; c < PD && c < NC; ++c) read_sc(c);
      // the first reads go out ahead of the carried contractions (block
      // n-1, u = 1), which cover their latency; block n+3 is fetched into
      // the buffer of block n-1, finished before the last barrier
      __builtin_amdgcn_sched_barrier(0);
      carried_fetch(n + NBUF - 1);
      sn = zero16();
      dn = zero16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        sn = M::mma(qa[c], kf[c], sn);
        dn = M::mma(oa[c], vf[c], dn);
        if (c + PD < NC) read_sc(c + PD);
#pragma unroll
        for (int g = c * NGA / NC; g < (c + 1) * NGA / NC; ++g) read_tr(g);
        step_extras(c);
      }
      __builtin_amdgcn_sched_barrier(0);
      prescale_write(n + 1, lx);
      const typename M::frag pf = frag_from_acc(ps, 0, T{}), sf = frag_from_acc(ds, 0, T{});
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        __builtin_amdgcn_sched_barrier(0);
        dvacc[d] = M::mma(ta[d], pf, dvacc[d]);
        dkacc[d] = M::mma(tb[d], sf, dkacc[d]);
        if (d + NGA < NG) read_tr(d + NGA);
        step_extras(NC + d);
      }
      __builtin_amdgcn_sched_barrier(0);
      cpf = frag_from_acc(ps, 1, T{});   // u = 1: carried into the next iteration
      csf = frag_from_acc(ds, 1, T{});
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<AHEAD * NPW>();    // block n+2 landed, later ones in flight
      __syncthreads();
    }
  };
  auto body = [&](auto masked, auto par, int n) {
    if constexpr (BF) {
      fused(masked, par, n);
    } else {
      prescale_write(n + 1, prescale_read(n + 1));
      fetch(n + NBUF - 1);     // into the buffer of block n-1, finished before the last barrier
      sdp(n + 1, pipe.next(par).s, pipe.next(par).dp);
      finish(masked, n, pipe.cur(par).s, pipe.cur(par).dp);
      wait_vm<AHEAD * NPW>();  // block n+2 landed, later ones in flight
      __syncthreads();
    }
  };
  // causal: the first BKV/NB blocks cross the diagonal (or all of them if
  // fewer remain); non-causal: none
  int n = n0, par = 0;
  pipe.run(body, std::true_type{}, n, min(nm, nl), par);
  pipe.run(body, std::false_type{}, n, nl, par);
  if constexpr (BF) carried();  // the last carried block
  pipe.last(finish, nl < nm, nl, par);
  wait_vm<0>();                // the fetches of blocks past the end write LDS: drain them

  // dK_j (scaled), dV_j for this lane's key: C tile column = key, rows = d
  const rsrc_t rdK = make_rsrc(p.dK + hoff, head_bytes);
  const rsrc_t rdV = make_rsrc(p.dV + hoff, head_bytes);
  const uint32_t krow = (uint32_t)kj * ROWB;   // keys past the end are dropped
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = d * 32 + 8 * g + 4 * h;
      if (G::HDP == HD || dd < HD) {
        store4<T>(rdK, krow + dd * sizeof(T), dkacc[d], g, p.scale);
        store4<T>(rdV, krow + dd * sizeof(T), dvacc[d], g, 1.f);
      }
    }
  }
}

// ---------------------------------------------------------- query workgroups
// One LDS buffer: the images of the K and V blocks, as Dma<..., 2, false>
// lays them out.
template <typename T, int HD, int NW>
struct QueryBuf {
  using DM = Dma<T, HD, NW, 2, false>;
  static constexpr size_t BYTES = DM::BYTES;
  static constexpr int NBUF = 4;   // rotating buffers (two bf16 workgroups fit per CU)
  T* k; T* v;
  __device__ QueryBuf(char* base) {
    k = reinterpret_cast<T*>(base);
    v = reinterpret_cast<T*>(base + DM::TILE);
  }
};

// DROP: dS^T = P o (M o dP - D) with the forward's regenerated mask M.
template <typename T, int HD, int NW, bool DROP>
__device__ __forceinline__ void query_role(const BwdParams<T>& p, int bh, int qq, char* smem) {
  using G = BlockGeo<T, HD, NW>;
  using M = typename G::M;
  using QB = QueryBuf<T, HD, NW>;
  constexpr bool BF = G::BF;
  constexpr int NB = G::NB, NDB = G::NDB, NC = G::NC, NU = G::NU;
  constexpr uint32_t ROWB = G::ROWB;
  constexpr int BQ = NW * 32;

  const int S = p.S;
  const int l = lane(), h = l >> 5, w = threadIdx.x >> 6;
  const size_t hoff = (size_t)bh * S * HD;
  const uint32_t head_bytes = (uint32_t)S * ROWB;
  const rsrc_t rQ = make_rsrc(p.Q + hoff, head_bytes);
  const rsrc_t rdO = make_rsrc(p.dO + hoff, head_bytes);
  const rsrc_t rL = make_rsrc(p.Lse + (size_t)bh * S, (uint32_t)S * 4u);
  const rsrc_t rD = make_rsrc(p.Dl + (size_t)bh * S, (uint32_t)S * 4u);

  const int q0 = qq * BQ;
  const int qi = q0 + 32 * w + (l & 31);         // this lane's query
  const int q_last = min(q0 + BQ, S) - 1;
  const int nb = p.causal ? q_last / NB + 1 : (S + NB - 1) / NB;   // key blocks
  // blocks [nm, nb) cross the diagonal of this workgroup's queries
  const int nm = p.causal ? q0 / NB : nb;
  const int nl = nb - 1;
  // last key block any query of this wave sees: from iteration n_wave + 1
  // on (blocks n and n+1 both past it) the wave only keeps the block ring
  // going (its strips, the wait and the barrier, as many as the other waves)
  // and leaves the other workgroup on its SIMD the cycles
  const int n_wave = p.causal ? __builtin_amdgcn_readfirstlane(min(q0 + 32 * w + 31, S - 1) / NB) : nl;

  constexpr int NBUF = QB::NBUF;
  auto buf = [&](int n) { return QB(smem + (size_t)((unsigned)n % NBUF) * QB::BYTES); };
  const TileRead<T, HD, NW> rd;

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
  float L2 = bload4(rL, (uint32_t)qi * 4u) * kLog2e;
  float Di = bload4(rD, (uint32_t)qi * 4u);
  // dropout: element v of block n is key n NB + 8 (v / 4) + 4 h + v % 4 of
  // this lane's query, flat index (bh S + qi) S + key; igold = index * kGolden
  const uint64_t lane_g = ((uint64_t)bh * (uint64_t)S + (uint64_t)qi) * (uint64_t)S * kGolden;
  auto block_g = [&](int n) { return lane_g + (uint64_t)(n * NB + 4 * h) * kGolden; };
  auto mask = [&](uint64_t bg, int v) {
    if constexpr (DROP) {
      const uint64_t ig = bg + (uint64_t)(8 * (v >> 2) + (v & 3)) * kGolden;
      return drop_keep(p.drop.seed, ig, p.drop.thresh) ? p.drop.inv_keep : 0.f;
    } else {
      return 1.f;
    }
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) dqacc[d] = zero16();

  // Blocks rotate through four LDS buffers filled by DMA: block m is fetched
  // two iterations before it is read.
  using DM = typename QB::DM;
  constexpr int NPW = DM::NPW;
  DM dma;
  const u32x4s dK = make_desc(p.K + hoff, head_bytes);
  dma.init({dK, make_desc(p.V + hoff, head_bytes)}, dK, dK);
  const uint32_t smem0 = lds_addr(smem);
  auto fetch = [&](int n) { dma.issue(smem0 + (uint32_t)((unsigned)n % NBUF) * QB::BYTES, n * NB); };
  constexpr int AHEAD = NBUF - 2;   // blocks still in flight when a block is waited for

  // S^T and dP^T of block n: C tiles with column = this lane's query, rows = keys
  auto sdp = [&](int n, f32x16& s, f32x16& dp) {
    QB b = buf(n);
    s = zero16();
    dp = zero16();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      s = M::mma(rd.nat(b.k, c), qf[c], s);
      dp = M::mma(rd.nat(b.v, c), of[c], dp);
    }
  };

  // dS^T = p (dp - D) with p = 2^(s c - L log2 e); dQ^T += K^T.dS^T
  auto finish = [&](auto masked, int n, f32x16 s, f32x16 dp) {
    QB b = buf(n);
    const uint64_t bg = block_g(n);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], p.c_log2, -L2));
      dp[v] = pr * (dp[v] * mask(bg, v) - Di);
    }
    if constexpr (decltype(masked)::value) {
      // key j is seen by query qi iff j <= qi
      const int rel = qi - (n * NB + 4 * h);
#pragma unroll
      for (int v = 0; v < 16; ++v) dp[v] = (8 * (v >> 2) + (v & 3) > rel) ? 0.f : dp[v];
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const typename M::frag sf = frag_from_acc(dp, u, T{});
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        typename M::frag af;
        af = rd.tr(b.k, u, d);
        dqacc[d] = M::mma(af, sf, dqacc[d]);
      }
    }
  };

  // the compiler's own loads (qf, of, L, D) land before the DMA starts
  settle(L2);
  settle(Di);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    settle(qf[c]);
    settle(of[c]);
  }
  // causal: blocks [0, nm) are unmasked and the rest cross the diagonal;
  // non-causal: all are unmasked
  int n = 0, par = 0;
  if constexpr (BF) {
    // As in the key workgroups: iteration n forms S^T and dP^T of block n+1
    // while it finishes block n, with the LDS reads spread over the
    // contraction steps (K and V rows of block n+1 PD steps ahead, the
    // transposed K operands of block n NGA pairs during the score steps and
    // the rest NGA ahead during the gradient steps).
    constexpr int EPC = (16 + NC - 1) / NC;  // score elements finished per contraction step
    constexpr int NG = NU * NDB;             // gradient contractions
    constexpr int PD = 1;
    constexpr int NGA = 2;
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) fetch(i);
    wait_vm<(NBUF - 3) * NPW>();   // blocks 0 and 1 landed, the rest in flight
    __syncthreads();
    f32x16 sa, pa, sb, pb;
    sdp(0, sa, pa);
    Pipe pipe(sa, pa, sb, pb);
    auto body = [&](auto masked, auto par, int n) {
      // block n+3 goes into the buffer of block n-1, finished before the
      // last barrier; its strips are issued between the dQ contractions
      const uint32_t fb = smem0 + (uint32_t)((unsigned)(n + NBUF - 1) % NBUF) * QB::BYTES;
      QB bn = buf(n + 1), bc = buf(n);
      f32x16& sn = pipe.next(par).s;
      f32x16& dn = pipe.next(par).dp;
      f32x16 s = pipe.cur(par).s, dp = pipe.cur(par).dp;
      const int rel = qi - (n * NB + 4 * h);   // masked: key row r is seen iff r <= rel
      const uint64_t bg = block_g(n);
      typename M::frag ka[NC], va[NC], ta[NG];
      auto read_sc = [&](int c) {
        ka[c] = rd.nat(bn.k, c);
        va[c] = rd.nat(bn.v, c);
      };
      auto read_tr = [&](int g) { ta[g] = rd.tr(bc.k, g / NDB, g % NDB); };
#pragma unroll
      for (int c = 0; c < PD && c < NC; ++c) read_sc(c);
      sn = zero16();
      dn = zero16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        sn = M::mma(ka[c], qf[c], sn);
        dn = M::mma(va[c], of[c], dn);
        if (c + PD < NC) read_sc(c + PD);
#pragma unroll
        for (int g = c * NGA / NC; g < (c + 1) * NGA / NC; ++g) read_tr(g);
#pragma unroll
        for (int v = c * EPC; v < (c + 1) * EPC && v < 16; ++v) {
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], p.c_log2, -L2));
          float ds = pr * (dp[v] * mask(bg, v) - Di);
          if constexpr (decltype(masked)::value) ds = (8 * (v >> 2) + (v & 3) > rel) ? 0.f : ds;
          dp[v] = ds;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      typename M::frag sf[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) sf[u] = frag_from_acc(dp, u, T{});
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        dqacc[g % NDB] = M::mma(ta[g], sf[g / NDB], dqacc[g % NDB]);
        if (g < NPW) dma.issue_one(fb, (n + NBUF - 1) * NB, g);
        if (g + NGA < NG) read_tr(g + NGA);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = NG; t < NPW; ++t) dma.issue_one(fb, (n + NBUF - 1) * NB, t);
      wait_vm<(NBUF - 3) * NPW>();   // block n+2 landed, later ones in flight
      __syncthreads();
    };
    Pipe::run(body, std::false_type{}, n, min(nm, nl), par);
    Pipe::run(body, std::true_type{}, n, min(nl, n_wave + 1), par);
    for (; n < nl; ++n) {
      const uint32_t fb = smem0 + (uint32_t)((unsigned)(n + NBUF - 1) % NBUF) * QB::BYTES;
#pragma unroll
      for (int t = 0; t < NPW; ++t) dma.issue_one(fb, (n + NBUF - 1) * NB, t);
      wait_vm<(NBUF - 3) * NPW>();
      __syncthreads();
    }
    if (nl <= n_wave) pipe.last(finish, nl >= nm, nl, par);
  } else {
    // fp32: one block per iteration, score and gradient contractions back
    // to back
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) fetch(i);
    wait_vm<AHEAD * NPW>();      // block 0 landed, the rest in flight
    __syncthreads();
    auto body = [&](auto masked, auto, int n) {
      fetch(n + NBUF - 1);       // into the buffer of block n-1, finished before the last barrier
      f32x16 s, dp;
      sdp(n, s, dp);
      finish(masked, n, s, dp);
      wait_vm<AHEAD * NPW>();    // block n+1 landed, later ones in flight
      __syncthreads();
    };
    Pipe::run(body, std::false_type{}, n, min(nm, nl), par);
    Pipe::run(body, std::true_type{}, n, nl, par);
    f32x16 s, dp;
    sdp(nl, s, dp);
    if (nl >= nm) finish(std::true_type{}, nl, s, dp);
    else finish(std::false_type{}, nl, s, dp);
  }
  wait_vm<0>();                // the fetches of blocks past the end write LDS: drain them

  // dQ_i (scaled): C tile column = query, rows = d
  const rsrc_t rdQ = make_rsrc(p.dQ + hoff, head_bytes);
  const uint32_t qrow = (uint32_t)qi * ROWB;   // queries past the end are dropped
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = d * 32 + 8 * g + 4 * h;
      if (G::HDP == HD || dd < HD) store4<T>(rdQ, qrow + dd * sizeof(T), dqacc[d], g, p.scale);
    }
  }
}

// ------------------------------------------------------------------ kernel
template <typename T, int HD>
struct BwdCfg {
  static constexpr int NW = 4;
  static constexpr size_t KEY_BYTES = KeyBuf<T, HD, NW>::NBUF * KeyBuf<T, HD, NW>::BYTES;
  static constexpr size_t QUERY_BYTES = QueryBuf<T, HD, NW>::NBUF * QueryBuf<T, HD, NW>::BYTES;
  static constexpr size_t SMEM = KEY_BYTES > QUERY_BYTES ? KEY_BYTES : QUERY_BYTES;
};

// Two launches on the caller's stream.  Key workgroups (heaviest first: the
// earliest keys see the most queries) need the whole register file, one wave
// per SIMD; query workgroups (heaviest first: the last queries see the most
// keys) fit two waves per SIMD for bf16.  Both dispatch heads in groups
// (head_group) with the group's tiles interleaved (group_order), a group's
// workgroups on one XCD.
template <typename T, int HD, bool DROP>
__global__ __launch_bounds__((BwdCfg<T, HD>::NW * 64), 1) void bwd_key_kernel(BwdParams<T> p, int nkt, int nwg, int BH, int hg) {
  using C = BwdCfg<T, HD>;
  __shared__ __attribute__((aligned(16))) char smem[C::KEY_BYTES];
  int bh, rank;
  group_order(xcd_logical(blockIdx.x, nwg), nkt, BH, hg, bh, rank);
  key_role<T, HD, C::NW, DROP>(p, bh, rank, smem);
}

// (with dropout the generator's 64-bit arithmetic needs more than half the
// register file: one workgroup per CU)
template <typename T, int HD, bool DROP>
__global__ __launch_bounds__((BwdCfg<T, HD>::NW * 64), (sizeof(T) == 2 && !DROP ? 2 : 1)) void bwd_query_kernel(
    BwdParams<T> p, int nqq, int nwg, int BH, int hg) {
  using C = BwdCfg<T, HD>;
  __shared__ __attribute__((aligned(16))) char smem[C::QUERY_BYTES];
  int bh, rank;
  group_order(xcd_logical(blockIdx.x, nwg), nqq, BH, hg, bh, rank);
  query_role<T, HD, C::NW, DROP>(p, bh, nqq - 1 - rank, smem);
}

template <typename T, int HD>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  using C = BwdCfg<T, HD>;
  constexpr int BKV = C::NW * 32;                // keys per key workgroup
  constexpr int BQQ = C::NW * 32;                // queries per query workgroup
  const int nkt = (int)((a.S + BKV - 1) / BKV);
  const int nqq = (int)((a.S + BQQ - 1) / BQQ);
  BwdParams<T> p{(const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout, a.lse, a.delta,
                 (T*)a.dq, (T*)a.dk, (T*)a.dv, (int)a.S, a.scale, a.scale * kLog2e, a.causal, a.drop};
  const int nk = (int)(a.BH * nkt), nq = (int)(a.BH * nqq);
  if (a.drop.thresh)
    hipLaunchKernelGGL((bwd_key_kernel<T, HD, true>), dim3(nk), dim3(C::NW * 64), 0, a.stream, p, nkt, nk, (int)a.BH, head_group(nkt));
  else
    hipLaunchKernelGGL((bwd_key_kernel<T, HD, false>), dim3(nk), dim3(C::NW * 64), 0, a.stream, p, nkt, nk, (int)a.BH, head_group(nkt));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.drop.thresh)
    hipLaunchKernelGGL((bwd_query_kernel<T, HD, true>), dim3(nq), dim3(C::NW * 64), 0, a.stream, p, nqq, nq, (int)a.BH, head_group(nqq));
  else
    hipLaunchKernelGGL((bwd_query_kernel<T, HD, false>), dim3(nq), dim3(C::NW * 64), 0, a.stream, p, nqq, nq, (int)a.BH, head_group(nqq));
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

// This file is compiled with matrix-core results in VGPRs (the build's
// per-file flags) and instantiates the bf16 kernels; xfa_bwd_f32.hip includes
// it with XFA_BWD_F32 defined and instantiates the fp32 kernels without that
// option (the fp32 hd 128 key kernel with dropout would spill under it).
#ifndef XFA_BWD_F32
hipError_t launch_bwd_f32(const BwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a) {
  return a.bf16 ? bwd_dispatch<bf16>(a) : launch_bwd_f32(a);
}
#else
hipError_t launch_bwd_f32(const BwdArgs& a) { return bwd_dispatch<float>(a); }
#endif

}  // namespace xfa
