// Forward pass: online-softmax attention over KV blocks (T14 flash-attention
// design doc, section "What flash-attention is": the running-max / running-sum
// recurrence, out = acc / l and L = m + log l, the inlined causal mask and the
// skip of blocks wholly above the diagonal).
//
// Work split (differs from the page's one-block-per-query-row kernel, which
// left the GPU underfilled): one workgroup per (head, tile of 32*NW queries);
// wave w owns 32 consecutive queries.  Each wave computes the transposed
// scores S^T = K . Q^T so that every lane owns one query: the row max / row
// sum of the online softmax are then in-lane reductions plus one exchange
// between the two lane halves, and the per-query rescale factor is a per-lane
// scalar.  O^T += V^T . P^T takes P^T straight from registers as the B
// operand and V^T with the LDS transpose read from the row-major V image.
//
// 32-key blocks of K and V stream through four LDS buffers filled by DMA
// (block images and their bank-conflict-free layout: xfa_stage.h); block
// m + 3 is fetched while block m is processed, and one wait plus one barrier
// end each iteration.  bf16 iterations interleave the score contractions of
// block n+1 with the exponentials of block n and the reads of block n's V^T
// operands, then run block n's P.V contractions with the strips of block
// n+3's fetch issued between them (a wave stalls on each strip's issue, and
// a contraction in flight covers that stall).
//
// The exponent is taken in base 2: with c = scale * log2(e) and a reference
// maximum m (log2 units), p = 2^(x c - m) is one fused multiply-add and one
// exp2.  The reference only moves when a block's maximum exceeds it by more
// than 8, so most blocks skip the rescale of the accumulators (out = acc / l
// does not depend on the reference).  Only blocks that cross the diagonal or
// a ragged sequence end evaluate the mask, and the row sum l is taken over
// the bf16-rounded weights that enter P.V.
#include <type_traits>

#include "xfa_common.h"
#include "xfa_launch.h"
#include "xfa_stage.h"

namespace xfa {

// One LDS buffer: the images of a K block and a V block.
template <typename T, int HD, int NW>
struct FwdBuf {
  using DM = Dma<T, HD, NW, 2, false>;
  static constexpr size_t BYTES = DM::BYTES;
  static constexpr int NBUF = 4;   // rotating buffers (two bf16 workgroups fit per CU)
  T* k; T* v;
  __device__ FwdBuf(char* base) {
    k = reinterpret_cast<T*>(base);
    v = reinterpret_cast<T*>(base + DM::TILE);
  }
};

// DROP: attention-probabilities dropout (keep bits regenerated from the seed
// and the element index, never stored): the row sum l is taken over the
// undropped weights, and P.V uses the kept weights times 1 / (1 - p).
template <typename T, int HD, int NW, bool DROP>
__global__ __launch_bounds__(NW * 64, (sizeof(T) == 2 ? 2 : 1)) void fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, T* __restrict__ O,
    float* __restrict__ Lse, int S, float c_log2, int causal, int nqt, int nwg, int BH, int hg, DropArgs drop) {
  using G = BlockGeo<T, HD, NW>;
  using M = typename G::M;
  using FB = FwdBuf<T, HD, NW>;
  using DM = typename FB::DM;
  constexpr bool BF = G::BF;
  constexpr int NB = G::NB, NDB = G::NDB, NC = G::NC, NU = G::NU;
  constexpr int NBUF = FB::NBUF, NPW = DM::NPW;
  constexpr uint32_t ROWB = G::ROWB;
  constexpr int BQ = NW * 32;
  __shared__ __attribute__((aligned(16))) char smem[NBUF * FB::BYTES];

  const int l = lane(), h = l >> 5, w = threadIdx.x >> 6;

  // heaviest query tiles first, hg heads' tiles together per XCD
  int bh, rank;
  group_order(xcd_logical(blockIdx.x, nwg), nqt, BH, hg, bh, rank);
  const int qt = nqt - 1 - rank;

  const size_t hoff = (size_t)bh * S * HD;
  const uint32_t head_bytes = (uint32_t)S * ROWB;
  const int q0 = qt * BQ;
  const int qi = q0 + 32 * w + (l & 31);         // this lane's query
  const int q_last = min(q0 + BQ, S) - 1;        // last real query of the workgroup
  // key blocks [0, nl]; blocks [nm, nl] evaluate the mask (the causal
  // diagonal, or a ragged end of the sequence)
  const int nl = causal ? q_last / NB : (S + NB - 1) / NB - 1;
  const int nm = causal ? q0 / NB : (S % NB ? nl : nl + 1);
  const int key_lim = causal ? min(qi, S - 1) : S - 1;   // last key this lane's query sees
  // last key block any query of this wave sees: from iteration n_wave + 1
  // on (blocks n and n+1 both past it) the wave only keeps the block ring
  // going (its strips, the wait and the barrier, as many as the other waves)
  // and leaves the other workgroup on its SIMD the cycles
  const int n_wave = causal ? __builtin_amdgcn_readfirstlane(min(q0 + 32 * w + 31, S - 1) / NB) : nl;

  // Q fragments: B operand of S^T = K . Q^T (column = query, natural d order)
  const rsrc_t rQ = make_rsrc(Q + hoff, head_bytes);
  typename M::frag qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t off = (uint32_t)qi * ROWB + (c * M::KD + M::KW * h) * sizeof(T);
    if constexpr (BF) qf[c] = bload16<bf16>(rQ, off);
    else qf[c] = bload4(rQ, off);
  }
  // the compiler's own loads land before the DMA starts (wait counts)
#pragma unroll
  for (int c = 0; c < NC; ++c) settle(qf[c]);

  auto buf = [&](int n) { return FB(smem + (size_t)((unsigned)n % NBUF) * FB::BYTES); };
  const TileRead<T, HD, NW> rd;
  DM dma;
  const u32x4s dK = make_desc(K + hoff, head_bytes);
  dma.init({dK, make_desc(V + hoff, head_bytes)}, dK, dK);
  const uint32_t smem0 = lds_addr(smem);
  auto fetch = [&](int n) { dma.issue(smem0 + (uint32_t)((unsigned)n % NBUF) * FB::BYTES, n * NB); };

  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) oacc[d] = zero16();
  // The reference maximum m_ref (log2 units) only moves when some lane's
  // block maximum exceeds it by more than kRescale; until then p stays below
  // 2^kRescale and the accumulators need no rescaling.
  constexpr float kRescale = 8.f;
  float m_ref = kNegInf;
  float l_run = 0.f;       // running sum over the keys this lane half holds

  // S^T of block n: C tile with rows = keys, column = this lane's query
  auto sblock = [&](int n, f32x16& s) {
    FB b = buf(n);
    s = zero16();
#pragma unroll
    for (int c = 0; c < NC; ++c) s = M::mma(rd.nat(b.k, c), qf[c], s);
  };
  // mask (keys past the query or past the sequence end), block maximum and
  // the rescale of the running state when the reference moves
  auto prepare = [&](auto masked, int n, f32x16& s) __attribute__((always_inline)) {
    if constexpr (decltype(masked)::value) {
      const int rel = key_lim - (n * NB + 4 * h);
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = (8 * (v >> 2) + (v & 3) > rel) ? kNegInf : s[v];
    }
    float mt = s[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mt = fmaxf(mt, s[v]);
    mt = fmaxf(mt, swap_halves(mt)) * c_log2;     // block maximum, log2 units (scale > 0)
    if (__builtin_amdgcn_ballot_w64(mt > m_ref + kRescale)) {
      const float m_new = fmaxf(m_ref, mt);       // key 0 is visible to every query
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d) oacc[d] *= alpha;
    }
  };
  // the mask alone (idempotent); the pipelined bf16 body leaves the block
  // maximum out and checks the weights instead (see below)
  auto mask_only = [&](auto masked, int n, f32x16& s) {
    if constexpr (decltype(masked)::value) {
      const int rel = key_lim - (n * NB + 4 * h);
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = (8 * (v >> 2) + (v & 3) > rel) ? kNegInf : s[v];
    }
  };
  // weight of element v and its contribution to the row sum (bf16: the
  // rounded weight that enters P.V)
  auto weight = [&](const f32x16& s, int v) { return __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], c_log2, -m_ref)); };
  // dropout: element v of block n is key n NB + 8 (v / 4) + 4 h + v % 4 of
  // this lane's query, flat index (bh S + qi) S + key; igold = index * kGolden
  const uint64_t lane_g = ((uint64_t)bh * (uint64_t)S + (uint64_t)qi) * (uint64_t)S * kGolden;
  auto block_g = [&](int n) { return lane_g + (uint64_t)(n * NB + 4 * h) * kGolden; };
  // weight of element v as it enters P.V; with dropout the row sum takes the
  // undropped weight here (pfrag then skips it)
  auto dropped = [&](float pv, uint64_t bg, int v) {
    if constexpr (DROP) {
      if constexpr (BF) l_run += (float)(bf16)pv;
      else l_run += pv;
      const uint64_t ig = bg + (uint64_t)(8 * (v >> 2) + (v & 3)) * kGolden;
      pv = drop_keep(drop.seed, ig, drop.thresh) ? pv * drop.inv_keep : 0.f;
    }
    return pv;
  };
  // P^T fragment u of block n's weights; the row sum over the values it holds
  auto pfrag = [&](const f32x16& p, int u) {
    const typename M::frag pf = frag_from_acc(p, u, T{});
    if constexpr (DROP) {
      // the row sum was taken in dropped()
    } else if constexpr (BF) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 one2{(bf16)1.f, (bf16)1.f};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[2 * e], pf[2 * e + 1]}, one2, l_run, false);
    } else {
      l_run += pf;
    }
    return pf;
  };
  // bf16 P^T fragments of a block's weights and this lane's sum of them
  constexpr float kSumMax = 128.f;   // 2^7: a block sum this small bounds every weight by it
  auto block_sum = [&](const f32x16& p, typename M::frag (&pf)[NU]) {
    float lb = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      pf[u] = frag_from_acc(p, u, T{});
      if constexpr (BF) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one2{(bf16)1.f, (bf16)1.f};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          lb = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[u][2 * e], pf[u][2 * e + 1]}, one2, lb, false);
      } else {
        lb += pf[u];
      }
    }
    return lb;
  };
  // the whole of block n: weights, row sum and O^T += V^T . P^T (the fourth
  // argument, the pipeline's second tile, is unused here)
  auto finish = [&](auto masked, int n, f32x16 s, const f32x16&) __attribute__((always_inline)) {
    FB b = buf(n);
    prepare(masked, n, s);
    const uint64_t bg = block_g(n);
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = dropped(weight(s, v), bg, v);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const typename M::frag pf = pfrag(s, u);
#pragma unroll
      for (int d = 0; d < NDB; ++d) oacc[d] = M::mma(rd.tr(b.v, u, d), pf, oacc[d]);
    }
  };

  int n = 0, par = 0;
  if constexpr (BF) {
    constexpr int EPC = (16 + NC - 1) / NC;  // weights per score contraction step
    constexpr int NG = NU * NDB;             // P.V contractions
    constexpr int PD = 2;                    // K operands read PD steps ahead
    constexpr int NGA = NG / 2;              // V^T operands read during the score steps
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) fetch(i);
    wait_vm<(NBUF - 3) * NPW>();   // blocks 0 and 1 landed, the rest in flight
    __syncthreads();
    f32x16 sa, sb, pa, pb;          // score tiles of blocks n and n+1 (pa, pb unused)
    sblock(0, sa);
    // block 0 sets the reference maximum (m_ref starts at -inf)
    if (0 >= nm) prepare(std::true_type{}, 0, sa);
    else prepare(std::false_type{}, 0, sa);
    Pipe pipe(sa, pa, sb, pb);
    auto body = [&](auto masked, auto par, int n) {
      FB bn = buf(n + 1), bc = buf(n);
      f32x16& sn = pipe.next(par).s;
      f32x16 s = pipe.cur(par).s;
      typename M::frag ka[NC], va[NG], pf[NU];
      auto read_k = [&](int c) { ka[c] = rd.nat(bn.k, c); };
      auto read_v = [&](int g) { va[g] = rd.tr(bc.v, g / NDB, g % NDB); };
#pragma unroll
      for (int c = 0; c < PD && c < NC; ++c) read_k(c);
      // block n+3 goes into the buffer of block n-1, finished before the
      // last barrier; its strips are issued between the P.V contractions
      const uint32_t fb = smem0 + (uint32_t)((unsigned)(n + NBUF - 1) % NBUF) * FB::BYTES;
      if constexpr (DROP) prepare(masked, n, s);
      else mask_only(masked, n, s);
      const uint64_t bg = block_g(n);
      sn = zero16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        sn = M::mma(ka[c], qf[c], sn);
        if (c + PD < NC) read_k(c + PD);
#pragma unroll
        for (int g = c * NGA / NC; g < (c + 1) * NGA / NC; ++g) read_v(g);
#pragma unroll
        for (int v = c * EPC; v < (c + 1) * EPC && v < 16; ++v) {
          // pinned here: otherwise the compiler sinks the arithmetic to the
          // fragment conversion, where no contraction overlaps it
          float pv = dropped(weight(s, v), bg, v);
          settle(pv);
          s[v] = pv;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (DROP) {
#pragma unroll
        for (int u = 0; u < NU; ++u) pf[u] = pfrag(s, u);
      } else {
        // The weights were formed against the reference maximum without
        // the block maximum.  While each lane's block sum stays at most
        // 2^kRescale every weight does too, which is all the reference has
        // to guarantee; otherwise (the first blocks of a row, a jump of the
        // logits, an overflow) the block is redone the full way: its scores
        // again from the K tile still in LDS, mask, maximum and rescale,
        // weights.  m_ref moves exactly as with the maximum taken first.
        float lb = block_sum(s, pf);
        if (__builtin_amdgcn_ballot_w64(!(lb <= kSumMax))) {
          sblock(n, s);
          prepare(masked, n, s);
#pragma unroll
          for (int v = 0; v < 16; ++v) s[v] = weight(s, v);
          lb = block_sum(s, pf);
        }
        l_run += lb;
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        oacc[g % NDB] = M::mma(va[g], pf[g / NDB], oacc[g % NDB]);
        if (g < NPW) dma.issue_one(fb, (n + NBUF - 1) * NB, g);
        if (g + NGA < NG) read_v(g + NGA);
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
      const uint32_t fb = smem0 + (uint32_t)((unsigned)(n + NBUF - 1) % NBUF) * FB::BYTES;
#pragma unroll
      for (int t = 0; t < NPW; ++t) dma.issue_one(fb, (n + NBUF - 1) * NB, t);
      wait_vm<(NBUF - 3) * NPW>();
      __syncthreads();
    }
    if (nl <= n_wave) pipe.last(finish, nl >= nm, nl, par);
  } else {
    // fp32: one block per iteration
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) fetch(i);
    wait_vm<(NBUF - 2) * NPW>();   // block 0 landed, the rest in flight
    __syncthreads();
    auto body = [&](auto masked, auto, int n) {
      fetch(n + NBUF - 1);         // into the buffer of block n-1, finished before the last barrier
      f32x16 s;
      sblock(n, s);
      finish(masked, n, s, s);
      wait_vm<(NBUF - 2) * NPW>();   // block n+1 landed, later ones in flight
      __syncthreads();
    };
    Pipe::run(body, std::false_type{}, n, min(nm, nl), par);
    Pipe::run(body, std::true_type{}, n, nl, par);
    f32x16 s;
    sblock(nl, s);
    if (nl >= nm) finish(std::true_type{}, nl, s, s);
    else finish(std::false_type{}, nl, s, s);
  }
  wait_vm<0>();                    // the fetches of blocks past the end write LDS: drain them

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
      if (G::HDP == HD || dd < HD)
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
  constexpr int BQ = NW * 32;
  const int nqt = (int)((a.S + BQ - 1) / BQ);
  const int nwg = (int)(a.BH * nqt);
  if (a.drop.thresh)
    hipLaunchKernelGGL((fwd_kernel<T, HD, NW, true>), dim3(nwg), dim3(NW * 64), 0, a.stream,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.S,
                       a.scale * kLog2e, a.causal, nqt, nwg, (int)a.BH, head_group(nqt), a.drop);
  else
    hipLaunchKernelGGL((fwd_kernel<T, HD, NW, false>), dim3(nwg), dim3(NW * 64), 0, a.stream,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.S,
                       a.scale * kLog2e, a.causal, nqt, nwg, (int)a.BH, head_group(nqt), a.drop);
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
