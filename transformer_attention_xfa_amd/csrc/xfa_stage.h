// Streaming of 32-row blocks of [S][HD] tensors from HBM into LDS, shared by
// the forward and backward kernels: explicit-wait global loads, staging
// units written row-major and/or transposed, and the parity runner of the
// hand-unrolled loops.
#pragma once

#include <type_traits>

#include "xfa_common.h"

namespace xfa {

// Geometry of a streamed block of NB = 32 rows of a [S][HD] tensor.
template <typename T, int HD, int NW>
struct BlockGeo {
  using M = Mma<T>;
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int NB = 32;
  static constexpr int NT = NW * 64;
  static constexpr int HDP = HD < 32 ? 32 : HD;
  static constexpr int NDB = HDP / 32;           // 32-row d blocks
  static constexpr int NC = HD / M::KD;          // instructions along d
  static constexpr int NU = 32 / M::KD;          // instructions per 32-wide k block
  static constexpr int VE = Vec16<T>::N;
  static constexpr int CPR = HD / VE;            // 16-byte chunks per row
  static constexpr int UPT = (NB / 4) * CPR;     // 4-row x 1-chunk units per block of a tensor
  static constexpr int PFU = (2 * UPT + NT - 1) / NT;   // units per thread (two tensors)
  // row-major tiles: a row stride of 4 (mod 8) dwords reads conflict-free
  static constexpr int LD = HDP + (BF ? 8 : 4);
  static constexpr int NE = NB * LD;             // elements of a row-major block
  static constexpr int TE = BF ? HDP * NB : 0;   // elements of a transposed block
  static constexpr uint32_t ROWB = HD * sizeof(T);
  static_assert(HD % M::KD == 0 && HD % VE == 0, "unsupported head dim");
};
using TB = TTile<32>;

// Four rows x two bf16 columns of a block -> the transposed block.
__device__ inline void put_t(unsigned* t, int c, int r, const unsigned x[4]) {
  u32x2 col0, col1;
  transpose_4x2(x, col0, col1);
  const int p = swap23(r);
  const bool odd_first = (lane() >> 3) & 1;
  const int c_first = c + (odd_first ? 1 : 0);
  const int dw_half = 2 * ((p >> 2) & 1);
  *reinterpret_cast<u32x2*>(t + TB::chunk_dw(c_first, p >> 3) + dw_half) = odd_first ? col1 : col0;
  *reinterpret_cast<u32x2*>(t + TB::chunk_dw(c_first ^ 1, p >> 3) + dw_half) = odd_first ? col0 : col1;
}

// Global loads of the streamed blocks are issued through inline assembly and
// waited for explicitly: the compiler's own wait-count placement merges the
// states of the unrolled loop bodies conservatively and then waits for every
// load in flight, including the ones issued just before, which exposes the
// full load latency once per iteration.  These loads are the only vector
// memory operations inside the loops; every load the compiler issues itself
// (the per-lane K/V or Q/dO rows) has been waited for before the first of
// them (see settle()).  The compiler takes an asm load's result register as
// written when the instruction issues, so every such register is kept live
// (used by a settle() after the matching wait) until its load has landed;
// otherwise it could hand the register to another value that the late load
// data would then overwrite.
typedef unsigned u32x4s __attribute__((ext_vector_type(4)));

// A raw buffer descriptor in scalar registers: 48-bit base, no stride,
// nbytes records, 32-bit raw data (same fields make_buffer_rsrc produces).
__device__ inline u32x4s make_desc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4s{(unsigned)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                (unsigned)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                (unsigned)__builtin_amdgcn_readfirstlane((int)nbytes), (unsigned)kRsrcWord3};
}
// The loads are volatile (never removed, duplicated or moved across another
// volatile statement or memory access), so the count of loads issued after a
// set is exactly what the code says; a load's result is only read through the
// wait that covers it (wait_vm with the registers as operands).
__device__ inline u32x4 asm_load16(const u32x4s& d, uint32_t off) {
  u32x4 r;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(r) : "v"(off), "s"(d));
  return r;
}
__device__ inline float asm_load4(const u32x4s& d, uint32_t off) {
  float r;
  asm volatile("buffer_load_dword %0, %1, %2, 0 offen" : "=v"(r) : "v"(off), "s"(d));
  return r;
}
// Wait until at most N of this wave's vector memory operations are in flight.
template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N));
}
// The same wait, also marking the registers of the loads it covers as
// (re)defined by it, so that no use of them can move above it.
template <int N>
__device__ inline void wait_vm(u32x4 (&x)[1][4]) {
  asm volatile("s_waitcnt vmcnt(%4)" : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3]) : "n"(N));
}
template <int N>
__device__ inline void wait_vm(u32x4 (&x)[2][4]) {
  asm volatile("s_waitcnt vmcnt(%8)"
               : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3]), "+v"(x[1][0]), "+v"(x[1][1]),
                 "+v"(x[1][2]), "+v"(x[1][3])
               : "n"(N));
}
template <int N>
__device__ inline void wait_vm(u32x4 (&x)[1][4], float& a, float& b) {
  asm volatile("s_waitcnt vmcnt(%6)"
               : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3]), "+v"(a), "+v"(b)
               : "n"(N));
}
template <int N>
__device__ inline void wait_vm(u32x4 (&x)[2][4], float& a, float& b) {
  asm volatile("s_waitcnt vmcnt(%10)"
               : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3]), "+v"(x[1][0]), "+v"(x[1][1]),
                 "+v"(x[1][2]), "+v"(x[1][3]), "+v"(a), "+v"(b)
               : "n"(N));
}
// Mark a register as (re)defined here, after the preceding wait: uses of it
// cannot move above this point.
template <typename X>
__device__ inline void settle(X& x) {
  asm volatile("" : "+v"(x));
}

// Staging of one block of two tensors A and B ([S][HD] rows row0..row0+31) in
// 4-row x 1-chunk units, rows fastest across lanes (see chunk()).  The first
// NW/2 waves stage A and the others B, so the tensor is wave-uniform.  Every
// thread issues exactly NLOAD loads per block (threads without a unit read
// past the buffer end, which returns zeros), so all waves count the same
// loads in flight.  A (B) is written row-major when NA (NB_) is set and
// transposed when TRA (TRB) is set (bf16 only).
template <typename T, int HD, int NW, bool NA, bool NB_, bool TRA, bool TRB>
struct Stage2 {
  using G = BlockGeo<T, HD, NW>;
  static constexpr int HALF = G::NT / 2;                   // threads per tensor
  static constexpr int PFU = (G::UPT + HALF - 1) / HALF;   // units per thread
  static constexpr int NLOAD = 4 * PFU;
  u32x4 x[PFU][4];

  __device__ static inline bool wave_a() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x) < HALF; }
  __device__ static inline int unit(int i) { return (int)(threadIdx.x % HALF) + i * HALF; }
  // unit u covers rows 4 * (u % 8) .. +3 and 16-byte chunk chunk(u): the
  // chunks of eight consecutive units are rotated by two for the upper four
  // row groups, which spreads the row-major writes of a 16-lane pass over all
  // banks (row stride LD = 4 mod 16 dwords); the transposed writes stay
  // conflict-free with it
  static constexpr int J = G::CPR < 8 ? G::CPR : 8;
  __device__ static inline int chunk(int u) {
    const int j = (u >> 3) % J, hi = (u >> 3) / J;
    return (j + 2 * ((u & 7) >> 2)) % J + J * hi;
  }

  __device__ inline void load(const u32x4s& da, const u32x4s& db, int row0) {
    const u32x4s d = wave_a() ? da : db;
#pragma unroll
    for (int i = 0; i < PFU; ++i) {
      const int u = unit(i);
      const uint32_t off = (G::UPT % HALF == 0 || u < G::UPT)
                               ? (uint32_t)(row0 + 4 * (u & 7)) * G::ROWB + (uint32_t)chunk(u) * 16u
                               : 0x80000000u;
#pragma unroll
      for (int k = 0; k < 4; ++k) x[i][k] = asm_load16(d, off + k * G::ROWB);
    }
  }
  __device__ inline void settle_all() {
#pragma unroll
    for (int i = 0; i < PFU; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) settle(x[i][k]);
  }
  // Part k (0..3) of store(): row k of each unit row-major and column pair
  // k transposed, so the writes can be spread between other work.
  __device__ inline void store_part(int k, T* a, T* b, T* at, T* bt) const {
    const bool is_a = wave_a();
#pragma unroll
    for (int i = 0; i < PFU; ++i) {
      const int u = unit(i);
      if (G::UPT % HALF == 0 || u < G::UPT) {
        const int r = 4 * (u & 7), c = chunk(u) * G::VE;
        T* dst = (is_a ? a : b) + r * G::LD + c;
        if ((NA && is_a) || (NB_ && !is_a)) *reinterpret_cast<u32x4*>(dst + k * G::LD) = x[i][k];
        if constexpr ((TRA || TRB) && G::BF) {
          if ((TRA && is_a) || (TRB && !is_a)) {
            const unsigned col[4] = {x[i][0][k], x[i][1][k], x[i][2][k], x[i][3][k]};
            put_t(reinterpret_cast<unsigned*>(is_a ? at : bt), c + 2 * k, r, col);
          }
        }
      }
    }
  }
  // a, b: row-major blocks (row stride LD); at, bt: their transposed blocks
  __device__ inline void store(T* a, T* b, T* at, T* bt) const {
    const bool is_a = wave_a();
#pragma unroll
    for (int i = 0; i < PFU; ++i) {
      const int u = unit(i);
      if (G::UPT % HALF == 0 || u < G::UPT) {
        const int r = 4 * (u & 7), c = chunk(u) * G::VE;
        T* dst = (is_a ? a : b) + r * G::LD + c;
        if ((NA && is_a) || (NB_ && !is_a)) {
#pragma unroll
          for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(dst + k * G::LD) = x[i][k];
        }
        if constexpr ((TRA || TRB) && G::BF) {
          if ((TRA && is_a) || (TRB && !is_a)) {
            unsigned* t = reinterpret_cast<unsigned*>(is_a ? at : bt);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const unsigned col[4] = {x[i][0][m], x[i][1][m], x[i][2][m], x[i][3][m]};
              put_t(t, c + 2 * m, r, col);
            }
          }
        }
      }
    }
  }
};

// Four consecutive C-tile results, scaled, to one row of an output tensor.
template <typename T>
__device__ inline void store4(rsrc_t r, uint32_t off, const f32x16& a, int g, float s) {
  bstore_row4(r, off, a[4 * g] * s, a[4 * g + 1] * s, a[4 * g + 2] * s, a[4 * g + 3] * s, T{});
}

// Zero the d >= HD padding of the blocks (hd = 16 only); padded rows and
// columns feed only C-tile rows that are never stored.
template <typename T, int HD, int NW>
__device__ inline void zero_pad(T* nat, T* tr) {
  using G = BlockGeo<T, HD, NW>;
  if constexpr (G::HDP != HD) {
    for (int e = threadIdx.x; e < G::NB * (G::HDP - HD); e += G::NT) {
      const int r = e / (G::HDP - HD), c = HD + e % (G::HDP - HD);
      nat[r * G::LD + c] = (T)0.f;
    }
    if constexpr (G::BF)
      if (tr != nullptr)
        for (int e = threadIdx.x; e < (G::HDP - HD) * G::NB; e += G::NT) tr[HD * G::NB + e] = (T)0.f;
  }
}

// Two sets of score tiles alternate between "block n being finished" and
// "block n+1 being formed"; which set plays which part is the iteration's
// parity, a compile-time constant in every loop body (loops are unrolled by
// two by hand: the workgroup barrier in the body keeps the compiler from
// unrolling them itself), so no tile is ever copied.
struct Pipe {
  struct Pair { f32x16& s; f32x16& dp; };
  Pair p0, p1;
  __device__ Pipe(f32x16& s0, f32x16& d0, f32x16& s1, f32x16& d1) : p0{s0, d0}, p1{s1, d1} {}
  template <int P> __device__ Pair cur(std::integral_constant<int, P>) { return P ? p1 : p0; }
  template <int P> __device__ Pair next(std::integral_constant<int, P>) { return P ? p0 : p1; }
  // Iterations [n, end) of body(masked, parity, n); par is the parity of
  // iteration n on entry and of iteration `end` on exit.  The parity
  // alternates from one body to the next across consecutive runs, so at the
  // entry of a body of parity P the staged set P was issued one body before
  // set 1-P, which is what the body's wait count relies on.
  template <typename Body, typename Masked>
  __device__ static void run(Body& body, Masked m, int& n, int end, int& par) {
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    if (n >= end) return;
    if (par) {
      body(m, P1{}, n);
      ++n;
      par = 0;
    }
    for (; n + 1 < end; n += 2) {
      body(m, P0{}, n);
      body(m, P1{}, n + 1);
    }
    if (n < end) {
      body(m, P0{}, n);
      ++n;
      par = 1;
    }
  }
  // the final block: finish(masked, n, s, dp) without a successor
  template <typename Finish>
  __device__ void last(Finish& finish, bool masked, int n, int par) {
    if (par) {
      if (masked) finish(std::true_type{}, n, p1.s, p1.dp);
      else finish(std::false_type{}, n, p1.s, p1.dp);
    } else {
      if (masked) finish(std::true_type{}, n, p0.s, p0.dp);
      else finish(std::false_type{}, n, p0.s, p0.dp);
    }
  }
};

}  // namespace xfa

namespace xfa {

// ------------------------------------------------ blocks copied by DMA
// The LDS image of a 32-row block of a [S][HD] tensor (row stride LD
// elements) is filled by buffer loads that write LDS directly
// (`buffer_load_dwordx4 ... lds`): each such load moves 64 x 16 bytes from
// per-lane global offsets to 1 KiB of consecutive LDS bytes starting at M0.
// Slot s of the image (16 bytes at byte 16 s) holds chunk s % SPR of block
// row s / SPR; the slots of the row padding and rows past the tensor read out
// of range, which writes zeros, so padding and ragged tails come out zero.
// No registers hold staged data.  Strips (1 KiB) of a block are dealt to the
// waves round robin; every wave issues the same number of loads per block,
// so a wave's wait count is a constant.
__device__ inline void dma16(const u32x4s& d, uint32_t off, uint32_t lds_byte) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(off), "s"(d), "{m0}"(lds_byte) : "memory");
}
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)((__attribute__((address_space(3))) const char*)p);
}

// NTEN tensors of [S][HD] rows plus, when ROWS_F32, two fp32 [S] vectors (L
// and D): per block the image is NTEN tiles of NI strips, then one strip for
// each vector (its first 128 bytes).  Each wave's strips are fixed, so their
// descriptors, LDS offsets and source offsets are worked out once (init) and
// a block costs NPW loads and a few scalar operations, with no branches.
template <typename T, int HD, int NW, int NTEN, bool ROWS_F32>
struct Dma {
  using G = BlockGeo<T, HD, NW>;
  static constexpr int SPR = G::LD * (int)sizeof(T) / 16;   // 16-byte slots per LDS row
  static constexpr int NI = (G::NB * SPR + 63) / 64;        // strips per tensor tile
  static constexpr int TILE = NI * 1024;                    // bytes of a tensor tile
  static constexpr int NS = NTEN * NI + (ROWS_F32 ? 2 : 0); // strips per block
  static constexpr int NPW = (NS + NW - 1) / NW;            // strips per wave per block
  static constexpr int BYTES = NTEN * TILE + (ROWS_F32 ? 2048 : 0);
  static_assert(G::LD * sizeof(T) % 16 == 0, "LDS rows must be whole slots");
  u32x4s desc[NPW];    // source tensor of each of this wave's strips
  uint32_t dst[NPW];   // its LDS byte offset in the image
  uint32_t step[NPW];  // source bytes per block row (ROWB or 4)
  uint32_t rel[NPW];   // this lane's source byte offset at block row 0

  __device__ inline void init(const u32x4s (&dt)[NTEN], const u32x4s& dl, const u32x4s& dd) {
    const int l = lane();
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
#pragma unroll
    for (int t = 0; t < NPW; ++t) {
      int j = w + NW * t;
      // a wave past the last strip loads one again: the same bytes to the
      // same place, so the duplicate is harmless and every wave counts NPW
      if (j >= NS) j -= NS;
      uint32_t r = 0x80000000u;                // out of range: writes zeros
      if (j < NTEN * NI) {
        const int ten = j / NI, i = j % NI;
        u32x4s d = dt[0];
#pragma unroll
        for (int e = 1; e < NTEN; ++e)
          if (ten == e) d = dt[e];
        desc[t] = d;
        dst[t] = (uint32_t)ten * TILE + (uint32_t)i * 1024u;
        step[t] = G::ROWB;
        const int s = 64 * i + l, row = s / SPR, ch = s % SPR;
        if (row < G::NB && ch < G::CPR) r = (uint32_t)row * G::ROWB + (uint32_t)ch * 16u;
      } else {
        desc[t] = (j == NTEN * NI) ? dl : dd;
        dst[t] = (uint32_t)NTEN * TILE + (uint32_t)(j - NTEN * NI) * 1024u;
        step[t] = 4u;
        if (l < G::NB / 4) r = (uint32_t)l * 16u;   // 4 fp32 rows per lane
      }
      rel[t] = r;
    }
  }
  // Issue this wave's strips of block rows [row0, row0 + NB) into the image
  // at LDS byte `base`.
  __device__ inline void issue(uint32_t base, int row0) const {
#pragma unroll
    for (int t = 0; t < NPW; ++t) {
      // an out-of-range slot stays out of range whatever the row offset
      const uint32_t off = (rel[t] + (uint32_t)row0 * step[t]) | (rel[t] & 0x80000000u);
      dma16(desc[t], off, base + dst[t]);
    }
  }
};

}  // namespace xfa
