// Streaming of 32-row blocks of [S][HD] tensors from HBM into LDS, shared by
// the forward and both backward kernels: the LDS layout of a block, its
// operand reads, the DMA that fills it, and the parity runner of the
// hand-unrolled loops.
#pragma once

#include <type_traits>

#include "xfa_common.h"

namespace xfa {

// Geometry of a streamed block of NB = 32 rows of a [S][HD] tensor and of its
// LDS image.  The image holds block row r in the P consecutive 16-byte slots
// starting at slot phys(r) * P: its CPR data slots first, then zeros.
//   fp32: P = HDP / 4 + 1 (one slot of padding), phys(r) = r: a row stride of
//         4 (mod 64) dwords, which the fp32 reads take without bank conflicts.
//   bf16: P = HDP / 8 + 1 (odd), and phys swaps the two low 2-bit fields of
//         the row index (r = 16a + 4b + c sits at 16a + 4c + b; the map is its
//         own inverse).  A slot's group (slot mod 16, four of the 64 banks)
//         is then distinct for the first slots of any 16 consecutive rows
//         (P is odd), which the natural 16-byte reads (16 rows at one column)
//         need, and the four rows 4b..4b+3 of a transposed read sit at
//         physical rows 4c + b, whose first slots are four groups apart, so
//         the transpose reads (4 rows x 64 bytes per 32 lanes) touch every
//         bank once too.  Rows r + 8 (r mod 16 < 8) and r + 16 sit 2 and 16
//         physical rows further on, so every read address is a per-lane base
//         plus a compile-time offset.  With the one slot of padding a 32-row
//         block of 256-byte rows is 544 slots, nine 1 KiB DMA strips (a
//         layout of 20-slot rows that needed no permutation took ten).
template <typename T, int HD, int NW>
struct BlockGeo {
  using M = Mma<T>;
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int NB = 32;
  static constexpr int HDP = HD < 32 ? 32 : HD;
  static constexpr int NDB = HDP / 32;           // 32-row d blocks
  static constexpr int NC = HD / M::KD;          // instructions along d
  static constexpr int NU = 32 / M::KD;          // instructions per 32-wide k block
  static constexpr int CPR = HD * (int)sizeof(T) / 16;   // 16-byte data slots per row
  static constexpr int P = BF ? HDP / 8 + 1 : HDP / 4 + 1;   // slots per LDS row
  static constexpr int LD = P * 16 / (int)sizeof(T);   // elements per LDS row
  static constexpr uint32_t ROWB = HD * sizeof(T);     // bytes per source row
  static_assert(HD % M::KD == 0 && HD * sizeof(T) % 16 == 0, "unsupported head dim");
  static_assert(!BF || P % 2 == 1, "an odd row length spreads 16 rows over the banks");
  // physical row of block row r (and block row of physical row r)
  __host__ __device__ static constexpr int phys(int r) { return BF ? (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3) : r; }
};

// Operand reads from a block image (bf16: natural 16-byte reads and the LDS
// transpose read; fp32: one dword per lane).  off_* are this lane's byte
// offsets into an image, fixed for the kernel.
template <typename T, int HD, int NW>
struct TileRead {
  using G = BlockGeo<T, HD, NW>;
  using M = typename G::M;
  uint32_t off_nat, off_tr;
  __device__ TileRead() {
    const int l = lane(), h = l >> 5;
    if constexpr (G::BF) {
      // natural: row l % 32, elements 8 h .. 8 h + 7 of each 16-wide k step
      const int r = l & 31;
      off_nat = 16u * (uint32_t)(G::phys(r) * G::P + h);
      // transposed: rows 4 h + t / 4 (+8, +16 u), bytes 32 nb + 8 (t % 4) of a
      // 64-byte column block (t = lane % 16, nb = bit 4 of the lane)
      const int t = l & 15, nb = (l >> 4) & 1, k = 4 * h + (t >> 2);
      off_tr = 16u * (uint32_t)(G::phys(k) * G::P) + 32u * nb + 8u * (t & 3);
    } else {
      off_nat = 4u * (uint32_t)((l & 31) * G::LD + h * M::KW);
      off_tr = 4u * (uint32_t)(4 * h * G::LD + (l & 31));
    }
  }
  // A or B operand of the c-th contraction step along d, with the block's
  // rows as the operand's m (or n) index
  __device__ typename M::frag nat(const T* img, int c) const {
    const char* p = reinterpret_cast<const char*>(img) + off_nat;
    if constexpr (G::BF) return *reinterpret_cast<const bf16x8*>(p + 32 * c);
    else return *reinterpret_cast<const float*>(p + 4 * c * M::KD);
  }
  // Result-order operand of the u-th contraction step of the 32-row k block
  // (the block's rows as k), for the 32 columns starting at 32 d.
  __device__ typename M::frag tr(const T* img, int u, int d) const {
    const char* p = reinterpret_cast<const char*>(img) + off_tr;
    if constexpr (G::BF) {
      const char* p0 = p + 16 * (16 * u * G::P) + 64 * d;
      const char* p1 = p0 + 16 * (2 * G::P);   // rows + 8: two physical rows on
      const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
      const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
      const bf16x4 fa = __builtin_bit_cast(bf16x4, a);
      const bf16x4 fb = __builtin_bit_cast(bf16x4, b);
      return bf16x8{fa[0], fa[1], fa[2], fa[3], fb[0], fb[1], fb[2], fb[3]};
    } else {
      // k = 8 (u / 4) + 4 h + u % 4
      return *reinterpret_cast<const float*>(p + 4 * ((8 * (u >> 2) + (u & 3)) * G::LD + 32 * d));
    }
  }
};

typedef unsigned u32x4s __attribute__((ext_vector_type(4)));

// A raw buffer descriptor in scalar registers: 48-bit base, no stride,
// nbytes records, 32-bit raw data (same fields make_buffer_rsrc produces).
__device__ inline u32x4s make_desc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4s{(unsigned)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                (unsigned)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                (unsigned)__builtin_amdgcn_readfirstlane((int)nbytes), (unsigned)kRsrcWord3};
}
// Wait until at most N of this wave's vector memory operations are in flight.
template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N));
}
// Mark a register as (re)defined here: uses of it cannot move above this
// point, so a compiler-issued load of it has been waited for by now.
template <typename X>
__device__ inline void settle(X& x) {
  asm volatile("" : "+v"(x));
}

// Four consecutive C-tile results, scaled, to one row of an output tensor.
template <typename T>
__device__ inline void store4(rsrc_t r, uint32_t off, const f32x16& a, int g, float s) {
  bstore_row4(r, off, a[4 * g] * s, a[4 * g + 1] * s, a[4 * g + 2] * s, a[4 * g + 3] * s, T{});
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
  // iteration n on entry and of iteration `end` on exit, so the parity
  // alternates from one body to the next across consecutive runs.
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

// ------------------------------------------------ blocks copied by DMA
// Block images are filled by buffer loads that write LDS directly
// (`buffer_load_dwordx4 ... lds`): each such load moves 64 x 16 bytes from
// per-lane global offsets to 1 KiB of consecutive LDS bytes starting at M0.
// Slot s of an image takes the source chunk the layout above puts there; the
// padding slots and the rows past the tensor end read out of range, which
// writes zeros, so padding and ragged tails come out zero.  No registers
// hold staged data.  Strips (1 KiB) of a block are dealt to the waves round
// robin; every wave issues the same number of loads per block, so a wave's
// wait count is a constant.  The loads are volatile asm with a memory
// clobber, so the compiler neither drops nor moves them across other memory
// accesses; their completion is waited for with wait_vm.
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
  static constexpr int NI = (G::NB * G::P + 63) / 64;       // strips per tensor tile
  static constexpr int TILE = NI * 1024;                    // bytes of a tensor tile
  static constexpr int NS = NTEN * NI + (ROWS_F32 ? 2 : 0); // strips per block
  static constexpr int NPW = (NS + NW - 1) / NW;            // strips per wave per block
  static constexpr int BYTES = NTEN * TILE + (ROWS_F32 ? 2048 : 0);
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
        const int s = 64 * i + l, pr = s / G::P, ch = s % G::P;
        if (pr < G::NB && ch < G::CPR) r = (uint32_t)G::phys(pr) * G::ROWB + (uint32_t)ch * 16u;
      } else {
        desc[t] = (j == NTEN * NI) ? dl : dd;
        dst[t] = (uint32_t)NTEN * TILE + (uint32_t)(j - NTEN * NI) * 1024u;
        step[t] = 4u;
        if (l < G::NB / 4) r = (uint32_t)l * 16u;   // 4 fp32 rows per lane
      }
      rel[t] = r;
    }
  }
  // Issue strip t of this wave (t < NPW) of block rows [row0, row0 + NB)
  // into the image at LDS byte `base`.  A wave's issue stalls while the
  // load unit takes each strip, so kernels spread a block's strips between
  // contractions instead of issuing them back to back.
  __device__ inline void issue_one(uint32_t base, int row0, int t) const {
    // an out-of-range slot (rel = 2^31) stays at or above 2^31 without
    // wrapping: the entry points keep (S + 256) rows of fp32 below 2^31 bytes
    dma16(desc[t], rel[t] + (uint32_t)row0 * step[t], base + dst[t]);
  }
  // All of this wave's strips of the block, back to back.
  __device__ inline void issue(uint32_t base, int row0) const {
#pragma unroll
    for (int t = 0; t < NPW; ++t) issue_one(base, row0, t);
  }
};

}  // namespace xfa
