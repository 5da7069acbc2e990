// Shared device-side building blocks of the xfa kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used by every kernel
// ---------------------------------------------
// All contractions run on 32x32 MFMA tiles with fp32 accumulation:
//   bf16: v_mfma_f32_32x32x16_bf16  (each lane feeds 8 k-values, depth 16)
//   fp32: v_mfma_f32_32x32x2f32     (each lane feeds 1 k-value,  depth 2)
// Operand A[m][k]: lane l supplies row m = l % 32; operand B[k][n]: lane l
// supplies column n = l % 32; the lane half h = l / 32 selects which k-values
// the lane supplies.  The result C[m][n] (16 floats per lane) has column
// n = l % 32 and, for element v, row m = 8*(v/4) + 4*h + (v%4).
//
// Because a contraction only needs A and B to agree on which k sits in which
// (half, slot), two k-orders are used:
//   * natural order: slot s of half h holds k = KW*h + s.  Used when both
//     operands are read from memory laid out [row][k] (k contiguous).
//   * result order: slot s of the u-th instruction of a 32-wide k block holds
//     k = 8*(w/4) + 4*h + (w%4) with w = KW*u + s.  This is exactly how a C
//     tile held in registers lists its rows, so a C tile can be fed straight
//     back as an operand whose k runs over those rows.  The partner operand is
//     then read from memory laid out [k][n] (n contiguous); for bf16 that is
//     the gfx950 LDS transpose read (ds_read_b64_tr_b16), which hands lane t
//     of each 16-lane group element t of the four rows addressed by the group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xfa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Counter-based dropout generator (xtrain dropout design doc, "RNG: counter
// based"): element i of the [B*H, S, S] attention probabilities is kept iff
// the top 24 bits of splitmix64(seed XOR i * kGolden) reach thresh =
// ceil(p 2^24), the same decision as u = (h >> 40) / 2^24 >= p in float32.
// splitmix64 (Steele, Lea and Flood): one generator step from state z, i.e.
// z + kGolden passed through two xorshift-multiply rounds and a xorshift.
constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;
// igold = i * kGolden (mod 2^64), formed incrementally by the callers.
// Only bits 40..63 of the hash decide, and the final xorshift by 31 leaves
// them as they are, so the last product is formed for its top 32 bits only
// (its low-half carry included; the multiplier 0x94D049BB133111EB taken in
// 32-bit halves) and compared with thresh << 8.
__device__ inline bool drop_keep(uint64_t seed, uint64_t igold, uint32_t thresh) {
  uint64_t z = (seed ^ igold) + kGolden;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  const uint32_t lo = (uint32_t)z, hi = (uint32_t)(z >> 32);
  const uint32_t top = __umulhi(lo, 0x133111EBu) + lo * 0x94D049BBu + hi * 0x133111EBu;
  return top >= (thresh << 8);
}
constexpr float kNegInf = -__builtin_huge_valf();

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <typename T> struct Mma;

template <> struct Mma<bf16> {
  using frag = bf16x8;
  static constexpr int KW = 8;   // k-values per lane per instruction
  static constexpr int KD = 16;  // contraction depth per instruction
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag zero() { return frag{}; }
};

template <> struct Mma<float> {
  using frag = float;
  static constexpr int KW = 1;
  static constexpr int KD = 2;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag zero() { return 0.f; }
};

__device__ inline int lane() { return threadIdx.x & 63; }

// ---------------------------------------------------------------- operands
// Natural-order operand: p points at X[row][k0 + KW*h] of a [row][k] layout.
__device__ inline bf16x8 ld_nat(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ inline float ld_nat(const float* p) { return *p; }

// Result-order operand from an LDS tile X[k][n] (n contiguous, row stride ld
// elements): the u-th instruction of the 32-wide k block starting at row k0,
// for the 32 columns starting at n0.
__device__ inline bf16x8 ld_res(const bf16* X, int ld, int k0, int u, int n0) {
  const int l = lane();
  const int h = l >> 5, t = l & 15, nb = (l >> 4) & 1;
  const int k = k0 + 16 * u + 4 * h + (t >> 2);
  const int n = n0 + 16 * nb + 4 * (t & 3);
  const bf16* p0 = X + k * ld + n;
  const bf16* p1 = p0 + 8 * ld;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
  bf16x4 fa = __builtin_bit_cast(bf16x4, a);
  bf16x4 fb = __builtin_bit_cast(bf16x4, b);
  return bf16x8{fa[0], fa[1], fa[2], fa[3], fb[0], fb[1], fb[2], fb[3]};
}
__device__ inline float ld_res(const float* X, int ld, int k0, int u, int n0) {
  const int l = lane();
  const int k = k0 + 8 * (u >> 2) + 4 * (l >> 5) + (u & 3);
  return X[k * ld + n0 + (l & 31)];
}

// Result-order operand taken from a C tile held in registers.
__device__ inline bf16x8 frag_from_acc(const f32x16& c, int u, bf16) {
  bf16x8 r;
#pragma unroll
  for (int s = 0; s < 8; ++s) r[s] = (bf16)c[8 * u + s];
  return r;
}
__device__ inline float frag_from_acc(const f32x16& c, int u, float) { return c[u]; }

// Value of the same element in the other lane half (lane l ^ 32).
__device__ inline float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes 0..31: r[1] holds lane l+32's x; lanes 32..63: r[0] holds lane l-32's x
  return __uint_as_float((lane() < 32) ? r[1] : r[0]);
}

__device__ inline f32x16 zero16() { return f32x16{}; }

// ------------------------------------------------------- 16-byte transfers
template <typename T> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int N = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };

template <typename T>
__device__ inline typename Vec16<T>::type ld16(const T* p) {
  return *reinterpret_cast<const typename Vec16<T>::type*>(p);
}

// ------------------------------------------------ buffer-resource access
// Global memory is addressed through buffer resources: a uniform base and
// size in scalar registers plus a 32-bit per-lane byte offset.  Loads past
// the end return zeros and stores past the end are dropped by the hardware,
// which handles ragged sequence tails without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr int kRsrcWord3 = 0x00020000;   // raw (unformatted) 32-bit data

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, kRsrcWord3);
}
template <typename T>
__device__ inline typename Vec16<T>::type bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(typename Vec16<T>::type, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline float bload4(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void bstore16(rsrc_t r, uint32_t off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0); }
__device__ inline void bstore8(rsrc_t r, uint32_t off, u32x2 v) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0); }
__device__ inline void bstore4(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// Four consecutive results of a C tile as an 8-byte (bf16) or 16-byte (fp32) store.
__device__ inline void bstore_row4(rsrc_t r, uint32_t off, float a, float b, float c, float d, bf16) {
  bf16x4 x{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  bstore8(r, off, __builtin_bit_cast(u32x2, x));
}
__device__ inline void bstore_row4(rsrc_t r, uint32_t off, float a, float b, float c, float d, float) {
  bstore16(r, off, u32x4{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)});
}

// Workgroup order for 8 XCDs: the hardware hands consecutive workgroup ids to
// the XCDs in turn.  Remap so that each XCD walks a contiguous range of the
// logical order (keeping one head's workgroups, which share K/V or Q/dO, in
// one L2), and, inside it, the order the kernel asks for.
__device__ inline int xcd_logical(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = bid & 7, slot = bid >> 3;
  return x * q + (x < r ? x : r) + slot;
}

// Logical order of the tile workgroups (forward, both backward roles): heads
// are taken in groups of G and the tiles of the group's heads interleaved,
// heaviest first (rank 0 = the tile with the most causal work); a short last
// group takes the heads that remain.  Dispatching each head's tiles heaviest
// first on its own leaves a head's light tiles finishing together and the
// next head's heavy tiles starting late (a ~10 % tail in a greedy-dispatch
// model of one XCD), while one longest-first list per group keeps the CUs
// level and still confines the streamed blocks to G heads per L2.  Measured
// on C4 (forward time; preprocess + backward time): two-head groups against
// one head at a time, forward and query kernel about 4 % each, backward 1.4 %
// more with the key kernel's tiles grouped too; four-head groups against two,
// forward 2.0 %, backward 1.0 % (query kernel) and 0.7 % (key kernel); eight
// or more heads, or three or six, made the key kernel slower.
__device__ inline void group_order(int lid, int nt, int BH, int G, int& bh, int& rank) {
  const int grp = lid / (G * nt);
  const int r = lid - grp * G * nt;
  const int nh = min(G, BH - G * grp);   // heads in this group (fewer in the last)
  bh = G * grp + r % nh;
  rank = r / nh;
}
// Heads per group for nt tiles per head: up to kGroupTiles tiles per group,
// at most four heads (C4, 32 tiles per head: four; S = 16384, 128 tiles per
// head: two, which measured 0.4-0.9 % faster than one or four there).
constexpr int kGroupTiles = 256;
inline int head_group(int64_t nt) {
  const int64_t g = kGroupTiles / (nt > 0 ? nt : 1);
  return (int)(g < 1 ? 1 : (g > 4 ? 4 : g));
}

}  // namespace xfa
