// kq_dev.h — device-side building blocks shared by the GEMV and expert kernels.
//
// Decode reads every weight once per token (Kinetic docs, "What makes it
// fast"), so these kernels are a codec over a weight stream: load packed
// blocks with wide loads, turn quants into fp16 in registers, and multiply
// against fp16 activations with fp32 accumulation, applying each block's fp16
// scale (and bias, affine4) once per 32 weights.
//
// Dequantization trick (exact): the fp16 bit pattern 0x6400 | u (u < 1024) is
// the number 1024 + u. v_perm_b32 builds two such halves from two bytes in
// one instruction, and v_dot2_f32_f16 multiplies a pair by two activations
// and adds into fp32 in one more. The offset is removed per block with the
// block's activation sum sx = sum_k x_k:
//   Q8_0    (bytes q ^ 0x80 = q + 128):  sum (1152 + q) x = sum q x + 1152 sx
//   Q4_0    (nibble q):                  sum (1024 + q) x = sum (q - 8) x + 1032 sx
//   affine4 (nibble q):                  sum (1024 + q) x = sum q x + 1024 sx
//   Q5_0    (nibble | fifth bit << 4):   sum (1024 + q) x = sum (q - 16) x + 1040 sx
//   Q5_1    (nibble | fifth bit << 4):   sum (1024 + q) x = sum q x + 1024 sx
// (1024 + q stays exact in fp16 for q < 1024; the fifth bit is OR-ed into bit 4
// of each half, or bit 8 where the high nibble is kept in place as 16 q.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kqd {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

enum { F_Q8_0 = 0, F_Q4_0 = 1, F_AFFINE4 = 2, F_Q5_0 = 3, F_Q5_1 = 4 };

// BB: bytes per block; UB: blocks per load unit (smallest dword-aligned group);
// UDW: dwords per unit.
template <int FMT> struct Fmt;
template <> struct Fmt<F_AFFINE4> { static constexpr int BB = 20, UB = 1, UDW = 5; };
template <> struct Fmt<F_Q4_0> { static constexpr int BB = 18, UB = 2, UDW = 9; };
template <> struct Fmt<F_Q8_0> { static constexpr int BB = 34, UB = 2, UDW = 17; };
template <> struct Fmt<F_Q5_0> { static constexpr int BB = 22, UB = 2, UDW = 11; };
template <> struct Fmt<F_Q5_1> { static constexpr int BB = 24, UB = 1, UDW = 6; };

// Per-format constants of the fix-up: the offset removed from the 1024 + q
// halves (per half of a block in the split form, where the high nibbles stand
// for 16 q and their offset is divided by 16 with them) and whether a bias
// (affine4's b, Q5_1's m) times the block's activation sum is added.
template <int FMT> struct Fix;
template <> struct Fix<F_Q8_0> { static constexpr float lo = -1152.0f, hi = -1152.0f; static constexpr bool bias = false; };
template <> struct Fix<F_Q4_0> { static constexpr float lo = -1032.0f, hi = -1152.0f; static constexpr bool bias = false; };
template <> struct Fix<F_AFFINE4> { static constexpr float lo = -1024.0f, hi = -1024.0f; static constexpr bool bias = true; };
template <> struct Fix<F_Q5_0> { static constexpr float lo = -1040.0f, hi = -1280.0f; static constexpr bool bias = false; };
template <> struct Fix<F_Q5_1> { static constexpr float lo = -1024.0f, hi = -1024.0f; static constexpr bool bias = true; };


constexpr uint32_t MAGIC = 0x64646464u;   // four 0x64 bytes: high byte of fp16 1024
constexpr uint32_t SEL_LO = 0x04010400u;  // (u0, 64, u1, 64) -> fp16 pair (1024+u0, 1024+u1)
constexpr uint32_t SEL_HI = 0x04030402u;  // (u2, 64, u3, 64)
constexpr uint32_t ONES = 0x3C003C00u;    // fp16 pair (1, 1)
constexpr int RSRC_FLAGS = 0x00020000;    // raw 32-bit buffer, range-checked

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xffffu));
}

__device__ __forceinline__ uint32_t f2h_bits(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}

// Index of this wave in its workgroup, as a wave-uniform (scalar) value so
// that addresses derived from it stay in SGPRs (buffer resources must).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// v plus the value of lane ^ 16 (permlane16 swap) or lane ^ 32 (permlane32
// swap) as one fp32 add. The swap is written out: this compiler reads the
// first result register for both results when one instruction consumes the
// two results of the swap builtin. s_nop 1 gives the swap's VGPR reads the
// wait states they need after a VALU write.
__device__ __forceinline__ float add_lane_xor16(float v) {
  uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float add_lane_xor32(float v) {
  uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over the G lanes of a group (G a power of two, groups aligned): a
// butterfly in fixed order, so it is deterministic and every lane of the group
// ends with the same value. Partners 1 and 2 apart come through DPP quad
// permutes; once each quad (each 8) holds one value, the row half-mirror
// (mirror) pairs it with the neighbouring quad (8); the gfx950 permlane swaps
// give the lane 16 and 32 apart. No step goes through LDS.
__device__ __forceinline__ float group_sum(float v, int G) {
  if (G >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  if (G >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  if (G >= 8) v += dpp_f<0x141>(v);   // row_half_mirror: the other quad of 8
  if (G >= 16) v += dpp_f<0x140>(v);  // row_mirror: the other 8 of 16
  if (G >= 32) v = add_lane_xor16(v);
  if (G >= 64) v = add_lane_xor32(v);
  return v;
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t alignbyte2(uint32_t hi, uint32_t lo) {
  return __builtin_amdgcn_alignbyte(hi, lo, 2u);
}

// Buffer resource over [base, base + bytes): loads past the end return 0
// instead of faulting.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           RSRC_FLAGS);
}

__device__ __forceinline__ u32x4 ld128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Load one unit (UB blocks, UDW dwords) at byte offset `off` (4-aligned):
// 16-byte pieces, then one 4-, 8- or 12-byte load for the rest.
template <int FMT>
__device__ __forceinline__ void load_unit(rsrc_t r, uint32_t off, uint32_t* D) {
  constexpr int NV = Fmt<FMT>::UDW / 4;  // full 16-byte pieces
  constexpr int REM = Fmt<FMT>::UDW % 4;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const u32x4 t = ld128(r, off + 16u * v);
    D[4 * v + 0] = t.x;
    D[4 * v + 1] = t.y;
    D[4 * v + 2] = t.z;
    D[4 * v + 3] = t.w;
  }
  if constexpr (REM == 1) {
    D[4 * NV] = ld32(r, off + 16u * NV);
  } else if constexpr (REM == 2) {
    const u32x2v t = __builtin_amdgcn_raw_buffer_load_b64(r, off + 16u * NV, 0, 0);
    D[4 * NV] = t.x;
    D[4 * NV + 1] = t.y;
  } else if constexpr (REM == 3) {
    const u32x3 t = __builtin_amdgcn_raw_buffer_load_b96(r, off + 16u * NV, 0, 0);
    D[4 * NV] = t.x;
    D[4 * NV + 1] = t.y;
    D[4 * NV + 2] = t.z;
  }
}

// One 5-bit block (2-byte-aligned halfwords at blk) against 32 fp16 x in fp32,
// plain dequantization: the generic kernels for rows of 2-byte-aligned blocks.
template <int FMT>
__device__ __forceinline__ float q5_block_plain(const uint16_t* blk, const uint16_t* xb, float acc) {
  constexpr int HB = FMT == F_Q5_0 ? 1 : 2;   // the fifth-bit word, in halfwords
  const float s = h2f(blk[0]);
  const float mn = FMT == F_Q5_1 ? h2f(blk[1]) : 0.0f;
  const uint32_t qh = (uint32_t)blk[HB] | ((uint32_t)blk[HB + 1] << 16);
  const uint16_t* nib = blk + HB + 2;
  for (int j = 0; j < 8; ++j) {
    const uint32_t two = nib[j];
    const int e = 2 * j;  // bytes 2j, 2j+1 hold elements 2j, 2j+16, 2j+1, 2j+17
    const int el[4] = {e, e + 16, e + 1, e + 17};
    const uint32_t q4[4] = {two & 15u, (two >> 4) & 15u, (two >> 8) & 15u, (two >> 12) & 15u};
    for (int i = 0; i < 4; ++i) {
      const int q = (int)(q4[i] | (((qh >> el[i]) & 1u) << 4));
      const float w = FMT == F_Q5_1 ? __builtin_fmaf(s, (float)q, mn) : s * (float)(q - 16);
      acc = __builtin_fmaf(w, h2f(xb[el[i]]), acc);
    }
  }
  return acc;
}

// (value, index) pairs for the argmax: the larger value wins; on equal values
// the lower index; NaN never wins. Index INT32_MAX marks "nothing yet".
struct Best {
  float v;
  int32_t i;
};

__device__ __forceinline__ Best better(Best a, Best b) {
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

// The same order as one 64-bit key, for atomic max: high word the value
// mapped to an unsigned order (NaN -> 0, below every number; -0 as +0, as
// they compare equal), low word the complement of the index (the lower index
// is the larger key). Key 0 is "nothing yet".
__device__ __forceinline__ unsigned long long best_key(float v, int32_t i) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v) == 0x80000000u ? 0u : __builtin_bit_cast(uint32_t, v);
  const uint32_t o = v != v ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
  return o == 0u ? 0ull : ((unsigned long long)o << 32) | (uint32_t)~(uint32_t)i;
}

__device__ __forceinline__ Best best_of_key(unsigned long long k) {
  if (k == 0ull) return Best{-__builtin_inff(), INT32_MAX};
  const uint32_t o = (uint32_t)(k >> 32);
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return Best{__builtin_bit_cast(float, u), (int32_t)~(uint32_t)k};
}

// Four nibble dwords of one 4-bit block -> 16 fp16 pairs (1024 + q), ordered
// to pair with activation dwords 0..15 of the block (dword i = x[2i], x[2i+1]).
// Byte t of the nibble area holds element t (low nibble) and t+16 (high).
__device__ __forceinline__ void unpack_nibbles(const uint32_t (&n)[4], uint32_t* A) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t lo = n[t] & 0x0F0F0F0Fu;          // elements 4t..4t+3
    const uint32_t hi = (n[t] >> 4) & 0x0F0F0F0Fu;   // elements 16+4t..19+4t
    A[2 * t] = perm(MAGIC, lo, SEL_LO);
    A[2 * t + 1] = perm(MAGIC, lo, SEL_HI);
    A[8 + 2 * t] = perm(MAGIC, hi, SEL_LO);
    A[9 + 2 * t] = perm(MAGIC, hi, SEL_HI);
  }
}

// The fifth bits of a 5-bit block (bit j of `qh` is bit 4 of q_j) into the
// fp16 pairs of unpack_nibbles: bit 4 of each half, so both halves of the
// block read 1024 + q. HI_SHIFT is 4 there, 8 for the high-nibble halves of
// the split form, which stand for 1024 + 16 q.
// Two bits b0, b1 (bits 0-1 of v) times 0x80010 land at bits 4 and 19 (b0)
// and 5 and 20 (b1); masking with 0x100010 keeps b0 at bit 4 and b1 at bit 20,
// the bit of 16 in each fp16 half of a pair (0x1000100 for bit 8 of each half:
// the multiplier 0x800100). Two bits per extract, multiply and and-or.
template <int SHIFT>
__device__ __forceinline__ uint32_t spread2(uint32_t qh, int pos) {
  constexpr uint32_t mul = SHIFT == 4 ? 0x80010u : 0x800100u;
  constexpr uint32_t mask = SHIFT == 4 ? 0x100010u : 0x1000100u;
  return (__builtin_amdgcn_ubfe(qh, (uint32_t)pos, 2u) * mul) & mask;
}

template <int HI_SHIFT>
__device__ __forceinline__ void add_fifth_bits(uint32_t qh, uint32_t* A) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    A[2 * t] |= spread2<4>(qh, 4 * t);                  // elements 4t, 4t+1
    A[2 * t + 1] |= spread2<4>(qh, 4 * t + 2);          // elements 4t+2, 4t+3
    A[8 + 2 * t] |= spread2<HI_SHIFT>(qh, 16 + 4 * t);  // elements 16+4t, 17+4t
    A[9 + 2 * t] |= spread2<HI_SHIFT>(qh, 18 + 4 * t);  // elements 18+4t, 19+4t
  }
}

// Eight int8 dwords of one Q8_0 block -> 16 fp16 pairs (1152 + q).
__device__ __forceinline__ void unpack_int8(const uint32_t (&q)[8], uint32_t* A) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t u = q[t] ^ 0x80808080u;
    A[2 * t] = perm(MAGIC, u, SEL_LO);
    A[2 * t + 1] = perm(MAGIC, u, SEL_HI);
  }
}

// Four nibble dwords -> 16 fp16 pairs, high nibbles shifted down (SPLIT
// false) or kept in place as 16 q (SPLIT true).
template <bool SPLIT>
__device__ __forceinline__ void unpack_nibbles_t(const uint32_t (&n)[4], uint32_t* A) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t lo = n[t] & 0x0F0F0F0Fu;
    const uint32_t hi = SPLIT ? (n[t] & 0xF0F0F0F0u) : ((n[t] >> 4) & 0x0F0F0F0Fu);
    A[2 * t] = perm(MAGIC, lo, SEL_LO);
    A[2 * t + 1] = perm(MAGIC, lo, SEL_HI);
    A[8 + 2 * t] = perm(MAGIC, hi, SEL_LO);
    A[9 + 2 * t] = perm(MAGIC, hi, SEL_HI);
  }
}

// Q5_0 unit (two 22-byte blocks, 11 dwords). Block a: d at bytes 0-1, fifth
// bits 2-5, nibbles 6-21; block b: d at 22-23, fifth bits 24-27, nibbles 28-43.
template <bool SPLIT>
__device__ __forceinline__ void q5_0_unit(const uint32_t* D, uint32_t* A, float* scale, float* bias) {
  const uint32_t na[4] = {alignbyte2(D[2], D[1]), alignbyte2(D[3], D[2]), alignbyte2(D[4], D[3]),
                          alignbyte2(D[5], D[4])};
  const uint32_t nb[4] = {D[7], D[8], D[9], D[10]};
  unpack_nibbles_t<SPLIT>(na, A);
  unpack_nibbles_t<SPLIT>(nb, A + 16);
  add_fifth_bits<SPLIT ? 8 : 4>(alignbyte2(D[1], D[0]), A);
  add_fifth_bits<SPLIT ? 8 : 4>(D[6], A + 16);
  scale[0] = h2f(D[0]);
  scale[1] = h2f(D[5] >> 16);
  bias[0] = bias[1] = 0.0f;
}

// Q5_1 unit (one 24-byte block, 6 dwords): d, m, fifth bits, nibbles.
template <bool SPLIT>
__device__ __forceinline__ void q5_1_unit(const uint32_t* D, uint32_t* A, float* scale, float* bias) {
  const uint32_t n[4] = {D[2], D[3], D[4], D[5]};
  unpack_nibbles_t<SPLIT>(n, A);
  add_fifth_bits<SPLIT ? 8 : 4>(D[1], A);
  scale[0] = h2f(D[0]);
  bias[0] = h2f(D[0] >> 16);
}

// A unit unpacked: 16 * UB fp16 pairs, and per block the fp32 factors of the
// fix-up y += c1 * (acc + c0 * sx) + c2 * sx.
template <int FMT>
struct Unpacked {
  uint32_t A[16 * Fmt<FMT>::UB];
  float scale[Fmt<FMT>::UB];
  float bias[Fmt<FMT>::UB];  // affine4 only
};

template <int FMT>
__device__ __forceinline__ void unpack_unit(const uint32_t* D, Unpacked<FMT>& u) {
  if constexpr (FMT == F_AFFINE4) {
    const uint32_t n[4] = {D[1], D[2], D[3], D[4]};
    unpack_nibbles(n, u.A);
    u.scale[0] = h2f(D[0]);
    u.bias[0] = h2f(D[0] >> 16);
  } else if constexpr (FMT == F_Q4_0) {
    // block a: d at bytes 0-1, nibbles at bytes 2-17; block b: d at 18-19, nibbles 20-35
    const uint32_t na[4] = {alignbyte2(D[1], D[0]), alignbyte2(D[2], D[1]), alignbyte2(D[3], D[2]),
                            alignbyte2(D[4], D[3])};
    const uint32_t nb[4] = {D[5], D[6], D[7], D[8]};
    unpack_nibbles(na, u.A);
    unpack_nibbles(nb, u.A + 16);
    u.scale[0] = h2f(D[0]);
    u.scale[1] = h2f(D[4] >> 16);
    u.bias[0] = u.bias[1] = 0.0f;
  } else if constexpr (FMT == F_Q5_0) {
    q5_0_unit<false>(D, u.A, u.scale, u.bias);
  } else if constexpr (FMT == F_Q5_1) {
    q5_1_unit<false>(D, u.A, u.scale, u.bias);
  } else {
    // block a: d at bytes 0-1, quants 2-33; block b: d at 34-35, quants 36-67
    uint32_t qa[8], qb[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      qa[t] = alignbyte2(D[t + 1], D[t]);
      qb[t] = D[9 + t];
    }
    unpack_int8(qa, u.A);
    unpack_int8(qb, u.A + 16);
    u.scale[0] = h2f(D[0]);
    u.scale[1] = h2f(D[8] >> 16);
    u.bias[0] = u.bias[1] = 0.0f;
  }
}

template <int FMT> struct Offset { static constexpr float v = Fix<FMT>::lo; };

// Dot of one block (16 pairs) with 16 activation dwords; add its
// dequantized contribution to y.
template <int FMT>
__device__ __forceinline__ float block_dot(const uint32_t* A, const uint32_t* X, float sx,
                                           float scale, float bias, float y) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc = dot2(A[i], X[i], acc);
  const float t = __builtin_fmaf(Offset<FMT>::v, sx, acc);   // sum of (q, q-8 or q-16) * x
  y = __builtin_fmaf(scale, t, y);
  if constexpr (Fix<FMT>::bias) y = __builtin_fmaf(bias, sx, y);
  return y;
}

// Activation sum of one block (16 dwords = 32 fp16).
__device__ __forceinline__ float block_xsum(const uint32_t* X) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s = dot2(X[i], ONES, s);
  return s;
}

// Load the activations of one unit for one column: 16 * UB dwords.
template <int FMT>
__device__ __forceinline__ void load_x_unit(const uint16_t* xcol, int unit, uint32_t* X) {
  constexpr int UK = 32 * Fmt<FMT>::UB;
  const u32x4* p = reinterpret_cast<const u32x4*>(xcol + (int64_t)unit * UK);
#pragma unroll
  for (int v = 0; v < UK / 8; ++v) {
    const u32x4 t = p[v];
    X[4 * v + 0] = t.x;
    X[4 * v + 1] = t.y;
    X[4 * v + 2] = t.z;
    X[4 * v + 3] = t.w;
  }
}

// One wave's share of a GEMV: R rows per lane, MT columns, lanes in groups of
// G = 2^log2g along K. Lane (rho = lane >> log2g, g = lane & (G-1)) handles
// tile rows rho + rpw*r (r < R, rpw = 64/G) and units g, g+G, g+2G, ...
// `rs` covers the tile's rows (rows past the matrix end read as zero).
// On return every lane of a group holds the group's full sums (butterfly
// reduction in a fixed order, so results are deterministic).
template <int FMT, int MT, int R>
__device__ __forceinline__ void valu_tile(rsrc_t rs, uint32_t row_bytes, int units, int log2g,
                                          const uint16_t* const (&xc)[MT], float (&acc)[R][MT]) {
  constexpr int UB = Fmt<FMT>::UB;
  constexpr int UBYTES = Fmt<FMT>::BB * UB;
  const int lane = threadIdx.x & 63;
  const int G = 1 << log2g;
  const int rpw = 64 >> log2g;
  const int rho = lane >> log2g;
  const int g = lane & (G - 1);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  uint32_t roff[R];
#pragma unroll
  for (int r = 0; r < R; ++r) roff[r] = (uint32_t)(rho + rpw * r) * row_bytes;

  for (int u = g; u < units; u += G) {
    uint32_t D[R][Fmt<FMT>::UDW];
#pragma unroll
    for (int r = 0; r < R; ++r) load_unit<FMT>(rs, roff[r] + (uint32_t)u * UBYTES, D[r]);
    Unpacked<FMT> up[R];
#pragma unroll
    for (int r = 0; r < R; ++r) unpack_unit<FMT>(D[r], up[r]);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      uint32_t X[16 * UB];
      load_x_unit<FMT>(xc[m], u, X);
#pragma unroll
      for (int b = 0; b < UB; ++b) {
        const float sx = block_xsum(X + 16 * b);
#pragma unroll
        for (int r = 0; r < R; ++r)
          acc[r][m] = block_dot<FMT>(up[r].A + 16 * b, X + 16 * b, sx, up[r].scale[b],
                                     up[r].bias[b], acc[r][m]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = group_sum(acc[r][m], G);
}


// ------------------------------------------------------------------------
// Latency-bound layout (used for small M): a lane issues the loads of ALL the
// units it owns before any arithmetic, so a whole tile costs one memory round
// trip, and the activations are staged once per workgroup in LDS (copied
// with LDS-DMA loads that need no registers) while those loads are in flight.

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Padded staging of activations. The lane groups of a wave read x of
// consecutive load units (UP = 4 UB pieces of 16 bytes each) at the same
// piece offset, so with the pieces back to back the lanes of one LDS read
// fall into two 16-byte bank slots (8-way conflicts on 32 banks). With one
// idle piece after every unit the unit stride is UP + 1 pieces, an odd number
// that walks every bank slot: piece P of the staged run sits at slot
// xphys(P) = P + P / UP, and a run of n16 pieces (a multiple of UP) takes
// xrun_pieces(n16) slots. Offsets within a unit stay immediate.
template <int UP>
__host__ __device__ constexpr int xphys(int P) { return UP ? P + P / UP : P; }
template <int UP>
__host__ __device__ constexpr int xrun_pieces(int n16) { return UP ? n16 + n16 / UP : n16; }

// Copy n16 16-byte pieces from global `src` (16-byte aligned) into LDS `dst`
// in the padded layout, with buffer-to-LDS loads (a wave instruction fills 64
// consecutive slots, lane L slot wave_first + L): slot s holds piece
// s - s / (UP + 1) unless it is a unit's idle slot (s % (UP + 1) == UP), which
// is not written. Every thread of the workgroup (nthreads of them) must call
// it; a later __syncthreads() waits for the copies. Buffer loads, not flat
// ones: the compiler then counts them like the other loads, and a barrier
// after later weight loads waits for the copies alone.
template <int UP>
__device__ __forceinline__ void stage_to_lds_padded(const void* src, uint32_t* dst, int n16, int nthreads) {
  const int nslot = xrun_pieces<UP>(n16);
  const rsrc_t rs = make_rsrc(src, (uint32_t)n16 * 16u);
  for (int i = threadIdx.x; i < nslot; i += nthreads) {
    const int q = i / (UP + 1), r = i - q * (UP + 1);
    if (r < UP) {
      const int wave_first = i - (int)(threadIdx.x & 63);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + 4 * wave_first), 16,
                                               (uint32_t)(q * UP + r) * 16u, 0, 0, 0);
    }
  }
}

// Offset that lies past every buffer's num_records: loads there return 0.
constexpr uint32_t OOB = 0x80000000u;

template <int FMT, int ITERS>
struct Loaded {
  uint32_t D[ITERS][Fmt<FMT>::UDW];
};

// Issue the loads of units first, first+G, ... (ITERS of them) of the row at
// byte offset `roff` of `rs`; units at or past `units` read as zero.
template <int FMT, int ITERS>
__device__ __forceinline__ void issue_units(rsrc_t rs, uint32_t roff, int first, int G, int units,
                                            Loaded<FMT, ITERS>& w) {
  constexpr uint32_t UBYTES = Fmt<FMT>::BB * Fmt<FMT>::UB;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int u = first + it * G;
    const uint32_t off = u < units ? roff + (uint32_t)u * UBYTES : OOB;
    load_unit<FMT>(rs, off, w.D[it]);
  }
}

// Four nibble dwords of one 4-bit block -> 16 fp16 pairs without shifts:
// low nibbles give 1024 + q (elements 0..15), high nibbles masked in place
// give 1024 + 16 q (elements 16..31). The 16x is removed in the fix-up.
__device__ __forceinline__ void unpack_nibbles_split(const uint32_t (&n)[4], uint32_t* A) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t lo = n[t] & 0x0F0F0F0Fu;
    const uint32_t hi = n[t] & 0xF0F0F0F0u;
    A[2 * t] = perm(MAGIC, lo, SEL_LO);
    A[2 * t + 1] = perm(MAGIC, lo, SEL_HI);
    A[8 + 2 * t] = perm(MAGIC, hi, SEL_LO);
    A[9 + 2 * t] = perm(MAGIC, hi, SEL_HI);
  }
}

template <int FMT>
__device__ __forceinline__ void unpack_unit_split(const uint32_t* D, Unpacked<FMT>& u) {
  if constexpr (FMT == F_AFFINE4) {
    const uint32_t n[4] = {D[1], D[2], D[3], D[4]};
    unpack_nibbles_split(n, u.A);
    u.scale[0] = h2f(D[0]);
    u.bias[0] = h2f(D[0] >> 16);
  } else if constexpr (FMT == F_Q4_0) {
    const uint32_t na[4] = {alignbyte2(D[1], D[0]), alignbyte2(D[2], D[1]), alignbyte2(D[3], D[2]),
                            alignbyte2(D[4], D[3])};
    const uint32_t nb[4] = {D[5], D[6], D[7], D[8]};
    unpack_nibbles_split(na, u.A);
    unpack_nibbles_split(nb, u.A + 16);
    u.scale[0] = h2f(D[0]);
    u.scale[1] = h2f(D[4] >> 16);
    u.bias[0] = u.bias[1] = 0.0f;
  } else if constexpr (FMT == F_Q5_0) {
    q5_0_unit<true>(D, u.A, u.scale, u.bias);
  } else if constexpr (FMT == F_Q5_1) {
    q5_1_unit<true>(D, u.A, u.scale, u.bias);
  } else {
    unpack_unit<FMT>(D, u);
  }
}

// One block against 16 activation dwords, with the block's activation sums
// (elements 0..15 and 16..31) precomputed. Adds the block's dequantized dot
// product to y.
template <int FMT>
__device__ __forceinline__ float block_dot_split(const uint32_t* A, const uint32_t* X, float sx_lo,
                                                 float sx_hi, float scale, float bias, float y) {
  if constexpr (FMT == F_Q8_0) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = dot2(A[i], X[i], acc);
    const float t = __builtin_fmaf(-1152.0f, sx_lo + sx_hi, acc);   // sum q x
    return __builtin_fmaf(scale, t, y);
  } else {
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) lo = dot2(A[i], X[i], lo);
#pragma unroll
    for (int i = 8; i < 16; ++i) hi = dot2(A[i], X[i], hi);
    // Q4_0: sum (q-8) x  = (lo - 1032 sx_lo) + (hi - 1152 sx_hi) / 16
    // Q5_0: sum (q-16) x = (lo - 1040 sx_lo) + (hi - 1280 sx_hi) / 16
    // affine4, Q5_1: sum q x = (lo - 1024 sx_lo) + (hi - 1024 sx_hi) / 16
    const float t_lo = __builtin_fmaf(Fix<FMT>::lo, sx_lo, lo);
    const float t_hi = __builtin_fmaf(Fix<FMT>::hi, sx_hi, hi);
    y = __builtin_fmaf(scale, t_lo, y);
    y = __builtin_fmaf(scale * 0.0625f, t_hi, y);
    if constexpr (Fix<FMT>::bias) {
      y = __builtin_fmaf(bias, sx_lo, y);
      y = __builtin_fmaf(bias, sx_hi, y);
    }
    return y;
  }
}

// Per-block activation sums for MT columns staged in LDS (column m at
// xl + m * kdw dwords, so the columns are one contiguous run): for column m
// and block b, xs[(m * nblk + b) * 2 + {0,1}] = sum of elements 0..15 / 16..31,
// i.e. xs[h] is the sum of half-block h of the run. Every thread of the
// workgroup (nthreads, as for stage_to_lds_padded) takes part; follow with
// __syncthreads().
template <int UP = 0>
__device__ __forceinline__ void block_sums_to_lds(const uint32_t* xl, int kdw, int mt, float* xs, int nthreads) {
  const int halves = mt * kdw / 8;
  for (int h = threadIdx.x; h < halves; h += nthreads) {
    const u32x4* p = reinterpret_cast<const u32x4*>(xl) + xphys<UP>(2 * h);   // both pieces in one unit
    const u32x4 a = p[0], c = p[1];
    float s = 0.0f;
    s = dot2(a.x, ONES, s);
    s = dot2(a.y, ONES, s);
    s = dot2(a.z, ONES, s);
    s = dot2(a.w, ONES, s);
    s = dot2(c.x, ONES, s);
    s = dot2(c.y, ONES, s);
    s = dot2(c.z, ONES, s);
    s = dot2(c.w, ONES, s);
    xs[h] = s;
  }
}

// Consume loaded units against MT activation columns held in LDS (column m
// at xl + m * kdw dwords, or at piece m * K / 8 of the padded layout when
// PAD) with their per-block sums in xs.
template <int FMT, int MT, int ITERS, bool PAD = false>
__device__ __forceinline__ void consume_units(const Loaded<FMT, ITERS>& w, const uint32_t* xl,
                                              const float* xs, int kdw, int first, int G, int units,
                                              float (&acc)[MT]) {
  constexpr int UB = Fmt<FMT>::UB;
  constexpr int UP = PAD ? 4 * UB : 0;
  const int nblk = kdw / 16;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int u = first + it * G;
    if (u < units) {
      Unpacked<FMT> up;
      unpack_unit_split<FMT>(w.D[it], up);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4* xp = reinterpret_cast<const u32x4*>(xl) + xphys<UP>(m * (kdw / 4) + 4 * UB * u);
        const float2* sp = reinterpret_cast<const float2*>(xs) + m * nblk + u * UB;
        uint32_t X[16 * UB];
#pragma unroll
        for (int v = 0; v < 4 * UB; ++v) {
          const u32x4 t = xp[v];
          X[4 * v] = t.x;
          X[4 * v + 1] = t.y;
          X[4 * v + 2] = t.z;
          X[4 * v + 3] = t.w;
        }
#pragma unroll
        for (int b = 0; b < UB; ++b) {
          const float2 sx = sp[b];
          acc[m] = block_dot_split<FMT>(up.A + 16 * b, X + 16 * b, sx.x, sx.y, up.scale[b],
                                        up.bias[b], acc[m]);
        }
      }
    }
  }
}

template <int MT>
__device__ __forceinline__ void group_reduce(float (&acc)[MT], int G) {
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = group_sum(acc[m], G);
}

}  // namespace kqd
