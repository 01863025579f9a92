// kq_mfma.hip — block-quantized GEMV for several activation columns on the
// matrix cores of gfx950 (v_mfma_f32_16x16x32_f16).
//
// A speculative-decoding verify pass checks several guessed tokens in one
// pass over the weights, and several requests can share a pass (Kinetic docs,
// "What makes it fast"; Kapitsa README, "How it works": a verify pass of 8
// rows; "What's new": three requests sharing one pass). With M >= 2 columns
// the per-weight multiply work grows with M while the bytes do not, so the
// products go to the MFMA units and the VALU only dequantizes:
//
//   D[m][n] = sum_k x[m][k] * (1024 + q[n][k])     (one MFMA per 32-block)
//   Dx[m]   = sum_k x[m][k]                          (an MFMA against ones)
//   y[m][n] += s[n] * D + (b[n] - 1024 s[n]) * Dx    (affine4, per block)
//   (Q4_0: c = -1032 d; Q8_0: 1152 + q, c = -1152 d; no bias)
//
// Work split: a workgroup owns 16 weight rows; its S waves (up to 16) split K
// into contiguous ranges of 4-block groups and sum their partial results in
// LDS in a fixed order (deterministic). Decode shapes have few rows and short
// K ranges per wave, so a wave is latency-bound unless many loads are in
// flight: each wave issues the loads of its first P groups (weights and
// activations alike, as range-checked buffer loads, so invalid rows, columns
// and blocks read zero with no branch) before any arithmetic, and refills a
// group's registers as soon as it has consumed it. A lane (n = lane % 16,
// g = lane / 16) loads block b0 + g of row n, then four lanes exchange 16-lane
// groups with permlane swaps so that lane group g holds quant dword g of all
// four blocks: the MFMA's 32 k of a block are, for lane group g, the elements
// 4g..4g+3 and 16+4g..19+4g (both nibbles of byte 4g..4g+3), and the
// activations use the same order.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "kq_dev.h"
#include "kq_internal.h"

namespace kqd {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half8_t as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8_t, v);
}

// 4x4 transpose of 16-lane groups across four registers: afterwards r[j] at
// lane group g holds what r[g] held at lane group j.
__device__ __forceinline__ void transpose4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
  auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = c[0];
  r1 = c[1];
  r2 = d[0];
  r3 = d[1];
}

// Raw data of one 4-block group, as loaded by a lane (block b0 + g of row n).
template <int FMT> struct GroupRaw;
template <> struct GroupRaw<F_AFFINE4> { uint32_t D[5]; };    // s|b, 4 nibble dwords
template <> struct GroupRaw<F_Q4_0> { uint32_t D[6]; };       // from the aligned dword before the nibbles
template <> struct GroupRaw<F_Q8_0> { uint32_t D[10]; };      // idem, 8 quant dwords
template <> struct GroupRaw<F_Q5_0> { uint32_t D[7]; };       // idem, fifth-bit word + 4 nibble dwords
template <> struct GroupRaw<F_Q5_1> { uint32_t D[6]; };       // d|m, fifth-bit word, 4 nibble dwords

// byte offset of block `blk` of the row at `roff`
template <int FMT>
__device__ __forceinline__ void load_group(rsrc_t rs, uint32_t roff, int blk, bool valid, GroupRaw<FMT>& r) {
  const uint32_t off = roff + (uint32_t)blk * Fmt<FMT>::BB;
  if constexpr (FMT == F_AFFINE4) {
    const uint32_t o = valid ? off : OOB;
    const u32x4 t = ld128(rs, o);
    r.D[0] = t.x; r.D[1] = t.y; r.D[2] = t.z; r.D[3] = t.w;
    r.D[4] = ld32(rs, o + 16);
  } else if constexpr (FMT == F_Q5_1) {   // 24-byte blocks: 8-byte aligned
    const uint32_t o = valid ? off : OOB;
    const u32x4 t = ld128(rs, o);
    const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(rs, o + 16u, 0, 0);
    r.D[0] = t.x; r.D[1] = t.y; r.D[2] = t.z; r.D[3] = t.w;
    r.D[4] = u.x; r.D[5] = u.y;
  } else {
    // Quants start at qs = off + 2, 2-byte aligned. Load the aligned dwords
    // from qs & ~3 (D[1]...), and the dword before them (D[0]) only when the
    // scale sits there (qs 4-aligned): every offset stays >= 0.
    const uint32_t qs = off + 2;
    const uint32_t base = qs & ~3u;
    const uint32_t o = valid ? base : OOB;
    r.D[0] = ld32(rs, valid && (qs & 3u) == 0 ? base - 4u : OOB);
    const u32x4 t = ld128(rs, o);
    r.D[1] = t.x; r.D[2] = t.y; r.D[3] = t.z; r.D[4] = t.w;
    if constexpr (FMT == F_Q4_0) {
      r.D[5] = ld32(rs, o + 16);
    } else if constexpr (FMT == F_Q5_0) {
      const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(rs, o + 16u, 0, 0);
      r.D[5] = u.x; r.D[6] = u.y;
    } else {
      const u32x4 u = ld128(rs, o + 16);
      r.D[5] = u.x; r.D[6] = u.y; r.D[7] = u.z; r.D[8] = u.w;
      r.D[9] = ld32(rs, o + 32);
    }
  }
}

// A lane's own block of a group, from its raw load: the header word (scale;
// scale|bias for affine4; d|m for Q5_1), the quant dwords (q, and p for Q8_0's
// second half) and the fifth-bit word (Q5_0, Q5_1).
struct OwnBlock {
  uint32_t hdr, q[4], p[4], qh;
};

template <int FMT>
__device__ __forceinline__ OwnBlock own_block(const GroupRaw<FMT>& cur, uint32_t roff, int blk) {
  OwnBlock b;
  b.qh = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) b.p[t] = 0;
  if constexpr (FMT == F_AFFINE4) {
    b.hdr = cur.D[0];
#pragma unroll
    for (int t = 0; t < 4; ++t) b.q[t] = cur.D[1 + t];
  } else if constexpr (FMT == F_Q5_1) {
    b.hdr = cur.D[0];
    b.qh = cur.D[1];
#pragma unroll
    for (int t = 0; t < 4; ++t) b.q[t] = cur.D[2 + t];
  } else {
    // the data after the 2-byte scale starts 0 or 2 bytes into D[1]
    const uint32_t r2 = ((roff + (uint32_t)blk * Fmt<FMT>::BB + 2u) & 3u) * 8u;  // bit shift 0/16
    b.hdr = r2 ? (cur.D[1] & 0xffffu) : (cur.D[0] >> 16);
    const uint32_t sh = r2 >> 3;   // byte shift 0 or 2
    if constexpr (FMT == F_Q5_0) {
      b.qh = __builtin_amdgcn_alignbyte(cur.D[2], cur.D[1], sh);
#pragma unroll
      for (int t = 0; t < 4; ++t) b.q[t] = __builtin_amdgcn_alignbyte(cur.D[3 + t], cur.D[2 + t], sh);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) b.q[t] = __builtin_amdgcn_alignbyte(cur.D[2 + t], cur.D[1 + t], sh);
      if constexpr (FMT == F_Q8_0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) b.p[t] = __builtin_amdgcn_alignbyte(cur.D[6 + t], cur.D[5 + t], sh);
      }
    }
  }
  return b;
}

// Per-block fix-up: y += sc * D + c * (sum of x over the block), D the product
// with the magic-number operands 1024 + q (Q8_0: 1152 + q). c removes the
// 1024 and applies the format's offset or minimum.
template <int FMT>
__device__ __forceinline__ float fix_const(uint32_t hdr, float sc) {
  if constexpr (FMT == F_AFFINE4 || FMT == F_Q5_1) return __builtin_fmaf(-1024.0f, sc, h2f(hdr >> 16));
  else if constexpr (FMT == F_Q4_0) return -1032.0f * sc;
  else if constexpr (FMT == F_Q5_0) return -1040.0f * sc;
  else return -1152.0f * sc;
}

// A group's blocks in operand order: after the exchange, lane group g holds
// for block j of the group its quant dword g (and Q8_0's dword 4 + g), its
// header word and its fifth-bit word.
struct GroupOps {
  uint32_t qs[4], ps[4], hs[4], qhs[4];
};

template <int FMT>
__device__ __forceinline__ void exchange(const OwnBlock& b, GroupOps& o) {
  uint32_t q0 = b.q[0], q1 = b.q[1], q2 = b.q[2], q3 = b.q[3];
  transpose4(q0, q1, q2, q3);
  o.qs[0] = q0; o.qs[1] = q1; o.qs[2] = q2; o.qs[3] = q3;
  if constexpr (FMT == F_Q8_0) {
    uint32_t p0 = b.p[0], p1 = b.p[1], p2 = b.p[2], p3 = b.p[3];
    transpose4(p0, p1, p2, p3);
    o.ps[0] = p0; o.ps[1] = p1; o.ps[2] = p2; o.ps[3] = p3;
  }
  uint32_t h0 = b.hdr, h1 = b.hdr, h2 = b.hdr, h3 = b.hdr;
  transpose4(h0, h1, h2, h3);
  o.hs[0] = h0; o.hs[1] = h1; o.hs[2] = h2; o.hs[3] = h3;
  if constexpr (FMT == F_Q5_0 || FMT == F_Q5_1) {
    uint32_t e0 = b.qh, e1 = b.qh, e2 = b.qh, e3 = b.qh;
    transpose4(e0, e1, e2, e3);
    o.qhs[0] = e0; o.qhs[1] = e1; o.qhs[2] = e2; o.qhs[3] = e3;
  }
}

// B operand of block j for lane group g: 8 fp16 (1024 + q, Q8_0 1152 + q) for
// elements {4g..4g+3, 16+4g..19+4g}; a 5-bit format's fifth bits (bit i of
// the word for element i) become +16 in those fp16 halves.
template <int FMT>
__device__ __forceinline__ half8_t b_operand(const GroupOps& o, int j, int g) {
  uint32_t b0, b1, b2, b3;
  if constexpr (FMT == F_Q8_0) {
    const uint32_t u = o.qs[j] ^ 0x80808080u, v = o.ps[j] ^ 0x80808080u;
    b0 = perm(MAGIC, u, SEL_LO); b1 = perm(MAGIC, u, SEL_HI);
    b2 = perm(MAGIC, v, SEL_LO); b3 = perm(MAGIC, v, SEL_HI);
  } else {
    const uint32_t lo = o.qs[j] & 0x0F0F0F0Fu, hi = (o.qs[j] >> 4) & 0x0F0F0F0Fu;
    b0 = perm(MAGIC, lo, SEL_LO); b1 = perm(MAGIC, lo, SEL_HI);
    b2 = perm(MAGIC, hi, SEL_LO); b3 = perm(MAGIC, hi, SEL_HI);
    if constexpr (FMT == F_Q5_0 || FMT == F_Q5_1) {
      const uint32_t qh = o.qhs[j];
      b0 |= spread2<4>(qh, 4 * g);
      b1 |= spread2<4>(qh, 4 * g + 2);
      b2 |= spread2<4>(qh, 16 + 4 * g);
      b3 |= spread2<4>(qh, 18 + 4 * g);
    }
  }
  return as_half8(b0, b1, b2, b3);
}

// Activations of one 4-block group for one 16-column tile: for block j the
// lane's A operand is x[col][32 b + 4g .. 4g+3] and x[col][32 b + 16 + 4g .. +3].
struct GroupX {
  u32x2 lo[4], hi[4];
};

// `xs` covers the M columns of x; `xoff` is this lane's column start in bytes,
// or OOB for a column past M (all its loads read zero).
__device__ __forceinline__ void load_group_x(rsrc_t xs, uint32_t xoff, int b0, int nblk, int g, GroupX& gx) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = b0 + j;
    const uint32_t o = b < nblk ? xoff + 64u * (uint32_t)b + 8u * (uint32_t)g : OOB;
    gx.lo[j] = __builtin_amdgcn_raw_buffer_load_b64(xs, o, 0, 0);
    gx.hi[j] = __builtin_amdgcn_raw_buffer_load_b64(xs, o + 32u, 0, 0);
  }
}

// One 4-block group of one row tile against T column tiles: exchange the
// loaded blocks into MFMA operand order, dequantize, multiply, fix up.
template <int FMT, int T>
__device__ __forceinline__ void consume_group(const GroupRaw<FMT>& cur, const GroupX (&cx)[T], uint32_t roff,
                                              int gi, int g, int nblk, float4_t (&acc)[T]) {
  const half8_t ones = as_half8(ONES, ONES, ONES, ONES);
  GroupOps o;
  exchange<FMT>(own_block<FMT>(cur, roff, 4 * gi + g), o);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (4 * gi + j >= nblk) break;      // uniform
    const half8_t B = b_operand<FMT>(o, j, g);
    const float sc = h2f(o.hs[j]);
    const float c = fix_const<FMT>(o.hs[j], sc);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const half8_t A = as_half8(cx[t].lo[j].x, cx[t].lo[j].y, cx[t].hi[j].x, cx[t].hi[j].y);
      const float4_t D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      const float4_t Dx = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ones, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        acc[t][v] = __builtin_fmaf(sc, D[v], acc[t][v]);
        acc[t][v] = __builtin_fmaf(c, Dx[v], acc[t][v]);
      }
    }
  }
}

// Grid: one workgroup per 16 rows, S = blockDim.x / 64 waves, wave w owns
// groups [w * gpw, (w + 1) * gpw) of the rows (clipped to the row length).
// Dynamic LDS: S * T * 64 float4 partial results.
// Waves per workgroup at most: 16, or 8 with three or more column tiles (their
// activations need more than the 128 registers a 16-wave workgroup allows).
template <int T> struct MfmaMaxWaves { static constexpr int v = T >= 3 ? 8 : 16; };

template <int FMT, int T, int P>
__global__ __launch_bounds__(64 * MfmaMaxWaves<T>::v) void k_gemv_mfma(const uint8_t* __restrict__ W,
                                                   const uint16_t* __restrict__ x,
                                                   float* __restrict__ y, int N, int K, int M, int gpw) {
  extern __shared__ float4_t red[];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int S = blockDim.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int nblk = K / 32;
  const int ngroups = (nblk + 3) / 4;
  const int gb = wave * gpw;
  const int ge = min(gb + gpw, ngroups);
  const uint32_t row_bytes = (uint32_t)nblk * Fmt<FMT>::BB;
  const int valid_rows = (int)min<int64_t>(16, N - row0);
  // Range rounded up to whole dwords: Q4_0/Q8_0 blocks are only 2-byte
  // aligned, so the last block's final dword may hang 2 bytes past the end
  // (same dword, same page).
  const rsrc_t rs = make_rsrc(W + row0 * row_bytes, ((uint32_t)valid_rows * row_bytes + 3u) & ~3u);
  const uint32_t roff = (uint32_t)n * row_bytes;
  const bool row_ok = n < valid_rows;
  const rsrc_t xs = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  uint32_t xoff[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int col = 16 * t + n;
    xoff[t] = col < M ? (uint32_t)col * (uint32_t)K * 2u : OOB;
  }

  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  GroupRaw<FMT> wr[P];
  GroupX xr[P][T];
  // Loads first: the first P groups of this wave's range (past its end: zero).
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int gi = gb + p;
    load_group<FMT>(rs, roff, 4 * gi + g, gi < ge && row_ok && 4 * gi + g < nblk, wr[p]);
#pragma unroll
    for (int t = 0; t < T; ++t) load_group_x(xs, gi < ge ? xoff[t] : OOB, 4 * gi, nblk, g, xr[p][t]);
    __builtin_amdgcn_sched_barrier(0);   // groups are issued in order: consuming one waits for it alone
  }
  for (int base = gb; base < ge; base += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int gi = base + p;
      if (gi < ge) consume_group<FMT, T>(wr[p], xr[p], roff, gi, g, nblk, acc);   // uniform
      // Refill the slot with the group one round ahead. Past the range the
      // loads read zero; they are issued anyway, so that every path leaves the
      // same loads in flight in the same order and each consume waits only
      // for its own group.
      const int gn = gi + P;
      load_group<FMT>(rs, roff, 4 * gn + g, gn < ge && row_ok && 4 * gn + g < nblk, wr[p]);
#pragma unroll
      for (int t = 0; t < T; ++t) load_group_x(xs, gn < ge ? xoff[t] : OOB, 4 * gn, nblk, g, xr[p][t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // fixed-order sum of the S waves' partial results
#pragma unroll
  for (int t = 0; t < T; ++t) red[(wave * T + t) * 64 + lane] = acc[t];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float4_t s = red[t * 64 + lane];
      for (int w = 1; w < S; ++w) {
        const float4_t o = red[(w * T + t) * 64 + lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) s[v] += o[v];
      }
      // lane holds D[col = 16t + 4g + v][row n]
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int col = 16 * t + 4 * g + v;
        if (col < M && row_ok) y[(int64_t)col * N + row0 + n] = s[v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Activations staged in LDS (M <= 16 and the copy fits): the workgroup copies
// x once, with 16-byte loads, into the MFMA operand order, so that a wave's
// per-group memory instructions are its weight loads alone (otherwise the
// texture address path, not HBM, bounds the kernel). With Mp = M rounded up
// to a power of two and K rounded up to whole 4-block groups (zeros past K):
//   x slots: for block b, lane group g, column c, 16 bytes at ((4 b + g) Mp + c') 16
//            with c' = c ^ xsw(b, g), holding x[c][32 b + 4 g .. +3] then
//            x[c][32 b + 16 + 4 g .. +3]. The lanes of one operand read take one
//            contiguous row (no bank conflicts); the column swizzle
//            xsw(b, g) = ((b & 3) << 1 | g >> 1) & (Mp - 1) spreads the writes of
//            the staging, whose lanes hold consecutive pieces of one column;
//   sums:    sx[b][c] = sum of block b of column c, fp32 (not swizzled).
// The per-block fix-up splits in two. The scale term sc * D needs D per block
// (4 FMAs per lane). The offset term sum_b c[row][b] sx[c][b] is itself a small
// product, done per group as one fp32 MFMA (16x16x4) whose B operand is the
// constant of the lane's own loaded block, so it needs no exchange. Blocks
// past K have zero weights (loads out of range), zero x and zero sums, so they
// add exactly zero and need no test.
//
// Grid: R 16-row tiles per workgroup, S waves per tile (R S <= 16); wave
// (r, s) owns groups [s P, (s + 1) P) of tile r, all loaded before any
// arithmetic. Columns >= M: their lanes read a real column and their outputs
// are discarded.
constexpr int XST_MAX = 12;   // 16-byte x pieces per thread while staging

// floor(a / b) for 0 <= a < 2^16 and b >= 1 without an integer division
// sequence (tens of scalar instructions ahead of a kernel's first load): the
// quotient (a + 1/2) / b is at least 1 / (2 b) away from an integer, far more
// than the error of the reciprocal and the product.
__device__ __forceinline__ int div_small(int a, int b) {
  return (int)(((float)a + 0.5f) * __builtin_amdgcn_rcpf((float)b));
}

// Column swizzle of the x slots of block b, lane group g.
__device__ __forceinline__ int xsw(int b, int g, int Mp) { return (((b & 3) << 1) | (g >> 1)) & (Mp - 1); }

template <int FMT, int P, bool SX, int XM>
__global__ __launch_bounds__(1024) void k_gemv_mfma_lds(const uint8_t* __restrict__ W,
                                                       const uint16_t* __restrict__ x,
                                                       float* __restrict__ y, int N, int K, int M, int R,
                                                       int S, int log2mp, int nsplit);

// One 4-block group of a 16-row tile (the lane's raw block `cur`, block
// index 4 gi + g) against the staged x: the group's offset term as one fp32
// MFMA, then per block D = x . (offset + q) and acc += scale * D.
template <int FMT, bool SX = true>
__device__ __forceinline__ void mfma_group(const GroupRaw<FMT>& cur, uint32_t roff, int gi, int gl, int g, int ncol,
                                           const u32x4* xa, const float* sxa, int Mp, float4_t& acc) {
  const OwnBlock own = own_block<FMT>(cur, roff, 4 * gi + g);
  if constexpr (SX) {
    const float so = h2f(own.hdr);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sxa[4 * gl * Mp], fix_const<FMT>(own.hdr, so), acc, 0, 0, 0);
  }
  GroupOps o;
  exchange<FMT>(own, o);
  const int bstride = 4 * Mp;
  float4_t D[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half8_t A = __builtin_bit_cast(half8_t, xa[(4 * gl + j) * bstride + (ncol ^ xsw(j, g, Mp))]);
    D[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, b_operand<FMT>(o, j, g), float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float sc = h2f(o.hs[j]);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(sc, D[j][v], acc[v]);
  }
  if constexpr (!SX) {
    // no block sums in LDS: the offset term per block from an MFMA against ones
    const half8_t ones = as_half8(ONES, ONES, ONES, ONES);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half8_t A = __builtin_bit_cast(half8_t, xa[(4 * gl + j) * bstride + (ncol ^ xsw(j, g, Mp))]);
      const float4_t Dx = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ones, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      const float sc = h2f(o.hs[j]);
      const float c = fix_const<FMT>(o.hs[j], sc);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(c, Dx[v], acc[v]);
    }
  }
}

// Stage x (M columns, K) into LDS in the operand order described above, plus
// the block sums. Called by every thread of the workgroup; `issue_more` runs
// between issuing the x loads and writing them (the caller's weight loads),
// after a barrier that puts every wave's x loads ahead of them in the queue.
// With a K split, the staged range starts at piece k8_0 of every column
// (column stride stays K) and covers ngroups groups.
template <bool SX, typename F, bool XF = false>
__device__ __forceinline__ void stage_x_mfma(const uint16_t* __restrict__ x, int M, int K, int ngroups,
                                             int log2mp, uint8_t* xlb, int nthreads, F issue_more, int k8_0 = 0) {
  const int Mp = 1 << log2mp;
  const int kq8 = K / 8, kq8p = 16 * ngroups;
  const int k8_lim = kq8 - k8_0;   // pieces of the column from the range start on
  const uint32_t sx_base = (uint32_t)kq8p * (uint32_t)Mp * 16u;
  const int nwaves = nthreads >> 6;   // nthreads: the workgroup size, from the caller's arguments
  const int lane = (int)threadIdx.x & 63;
  const int wv = wave_id();
  const rsrc_t xs = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  // Wave chunk q = wv + nwaves * c: 64 consecutive 16-byte pieces of one
  // column, column q & (Mp - 1), pieces 64 (q >> log2mp) + lane, so the lanes
  // of one load read 1 KB of contiguous memory. Chunks past the nq the
  // staging needs, and chunks of the padding columns M..Mp - 1 (whose slots no
  // operand read uses), are not issued at all (a branch uniform over the
  // wave): a load that reads nothing still takes the CU's address unit as
  // long as a real one, and every workgroup on the CU stages its own copy of x.
  const int nq = Mp * ((kq8p + 63) / 64);
  u32x4 xr[XST_MAX];
#pragma unroll
  for (int c = 0; c < XST_MAX; ++c) {
    const int q = wv + nwaves * c;
    const int col = q & (Mp - 1), k8 = 64 * (q >> log2mp) + lane;
    const bool ok = k8 < k8_lim;
    xr[c] = q < nq && col < M ? ld128(xs, ok ? ((uint32_t)col * (uint32_t)kq8 + (uint32_t)(k8_0 + k8)) * 16u : OOB)
                              : u32x4{0u, 0u, 0u, 0u};
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!XF) {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_more();
    __builtin_amdgcn_sched_barrier(0);
  }
  {
    // piece k8 = 4 b + h: elements 0-3 go to lane group g0 = 2 (h & 1), 4-7 to
    // g0 + 1, at byte 8 (h >> 1) of the slot; b & 3 and h are the lane's own.
    const int h = lane & 3, g0 = 2 * (h & 1);
    const int sw = xsw(lane >> 2, g0, Mp);
    const uint32_t part = 8u * (uint32_t)(h >> 1);
#pragma unroll
    for (int c = 0; c < XST_MAX; ++c) {
      const int q = wv + nwaves * c;
      const int col = q & (Mp - 1), k8 = 64 * (q >> log2mp) + lane;
      if (q < nq && k8 < kq8p) {   // pieces past the padded K have no slot
        const uint32_t a0 = (uint32_t)((4 * (k8 >> 2) + g0) * Mp + (col ^ sw)) * 16u + part;
        *reinterpret_cast<u32x2*>(xlb + a0) = u32x2{xr[c].x, xr[c].y};
        *reinterpret_cast<u32x2*>(xlb + a0 + (uint32_t)Mp * 16u) = u32x2{xr[c].z, xr[c].w};
      }
    }
  }
  if constexpr (XF) {
    __builtin_amdgcn_sched_barrier(0);
    issue_more();
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  if constexpr (!SX) return;
  const u32x4* xl4 = reinterpret_cast<const u32x4*>(xlb);
  float* sx = reinterpret_cast<float*>(xlb + sx_base);
  const int ntask = 4 * ngroups * Mp;
  for (int t = (int)threadIdx.x; t < ntask; t += nthreads) {
    const int bb = t >> log2mp, col = t & (Mp - 1);
    float v = 0.0f;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const u32x4 q = xl4[(4 * bb + gg) * Mp + (col ^ xsw(bb, gg, Mp))];
      v = dot2(q.x, ONES, v);
      v = dot2(q.y, ONES, v);
      v = dot2(q.z, ONES, v);
      v = dot2(q.w, ONES, v);
    }
    sx[t] = v;
  }
  __syncthreads();
}

// x by buffer-to-LDS DMA for the teams kernel, column-major: piece p of column c (x[c][8 (k8_0 + p) .. +7],
// p < P = 16 ngroups) at slot c P + (p ^ (c & 15)). One load instruction of a
// wave fills 64 consecutive slots, so its lanes read one column's 1 KB with
// the pieces permuted inside aligned runs of 16 (every quad of lanes still
// reads one 64-byte run); pieces past the column's end are written as zeros.
// Nothing passes through registers: the caller's weight loads are issued
// right behind x, and the barrier after them waits for both. The swizzle puts
// the pieces the 16 lanes of an operand read (one column each) in distinct
// bank groups.
template <bool SX, typename F>
__device__ __forceinline__ void stage_x_cm(const uint16_t* __restrict__ x, int M, int K, int ngroups, int log2mp,
                                           uint8_t* xlb, int nthreads, F issue_more, int k8_0) {
  const int P = 16 * ngroups, nslot = M * P, kq8 = K / 8;
  const int lane = (int)threadIdx.x & 63, nwaves = nthreads >> 6;
  const rsrc_t xs = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  for (int base = 64 * wave_id(); base < nslot; base += 64 * nwaves) {   // uniform over the wave
    const int s = base + lane;
    const int c = div_small(s, P);   // s < 2^16: the slots fit in LDS
    const int p = (s - c * P) ^ (c & 15);
    if (s < nslot) {
      if (k8_0 + p < kq8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (lds_void_t*)(xlb + 16 * base), 16,
                                                 ((uint32_t)c * (uint32_t)kq8 + (uint32_t)(k8_0 + p)) * 16u, 0, 0, 0);
      else
        *reinterpret_cast<u32x4*>(xlb + 16 * s) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  issue_more();
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  if constexpr (!SX) return;
  // block sums sx[b][c] (fp32, at the offset and in the order stage_x_mfma
  // leaves them), for the real columns: no operand read uses the others
  const int Mp = 1 << log2mp;
  float* sx = reinterpret_cast<float*>(xlb + (uint32_t)P * (uint32_t)Mp * 16u);
  const int ntask = 4 * ngroups * Mp;
  for (int t = (int)threadIdx.x; t < ntask; t += nthreads) {
    const int bb = t >> log2mp, col = t & (Mp - 1);
    if (col >= M) continue;
    // the elements in the order of the operand-order sums: lane group gg's
    // x[32 bb + 4 gg .. +3], then x[32 bb + 16 + 4 gg .. +3]
    const uint8_t* xc = xlb + (uint32_t)(col * P) * 16u;
    float v = 0.0f;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const uint32_t half = 8u * (uint32_t)(gg & 1);
      const int p0 = 4 * bb + (gg >> 1);
      const u32x2 lo = *reinterpret_cast<const u32x2*>(xc + 16u * (uint32_t)(p0 ^ (col & 15)) + half);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(xc + 16u * (uint32_t)((p0 + 2) ^ (col & 15)) + half);
      v = dot2(lo.x, ONES, v);
      v = dot2(lo.y, ONES, v);
      v = dot2(hi.x, ONES, v);
      v = dot2(hi.y, ONES, v);
    }
    sx[t] = v;
  }
  __syncthreads();
}

// mfma_group on x staged by stage_x_cm: xc is the first slot
// of the lane's column, csw its swizzle; the A operand of block j is read as
// two 8-byte halves, x[c][32 b + 4 g .. +3] and x[c][32 b + 16 + 4 g .. +3].
template <int FMT, bool SX>
__device__ __forceinline__ void mfma_group_cm(const GroupRaw<FMT>& cur, uint32_t roff, int gi, int gl, int g,
                                              const uint8_t* xc, int csw, const float* sxa, int Mp, float4_t& acc) {
  const OwnBlock own = own_block<FMT>(cur, roff, 4 * gi + g);
  if constexpr (SX) {
    const float so = h2f(own.hdr);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sxa[4 * gl * Mp], fix_const<FMT>(own.hdr, so), acc, 0, 0, 0);
  }
  GroupOps o;
  exchange<FMT>(own, o);
  const uint32_t half = 8u * (uint32_t)(g & 1);
  half8_t A[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p0 = 4 * (4 * gl + j) + (g >> 1);
    const u32x2 lo = *reinterpret_cast<const u32x2*>(xc + 16u * (uint32_t)(p0 ^ csw) + half);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(xc + 16u * (uint32_t)((p0 + 2) ^ csw) + half);
    A[j] = as_half8(lo.x, lo.y, hi.x, hi.y);
  }
  float4_t D[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    D[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[j], b_operand<FMT>(o, j, g), float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float sc = h2f(o.hs[j]);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(sc, D[j][v], acc[v]);
  }
  if constexpr (SX) return;
  const half8_t ones = as_half8(ONES, ONES, ONES, ONES);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4_t Dx = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[j], ones, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    const float sc = h2f(o.hs[j]);
    const float c = fix_const<FMT>(o.hs[j], sc);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(c, Dx[v], acc[v]);
  }
}

// Many tiles (large N): persistent waves. x is staged once per workgroup;
// then every wave on its own streams whole 16-row tiles (no K split, so no
// reduction), tiles t0, t0 + T, ... (T = waves in the grid, `tpw` tiles per
// wave at most), as one sequence of 4-block groups with P groups in flight:
// a slot is refilled with the group P steps ahead (of this tile or the next)
// as soon as it has been consumed. A finished tile's outputs are stored at
// once by the wave that owns it.
// Few tiles (small N): a workgroup of R tiles x S waves; wave (r, s) owns
// groups [s P, (s + 1) P) of tile r, all loaded before any arithmetic, and the
// S partial results of a tile are summed in LDS in a fixed order. SX: block
// sums in LDS (else, when x alone just fits, from an MFMA per block). XM, how
// x is staged: 2 by DMA in column-major order (stage_x_cm), 1 through
// registers in operand order before the weight loads are issued, 0 through
// registers with the weight loads issued first (stage_x_mfma).
template <int FMT, int P, bool SX, int XM>
__global__ __launch_bounds__(1024) void k_gemv_mfma_lds(const uint8_t* __restrict__ W,
                                                       const uint16_t* __restrict__ x,
                                                       float* __restrict__ y, int N, int K, int M, int R,
                                                       int S, int log2mp, int nsplit) {
  extern __shared__ u32x4 xl4[];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int r = div_small(wave, S), s = wave - r * S;
  const int n = lane & 15, g = lane >> 4;
  const int64_t row0 = ((int64_t)blockIdx.x * R + r) * 16;
  const int nblk = K / 32;
  // K split (grid y): this workgroup's groups [gs0, gs1) of the row, its
  // output the partial sums y[blockIdx.y][M][N] (one split: y itself)
  const int ngroups_all = (nblk + 3) / 4;   // nsplit = the grid's y extent (an argument)
  const int gs0 = nsplit == 1 ? 0 : div_small((int)blockIdx.y * ngroups_all, nsplit);
  const int gs1 = nsplit == 1 ? ngroups_all : div_small(((int)blockIdx.y + 1) * ngroups_all, nsplit);
  const int ngroups = gs1 - gs0;
  y += (int64_t)blockIdx.y * M * N;
  const int Mp = 1 << log2mp;
  const int gb = gs0 + s * P;
  const uint32_t row_bytes = (uint32_t)nblk * Fmt<FMT>::BB;
  const int valid_rows = row0 < N ? (int)min<int64_t>(16, N - row0) : 0;
  const rsrc_t rs = make_rsrc(W + (valid_rows ? row0 * row_bytes : 0), ((uint32_t)valid_rows * row_bytes + 3u) & ~3u);
  const uint32_t roff = (uint32_t)n * row_bytes;
  const bool row_ok = n < valid_rows;
  uint8_t* xlb = reinterpret_cast<uint8_t*>(xl4);
  GroupRaw<FMT> wr[P];
  auto issue = [&]() {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int gi = gb + p;
      load_group<FMT>(rs, roff, 4 * gi + g, gi < gs1 && row_ok && 4 * gi + g < nblk, wr[p]);
    }
  };
  if constexpr (XM == 2)
    stage_x_cm<SX>(x, M, K, ngroups, log2mp, xlb, 64 * R * S, issue, 16 * gs0);
  else
    stage_x_mfma<SX, decltype(issue), XM == 1>(x, M, K, ngroups, log2mp, xlb, 64 * R * S, issue, 16 * gs0);
  const int ncol = n < M ? n : M - 1;
  const u32x4* xa = xl4 + g * Mp;
  const float* sxa = reinterpret_cast<const float*>(xlb + (uint32_t)(16 * ngroups) * (uint32_t)Mp * 16u) + g * Mp + ncol;
  const uint8_t* xc = xlb + (uint32_t)(16 * ngroups) * (uint32_t)ncol * 16u;
  float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int gi = gb + p;
    if (gi >= gs1) break;   // uniform
    if constexpr (XM == 2)
      mfma_group_cm<FMT, SX>(wr[p], roff, gi, gi - gs0, g, xc, ncol & 15, sxa, Mp, acc);
    else
      mfma_group<FMT, SX>(wr[p], roff, gi, gi - gs0, g, ncol, xa, sxa, Mp, acc);
  }
  // fixed-order sum over the S waves of each tile (the x area is reused)
  __syncthreads();
  float4_t* red = reinterpret_cast<float4_t*>(xl4);
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (s == 0 && valid_rows > 0) {
    float4_t t = red[(r * S) * 64 + lane];
    for (int w = 1; w < S; ++w) {
      const float4_t o = red[(r * S + w) * 64 + lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) t[v] += o[v];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int col = 4 * g + v;
      if (col < M && row_ok) y[(int64_t)col * N + row0 + n] = t[v];
    }
  }
}

// Many columns (T tiles of 16) or long rows: the workgroup walks K in chunks
// of CG 4-block groups (CG a power of two), staging x of the chunk for all T
// column tiles at once (tile t at t * 4096 CG bytes, each in the operand
// order above with Mp = 16), with block sums. Per chunk, each wave loads its
// P groups of the chunk, then consumes them: the dequantized weights of a
// block serve all T column tiles. R row tiles x S waves per workgroup (at most
// 8 waves: the staged pieces, the loaded groups and T accumulators need more
// than the 128 registers of a 16-wave workgroup); the S partial results of a
// tile are summed in a fixed order at the end.
template <int FMT, int P, int T>
__global__ __launch_bounds__(512) void k_gemv_mfma_chunk(const uint8_t* __restrict__ W,
                                                         const uint16_t* __restrict__ x,
                                                         float* __restrict__ y, int N, int K, int M, int R,
                                                         int S, int log2cg) {
  extern __shared__ u32x4 xl4[];
  // Column groups of 16 T columns along the grid's y (one group when the
  // grid has no y extent): this workgroup's columns start at col0.
  {
    const int col0 = (int)blockIdx.y * 16 * T;
    x += (int64_t)col0 * K;
    y += (int64_t)col0 * N;
    M = min(M - col0, 16 * T);
  }
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int r = div_small(wave, S), s = wave - r * S;
  const int n = lane & 15, g = lane >> 4;
  const int64_t row0 = ((int64_t)blockIdx.x * R + r) * 16;
  const int nblk = K / 32;
  const int ngroups = (nblk + 3) / 4;
  const int CG = 1 << log2cg;
  const int nchunks = (ngroups + CG - 1) >> log2cg;
  const uint32_t row_bytes = (uint32_t)nblk * Fmt<FMT>::BB;
  const int valid_rows = row0 < N ? (int)min<int64_t>(16, N - row0) : 0;
  const rsrc_t rs = make_rsrc(W + (valid_rows ? row0 * row_bytes : 0), ((uint32_t)valid_rows * row_bytes + 3u) & ~3u);
  const uint32_t roff = (uint32_t)n * row_bytes;
  const bool row_ok = n < valid_rows;
  uint8_t* xlb = reinterpret_cast<uint8_t*>(xl4);
  const int kq8 = K / 8;
  const uint32_t tile_bytes = 4096u << log2cg;                 // x of one column tile, one chunk (4 CG blocks x 1 KB)
  const uint32_t sx_base = (uint32_t)T * tile_bytes;           // fp32 [T][4 CG][16]
  const uint32_t dummy = sx_base + (uint32_t)T * (64u << log2cg) * 4u;
  const int npieces = T * (256 << log2cg);
  // The workgroup size as the hardware reports it: written as 64 R S, the
  // piece addresses of the staging loop below were re-derived with 32-bit
  // multiplies per piece, and the 48-column verify pass took 8 % longer.
  const int nthreads = (int)blockDim.x;
  const rsrc_t xs = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  const half8_t ones = as_half8(ONES, ONES, ONES, ONES);
  (void)ones;

  for (int c = 0; c < nchunks; ++c) {
    const int cg0 = c * CG;
    const int gb = cg0 + s * P;                // this wave's first group of the chunk
    const int ge = min(gb + P, min(cg0 + CG, ngroups));
    // 1. x pieces of the chunk: piece i is column i >> (4 + log2cg) (tile
    //    column >> 4), chunk piece i & (16 CG - 1), so that the lanes of one
    //    load read contiguous runs of a column
    u32x4 xr[XST_MAX];
#pragma unroll
    for (int q = 0; q < XST_MAX; ++q) {
      const int i = (int)threadIdx.x + nthreads * q;
      const int col = i >> (4 + log2cg);
      const int k8 = 16 * cg0 + (i & ((16 << log2cg) - 1));
      const bool ok = i < npieces && col < M && k8 < kq8;
      xr[q] = ld128(xs, ok ? ((uint32_t)col * (uint32_t)kq8 + (uint32_t)k8) * 16u : OOB);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // 2. this wave's weights of the chunk
    GroupRaw<FMT> wr[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int gi = gb + p;
      load_group<FMT>(rs, roff, 4 * gi + g, gi < ge && row_ok && 4 * gi + g < nblk, wr[p]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // 3. x into LDS (branch-free, as above; slots swizzled as in the Mp = 16
    //    layout, and (k8 >> 2) & 3 and k8 & 3 are the lane's own)
#pragma unroll
    for (int q = 0; q < XST_MAX; ++q) {
      const int i = (int)threadIdx.x + nthreads * q;
      const int cl = i >> (4 + log2cg);
      const int t = cl >> 4, col = cl & 15, k8l = i & ((16 << log2cg) - 1);
      const int bb = k8l >> 2, h = k8l & 3;
      const int g0 = 2 * (h & 1);
      const int csw = col ^ xsw(bb, g0, 16);
      const uint32_t part = 8u * (uint32_t)(h >> 1);
      const bool ok = i < npieces;
      const uint32_t base = (uint32_t)t * tile_bytes;
      const uint32_t a0 = ok ? base + (uint32_t)((4 * bb + g0) * 16 + csw) * 16u + part : dummy;
      const uint32_t a1 = ok ? base + (uint32_t)((4 * bb + g0 + 1) * 16 + csw) * 16u + part : dummy + 8u;
      *reinterpret_cast<u32x2*>(xlb + a0) = u32x2{xr[q].x, xr[q].y};
      *reinterpret_cast<u32x2*>(xlb + a1) = u32x2{xr[q].z, xr[q].w};
    }
    __syncthreads();
    // 4. block sums of the chunk
    {
      float* sx = reinterpret_cast<float*>(xlb + sx_base);
      const int ntask = T * (64 << log2cg);
      for (int tk = (int)threadIdx.x; tk < ntask; tk += nthreads) {
        const int t = tk >> (6 + log2cg), rem = tk & ((64 << log2cg) - 1);
        const int bb = rem >> 4, col = rem & 15;
        const u32x4* xt = reinterpret_cast<const u32x4*>(xlb + (uint32_t)t * tile_bytes);
        float v = 0.0f;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const u32x4 qv = xt[(4 * bb + gg) * 16 + (col ^ xsw(bb, gg, 16))];
          v = dot2(qv.x, ONES, v);
          v = dot2(qv.y, ONES, v);
          v = dot2(qv.z, ONES, v);
          v = dot2(qv.w, ONES, v);
        }
        sx[tk] = v;
      }
    }
    __syncthreads();
    // 5. multiply: local group index gl = gi - cg0 addresses the chunk's LDS
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int gi = gb + p;
      if (gi >= ge) break;   // uniform
      const int gl = gi - cg0;
      const OwnBlock own = own_block<FMT>(wr[p], roff, 4 * gi + g);
      {
        const float so = h2f(own.hdr);
        const float cown = fix_const<FMT>(own.hdr, so);
        const float* sx = reinterpret_cast<const float*>(xlb + sx_base);
#pragma unroll
        for (int t = 0; t < T; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(sx[(t << (6 + log2cg)) + (4 * gl + g) * 16 + n], cown,
                                                        acc[t], 0, 0, 0);
      }
      GroupOps o;
      exchange<FMT>(own, o);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8_t B = b_operand<FMT>(o, j, g);
        const float sc = h2f(o.hs[j]);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const u32x4* xt = reinterpret_cast<const u32x4*>(xlb + (uint32_t)t * tile_bytes);
          const half8_t A = __builtin_bit_cast(half8_t, xt[(4 * (4 * gl + j) + g) * 16 + (n ^ xsw(j, g, 16))]);
          const float4_t D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[t][v] = __builtin_fmaf(sc, D[v], acc[t][v]);
        }
      }
    }
    __syncthreads();   // the chunk's LDS is restaged next
  }
  // fixed-order sum over the S waves of each tile (the x area is reused)
  float4_t* red = reinterpret_cast<float4_t*>(xl4);
#pragma unroll
  for (int t = 0; t < T; ++t) red[(wave * T + t) * 64 + lane] = acc[t];
  __syncthreads();
  if (s == 0 && valid_rows > 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float4_t sum = red[((r * S) * T + t) * 64 + lane];
      for (int w = 1; w < S; ++w) {
        const float4_t o = red[((r * S + w) * T + t) * 64 + lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) sum[v] += o[v];
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int col = 16 * t + 4 * g + v;
        if (col < M && row_ok) y[(int64_t)col * N + row0 + n] = sum[v];
      }
    }
  }
}

constexpr int MFMA_PERS_TPW = 8;   // tiles per wave at most

template <int FMT, int P, bool SX>
__global__ __launch_bounds__(512) void k_gemv_mfma_pers(const uint8_t* __restrict__ W,
                                                       const uint16_t* __restrict__ x,
                                                       float* __restrict__ y, int N, int K, int M,
                                                       int log2mp, int tpw, int nw, int nwg) {
  extern __shared__ u32x4 xl4[];
  const int lane = threadIdx.x & 63;   // nw: waves per workgroup, nwg: workgroups (arguments)
  const int n = lane & 15, g = lane >> 4;
  const int nblk = K / 32;
  const int ngroups = (nblk + 3) / 4;
  const int Mp = 1 << log2mp;
  const int64_t tiles = (N + 15) / 16;
  const int64_t T = (int64_t)nwg * nw;
  const int64_t t0 = (int64_t)blockIdx.x * nw + wave_id();
  const uint32_t row_bytes = (uint32_t)nblk * Fmt<FMT>::BB;
  const uint32_t roff = (uint32_t)n * row_bytes;
  // this wave's sequence: tiles t0 + k T (k < tpw, tile < tiles), groups 0..ngroups-1 each
  int64_t mine = 0;   // min(tpw, tiles of t0 + k T below `tiles`), tpw <= MFMA_PERS_TPW
#pragma unroll
  for (int k = 0; k < MFMA_PERS_TPW; ++k) mine += (k < tpw && t0 + (int64_t)k * T < tiles) ? 1 : 0;
  const int Q = (int)mine * ngroups;
  GroupRaw<FMT> wr[P];
  // issue pointer (tile index k, group) of the next group to load
  int ik = 0, ig = 0;
  auto issue = [&](GroupRaw<FMT>& slot, bool live) {
    const int64_t tile = t0 + (int64_t)ik * T;
    const int64_t row0 = tile * 16;
    const int valid_rows = live ? (int)min<int64_t>(16, N - row0) : 0;
    const rsrc_t rs = make_rsrc(W + (valid_rows ? row0 * row_bytes : 0), ((uint32_t)valid_rows * row_bytes + 3u) & ~3u);
    load_group<FMT>(rs, roff, 4 * ig + g, n < valid_rows && 4 * ig + g < nblk, slot);
    if (++ig == ngroups) { ig = 0; ++ik; }
  };
  uint8_t* xlb = reinterpret_cast<uint8_t*>(xl4);
  stage_x_mfma<SX>(x, M, K, ngroups, log2mp, xlb, 64 * nw, [&]() {
#pragma unroll
    for (int p = 0; p < P; ++p) issue(wr[p], p < Q);
  });
  const int ncol = n < M ? n : M - 1;
  const u32x4* xa = xl4 + g * Mp;
  const float* sxa = reinterpret_cast<const float*>(xlb + (uint32_t)(16 * ngroups) * (uint32_t)Mp * 16u) + g * Mp + ncol;
  float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
  // Finished tiles wait in registers (newest first) and are stored after the
  // loop: a store counts as a memory operation in flight too, and one taken
  // only at tile ends would make the loads' waits depend on the path.
  float4_t done[MFMA_PERS_TPW];
  int cg = 0;   // consume pointer (group within the current tile)
  for (int base = 0; base < Q; base += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int q = base + p;
      if (q < Q) {   // uniform
        mfma_group<FMT, SX>(wr[p], roff, cg, cg, g, ncol, xa, sxa, Mp, acc);
        if (++cg == ngroups) {   // tile complete: lane holds D[col 4g+v][row n]
#pragma unroll
          for (int k = MFMA_PERS_TPW - 1; k > 0; --k) done[k] = done[k - 1];
          done[0] = acc;
          acc = float4_t{0.f, 0.f, 0.f, 0.f};
          cg = 0;
        }
      }
      // refill the slot with the group P steps ahead (zero past the end: the
      // same loads on every path keep each wait to its own group)
      issue(wr[p], q + P < Q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int k = 0; k < MFMA_PERS_TPW; ++k) {
    if (k >= mine) break;   // uniform
    const int64_t row = (t0 + (mine - 1 - k) * T) * 16 + n;
    if (row < N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int col = 4 * g + v;
        if (col < M) y[(int64_t)col * N + row] = done[k][v];
      }
    }
  }
}

// Sum of the K-split partial results in split order (fixed, so the result is
// deterministic): y[i] = part[0][i] + part[1][i] + ... for i < mn.
__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ part, float* __restrict__ y, int64_t mn,
                                                   int nsplit) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= mn) return;
  float t = part[i];
  for (int s = 1; s < nsplit; ++s) t += part[(int64_t)s * mn + i];
  y[i] = t;
}

}  // namespace kqd

namespace kq {

using namespace kqd;

namespace {

// Groups in flight per wave, by register footprint (T column tiles of x).
template <int FMT, int T> struct MfmaDepth { static constexpr int v = T == 1 ? (FMT == F_Q8_0 ? 3 : 4) : (T == 2 && FMT != F_Q8_0 ? 2 : 1); };

struct MfmaCfg {
  int waves;   // per workgroup (16 rows)
  int gpw;     // 4-block groups per wave
};

// Waves per 16-row tile: at least enough to cover the row with P groups per
// wave, then doubled (up to smax) while the grid has fewer than 2048 waves, so
// that short or few rows still keep enough loads in flight. The mfma_s
// tuning override replaces it (sweeps and tests).
MfmaCfg mfma_cfg(int64_t N, int64_t K, int P, int smax) {
  const int ngroups = (int)((K / 32 + 3) / 4);
  const int64_t tiles = (N + 15) / 16;
  int S = (ngroups + P - 1) / P;
  if (S > smax) S = smax;
  while (S < smax && S < ngroups && tiles * S < 2048) S *= 2;
  if (S > smax) S = smax;
  {
    const int v = tune(TUNE_MFMA_S);
    if (v >= 1 && v <= smax) S = v;
  }
  if (S > ngroups) S = ngroups;
  const int gpw = (ngroups + S - 1) / S;
  S = (ngroups + gpw - 1) / gpw;   // no idle waves
  return {S, gpw};
}

template <int FMT, int T>
int launch_mfma_t(const GemvArgs& a, int m0, int mt) {
  constexpr int P = MfmaDepth<FMT, T>::v;
  const MfmaCfg c = mfma_cfg(a.N, a.K, P, MfmaMaxWaves<T>::v);
  const dim3 grid((unsigned)((a.N + 15) / 16)), block((unsigned)(64 * c.waves));
  const size_t lds = (size_t)c.waves * T * 64 * sizeof(float4_t);
  dispatch_log("k_gemv_mfma", a.fmt, a.N, a.K, mt, grid.x, 1, block.x, lds, "direct T=%d P=%d groups/wave=%d m0=%d",
               T, P, c.gpw, m0);
  hipLaunchKernelGGL((k_gemv_mfma<FMT, T, P>), grid, block, lds, a.stream, a.W, a.x + (int64_t)m0 * a.K,
                     a.y + (int64_t)m0 * a.N, (int)a.N, (int)a.K, mt, c.gpw);
  return (int)hipGetLastError();
}

constexpr int MFMA_LDS_MAX_BYTES = 160 * 1024;

// 16-byte pieces that stage_x_mfma loads: Mp columns of whole 64-piece
// chunks (x padded to whole 4-block groups, then to a multiple of 64 pieces).
int64_t mfma_x_pieces(int ngroups, int log2mp) {
  return ((int64_t)1 << log2mp) * 64 * ((16 * (int64_t)ngroups + 63) / 64);
}
// Groups per wave at most (registers within the 128 of a 16-wave workgroup).
template <int FMT> struct MfmaLdsMaxP { static constexpr int v = FMT == F_Q8_0 ? 4 : 6; };

struct MfmaLdsCfg {
  int R, S, P, log2mp;
  bool sx;     // block sums in LDS (else an MFMA per block)
  size_t lds;
  bool ok;
};

// LDS bytes of staged x (M columns padded to Mp, K to whole groups), with or
// without the block sums (gate|up at 8 columns: 40 KB, four workgroups per CU).
int64_t mfma_x_lds_bytes(int64_t K, int log2mp, bool sums) {
  const int64_t ngroups = (K / 32 + 3) / 4, Mp = (int64_t)1 << log2mp;
  return Mp * 16 * ngroups * 16 + (sums ? 4 * ngroups * Mp * 4 : 0);
}

// Waves per tile S: enough that each wave holds at most maxp groups,
// doubled while the grid has fewer than 1024 waves (measured against 2048 at
// M = 4, 8, 16 on the decode shapes: q|k|v 8.0 -> 7.0 us, o 7.3 -> 6.6 us at
// M = 8, with x issued first); then tiles per workgroup R
// (R S <= 8, so that several workgroups share a CU and one computes while
// another loads) while at least 1024 workgroups remain, so that one staged
// copy of x serves several tiles. Not usable (ok = false) when x does not fit in LDS
// or needs more than XST_MAX pieces per thread. no_sums: take the offset term
// from an MFMA against ones per block rather than block sums staged in LDS
// (measured faster at M = 8 and 16 on the decode shapes: the sums cost a
// pass over x and a barrier before the first product; q|k|v 8.24 -> 7.88 us,
// gate|up 13.99 -> 12.99 us at M = 8).
MfmaLdsCfg mfma_lds_cfg(int64_t N, int64_t K, int M, int maxp, bool no_sums) {
  MfmaLdsCfg c{1, 1, 1, 0, true, 0, false};
  const int ngroups = (int)((K / 32 + 3) / 4);
  const int64_t tiles = (N + 15) / 16;
  int S = (ngroups + maxp - 1) / maxp;
  if (S > 16) return c;
  int min_waves = 1024;
  if (tune(TUNE_MFMA_WAVES) > 0) min_waves = tune(TUNE_MFMA_WAVES);   // sweeps
  while (S < 16 && S < ngroups && tiles * S < min_waves) S *= 2;
  if (S > 16) S = 16;
  {
    const int v = tune(TUNE_MFMA_S);
    if (v >= 1 && v <= 16) S = v;
  }
  if (S > ngroups) S = ngroups;
  const int P1 = (ngroups + S - 1) / S;
  if (P1 > maxp) return c;
  S = (ngroups + P1 - 1) / P1;
  int R = 1;
  while (2 * R * S <= 8 && (tiles + 2 * R - 1) / (2 * R) >= 1024) R *= 2;
  {
    const int v = tune(TUNE_MFMA_R);
    if (v >= 1 && v * S <= 16) R = v;
  }
  int log2mp = 0;
  while ((1 << log2mp) < M) ++log2mp;
  const int64_t pieces = mfma_x_pieces(ngroups, log2mp);
  // enough threads to stage x (at most XST_MAX pieces each): more tiles per
  // workgroup while at least 128 workgroups remain, else more waves per tile
  // (one staged copy of x then serves two tiles: q|k|v at M = 16, 384 tiles,
  // 10.0 us as 384 workgroups of 7 waves against 7.4 us as 192 of 2 x 4)
  while (pieces > (int64_t)XST_MAX * 64 * R * S && 2 * R * S <= 16 && (tiles + 2 * R - 1) / (2 * R) >= 128) R *= 2;
  while (pieces > (int64_t)XST_MAX * 64 * R * S && R * (S + 1) <= 16 && S < ngroups) {
    ++S;
  }
  const int P2 = (ngroups + S - 1) / S;
  const int P = P2 < P1 ? P2 : P1;
  S = (ngroups + P - 1) / P;
  const int64_t rbytes = (int64_t)R * S * 64 * 16;
  if (pieces > (int64_t)XST_MAX * 64 * R * S) return c;
  for (int sums = no_sums ? 0 : 1; sums >= 0; --sums) {
    const int64_t xb = mfma_x_lds_bytes(K, log2mp, sums != 0);
    const int64_t lds = xb > rbytes ? xb : rbytes;
    if (lds <= MFMA_LDS_MAX_BYTES) return {R, S, P, log2mp, sums != 0, (size_t)lds, true};
  }
  return c;
}

// Teams kernel: x staged by DMA in column-major order (stage_x_cm) or through
// registers in operand order; the same bits either way. Measured per launch
// on the decode shapes (12 layers, cold, DMA against registers): q|k|v (384
// workgroups) -0.25..-0.41 us at 4, 6, 8, 12, 16 columns; down split along K
// (640) -0.09..-0.45 us; gate|up (1216 tiles) -0.56 us at 4, -0.43 at 6, even
// at 8, +0.23..+0.35 at 12 and 16; o (160 workgroups, fewer than the CUs)
// +0.16..+0.34 us. So DMA on grids of more than 256 workgroups, and from 1024
// tiles on only up to 8 columns. The mfma_xdma override (0 / 1) forces one way.
bool mfma_x_dma(int M, int64_t workgroups, int64_t tiles) {
  const int v = tune(TUNE_MFMA_XDMA);
  if (v != TUNE_UNSET) return v == 1;
  return workgroups > 256 && (tiles < 1024 || M <= 8);
}

template <int FMT, int P, bool SX>
int launch_mfma_lds_p(const GemvArgs& a, int m0, int mt, const MfmaLdsCfg& c) {
  const int64_t tiles = (a.N + 15) / 16;
  const dim3 grid((unsigned)((tiles + c.R - 1) / c.R)), block((unsigned)(64 * c.R * c.S));
  // x written to LDS before the weight loads are issued, except for grids of
  // at least 1024 tiles at 5..8 columns, which issue x loads, an issue-only
  // barrier, the weights, then the LDS writes. Measured with cold x on the
  // decode shapes: x first wins or ties at M = 2..16 on q|k|v, o and down
  // (o at M = 8 6.52 against 7.23 us) and on gate|up at M = 2..4 and 12..16
  // (M = 16 19.13 against 21.13 us), but gate|up (1216 tiles) at M = 5..8
  // takes 0.5-1.1 us longer that way (M = 8 14.1-14.3 against 13.0-13.8 us).
  // The mfma_xf tuning override (0 / 1) forces one order.
  const int exf = tune(TUNE_MFMA_XF);
  const bool xf = exf != TUNE_UNSET ? exf != 0 : !(c.log2mp == 3 && tiles >= 1024);
  dispatch_log("k_gemv_mfma_lds", a.fmt, a.N, a.K, mt, grid.x, 1, block.x, c.lds,
               "teams R=%d S=%d P=%d Mp=%d sums=%d x_first=%d x_dma=%d m0=%d", c.R, c.S, P, 1 << c.log2mp,
               SX ? 1 : 0, xf ? 1 : 0, mfma_x_dma(mt, grid.x, tiles) ? 1 : 0, m0);
  const uint16_t* xm = a.x + (int64_t)m0 * a.K;
  float* ym = a.y + (int64_t)m0 * a.N;
  if (mfma_x_dma(mt, grid.x, tiles)) {
    hipLaunchKernelGGL((k_gemv_mfma_lds<FMT, P, SX, 2>), grid, block, c.lds, a.stream, a.W, xm, ym, (int)a.N,
                       (int)a.K, mt, c.R, c.S, c.log2mp, 1);
    return (int)hipGetLastError();
  }
  if (xf)
    hipLaunchKernelGGL((k_gemv_mfma_lds<FMT, P, SX, 1>), grid, block, c.lds, a.stream, a.W, xm, ym, (int)a.N, (int)a.K,
                       mt, c.R, c.S, c.log2mp, 1);
  else
    hipLaunchKernelGGL((k_gemv_mfma_lds<FMT, P, SX, 0>), grid, block, c.lds, a.stream, a.W, xm, ym, (int)a.N, (int)a.K,
                       mt, c.R, c.S, c.log2mp, 1);
  return (int)hipGetLastError();
}

template <int FMT, bool SX>
int launch_mfma_lds_sx(const GemvArgs& a, int m0, int mt, const MfmaLdsCfg& c) {
  switch (c.P) {
    case 1: return launch_mfma_lds_p<FMT, 1, SX>(a, m0, mt, c);
    case 2: return launch_mfma_lds_p<FMT, 2, SX>(a, m0, mt, c);
    case 3: return launch_mfma_lds_p<FMT, 3, SX>(a, m0, mt, c);
    case 4: return launch_mfma_lds_p<FMT, 4, SX>(a, m0, mt, c);
    default:
      if constexpr (MfmaLdsMaxP<FMT>::v >= 6) {
        if (c.P == 5) return launch_mfma_lds_p<FMT, 5, SX>(a, m0, mt, c);
        return launch_mfma_lds_p<FMT, 6, SX>(a, m0, mt, c);
      }
      return (int)hipErrorInvalidValue;
  }
}

template <int FMT>
int launch_mfma_lds(const GemvArgs& a, int m0, int mt, const MfmaLdsCfg& c) {
  return c.sx ? launch_mfma_lds_sx<FMT, true>(a, m0, mt, c) : launch_mfma_lds_sx<FMT, false>(a, m0, mt, c);
}

// K split of the teams kernel (only with a caller's workspace, kq_gemv_ws):
// outputs with few row tiles and long rows run as tiles x splits workgroups,
// each staging x for its part of K only; a second kernel adds the partial
// results in split order. Measured on MI355X (2560 x 9728 affine4, the same
// bytes as 4 splits timed as a 10240 x 2432 matrix): 12.3 -> 8.2 us at 8
// columns before the sum, 15.8 -> 9.9 at 16; 2560 x 4096 gains nothing
// (6.1 against 5.7 us before the sum), so rows of fewer than 48 groups
// (6144 elements) are not split.
constexpr int SPLIT_MAX_TILES = 256;
constexpr int SPLIT_MIN_GROUPS = 48;
constexpr int SPLIT_GROUPS_EACH = 16;   // groups per split at least
constexpr int SPLIT_MAX = 8;

int split_count(const GemvArgs& a) {
  const int64_t tiles = (a.N + 15) / 16;
  const int ngroups = (int)((a.K / 32 + 3) / 4);
  if (a.M > 16 || a.M < 4) return 1;
  int ns = 1;
  if (tiles < SPLIT_MAX_TILES && ngroups >= SPLIT_MIN_GROUPS) {
    ns = ngroups / SPLIT_GROUPS_EACH;
    while (ns > 1 && tiles * ns > 4 * SPLIT_MAX_TILES) --ns;
    if (ns > 4) ns = 4;
  }
  const int v = tune(TUNE_MFMA_SPLIT);
  if (v >= 1 && v <= SPLIT_MAX && v <= ngroups) ns = v;
  return ns;
}

// teams configuration of one split (its groups as the row, the grid's tiles
// times the splits as the tile count)
MfmaLdsCfg split_cfg(const GemvArgs& a, int ns, int maxp, bool no_sums) {
  const int ngroups = (int)((a.K / 32 + 3) / 4);
  const int64_t kpart = (int64_t)((ngroups + ns - 1) / ns) * 128;
  return mfma_lds_cfg(a.N * ns, kpart, (int)a.M, maxp, no_sums);
}

template <int FMT>
int launch_mfma_split(const GemvArgs& a, int ns, const MfmaLdsCfg& c) {
  // the teams kernel with grid y = ns and its output in the workspace
  GemvArgs b = a;
  b.y = static_cast<float*>(a.ws);
  MfmaLdsCfg cc = c;
  const int64_t tiles = (a.N + 15) / 16;
  int err;
  {
    const int exf = tune(TUNE_MFMA_XF);
    const bool xf = exf != TUNE_UNSET ? exf != 0 : true;
    const dim3 grid((unsigned)((tiles + cc.R - 1) / cc.R), (unsigned)ns), block((unsigned)(64 * cc.R * cc.S));
    const bool xdma = mfma_x_dma((int)a.M, (int64_t)grid.x * ns, tiles);
    dispatch_log("k_gemv_mfma_lds", a.fmt, a.N, a.K, (int)a.M, grid.x, grid.y, block.x, cc.lds,
                 "teams K-split=%d R=%d S=%d P=%d Mp=%d sums=%d x_first=%d x_dma=%d", ns, cc.R, cc.S, cc.P,
                 1 << cc.log2mp, cc.sx ? 1 : 0, xf ? 1 : 0, xdma ? 1 : 0);
#define KQ_SPLIT_LAUNCH(PP, SXX)                                                                                  \
  do {                                                                                                           \
    if (xdma)                                                                                                    \
      hipLaunchKernelGGL((k_gemv_mfma_lds<FMT, PP, SXX, 2>), grid, block, cc.lds, a.stream, a.W, a.x, b.y,      \
                         (int)a.N, (int)a.K, (int)a.M, cc.R, cc.S, cc.log2mp, ns);                               \
    else if (xf)                                                                                                 \
      hipLaunchKernelGGL((k_gemv_mfma_lds<FMT, PP, SXX, 1>), grid, block, cc.lds, a.stream, a.W, a.x, b.y,      \
                         (int)a.N, (int)a.K, (int)a.M, cc.R, cc.S, cc.log2mp, ns);                               \
    else                                                                                                         \
      hipLaunchKernelGGL((k_gemv_mfma_lds<FMT, PP, SXX, 0>), grid, block, cc.lds, a.stream, a.W, a.x, b.y,      \
                         (int)a.N, (int)a.K, (int)a.M, cc.R, cc.S, cc.log2mp, ns);                               \
  } while (0)
    switch (cc.P) {
      case 1: if (cc.sx) KQ_SPLIT_LAUNCH(1, true); else KQ_SPLIT_LAUNCH(1, false); break;
      case 2: if (cc.sx) KQ_SPLIT_LAUNCH(2, true); else KQ_SPLIT_LAUNCH(2, false); break;
      case 3: if (cc.sx) KQ_SPLIT_LAUNCH(3, true); else KQ_SPLIT_LAUNCH(3, false); break;
      case 4: if (cc.sx) KQ_SPLIT_LAUNCH(4, true); else KQ_SPLIT_LAUNCH(4, false); break;
      default:
        if constexpr (MfmaLdsMaxP<FMT>::v >= 6) {
          if (cc.P == 5) { if (cc.sx) KQ_SPLIT_LAUNCH(5, true); else KQ_SPLIT_LAUNCH(5, false); }
          else { if (cc.sx) KQ_SPLIT_LAUNCH(6, true); else KQ_SPLIT_LAUNCH(6, false); }
        } else {
          return (int)hipErrorInvalidValue;
        }
    }
#undef KQ_SPLIT_LAUNCH
    err = (int)hipGetLastError();
  }
  if (err) return err;
  const int64_t mn = (int64_t)a.M * a.N;
  dispatch_log("k_split_sum", a.fmt, a.N, a.K, (int)a.M, (unsigned)((mn + 255) / 256), 1, 256, 0, "splits=%d", ns);
  hipLaunchKernelGGL(k_split_sum, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, a.stream,
                     static_cast<const float*>(a.ws), a.y, mn, ns);
  return (int)hipGetLastError();
}

struct MfmaChunkCfg {
  int R, S, P, log2cg;
  size_t lds;
  bool ok;
};

// Groups per wave per chunk at most, by registers (T column tiles).
template <int FMT, int T> struct MfmaChunkMaxP {
  static constexpr int v = T == 1 ? (FMT == F_Q8_0 ? 4 : 6) : (T == 2 ? 3 : 2);
};

// Chunk of CG groups: the largest power of two (at most the row's group count
// rounded up) whose x and block sums for all T tiles fit in 128 KB and need at
// most XST_MAX pieces per thread of an 8-wave workgroup. Waves per tile S:
// at most maxp groups each, more (smaller P) while the grid has fewer than
// 2048 waves. Tiles per workgroup R: only as many as staging x needs threads.
MfmaChunkCfg mfma_chunk_cfg(int64_t N, int64_t K, int T, int maxp) {
  MfmaChunkCfg c{1, 1, 1, 0, 0, false};
  const int ngroups = (int)((K / 32 + 3) / 4);
  const int64_t tiles = (N + 15) / 16;
  int log2cg = 0;
  while ((1 << log2cg) < ngroups) ++log2cg;
  auto x_bytes = [&](int l2) { return (int64_t)T * (4352 << l2) + 16; };   // x (4 KB per group) + sums (256 B per group)
  while (log2cg > 0 && (x_bytes(log2cg) > 128 * 1024 || (int64_t)T * (256 << log2cg) > (int64_t)XST_MAX * 512)) --log2cg;
  const int max_log2cg = log2cg;
  // With at least one tile per compute unit, chunks small enough for two
  // workgroups per CU (x of a chunk <= 64 KB): at M = 48, q|k|v 23.0 -> 15.7 us,
  // gate|up 40.9 -> 26.3 us and the Q8_0 lm_head 280 -> 165-180 us with
  // 4-group chunks instead of 8. With fewer tiles (o, down: 160) the extra
  // chunk rounds cost more (14.8 -> 18.4 us, 34.8 -> 45.6 us).
  if (tiles >= 256)
    while (log2cg > 0 && x_bytes(log2cg) > 64 * 1024) --log2cg;
  {
    const int v = tune(TUNE_MFMA_CHUNK_L2CG);   // sweeps
    if (v >= 0 && v <= max_log2cg) log2cg = v;
  }
  const int CG = 1 << log2cg;
  int P = maxp < CG ? maxp : CG;
  int S = (CG + P - 1) / P;
  while (S < 8 && P > 1 && tiles * S < 2048) {
    --P;
    S = (CG + P - 1) / P;
  }
  if (S > 8) return c;
  int R = 1;
  const int64_t pieces = (int64_t)T * (256 << log2cg);
  while (pieces > (int64_t)XST_MAX * 64 * R * S && 2 * R * S <= 8) R *= 2;
  while (pieces > (int64_t)XST_MAX * 64 * R * S && R * (S + 1) <= 8 && S < CG) ++S;
  if (pieces > (int64_t)XST_MAX * 64 * R * S) return c;
  const int64_t xb = x_bytes(log2cg), rb = (int64_t)R * S * T * 1024;
  const int64_t lds = xb > rb ? xb : rb;
  if (lds > MFMA_LDS_MAX_BYTES) return c;
  return {R, S, P, log2cg, (size_t)lds, true};
}

template <int FMT, int P, int T>
int launch_mfma_chunk_p(const GemvArgs& a, int m0, int mt, const MfmaChunkCfg& c) {
  const int64_t tiles = (a.N + 15) / 16;
  const unsigned cgroups = (unsigned)((mt + 16 * T - 1) / (16 * T));   // column groups of 16 T along y
  const dim3 grid((unsigned)((tiles + c.R - 1) / c.R), cgroups), block((unsigned)(64 * c.R * c.S));
  dispatch_log("k_gemv_mfma_chunk", a.fmt, a.N, a.K, mt, grid.x, grid.y, block.x, c.lds,
               "T=%d R=%d S=%d P=%d groups/chunk=%d m0=%d", T, c.R, c.S, P, 1 << c.log2cg, m0);
  hipLaunchKernelGGL((k_gemv_mfma_chunk<FMT, P, T>), grid, block, c.lds, a.stream, a.W, a.x + (int64_t)m0 * a.K,
                     a.y + (int64_t)m0 * a.N, (int)a.N, (int)a.K, mt, c.R, c.S, c.log2cg);
  return (int)hipGetLastError();
}

template <int FMT, int T>
int launch_mfma_chunk(const GemvArgs& a, int m0, int mt) {
  const MfmaChunkCfg c = mfma_chunk_cfg(a.N, a.K, T, MfmaChunkMaxP<FMT, T>::v);
  if (!c.ok) return -1;   // not applicable: the caller falls back
  switch (c.P) {
    case 1: return launch_mfma_chunk_p<FMT, 1, T>(a, m0, mt, c);
    case 2: return launch_mfma_chunk_p<FMT, 2, T>(a, m0, mt, c);
    case 3:
      if constexpr (MfmaChunkMaxP<FMT, T>::v >= 3) return launch_mfma_chunk_p<FMT, 3, T>(a, m0, mt, c);
      return (int)hipErrorInvalidValue;
    case 4:
      if constexpr (MfmaChunkMaxP<FMT, T>::v >= 4) return launch_mfma_chunk_p<FMT, 4, T>(a, m0, mt, c);
      return (int)hipErrorInvalidValue;
    case 5:
      if constexpr (MfmaChunkMaxP<FMT, T>::v >= 5) return launch_mfma_chunk_p<FMT, 5, T>(a, m0, mt, c);
      return (int)hipErrorInvalidValue;
    default:
      if constexpr (MfmaChunkMaxP<FMT, T>::v >= 6) return launch_mfma_chunk_p<FMT, 6, T>(a, m0, mt, c);
      return (int)hipErrorInvalidValue;
  }
}

// Persistent waves for many tiles: 8 waves per workgroup, as many workgroups
// as fit at once (up to one wave per tile), tiles dealt evenly: tpw =
// ceil(tiles / waves) (at most MFMA_PERS_TPW), then only as many waves as
// that needs.
template <int FMT, int P, bool SX>
int launch_mfma_pers_p(const GemvArgs& a, int log2mp, size_t lds) {
  static int cus_of[64] = {0};   // compute units per device, looked up once
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
  if (!cus_of[dev] && hipDeviceGetAttribute(&cus_of[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return (int)hipErrorInvalidDevice;
  const int cus = cus_of[dev];
  // waves per workgroup: 8, or fewer (more workgroups, each staging x once)
  // where enough threads remain to stage x
  int nw = 8;
  {
    const int v = tune(TUNE_MFMA_PERS_WAVES);
    if (v >= 1 && v <= 8 && mfma_x_pieces((int)((a.K / 32 + 3) / 4), log2mp) <= (int64_t)XST_MAX * 64 * v) nw = v;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gemv_mfma_pers<FMT, P, SX>, 64 * nw, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int64_t tiles = (a.N + 15) / 16;
  const int64_t max_waves = (int64_t)cus * per_cu * nw;
  int64_t tpw = (tiles + max_waves - 1) / max_waves;
  if (tpw > MFMA_PERS_TPW) tpw = MFMA_PERS_TPW;   // more workgroups than fit at once
  {
    const int v = tune(TUNE_MFMA_PERS_TPW);     // tests: several tiles per wave at any size
    if (v >= 1 && v <= MFMA_PERS_TPW) tpw = v;
  }
  const int64_t waves = (tiles + tpw - 1) / tpw;
  const dim3 grid((unsigned)((waves + nw - 1) / nw)), block((unsigned)(64 * nw));
  dispatch_log("k_gemv_mfma_pers", a.fmt, a.N, a.K, (int)a.M, grid.x, 1, 64 * nw, lds,
               "persistent P=%d tiles/wave=%d Mp=%d", P, (int)tpw, 1 << log2mp);
  hipLaunchKernelGGL((k_gemv_mfma_pers<FMT, P, SX>), grid, block, lds, a.stream, a.W, a.x, a.y, (int)a.N, (int)a.K,
                     (int)a.M, log2mp, (int)tpw, nw, (int)grid.x);
  return (int)hipGetLastError();
}

// Groups in flight per wave. Deeper rings win even where they cost occupancy
// (measured at M = 8 on 151936 x 2560: Q8_0 P = 6 / 8: 95.6 / 94.0 us, Q4_0
// P = 8 / 10: 78.1 / 65.6 us, affine4 P = 8 / 12: 74.1 / 64.8 us).
template <int FMT> struct MfmaPersP {
  static constexpr int v = FMT == F_Q8_0 ? 8 : (FMT == F_AFFINE4 ? 12 : 10);   // 5-bit formats: 6-7 dwords a group
};
// From this many 16-row tiles on, persistent waves (one tile at a time per
// wave) fill the device; below it, tiles are split over the waves of a workgroup.
constexpr int64_t MFMA_PERS_MIN_TILES = 4096;

// Order: persistent waves (many tiles, M <= 16), split-K teams with all of x
// in LDS (M <= 16), K-chunked staging (any M up to 64 per launch), and per-wave
// activation loads as the fallback. The mfma_variant tuning override (tests and sweeps) forces
// one kernel where it applies: "pers", "teams", "teams_sx" (block sums staged
// in LDS instead of an MFMA against ones per block), "chunk" or "direct";
// past 16 columns "chunk_whole" / "chunk_split" force one workgroup per tile
// for all columns / per tile and 16 columns (measured at M = 48: the split
// wins below 256 tiles, o 15.1 -> 12.8 us and down 34.8 -> 24.8 us, and
// loses above, q|k|v 15.6 -> 25.5 us, gate|up 26.2 -> 41.3 us).
template <int FMT>
int launch_mfma_fmt(const GemvArgs& a) {
  const int var = tune(TUNE_MFMA_VARIANT);
  const bool want_direct = var == MV_DIRECT;
  const bool want_pers = var == MV_PERS;
  const bool want_teams = var == MV_TEAMS || var == MV_TEAMS_SX;
  const bool want_chunk = var == MV_CHUNK;
  if (a.M <= 16 && !want_direct) {
    const int64_t tiles = (a.N + 15) / 16;
    const int ngroups = (int)((a.K / 32 + 3) / 4);
    int log2mp = 0;
    while ((1 << log2mp) < a.M) ++log2mp;
    const int64_t pieces = mfma_x_pieces(ngroups, log2mp);
    const int64_t lds = mfma_x_lds_bytes(a.K, log2mp, true);
    if ((tiles >= MFMA_PERS_MIN_TILES || want_pers) && !want_teams && !want_chunk && lds <= MFMA_LDS_MAX_BYTES &&
        pieces <= (int64_t)XST_MAX * 512)
      return launch_mfma_pers_p<FMT, MfmaPersP<FMT>::v, true>(a, log2mp, (size_t)lds);
    if (!want_chunk) {
      // with a workspace, a K split where it pays (also where all of x would
      // not fit one workgroup's LDS)
      // Offset terms from block sums staged in LDS up to 4 columns, from an
      // MFMA against ones beyond (measured on the decode shapes, cold, M = 4:
      // q|k|v 6.62 -> 6.32 us, gate|up 12.29 -> 11.63, down with its K split
      // 10.97 -> 10.83, o 6.22 / 6.24; at 6..16 columns the sums lose, e.g.
      // gate|up 12.46 -> 13.45 at 8). "teams" / "teams_sx" force one way.
      const bool no_sums = !(var == MV_TEAMS_SX || (var != MV_TEAMS && a.M <= 4));
      const int ns = a.ws ? split_count(a) : 1;
      if (ns > 1) {
        const MfmaLdsCfg cs = split_cfg(a, ns, MfmaLdsMaxP<FMT>::v, no_sums);
        if (cs.ok && a.ws_bytes >= (int64_t)ns * a.M * a.N * 4) return launch_mfma_split<FMT>(a, ns, cs);
      }
      const MfmaLdsCfg c = mfma_lds_cfg(a.N, a.K, (int)a.M, MfmaLdsMaxP<FMT>::v, no_sums);
      if (c.ok) return launch_mfma_lds<FMT>(a, 0, (int)a.M, c);
    }
  }
  for (int m0 = 0; m0 < a.M; m0 += 64) {
    const int mt = a.M - m0 < 64 ? a.M - m0 : 64;
    int err = -1;
    if (!want_direct) {
      // Fewer row tiles than compute units: one workgroup per (tile, 16
      // columns) instead of one per tile for all columns, so more CUs work
      // and each stages a third of x at 48 columns. The column groups of a
      // tile land on the same XCD when the grid's x extent is a multiple of
      // 8 (workgroups go to XCDs round-robin) and share its L2 for the
      // tile's weights: down at M = 48 fetches the same bytes past L2 in both
      // layouts (FETCH_SIZE 11.30 MiB per launch).
      const bool split = mt > 16 && ((a.N + 15) / 16 < 256 || var == MV_CHUNK_SPLIT) &&
                         var != MV_CHUNK_WHOLE;
      if (mt <= 16 || split) err = launch_mfma_chunk<FMT, 1>(a, m0, mt);
      else if (mt <= 32) err = launch_mfma_chunk<FMT, 2>(a, m0, mt);
      else if (mt <= 48) err = launch_mfma_chunk<FMT, 3>(a, m0, mt);
      else err = launch_mfma_chunk<FMT, 4>(a, m0, mt);
      if (err == 0) continue;
      if (err != -1) return err;
    }
    if (mt <= 16) err = launch_mfma_t<FMT, 1>(a, m0, mt);
    else if (mt <= 32) err = launch_mfma_t<FMT, 2>(a, m0, mt);
    else if (mt <= 48) err = launch_mfma_t<FMT, 3>(a, m0, mt);
    else err = launch_mfma_t<FMT, 4>(a, m0, mt);
    if (err) return err;
  }
  return 0;
}

// Batch-invariant matrix-core GEMV: every launch configuration is chosen from
// N and K alone, so a column's sum (the groups each wave takes, the order of
// the matrix-core products and scale FMAs, the fixed-order sum over the waves
// of a tile) is the same whatever M is; M only sets how many operand rows hold
// real columns (a matrix-core product's output element depends on its own row
// and column alone). Persistent waves (many tiles: each wave sums a tile's
// groups in order, no split) and the chunked and per-wave kernels (their
// configuration does not involve M) take columns 16 at a time; the split-K
// teams kernel takes them 8 at a time with the configuration it has at 8
// columns (the verify width), staged for as many as are real.
constexpr int INV_TEAMS_COLS = 8;

template <int FMT>
int launch_mfma_invariant_fmt(const GemvArgs& a) {
  const int64_t tiles = (a.N + 15) / 16;
  const int ngroups = (int)((a.K / 32 + 3) / 4);
  const bool pers = tiles >= MFMA_PERS_MIN_TILES && mfma_x_lds_bytes(a.K, 4, true) <= MFMA_LDS_MAX_BYTES &&
                    mfma_x_pieces(ngroups, 4) <= (int64_t)XST_MAX * 512;
  const MfmaLdsCfg teams = mfma_lds_cfg(a.N, a.K, INV_TEAMS_COLS, MfmaLdsMaxP<FMT>::v, true);
  const int width = (!pers && teams.ok) ? INV_TEAMS_COLS : 16;
  for (int m0 = 0; m0 < a.M; m0 += width) {
    const int mt = a.M - m0 < width ? a.M - m0 : width;
    int log2mp = 0;
    while ((1 << log2mp) < mt) ++log2mp;
    int err;
    if (pers) {
      GemvArgs b = a;
      b.x = a.x + (int64_t)m0 * a.K;
      b.y = a.y + (int64_t)m0 * a.N;
      b.M = mt;
      err = launch_mfma_pers_p<FMT, MfmaPersP<FMT>::v, true>(b, log2mp, (size_t)mfma_x_lds_bytes(a.K, log2mp, true));
    } else if (teams.ok) {
      MfmaLdsCfg c = teams;
      c.log2mp = log2mp;
      const int64_t xb = mfma_x_lds_bytes(a.K, log2mp, c.sx), rb = (int64_t)c.R * c.S * 64 * 16;
      c.lds = (size_t)(xb > rb ? xb : rb);
      err = launch_mfma_lds<FMT>(a, m0, mt, c);
    } else {
      err = launch_mfma_chunk<FMT, 1>(a, m0, mt);
      if (err == -1) err = launch_mfma_t<FMT, 1>(a, m0, mt);
    }
    if (err) return err;
  }
  return 0;
}

}  // namespace

int launch_gemv_mfma_invariant(const GemvArgs& a) {
  switch (a.fmt) {
    case KQ_Q8_0: return launch_mfma_invariant_fmt<F_Q8_0>(a);
    case KQ_Q4_0: return launch_mfma_invariant_fmt<F_Q4_0>(a);
    case KQ_Q5_0: return launch_mfma_invariant_fmt<F_Q5_0>(a);
    case KQ_Q5_1: return launch_mfma_invariant_fmt<F_Q5_1>(a);
    default: return launch_mfma_invariant_fmt<F_AFFINE4>(a);
  }
}

int64_t gemv_split_bytes(const GemvArgs& a) {
  // the splits the matrix-core path would take with a workspace (the teams
  // kernel applies, its split configuration fits)
  if (a.M < 4 || a.M > 16 || a.N < 1) return 0;
  const int64_t tiles = (a.N + 15) / 16;
  if (tiles >= MFMA_PERS_MIN_TILES) return 0;
  GemvArgs b = a;
  b.ws = reinterpret_cast<void*>(1);
  const int ns = split_count(b);
  if (ns <= 1) return 0;
  const int maxp = a.fmt == KQ_Q8_0 ? MfmaLdsMaxP<F_Q8_0>::v : MfmaLdsMaxP<F_AFFINE4>::v;
  if (!split_cfg(a, ns, maxp, true).ok) return 0;
  return (int64_t)ns * a.M * a.N * 4;
}

int launch_gemv_mfma(const GemvArgs& a) {
  switch (a.fmt) {
    case KQ_Q8_0: return launch_mfma_fmt<F_Q8_0>(a);
    case KQ_Q4_0: return launch_mfma_fmt<F_Q4_0>(a);
    case KQ_Q5_0: return launch_mfma_fmt<F_Q5_0>(a);
    case KQ_Q5_1: return launch_mfma_fmt<F_Q5_1>(a);
    default: return launch_mfma_fmt<F_AFFINE4>(a);
  }
}

}  // namespace kq
