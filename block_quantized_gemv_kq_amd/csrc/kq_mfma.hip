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
// Work split: a workgroup owns 16 weight rows; its 8 waves split K into
// contiguous ranges of 4-block groups and sum their partial results in LDS in
// a fixed order (deterministic). A lane (n = lane % 16, g = lane / 16) loads
// block b0 + g of row n, then four lanes exchange 16-lane groups with
// permlane swaps so that lane group g holds quant dword g of all four blocks:
// the MFMA's 32 k of a block are, for lane group g, the elements 4g..4g+3 and
// 16+4g..19+4g (both nibbles of byte 4g..4g+3), and the activations use the
// same order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_dev.h"
#include "kq_internal.h"

namespace kqd {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int MF_WAVES = 8;

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

// byte offset of block `blk` of the row at `roff`
template <int FMT>
__device__ __forceinline__ void load_group(rsrc_t rs, uint32_t roff, int blk, bool valid, GroupRaw<FMT>& r) {
  const uint32_t off = roff + (uint32_t)blk * Fmt<FMT>::BB;
  if constexpr (FMT == F_AFFINE4) {
    const uint32_t o = valid ? off : OOB;
    const u32x4 t = ld128(rs, o);
    r.D[0] = t.x; r.D[1] = t.y; r.D[2] = t.z; r.D[3] = t.w;
    r.D[4] = ld32(rs, o + 16);
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
    } else {
      const u32x4 u = ld128(rs, o + 16);
      r.D[5] = u.x; r.D[6] = u.y; r.D[7] = u.z; r.D[8] = u.w;
      r.D[9] = ld32(rs, o + 32);
    }
  }
}

// Activations of one 4-block group for one 16-column tile: for block j the
// lane's A operand is x[col][32 b + 4g .. 4g+3] and x[col][32 b + 16 + 4g .. +3].
struct GroupX {
  u32x2 lo[4], hi[4];
};

__device__ __forceinline__ void load_group_x(const uint16_t* __restrict__ xcol, bool col_ok, int b0,
                                             int nblk, int g, GroupX& gx) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = b0 + j;
    if (col_ok && b < nblk) {
      const u32x2* p = reinterpret_cast<const u32x2*>(xcol + 32 * b + 4 * g);
      gx.lo[j] = p[0];
      gx.hi[j] = p[4];   // + 16 elements
    } else {
      gx.lo[j] = u32x2{0u, 0u};
      gx.hi[j] = u32x2{0u, 0u};
    }
  }
}

template <int FMT, int T>
__global__ __launch_bounds__(64 * MF_WAVES) void k_gemv_mfma(const uint8_t* __restrict__ W,
                                                            const uint16_t* __restrict__ x,
                                                            float* __restrict__ y, int N, int K, int M) {
  __shared__ float4_t red[MF_WAVES][T][64];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int nblk = K / 32;
  const int ngroups = (nblk + 3) / 4;
  const int gb = ngroups * wave / MF_WAVES, ge = ngroups * (wave + 1) / MF_WAVES;
  const uint32_t row_bytes = (uint32_t)nblk * Fmt<FMT>::BB;
  const int valid_rows = (int)min<int64_t>(16, N - row0);
  // Range rounded up to whole dwords: Q4_0/Q8_0 blocks are only 2-byte
  // aligned, so the last block's final dword may hang 2 bytes past the end
  // (same dword, same page).
  const rsrc_t rs = make_rsrc(W + row0 * row_bytes, ((uint32_t)valid_rows * row_bytes + 3u) & ~3u);
  const uint32_t roff = (uint32_t)n * row_bytes;
  const bool row_ok = n < valid_rows;

  const uint16_t* xc[T];
  bool col_ok[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int col = 16 * t + n;
    col_ok[t] = col < M;
    xc[t] = x + (int64_t)(col_ok[t] ? col : 0) * K;
  }

  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  const half8_t ones = as_half8(ONES, ONES, ONES, ONES);

  GroupRaw<FMT> cur, nxt;
  GroupX cx[T], nx[T];
  if (gb < ge) {
    load_group<FMT>(rs, roff, 4 * gb + g, row_ok && 4 * gb + g < nblk, cur);
#pragma unroll
    for (int t = 0; t < T; ++t) load_group_x(xc[t], col_ok[t], 4 * gb, nblk, g, cx[t]);
  }
  for (int gi = gb; gi < ge; ++gi) {
    if (gi + 1 < ge) {
      load_group<FMT>(rs, roff, 4 * (gi + 1) + g, row_ok && 4 * (gi + 1) + g < nblk, nxt);
#pragma unroll
      for (int t = 0; t < T; ++t) load_group_x(xc[t], col_ok[t], 4 * (gi + 1), nblk, g, nx[t]);
    }
    // ---- this lane's block (b0 + g): scale/bias and quant dwords, then
    // exchange so lane group g holds quant dword(s) g of blocks b0..b0+3
    uint32_t hdr, q0, q1, q2, q3, p0 = 0, p1 = 0, p2 = 0, p3 = 0;
    if constexpr (FMT == F_AFFINE4) {
      hdr = cur.D[0];
      q0 = cur.D[1]; q1 = cur.D[2]; q2 = cur.D[3]; q3 = cur.D[4];
    } else {
      const uint32_t r2 = ((roff + (uint32_t)(4 * gi + g) * Fmt<FMT>::BB + 2u) & 3u) * 8u;  // bit shift 0/16
      hdr = r2 ? (cur.D[1] & 0xffffu) : (cur.D[0] >> 16);
      const uint32_t sh = r2 >> 3;   // byte shift 0 or 2
      q0 = __builtin_amdgcn_alignbyte(cur.D[2], cur.D[1], sh);
      q1 = __builtin_amdgcn_alignbyte(cur.D[3], cur.D[2], sh);
      q2 = __builtin_amdgcn_alignbyte(cur.D[4], cur.D[3], sh);
      q3 = __builtin_amdgcn_alignbyte(cur.D[5], cur.D[4], sh);
      if constexpr (FMT == F_Q8_0) {
        p0 = __builtin_amdgcn_alignbyte(cur.D[6], cur.D[5], sh);
        p1 = __builtin_amdgcn_alignbyte(cur.D[7], cur.D[6], sh);
        p2 = __builtin_amdgcn_alignbyte(cur.D[8], cur.D[7], sh);
        p3 = __builtin_amdgcn_alignbyte(cur.D[9], cur.D[8], sh);
      }
    }
    transpose4(q0, q1, q2, q3);
    if constexpr (FMT == F_Q8_0) transpose4(p0, p1, p2, p3);
    uint32_t h0 = hdr, h1 = hdr, h2 = hdr, h3 = hdr;
    transpose4(h0, h1, h2, h3);
    const uint32_t qs[4] = {q0, q1, q2, q3};
    const uint32_t ps[4] = {p0, p1, p2, p3};
    const uint32_t hs[4] = {h0, h1, h2, h3};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (4 * gi + j >= nblk) break;      // uniform
      // B operand: 8 fp16 (offset + q) for elements {4g..4g+3, 16+4g..19+4g}
      uint32_t b0, b1, b2, b3;
      if constexpr (FMT == F_Q8_0) {
        const uint32_t u = qs[j] ^ 0x80808080u, v = ps[j] ^ 0x80808080u;
        b0 = perm(MAGIC, u, SEL_LO); b1 = perm(MAGIC, u, SEL_HI);
        b2 = perm(MAGIC, v, SEL_LO); b3 = perm(MAGIC, v, SEL_HI);
      } else {
        const uint32_t lo = qs[j] & 0x0F0F0F0Fu, hi = (qs[j] >> 4) & 0x0F0F0F0Fu;
        b0 = perm(MAGIC, lo, SEL_LO); b1 = perm(MAGIC, lo, SEL_HI);
        b2 = perm(MAGIC, hi, SEL_LO); b3 = perm(MAGIC, hi, SEL_HI);
      }
      const half8_t B = as_half8(b0, b1, b2, b3);
      const float sc = h2f(hs[j]);
      float c;
      if constexpr (FMT == F_AFFINE4) c = __builtin_fmaf(-1024.0f, sc, h2f(hs[j] >> 16));
      else if constexpr (FMT == F_Q4_0) c = -1032.0f * sc;
      else c = -1152.0f * sc;
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
    if (gi + 1 < ge) {
      cur = nxt;
#pragma unroll
      for (int t = 0; t < T; ++t) cx[t] = nx[t];
    }
  }
  // fixed-order sum of the 8 waves' partial results
#pragma unroll
  for (int t = 0; t < T; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float4_t s = red[0][t][lane];
#pragma unroll
      for (int w = 1; w < MF_WAVES; ++w) {
        const float4_t o = red[w][t][lane];
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

}  // namespace kqd

namespace kq {

using namespace kqd;

namespace {

template <int FMT, int T>
int launch_mfma_t(const GemvArgs& a, int m0, int mt) {
  const dim3 grid((unsigned)((a.N + 15) / 16)), block(64 * MF_WAVES);
  hipLaunchKernelGGL((k_gemv_mfma<FMT, T>), grid, block, 0, a.stream, a.W, a.x + (int64_t)m0 * a.K,
                     a.y + (int64_t)m0 * a.N, (int)a.N, (int)a.K, mt);
  return (int)hipGetLastError();
}

template <int FMT>
int launch_mfma_fmt(const GemvArgs& a) {
  for (int m0 = 0; m0 < a.M; m0 += 64) {
    const int mt = a.M - m0 < 64 ? a.M - m0 : 64;
    int err;
    if (mt <= 16) err = launch_mfma_t<FMT, 1>(a, m0, mt);
    else if (mt <= 32) err = launch_mfma_t<FMT, 2>(a, m0, mt);
    else if (mt <= 48) err = launch_mfma_t<FMT, 3>(a, m0, mt);
    else err = launch_mfma_t<FMT, 4>(a, m0, mt);
    if (err) return err;
  }
  return 0;
}

}  // namespace

int launch_gemv_mfma(const GemvArgs& a) {
  switch (a.fmt) {
    case KQ_Q8_0: return launch_mfma_fmt<F_Q8_0>(a);
    case KQ_Q4_0: return launch_mfma_fmt<F_Q4_0>(a);
    default: return launch_mfma_fmt<F_AFFINE4>(a);
  }
}

}  // namespace kq
