// kq_shortlist.hip — Shortlist: the greedy argmax over a Q8_0 output layer
// computed from a bound copy, with exact scores only for the rows the bounds
// cannot rule out (Kinetic docs, "What makes it fast": picking the next token
// reads an output layer of up to a quarter of a million rows; a small copy
// bounds every row's score, and only rows that can still win are scored
// exactly).
//
// Each int8 quant splits as q = 8 (v - 16) + ql, v = floor(q / 8) + 16 in
// 0..31, ql in 0..7. The bound copy keeps the block scales d and v (as Q5_0
// nibbles and fifth bits), 22 of the 34 bytes of a Q8_0 block, and per row
// E, the least fp32 >= the 2-norm of the row's error d (ql - 3.5). With x the
// activation column:
//   yhat = sum_b d_b (8 sum_j (v_j - 16) x_j + 3.5 sum_j x_j)
//   |y - yhat| <= E ||x||_2                                (Cauchy-Schwarz)
//   u = yhat + r + s >= y >= l = yhat - r - s,  r = E ||x||_2,
//   s = T / 4 + r / 256 + 2^-80,  T = sum_b |d_b| sum_j |x_j|
// s covers fp32 rounding in yhat and in the exact scores: below 0.05 T
// together for K <= 16384 (the derivation is with the interface in kq.h).
//
// Four launches:
//   k_sl_bound  reads the bound copy: u per row, and each workgroup's largest
//               (l, row) key;
//   k_sl_pivot  one workgroup: the row c with the largest l, and its exact
//               score y_c (tau);
//   k_sl_exact  rows with u >= tau (NaN-safe: every row not shown to be below
//               tau) get their exact scores, each workgroup's best key;
//   k_sl_final  the best key over the workgroups: the index (and the count of
//               rows scored exactly).
// Exact scores run the one-column GEMV kernel's per-row arithmetic with its
// configuration for this N and K (lane-group size, units per lane, passes,
// the same x staging and block sums), so each score has the bits kq_gemv
// gives that row and the index is kq_gemv_argmax's. Every row left out scores
// below row c (u is an upper bound on its exact score), so the answer is the
// argmax over all rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_dev.h"
#include "kq_internal.h"

namespace kqd {

constexpr int SL_UB = 4;          // blocks per load unit of the bound copy
constexpr int SL_WPG = 4;         // waves per workgroup (bound and exact kernels)
// x in LDS with an idle 16-byte piece after each load unit's pieces (no LDS
// bank conflicts between lane groups): 16 pieces per bound-copy unit, 8 per
// Q8_0 unit of the exact scores
constexpr int SL_XUP = 4 * SL_UB;
constexpr int Q8_XUP = 4 * Fmt<F_Q8_0>::UB;

// Pivot record in the workspace: tau = exact score of row c (NaN: keep every row).
struct SlPivot {
  float tau;
  int32_t row;
};

// One load unit of a bound-copy row: 4 block scales, 4 fifth-bit words, 4
// blocks of nibbles.
struct SlUnit {
  uint32_t d[2];
  uint32_t f[4];
  uint32_t n[16];
};

template <int ITERS>
__device__ __forceinline__ void sl_issue(rsrc_t rs, uint32_t roff, int nb, int first, int G, int units,
                                         SlUnit (&w)[ITERS]) {
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int u = first + it * G;
    const bool ok = u < units;
    const uint32_t od = ok ? roff + 8u * (uint32_t)u : OOB;
    const uint32_t of = ok ? roff + 2u * (uint32_t)nb + 16u * (uint32_t)u : OOB;
    const uint32_t on = ok ? roff + 6u * (uint32_t)nb + 64u * (uint32_t)u : OOB;
    const u32x2v d = __builtin_amdgcn_raw_buffer_load_b64(rs, od, 0, 0);
    w[it].d[0] = d.x;
    w[it].d[1] = d.y;
    const u32x4 f = ld128(rs, of);
    w[it].f[0] = f.x; w[it].f[1] = f.y; w[it].f[2] = f.z; w[it].f[3] = f.w;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x4 t = ld128(rs, on + 16u * (uint32_t)p);
      w[it].n[4 * p] = t.x; w[it].n[4 * p + 1] = t.y; w[it].n[4 * p + 2] = t.z; w[it].n[4 * p + 3] = t.w;
    }
  }
}

// Four bits b0..b3 (bits pos..pos+3 of w) as bit 4 of four bytes: one
// 24-bit multiply places bit k at bit 7k, the mask keeps it, the shift moves
// it to bit 4 of byte k.
__device__ __forceinline__ uint32_t fifth_bytes(uint32_t w, int pos) {
  return ((__builtin_amdgcn_ubfe(w, (uint32_t)pos, 4u) * 0x00204081u) & 0x01010101u) << 4;
}

// Sum over the lane's units: acc += d sum_j (v_j - 16) x_j, C += d sum_j x_j,
// T += |d| sum_j |x_j|, per block. v goes into bytes (nibble | fifth bit << 4)
// before the magic-exponent permutes, so each fp16 half is 1024 + v and one
// fix-up -1040 sum x per block removes the offset.
template <int ITERS>
__device__ __forceinline__ void sl_consume(const SlUnit (&w)[ITERS], const uint32_t* xl, const float* xs,
                                           const float* xa, int first, int G, int units, float& acc, float& C,
                                           float& T) {
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int u = first + it * G;
    if (u < units) {
#pragma unroll
      for (int t = 0; t < SL_UB; ++t) {
        const int b = SL_UB * u + t;
        const uint32_t qh = w[it].f[t];
        uint32_t A[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t nb4 = w[it].n[4 * t + i];
          const uint32_t lo = (nb4 & 0x0F0F0F0Fu) | fifth_bytes(qh, 4 * i);        // elements 4i .. 4i+3
          const uint32_t hi = ((nb4 >> 4) & 0x0F0F0F0Fu) | fifth_bytes(qh, 16 + 4 * i);  // 16+4i .. 19+4i
          A[2 * i] = perm(MAGIC, lo, SEL_LO);
          A[2 * i + 1] = perm(MAGIC, lo, SEL_HI);
          A[8 + 2 * i] = perm(MAGIC, hi, SEL_LO);
          A[9 + 2 * i] = perm(MAGIC, hi, SEL_HI);
        }
        const u32x4* xp = reinterpret_cast<const u32x4*>(xl) + xphys<SL_XUP>(4 * b);
        float dot = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x4 q = xp[v];
          dot = dot2(A[4 * v], q.x, dot);
          dot = dot2(A[4 * v + 1], q.y, dot);
          dot = dot2(A[4 * v + 2], q.z, dot);
          dot = dot2(A[4 * v + 3], q.w, dot);
        }
        const float2 sx = reinterpret_cast<const float2*>(xs)[b];
        const float sxb = sx.x + sx.y;
        const float d = h2f(w[it].d[t >> 1] >> (16 * (t & 1)));
        acc = __builtin_fmaf(d, __builtin_fmaf(-1040.0f, sxb, dot), acc);
        C = __builtin_fmaf(d, sxb, C);
        T = __builtin_fmaf(__builtin_fabsf(d), xa[b], T);
      }
    }
  }
}

// x (one column, K halves) in registers: XCH 16-byte pieces for each of NT
// threads (NT * XCH * 8 >= K). Issued ahead of the weight loads, so that
// writing x to LDS waits for x alone.
template <int XCH, int NT>
__device__ __forceinline__ void sl_x_load(const uint16_t* __restrict__ x, int K, u32x4 (&xr)[XCH]) {
  const int n16 = K / 8;
  const u32x4* src = reinterpret_cast<const u32x4*>(x);
#pragma unroll
  for (int c = 0; c < XCH; ++c) {
    const int i = (int)threadIdx.x + NT * c;
    xr[c] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
  }
}

// x from registers into LDS at xl, then the half-block sums xs as the
// one-column GEMV kernel forms them; with ABS also the per-block sums of |x|
// (xa) and ||x||_2 (returned, the same value in every thread; s_red holds
// NT / 64 floats). Two barriers.
template <int XCH, int NT, bool ABS, int UP>
__device__ __forceinline__ float sl_x_store(const u32x4 (&xr)[XCH], int K, uint32_t* xl, float* xs, float* xa,
                                            float* s_red) {
  const int n16 = K / 8;
  u32x4* xl4 = reinterpret_cast<u32x4*>(xl);
  float sq = 0.0f;
#pragma unroll
  for (int c = 0; c < XCH; ++c) {
    const int i = (int)threadIdx.x + NT * c;
    if (i < n16) xl4[xphys<UP>(i)] = xr[c];
    if constexpr (ABS) {   // pieces past K are zero
      sq = dot2(xr[c].x, xr[c].x, sq);
      sq = dot2(xr[c].y, xr[c].y, sq);
      sq = dot2(xr[c].z, xr[c].z, sq);
      sq = dot2(xr[c].w, xr[c].w, sq);
    }
  }
  __syncthreads();
  block_sums_to_lds<UP>(xl, K / 2, 1, xs, NT);
  float nrm = 0.0f;
  if constexpr (ABS) {
    const int nb = K / 32;
    for (int b = (int)threadIdx.x; b < nb; b += NT) {
      const u32x4* p = xl4 + xphys<UP>(4 * b);
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const u32x4 q = p[v];
        s = dot2(q.x & 0x7fff7fffu, ONES, s);
        s = dot2(q.y & 0x7fff7fffu, ONES, s);
        s = dot2(q.z & 0x7fff7fffu, ONES, s);
        s = dot2(q.w & 0x7fff7fffu, ONES, s);
      }
      xa[b] = s;
    }
    sq = group_sum(sq, 64);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = sq;
  }
  __syncthreads();
  if constexpr (ABS) {
    float t = s_red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) t += s_red[w];
    nrm = __builtin_sqrtf(t);
  }
  return nrm;
}

// The workgroup's largest key: an LDS 64-bit atomic max per contribution,
// then every thread reads it after a barrier. `key` 0 contributes nothing.
__device__ __forceinline__ unsigned long long wg_max_key(unsigned long long key, unsigned long long* s_key) {
  if (key) atomicMax(s_key, key);
  __syncthreads();
  return *s_key;
}

template <int ITERS, int XCH>
__global__ __launch_bounds__(256) void k_sl_bound(const uint8_t* __restrict__ Wc, const uint16_t* __restrict__ x,
                                                  float* __restrict__ u, unsigned long long* __restrict__ part,
                                                  int N, int K, int log2g, int passes) {
  extern __shared__ u32x4 sl_lds[];
  uint32_t* xl = reinterpret_cast<uint32_t*>(sl_lds);
  const int nb = K / 32;
  float* xs = reinterpret_cast<float*>(xl + 4 * xrun_pieces<SL_XUP>(K / 8));
  float* xa = xs + 2 * nb;
  __shared__ float s_red[SL_WPG];
  __shared__ unsigned long long s_key;
  if (threadIdx.x == 0) s_key = 0ull;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * SL_WPG + wave_id();
  const int G = 1 << log2g;
  const int rpw = 64 >> log2g;
  const int64_t row_base = (int64_t)wave * rpw;
  const uint32_t row_bytes = 22u * (uint32_t)nb;
  const int units = nb / SL_UB;
  const int valid = row_base < N ? (int)min<int64_t>(rpw, N - row_base) : 0;
  const rsrc_t rs = make_rsrc(Wc + (valid ? row_base * row_bytes : 0), (uint32_t)valid * row_bytes);
  const int rho = lane >> log2g;
  const int g = lane & (G - 1);
  const uint32_t roff = (uint32_t)rho * row_bytes;
  const bool own = g == 0 && rho < valid;
  // x and the row norms (stored after all rows) go ahead of the weights
  u32x4 xr[XCH];
  sl_x_load<XCH, 256>(x, K, xr);
  const float* En = reinterpret_cast<const float*>(Wc + (int64_t)N * row_bytes);
  const float e = own ? En[row_base + rho] : 0.0f;
  __builtin_amdgcn_sched_barrier(0);
  SlUnit w[ITERS];
  sl_issue<ITERS>(rs, roff, nb, g, G, units, w);
  __builtin_amdgcn_sched_barrier(0);
  const float xnorm = sl_x_store<XCH, 256, true, SL_XUP>(xr, K, xl, xs, xa, s_red);
  float acc = 0.0f, C = 0.0f, T = 0.0f;
  const int span = G * ITERS;
  for (int p = 0;;) {
    sl_consume<ITERS>(w, xl, xs, xa, p * span + g, G, units, acc, C, T);
    if (++p >= passes) break;
    sl_issue<ITERS>(rs, roff, nb, p * span + g, G, units, w);
  }
  acc = group_sum(acc, G);
  C = group_sum(C, G);
  T = group_sum(T, G);
  unsigned long long key = 0ull;
  if (own) {
    const float yhat = __builtin_fmaf(8.0f, acc, 3.5f * C);
    const float r = e * xnorm;
    const float s = __builtin_fmaf(0.25f, T, __builtin_fmaf(0.00390625f, r, 0x1p-80f));
    const int32_t row = (int32_t)(row_base + rho);
    u[row] = (yhat + r) + s;
    key = best_key((yhat - r) - s, row);
  }
  const unsigned long long k = wg_max_key(key, &s_key);
  if (threadIdx.x == 0) part[blockIdx.x] = k;
}

// Exact score of one Q8_0 row with the one-column GEMV kernel's per-row
// arithmetic, from x and xs in LDS, after issue_units of the row's first pass
// into w (roff OOB: a lane group with no row, its score is not used). The
// value is in every lane of the group.
template <int ITERS>
__device__ __forceinline__ float q8_row_finish(Loaded<F_Q8_0, ITERS>& w, rsrc_t rs, uint32_t roff, const uint32_t* xl,
                                               const float* xs, int K, int g, int G, int passes) {
  const int units = K / 64;
  float acc[1] = {0.0f};
  const int span = G * ITERS;
  for (int p = 0;;) {
    consume_units<F_Q8_0, 1, ITERS, true>(w, xl, xs, K / 2, p * span + g, G, units, acc);
    if (++p >= passes) break;
    issue_units<F_Q8_0, ITERS>(rs, roff, p * span + g, G, units, w);
  }
  group_reduce<1>(acc, G);
  return acc[0];
}

constexpr int SL_PIVOT_NT = 512;    // threads of the pivot kernel (registers for 5 units per lane)
constexpr int SL_PIVOT_XCH = 4;     // K up to 16384
constexpr int SL_PIVOT_KEYS = 16;   // partial keys per thread and round, loaded together (8192 per round)
constexpr int SL_KEYS = 8;          // the same for the final kernel (2048 per round)

template <int ITERS>
__global__ __launch_bounds__(SL_PIVOT_NT) void k_sl_pivot(const uint8_t* __restrict__ W,
                                                          const uint16_t* __restrict__ x,
                                                          const unsigned long long* __restrict__ part,
                                                          int nparts, SlPivot* __restrict__ pv, int N, int K,
                                                          int log2g, int passes) {
  extern __shared__ u32x4 sl_lds[];
  uint32_t* xl = reinterpret_cast<uint32_t*>(sl_lds);
  float* xs = reinterpret_cast<float*>(xl + 4 * xrun_pieces<Q8_XUP>(K / 8));
  __shared__ unsigned long long s_key;
  if (threadIdx.x == 0) s_key = 0ull;
  u32x4 xr[SL_PIVOT_XCH];
  sl_x_load<SL_PIVOT_XCH, SL_PIVOT_NT>(x, K, xr);
  unsigned long long k = 0ull;
  for (int base = 0; base < nparts; base += SL_PIVOT_NT * SL_PIVOT_KEYS) {
    unsigned long long v[SL_PIVOT_KEYS];
#pragma unroll
    for (int j = 0; j < SL_PIVOT_KEYS; ++j) {
      const int i = base + (int)threadIdx.x + SL_PIVOT_NT * j;
      v[j] = i < nparts ? part[i] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < SL_PIVOT_KEYS; ++j) k = v[j] > k ? v[j] : k;
  }
  sl_x_store<SL_PIVOT_XCH, SL_PIVOT_NT, false, Q8_XUP>(xr, K, xl, xs, nullptr, nullptr);
  k = wg_max_key(k, &s_key);
  if (threadIdx.x >= 64) return;
  const Best b = best_of_key(k);
  const bool has = k != 0ull && b.i >= 0 && b.i < N;
  const uint32_t row_bytes = (uint32_t)(K / 32) * 34u;
  const rsrc_t rs = make_rsrc(W + (has ? (int64_t)b.i * row_bytes : 0), has ? row_bytes : 0u);
  const int G = 1 << log2g;
  const int g = (int)threadIdx.x & (G - 1);
  Loaded<F_Q8_0, ITERS> w;
  issue_units<F_Q8_0, ITERS>(rs, 0u, g, G, K / 64, w);
  const float yc = q8_row_finish<ITERS>(w, rs, 0u, xl, xs, K, g, G, passes);
  if (threadIdx.x == 0) {
    pv->tau = has ? yc : __builtin_nanf("");
    pv->row = has ? b.i : -1;
  }
}

template <int ITERS, int XCH>
__global__ __launch_bounds__(256) void k_sl_exact(const uint8_t* __restrict__ W, const uint16_t* __restrict__ x,
                                                  const float* __restrict__ u, const SlPivot* __restrict__ pv,
                                                  unsigned long long* __restrict__ part, int32_t* __restrict__ cnt,
                                                  int N, int K, int log2g, int passes) {
  extern __shared__ u32x4 sl_lds[];
  uint32_t* xl = reinterpret_cast<uint32_t*>(sl_lds);
  float* xs = reinterpret_cast<float*>(xl + 4 * xrun_pieces<Q8_XUP>(K / 8));
  __shared__ unsigned long long s_key;
  __shared__ int32_t s_cnt;
  if (threadIdx.x == 0) {
    s_key = 0ull;
    s_cnt = 0;
  }
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * SL_WPG + wave_id()) * 64;
  const int64_t r = row0 + lane;
  const float ur = r < N ? u[r] : 0.0f;
  u32x4 xr[XCH];
  sl_x_load<XCH, 256>(x, K, xr);
  const float tau = pv->tau;
  const bool keep = r < N && !(ur < tau);
  uint64_t mask = __ballot(keep);
  if (!__syncthreads_or(keep)) {
    if (threadIdx.x == 0) {
      part[blockIdx.x] = 0ull;
      cnt[blockIdx.x] = 0;
    }
    return;
  }
  if (lane == 0 && mask) atomicAdd(&s_cnt, (int32_t)__builtin_popcountll(mask));
  const int G = 1 << log2g;
  const int R = 64 >> log2g;
  const int rho = lane >> log2g;
  const int g = lane & (G - 1);
  const uint32_t row_bytes = (uint32_t)(K / 32) * 34u;
  const int units = K / 64;
  const rsrc_t rs = make_rsrc(W, (uint32_t)N * row_bytes);
  // Rounds of up to R kept rows (one per lane group; the mask is the same in
  // every lane). The first round's loads go out before x is written to LDS.
  auto next_row = [&](int64_t* row) {
    uint64_t m = mask;
    for (int i = 0; i < rho; ++i) m &= m - 1;
    for (int i = 0; i < R; ++i) mask &= mask - 1;
    *row = m ? row0 + __builtin_ctzll(m) : -1;
  };
  int64_t row;
  next_row(&row);
  Loaded<F_Q8_0, ITERS> w;
  uint32_t roff = row >= 0 ? (uint32_t)row * row_bytes : OOB;
  issue_units<F_Q8_0, ITERS>(rs, roff, g, G, units, w);
  sl_x_store<XCH, 256, false, Q8_XUP>(xr, K, xl, xs, nullptr, nullptr);
  unsigned long long best = 0ull;
  for (;;) {
    const float y = q8_row_finish<ITERS>(w, rs, roff, xl, xs, K, g, G, passes);
    if (row >= 0 && g == 0) {
      const unsigned long long k = best_key(y, (int32_t)row);
      best = k > best ? k : best;
    }
    if (!mask) break;
    next_row(&row);
    roff = row >= 0 ? (uint32_t)row * row_bytes : OOB;
    issue_units<F_Q8_0, ITERS>(rs, roff, g, G, units, w);
  }
  const unsigned long long k = wg_max_key(best, &s_key);
  if (threadIdx.x == 0) {
    part[blockIdx.x] = k;
    cnt[blockIdx.x] = s_cnt;
  }
}

__global__ __launch_bounds__(256) void k_sl_final(const unsigned long long* __restrict__ part,
                                                  const int32_t* __restrict__ cnt, int nparts,
                                                  int32_t* __restrict__ out, int32_t* __restrict__ kept) {
  __shared__ unsigned long long s_key;
  __shared__ int32_t s_cnt;
  if (threadIdx.x == 0) {
    s_key = 0ull;
    s_cnt = 0;
  }
  unsigned long long k = 0ull;
  int32_t c = 0;
  for (int base = 0; base < nparts; base += 256 * SL_KEYS) {
    unsigned long long v[SL_KEYS];
    int32_t n[SL_KEYS];
#pragma unroll
    for (int j = 0; j < SL_KEYS; ++j) {
      const int i = base + (int)threadIdx.x + 256 * j;
      v[j] = i < nparts ? part[i] : 0ull;
      n[j] = i < nparts ? cnt[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < SL_KEYS; ++j) {
      k = v[j] > k ? v[j] : k;
      c += n[j];
    }
  }
  __syncthreads();   // the initial values above are written
  if (c) atomicAdd(&s_cnt, c);
  k = wg_max_key(k, &s_key);
  if (threadIdx.x == 0) {
    const Best b = best_of_key(k);
    out[0] = k == 0ull ? 0 : b.i;
    if (kept) kept[0] = s_cnt;
  }
}

}  // namespace kqd

namespace kq {

using namespace kqd;

namespace {

int ilog2i(int v) {
  int l = 0;
  while ((1 << (l + 1)) <= v) ++l;
  return l;
}

struct SlCfg {
  int log2g, iters, passes;   // bound kernel
  int64_t parts1, parts2;     // workgroups of the bound and exact kernels
  RowCfg q8;                  // per-row configuration of the exact scores
};

SlCfg sl_cfg(int64_t N, int64_t K) {
  SlCfg c;
  const int units = (int)(K / 128);
  int G = 1;
  while (G < 64 && (units + G - 1) / G > 5) G <<= 1;   // at most 5 units (440 bytes) per lane
  const int tg = tune(TUNE_SL_G);
  if (tg == 1 || tg == 2 || tg == 4 || tg == 8 || tg == 16 || tg == 32 || tg == 64) G = tg;
  int iters = (units + G - 1) / G;
  if (iters > 5) iters = 5;
  c.log2g = ilog2i(G);
  c.iters = iters;
  c.passes = (units + G * iters - 1) / (G * iters);
  const int64_t rows_per_wg = (int64_t)SL_WPG * (64 / G);
  c.parts1 = (N + rows_per_wg - 1) / rows_per_wg;
  c.parts2 = (N + 64 * SL_WPG - 1) / (64 * SL_WPG);
  c.q8 = q8_row_cfg(N, K);
  return c;
}

int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

struct SlWs {
  float* u;
  unsigned long long* part1;
  SlPivot* pv;
  unsigned long long* part2;
  int32_t* cnt;
  int64_t bytes;
};

SlWs sl_ws(void* base, int64_t N, const SlCfg& c) {
  uint8_t* b = static_cast<uint8_t*>(base);
  SlWs w;
  int64_t off = 0;
  w.u = reinterpret_cast<float*>(b + off);
  off = align256(off + 4 * N);
  w.part1 = reinterpret_cast<unsigned long long*>(b + off);
  off = align256(off + 8 * c.parts1);
  w.pv = reinterpret_cast<SlPivot*>(b + off);
  off = align256(off + (int64_t)sizeof(SlPivot));
  w.part2 = reinterpret_cast<unsigned long long*>(b + off);
  off = align256(off + 8 * c.parts2);
  w.cnt = reinterpret_cast<int32_t*>(b + off);
  off = align256(off + 4 * c.parts2);
  w.bytes = off;
  return w;
}

template <int IT, int XCH>
int launch_bound_it(const ShortlistArgs& a, const SlCfg& c, const SlWs& w, size_t lds) {
  hipLaunchKernelGGL((k_sl_bound<IT, XCH>), dim3((unsigned)c.parts1), dim3(256), lds, a.stream, a.Wc, a.x, w.u,
                     w.part1, (int)a.N, (int)a.K, c.log2g, c.passes);
  return (int)hipGetLastError();
}

template <int IT, int XCH>
int launch_exact_it(const ShortlistArgs& a, const SlCfg& c, const SlWs& w, size_t lds) {
  hipLaunchKernelGGL((k_sl_pivot<IT>), dim3(1), dim3(SL_PIVOT_NT), lds, a.stream, a.W, a.x, w.part1,
                     (int)c.parts1, w.pv, (int)a.N, (int)a.K, c.q8.log2g, c.q8.passes);
  int err = (int)hipGetLastError();
  if (err) return err;
  hipLaunchKernelGGL((k_sl_exact<IT, XCH>), dim3((unsigned)c.parts2), dim3(256), lds, a.stream, a.W, a.x, w.u,
                     w.pv, w.part2, w.cnt, (int)a.N, (int)a.K, c.q8.log2g, c.q8.passes);
  return (int)hipGetLastError();
}

// x pieces per thread for 256 threads: 2 up to K = 4096, else 8 (K <= 16384).
template <int IT>
int launch_bound_x(const ShortlistArgs& a, const SlCfg& c, const SlWs& w, size_t lds) {
  return a.K <= 4096 ? launch_bound_it<IT, 2>(a, c, w, lds) : launch_bound_it<IT, 8>(a, c, w, lds);
}
template <int IT>
int launch_exact_x(const ShortlistArgs& a, const SlCfg& c, const SlWs& w, size_t lds) {
  return a.K <= 4096 ? launch_exact_it<IT, 2>(a, c, w, lds) : launch_exact_it<IT, 8>(a, c, w, lds);
}

}  // namespace

int64_t shortlist_workspace_bytes(int64_t N, int64_t K) {
  const SlCfg c = sl_cfg(N, K);
  return sl_ws(nullptr, N, c).bytes;
}

int launch_shortlist_argmax(const ShortlistArgs& a) {
  const SlCfg c = sl_cfg(a.N, a.K);
  const SlWs w = sl_ws(a.ws, a.N, c);
  // x (padded), half-block sums, block |x| sums / x (padded), half-block sums
  const size_t lds_bound = (size_t)16 * xrun_pieces<SL_XUP>((int)(a.K / 8)) + (size_t)(a.K / 32) * 12;
  const size_t lds_exact = (size_t)16 * xrun_pieces<Q8_XUP>((int)(a.K / 8)) + (size_t)(a.K / 32) * 8;
  dispatch_log("k_sl_bound", KQ_Q8_0, a.N, a.K, 1, (unsigned)c.parts1, 1, 256, lds_bound,
               "G=%d units/lane=%d passes=%d; exact rows G=%d units/lane=%d passes=%d", 1 << c.log2g, c.iters,
               c.passes, 1 << c.q8.log2g, c.q8.iters, c.q8.passes);
  int err;
  switch (c.iters) {
    case 1: err = launch_bound_x<1>(a, c, w, lds_bound); break;
    case 2: err = launch_bound_x<2>(a, c, w, lds_bound); break;
    case 3: err = launch_bound_x<3>(a, c, w, lds_bound); break;
    case 4: err = launch_bound_x<4>(a, c, w, lds_bound); break;
    default: err = launch_bound_x<5>(a, c, w, lds_bound); break;
  }
  if (err) return err;
  switch (c.q8.iters) {
    case 1: err = launch_exact_x<1>(a, c, w, lds_exact); break;
    case 2: err = launch_exact_x<2>(a, c, w, lds_exact); break;
    case 3: err = launch_exact_x<3>(a, c, w, lds_exact); break;
    case 4: err = launch_exact_x<4>(a, c, w, lds_exact); break;
    default: err = launch_exact_x<5>(a, c, w, lds_exact); break;
  }
  if (err) return err;
  hipLaunchKernelGGL(k_sl_final, dim3(1), dim3(256), 0, a.stream, w.part2, w.cnt, (int)c.parts2, a.out, a.kept);
  return (int)hipGetLastError();
}

}  // namespace kq
