// kq_gemv.hip — dense block-quantized GEMV for gfx950: y[M][N] = W'[N][K] x[M][K]^T.
//
// The decode step reads all of a dense model's weights once per token, and a
// speculative verify pass checks several guessed tokens "in one pass over the
// weights" (Kinetic docs, "What makes it fast"), so every kernel here streams
// each weight byte exactly once per call whatever M is.
//
// Paths:
//  * VALU path (kq_dev.h valu_tile): fp16 magic-number dequant + v_dot2_f32_f16,
//    used for small M (a few activation columns).
//  * MFMA path (kq_mfma.hip): v_mfma_f32_16x16x32_f16 for larger M.
//  * Generic path: Q4_0/Q8_0 rows whose length is an odd number of blocks are
//    only 2-byte aligned; a simple per-block kernel handles them.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "kq_dev.h"
#include "kq_internal.h"

namespace kqd {

// ----------------------------------------------------------------- VALU path

template <int FMT, int MT, int R>
__global__ __launch_bounds__(256) void k_gemv_valu(const uint8_t* __restrict__ W,
                                                   const uint16_t* __restrict__ x,
                                                   float* __restrict__ y, int N, int K, int log2g,
                                                   int m0) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + wave_id();
  const int rpw = 64 >> log2g;
  const int tile_rows = rpw * R;
  const int64_t row_base = (int64_t)wave * tile_rows;
  if (row_base >= N) return;
  const uint32_t row_bytes = (uint32_t)(K / 32) * Fmt<FMT>::BB;
  const int valid = (int)min<int64_t>(tile_rows, N - row_base);
  const rsrc_t rs = make_rsrc(W + row_base * row_bytes, (uint32_t)valid * row_bytes);
  const uint16_t* xc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xc[m] = x + (int64_t)(m0 + m) * K;
  float acc[R][MT];
  valu_tile<FMT, MT, R>(rs, row_bytes, K / (32 * Fmt<FMT>::UB), log2g, xc, acc);
  const int G = 1 << log2g;
  if ((lane & (G - 1)) == 0) {
    const int rho = lane >> log2g;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row_base + rho + rpw * r;
      if (row < N) {
#pragma unroll
        for (int m = 0; m < MT; ++m) y[(int64_t)(m0 + m) * N + row] = acc[r][m];
      }
    }
  }
}

// 16-byte activation chunks per thread in the register variant: enough for
// 1280 chunks per workgroup (one 10240-long column), 2560 for two columns (so
// that two 9728-long columns go through registers rather than LDS DMA).
template <int MT, int WPG> constexpr int xreg_chunks() {
  return ((MT == 2 ? 2560 : 1280) + 64 * WPG - 1) / (64 * WPG);
}

// ------------------------------------------- VALU path, loads-first + LDS x
// One row per lane group (G lanes), 64/G rows per wave. Each lane issues the
// loads of all ITERS units it owns, the workgroup stages the MT activation
// columns in LDS meanwhile, and only then does any arithmetic: one memory
// round trip per tile. `passes` > 1 only when units > G * ITERS.
// AM: also the argmax epilogue: the workgroup's best (value, row) of each
// column goes to part[column][blockIdx.x] (nparts per column), for
// k_argmax_final.
template <int FMT, int MT, int ITERS, bool XREG, int WPG = 4, bool AM = false>
__global__ __launch_bounds__(64 * WPG) void k_gemv_lds(const uint8_t* __restrict__ W,
                                                  const uint16_t* __restrict__ x,
                                                  float* __restrict__ y, int N, int K, int log2g,
                                                  int m0, int passes, Best* __restrict__ part, int nparts) {
  extern __shared__ u32x4 x_lds4[];
  uint32_t* xl = reinterpret_cast<uint32_t*>(x_lds4);
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * WPG + wave_id();
  const int G = 1 << log2g;
  __shared__ unsigned long long s_am_key[AM ? MT : 1];
  __shared__ uint32_t s_am_count;
  if constexpr (AM) {
    if (threadIdx.x == 0) {   // ordered before every update by the staging barrier below
#pragma unroll
      for (int m = 0; m < MT; ++m) s_am_key[m] = 0ull;
      s_am_count = 0u;
    }
  }
  const int rpw = 64 >> log2g;
  const int64_t row_base = (int64_t)wave * rpw;
  const uint32_t row_bytes = (uint32_t)(K / 32) * Fmt<FMT>::BB;
  const int units = K / (32 * Fmt<FMT>::UB);
  const int valid = row_base < N ? (int)min<int64_t>(rpw, N - row_base) : 0;
  const rsrc_t rs = make_rsrc(W + (valid ? row_base * row_bytes : 0), (uint32_t)valid * row_bytes);
  const int rho = lane >> log2g;
  const int g = lane & (G - 1);
  const uint32_t roff = (uint32_t)rho * row_bytes;
  const int kdw = K / 2;
  constexpr int UP = 4 * Fmt<FMT>::UB;   // pieces per load unit: x is staged with one idle piece after each
  float* xs = reinterpret_cast<float*>(xl + 4 * xrun_pieces<UP>(MT * K / 8));
  // XREG: the activations go ahead of the weights in this CU's memory queue,
  // loaded into registers (at most xreg_chunks 16-byte chunks per thread), so
  // writing them to LDS waits for them alone and the block sums below overlap
  // the weights' latency. Otherwise they are copied by LDS DMA (any K), also
  // ahead of the weights, so that the first barrier waits for the DMA alone
  // (loads complete in order). The two variants are separate kernels: with an
  // LDS DMA anywhere in the kernel the compiler would make the register
  // path's LDS writes wait for every load.
  constexpr int XCH = xreg_chunks<MT, WPG>();
  const int n16 = MT * K / 8;   // columns m0 .. m0+MT-1 are contiguous
  u32x4 xr[XCH];
  const u32x4* xsrc = reinterpret_cast<const u32x4*>(x + (int64_t)m0 * K);
  if constexpr (XREG) {
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      const int i = (int)threadIdx.x + 64 * WPG * c;
      xr[c] = i < n16 ? xsrc[i] : u32x4{0u, 0u, 0u, 0u};
    }
  } else {
    stage_to_lds_padded<UP>(x + (int64_t)m0 * K, xl, n16, 64 * WPG);
  }
  __builtin_amdgcn_sched_barrier(0);
  Loaded<FMT, ITERS> w;
  issue_units<FMT, ITERS>(rs, roff, g, G, units, w);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XREG) {
    u32x4* xl4 = reinterpret_cast<u32x4*>(xl);
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      const int i = (int)threadIdx.x + 64 * WPG * c;
      if (i < n16) xl4[xphys<UP>(i)] = xr[c];
    }
  }
  __syncthreads();
  block_sums_to_lds<UP>(xl, kdw, MT, xs, 64 * WPG);
  __syncthreads();
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
  const int span = G * ITERS;
  for (int p = 0;;) {
    consume_units<FMT, MT, ITERS, true>(w, xl, xs, kdw, p * span + g, G, units, acc);
    if (++p >= passes) break;
    issue_units<FMT, ITERS>(rs, roff, p * span + g, G, units, w);
  }
  group_reduce<MT>(acc, G);
  if (g == 0 && rho < valid) {
#pragma unroll
    for (int m = 0; m < MT; ++m) y[(int64_t)(m0 + m) * N + row_base + rho] = acc[m];
  }
  if constexpr (AM) {
    // No barrier: each row's (value, row) key goes into the workgroup's slot
    // by an LDS 64-bit atomic max, then the wave bumps a counter; the wave
    // that completes the count publishes the slot.
    if (g == 0 && rho < valid) {
#pragma unroll
      for (int m = 0; m < MT; ++m) atomicMax(&s_am_key[m], best_key(acc[m], (int32_t)(row_base + rho)));
    }
    if (lane == 0) {
      const uint32_t done = __hip_atomic_fetch_add(&s_am_count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (done == WPG - 1) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const unsigned long long k = __hip_atomic_load(&s_am_key[m], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
          part[(int64_t)(m0 + m) * nparts + blockIdx.x] = best_of_key(k);
        }
      }
    }
  }
}

// -------------------------------------------------------------- generic path
// One wave per row, one lane per block, 16-bit loads (blocks may be only
// 2-byte aligned), plain fp32 dequantization. Loops over all M columns.
template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_generic(const uint8_t* __restrict__ W,
                                                      const uint16_t* __restrict__ x,
                                                      float* __restrict__ y, int N, int K, int M) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  if (row >= N) return;
  const int nb = K / 32;
  const int64_t row_bytes = (int64_t)nb * Fmt<FMT>::BB;
  for (int m = 0; m < M; ++m) {
    float acc = 0.0f;
    for (int b = lane; b < nb; b += 64) {
      const uint16_t* blk = reinterpret_cast<const uint16_t*>(W + row * row_bytes + (int64_t)b * Fmt<FMT>::BB);
      const uint16_t* xb = x + (int64_t)m * K + b * 32;
      const float s = h2f(blk[0]);
      if constexpr (FMT == F_Q5_0 || FMT == F_Q5_1) {
        acc = q5_block_plain<FMT>(blk, xb, acc);
      } else if constexpr (FMT == F_Q8_0) {
        for (int j = 0; j < 16; ++j) {
          const uint32_t two = blk[1 + j];
          acc = __builtin_fmaf(s * (float)(int8_t)(two & 0xff), h2f(xb[2 * j]), acc);
          acc = __builtin_fmaf(s * (float)(int8_t)(two >> 8), h2f(xb[2 * j + 1]), acc);
        }
      } else {
        const float bias = FMT == F_AFFINE4 ? h2f(blk[1]) : 0.0f;
        const uint16_t* nib = blk + (FMT == F_AFFINE4 ? 2 : 1);
        for (int j = 0; j < 8; ++j) {
          const uint32_t two = nib[j];
          const int q0 = two & 15, q1 = (two >> 4) & 15, q2 = (two >> 8) & 15, q3 = (two >> 12) & 15;
          const int e = 2 * j;  // bytes 2j, 2j+1 hold elements 2j, 2j+16, 2j+1, 2j+17
          float w0, w1, w2, w3;
          if constexpr (FMT == F_AFFINE4) {
            w0 = __builtin_fmaf(s, (float)q0, bias);
            w1 = __builtin_fmaf(s, (float)q1, bias);
            w2 = __builtin_fmaf(s, (float)q2, bias);
            w3 = __builtin_fmaf(s, (float)q3, bias);
          } else {
            w0 = s * (float)(q0 - 8);
            w1 = s * (float)(q1 - 8);
            w2 = s * (float)(q2 - 8);
            w3 = s * (float)(q3 - 8);
          }
          acc = __builtin_fmaf(w0, h2f(xb[e]), acc);
          acc = __builtin_fmaf(w1, h2f(xb[e + 16]), acc);
          acc = __builtin_fmaf(w2, h2f(xb[e + 1]), acc);
          acc = __builtin_fmaf(w3, h2f(xb[e + 17]), acc);
        }
      }
    }
    acc = group_sum(acc, 64);
    if (lane == 0) y[(int64_t)m * N + row] = acc;
  }
}

}  // namespace kqd

namespace kq {

using namespace kqd;

const char* hip_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

int device_cus() {
  static std::atomic<int> cus_of[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;   // only shapes launches
  int v = cus_of[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) v = 256;
    cus_of[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

namespace {

int ilog2(int v) {
  int l = 0;
  while ((1 << (l + 1)) <= v) ++l;
  return l;
}

struct ValuCfg {
  int log2g;
  int R;
};

int tune_int(TuneKey k) {
  const int v = tune(k);
  return v == TUNE_UNSET ? 0 : v;
}

// Lanes per row (G) and rows per lane (R) for the VALU path. G is a power of
// two near units/4, so each lane walks a few units of a row; R grows while
// the grid still holds >= 2048 waves (8 per CU) to keep loads in flight.
// The valu_g / valu_r tuning overrides replace the choice (sweeps and tests).
ValuCfg valu_cfg(int64_t N, int units) {
  const int env_g = tune_int(TUNE_VALU_G);
  const int env_r = tune_int(TUNE_VALU_R);
  int G = 1 << ilog2(units / 4 > 0 ? units / 4 : 1);
  G = G < 4 ? 4 : (G > 64 ? 64 : G);
  if (env_g == 1 || env_g == 2 || env_g == 4 || env_g == 8 || env_g == 16 || env_g == 32 || env_g == 64) G = env_g;
  int R = 1;
  const int64_t rpw = 64 / G;
  for (int cand : {4, 2}) {
    if ((N + rpw * cand - 1) / (rpw * cand) >= 2048) { R = cand; break; }
  }
  if (env_r == 1 || env_r == 2 || env_r == 4) R = env_r;
  return {ilog2(G), R};
}

template <int FMT, int MT>
int launch_valu_mt(const GemvArgs& a, int m0, ValuCfg c) {
  const int64_t tile = (int64_t)(64 >> c.log2g) * c.R;
  const int64_t waves = (a.N + tile - 1) / tile;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  dispatch_log("k_gemv_valu", a.fmt, a.N, a.K, MT, grid.x, 1, 256, 0, "register-x G=%d R=%d m0=%d", 1 << c.log2g,
               c.R, m0);
  if (c.R == 4)
    hipLaunchKernelGGL((k_gemv_valu<FMT, MT, 4>), grid, block, 0, a.stream, a.W, a.x, a.y, (int)a.N, (int)a.K, c.log2g, m0);
  else if (c.R == 2)
    hipLaunchKernelGGL((k_gemv_valu<FMT, MT, 2>), grid, block, 0, a.stream, a.W, a.x, a.y, (int)a.N, (int)a.K, c.log2g, m0);
  else
    hipLaunchKernelGGL((k_gemv_valu<FMT, MT, 1>), grid, block, 0, a.stream, a.W, a.x, a.y, (int)a.N, (int)a.K, c.log2g, m0);
  return (int)hipGetLastError();
}

template <int FMT>
int launch_valu(const GemvArgs& a) {
  const int units = (int)(a.K / (32 * Fmt<FMT>::UB));
  const ValuCfg c = valu_cfg(a.N, units);
  for (int m0 = 0; m0 < a.M; m0 += 8) {
    const int mt = a.M - m0 < 8 ? a.M - m0 : 8;
    int err = 0;
    switch (mt) {
      case 1: err = launch_valu_mt<FMT, 1>(a, m0, c); break;
      case 2: err = launch_valu_mt<FMT, 2>(a, m0, c); break;
      case 3: err = launch_valu_mt<FMT, 3>(a, m0, c); break;
      case 4: err = launch_valu_mt<FMT, 4>(a, m0, c); break;
      case 5: err = launch_valu_mt<FMT, 5>(a, m0, c); break;
      case 6: err = launch_valu_mt<FMT, 6>(a, m0, c); break;
      case 7: err = launch_valu_mt<FMT, 7>(a, m0, c); break;
      default: err = launch_valu_mt<FMT, 8>(a, m0, c); break;
    }
    if (err) return err;
  }
  return 0;
}

constexpr int LDS_MAX_MT = 4;
// From 4 columns on, products go to the matrix cores; with 2 or 3 the VALU
// kernel is faster on every decode shape (2 columns on MI355X: gate|up 10.4
// vs 12.6 us, lm_head 98.5 vs 106 us). Rows of 2-byte-aligned blocks (an
// odd number of Q4_0/Q8_0 blocks) take the matrix cores from 2 columns on.
constexpr int MFMA_MIN_M = 4;
constexpr int MFMA_MIN_M_UNALIGNED = 2;
constexpr int LDS_MAX_BYTES = 96 * 1024;

// LDS bytes of the one-column-family kernel: x of mt columns in the padded
// layout (one idle 16-byte piece per load unit), then the half-block sums.
template <int FMT>
int64_t lds_kernel_bytes(int mt, int64_t K) {
  return 16 * (int64_t)xrun_pieces<4 * Fmt<FMT>::UB>((int)(mt * K / 8)) + (int64_t)mt * (K / 32) * 8;
}
constexpr int MAX_ITERS = 5;

struct LdsCfg {
  int log2g;
  int iters;
  int passes;
  int wpg;     // waves per workgroup (one staged copy of x per workgroup)
};

// G (lanes per row, power of two) and ITERS (units per lane per pass): G
// gives each lane about LANE_BYTES of weights (at most MAX_ITERS units; the
// larger G on a tie), then is doubled while the grid has fewer than 2048 waves
// (8 per CU) and lanes would still have work, so small matrices spread over
// more waves. On MI355X (cold weights, graph-replayed) this picks the fastest
// or nearly fastest G for the 4B-shaped projections and the Q8_0 lm_head.
// Outputs with at least LARGE_N rows (a vocabulary-sized output layer) have
// waves to spare, and there longer runs per lane (LANE_BYTES_LARGE) measure
// faster (Q8_0 151936 x 2560: 67 us at G = 16 against 78 us at G = 32).
constexpr int LANE_BYTES = 128;
constexpr int LANE_BYTES_LARGE = 200;
constexpr int64_t LARGE_N = 65536;

LdsCfg lds_cfg(int64_t N, int units, int unit_bytes) {
  int G = 64;
  int best = -1;
  const int target = N >= LARGE_N ? LANE_BYTES_LARGE : LANE_BYTES;
  for (int g = 64; g >= 1; g >>= 1) {
    const int iters = (units + g - 1) / g;
    if (iters > MAX_ITERS) break;
    const int dev = iters * unit_bytes > target ? iters * unit_bytes - target : target - iters * unit_bytes;
    if (best < 0 || dev < best) {
      best = dev;
      G = g;
    }
  }
  while (G < 64 && N * G / 64 < 2048 && G < units) G <<= 1;
  const int env_g = tune_int(TUNE_VALU_G);
  if (env_g == 1 || env_g == 2 || env_g == 4 || env_g == 8 || env_g == 16 || env_g == 32 || env_g == 64) G = env_g;
  int iters = (units + G - 1) / G;
  if (iters > MAX_ITERS) iters = MAX_ITERS;
  const int passes = (units + G * iters - 1) / (G * iters);
  // Waves per workgroup (one column): 4, or 12 where a row is 64 lanes of
  // exactly two units each and the grid fits the device at once (fewer
  // workgroups, each staging x for more rows). Measured on MI355X (cold,
  // graph-replayed, medians of 3, std about 0.01 us): 2560 x 4096 affine4 3.33
  // against 3.60 us, Q5_1 3.91 against 4.06; every other shape tried is as
  // fast or faster at 4 (q|k|v 4.16 against 4.22, down 5.80 against 6.15,
  // Q8_0 6144 x 2560 with two units on 32 lanes 5.58 against 6.73, the 0.6B
  // Q4_0 shapes with one unit per lane 2.7-3.3 against 3.3-3.7). Spreading
  // row waves evenly over the CUs (5 per workgroup on 2560 rows: 10 on every
  // CU instead of 12 on half and 8 on the rest) did not help: 3.58, 5.86 us.
  int wpg = 4;
  if (iters == 2 && G == 64 && passes == 1 && N <= 16 * (int64_t)device_cus()) wpg = 12;
  const int env_w = tune_int(TUNE_LDS_WPG);
  if (env_w == 4 || env_w == 8 || env_w == 12 || env_w == 16) wpg = env_w;
  return {ilog2(G), iters, passes, wpg};
}

template <int FMT, int MT, int ITERS, int WPG>
int launch_lds_wpg(const GemvArgs& a, int m0, LdsCfg c, Best* part) {
  const int64_t rpw = 64 >> c.log2g;
  const int64_t waves = (a.N + rpw - 1) / rpw;
  const int64_t nwg = (waves + WPG - 1) / WPG;
  const dim3 grid((unsigned)nwg), block(64 * WPG);
  const size_t lds = (size_t)lds_kernel_bytes<FMT>(MT, a.K);   // x (padded) + block sums
  const bool xreg = (int64_t)MT * a.K / 8 <= 64 * WPG * xreg_chunks<MT, WPG>() && tune(TUNE_LDS_XDMA) != 1;
  dispatch_log("k_gemv_lds", a.fmt, a.N, a.K, MT, grid.x, 1, 64 * WPG, lds,
               "G=%d units/lane=%d passes=%d x=%s m0=%d argmax=%d", 1 << c.log2g, ITERS, c.passes,
               xreg ? "registers" : "lds-dma", m0, part ? 1 : 0);
  if (MT == 1 && part) {   // the argmax epilogue (one column only)
    if (xreg)
      hipLaunchKernelGGL((k_gemv_lds<FMT, MT, ITERS, true, WPG, MT == 1>), grid, block, lds, a.stream, a.W, a.x, a.y,
                         (int)a.N, (int)a.K, c.log2g, m0, c.passes, part, (int)nwg);
    else
      hipLaunchKernelGGL((k_gemv_lds<FMT, MT, ITERS, false, WPG, MT == 1>), grid, block, lds, a.stream, a.W, a.x,
                         a.y, (int)a.N, (int)a.K, c.log2g, m0, c.passes, part, (int)nwg);
  } else if (xreg) {
    hipLaunchKernelGGL((k_gemv_lds<FMT, MT, ITERS, true, WPG>), grid, block, lds, a.stream, a.W, a.x, a.y,
                       (int)a.N, (int)a.K, c.log2g, m0, c.passes, nullptr, 0);
  } else {
    hipLaunchKernelGGL((k_gemv_lds<FMT, MT, ITERS, false, WPG>), grid, block, lds, a.stream, a.W, a.x, a.y,
                       (int)a.N, (int)a.K, c.log2g, m0, c.passes, nullptr, 0);
  }
  return (int)hipGetLastError();
}

template <int FMT, int MT, int ITERS>
int launch_lds_it(const GemvArgs& a, int m0, LdsCfg c, Best* part) {
  if constexpr (MT == 1) {
    switch (c.wpg) {
      case 8: return launch_lds_wpg<FMT, MT, ITERS, 8>(a, m0, c, part);
      case 12: return launch_lds_wpg<FMT, MT, ITERS, 12>(a, m0, c, part);
      case 16: return launch_lds_wpg<FMT, MT, ITERS, 16>(a, m0, c, part);
      default: break;
    }
  }
  return launch_lds_wpg<FMT, MT, ITERS, 4>(a, m0, c, part);
}

// Waves per workgroup the LDS kernel runs with (c.wpg applies to one column).
int lds_wpg(const LdsCfg& c, int mt) { return mt == 1 ? c.wpg : 4; }

template <int FMT, int MT>
int launch_lds_mt(const GemvArgs& a, int m0, LdsCfg c, Best* part = nullptr) {
  switch (c.iters) {
    case 1: return launch_lds_it<FMT, MT, 1>(a, m0, c, part);
    case 2: return launch_lds_it<FMT, MT, 2>(a, m0, c, part);
    case 3: return launch_lds_it<FMT, MT, 3>(a, m0, c, part);
    case 4: return launch_lds_it<FMT, MT, 4>(a, m0, c, part);
    default: return launch_lds_it<FMT, MT, 5>(a, m0, c, part);
  }
}

template <int FMT>
int launch_lds(const GemvArgs& a) {
  const int units = (int)(a.K / (32 * Fmt<FMT>::UB));
  const LdsCfg c = lds_cfg(a.N, units, Fmt<FMT>::BB * Fmt<FMT>::UB);
  for (int m0 = 0; m0 < a.M; m0 += LDS_MAX_MT) {
    const int mt = a.M - m0 < LDS_MAX_MT ? a.M - m0 : LDS_MAX_MT;
    int err;
    switch (mt) {
      case 1: err = launch_lds_mt<FMT, 1>(a, m0, c); break;
      case 2: err = launch_lds_mt<FMT, 2>(a, m0, c); break;
      case 3: err = launch_lds_mt<FMT, 3>(a, m0, c); break;
      default: err = launch_lds_mt<FMT, 4>(a, m0, c); break;
    }
    if (err) return err;
  }
  return 0;
}

template <int FMT>
int launch_generic(const GemvArgs& a) {
  const dim3 grid((unsigned)((a.N + 3) / 4)), block(256);
  dispatch_log("k_gemv_generic", a.fmt, a.N, a.K, a.M, grid.x, 1, 256, 0, "one wave per row");
  hipLaunchKernelGGL((k_gemv_generic<FMT>), grid, block, 0, a.stream, a.W, a.x, a.y, (int)a.N, (int)a.K, a.M);
  return (int)hipGetLastError();
}

template <int FMT>
int dispatch(const GemvArgs& a) {
  if (a.K % (32 * Fmt<FMT>::UB) != 0) return a.M >= MFMA_MIN_M_UNALIGNED ? launch_gemv_mfma(a) : launch_generic<FMT>(a);
  const int force = tune_int(TUNE_FORCE_PATH);  // tests: run a given path at any shape
  if (force == 'g') return launch_generic<FMT>(a);
  const bool lds_fits = lds_kernel_bytes<FMT>(a.M < LDS_MAX_MT ? a.M : LDS_MAX_MT, a.K) <= LDS_MAX_BYTES;
  if (force == 'v') return launch_valu<FMT>(a);     // register-x VALU kernel
  if (force == 'l' && lds_fits) return launch_lds<FMT>(a);
  if (force == 'm') return launch_gemv_mfma(a);
  if (a.M >= MFMA_MIN_M) return launch_gemv_mfma(a);
  if (a.M <= LDS_MAX_MT && lds_fits) return launch_lds<FMT>(a);
  return launch_valu<FMT>(a);
}

}  // namespace

RowCfg q8_row_cfg(int64_t N, int64_t K) {
  const LdsCfg c = lds_cfg(N, (int)(K / (32 * Fmt<F_Q8_0>::UB)), Fmt<F_Q8_0>::BB * Fmt<F_Q8_0>::UB);
  return {c.log2g, c.iters, c.passes};
}

int launch_gemv(const GemvArgs& a) {
  switch (a.fmt) {
    case KQ_Q8_0: return dispatch<F_Q8_0>(a);
    case KQ_Q4_0: return dispatch<F_Q4_0>(a);
    case KQ_Q5_0: return dispatch<F_Q5_0>(a);
    case KQ_Q5_1: return dispatch<F_Q5_1>(a);
    default: return dispatch<F_AFFINE4>(a);
  }
}

namespace {

// Batch-invariant dispatch: the matrix-core kernels with configurations that
// depend on N and K only, for every M including 1, so column m gets the bits
// of a one-column call of this entry point. Rows of 2-byte-aligned blocks take
// the generic kernel, which loops over the columns (also invariant).
template <int FMT>
int dispatch_invariant(const GemvArgs& a) {
  if (a.K % (32 * Fmt<FMT>::UB) != 0) return launch_generic<FMT>(a);
  return launch_gemv_mfma_invariant(a);
}

}  // namespace

namespace {

// GEMV + argmax of every column. For one column on the one-pass LDS kernel
// (rows of whole units, x fits), that kernel leaves each workgroup's best
// (value, row) in `ws` and one small kernel reduces them; otherwise the GEMV,
// then kq_argmax's two kernels. Measured on the 151936 x 2560 Q8_0 output
// layer: 72.4 against 75.4 us at M = 1; at M = 2 the fused form was 1.7 us
// slower, so it stops at one column.
template <int FMT>
bool argmax_fusable(const GemvArgs& a, LdsCfg* cfg) {
  if (a.K % (32 * Fmt<FMT>::UB) != 0 || a.M != 1) return false;
  if (lds_kernel_bytes<FMT>(a.M, a.K) > LDS_MAX_BYTES) return false;
  if (tune(TUNE_FORCE_PATH) != TUNE_UNSET) return false;
  const int units = (int)(a.K / (32 * Fmt<FMT>::UB));
  *cfg = lds_cfg(a.N, units, Fmt<FMT>::BB * Fmt<FMT>::UB);
  return true;
}

int64_t fused_parts(const GemvArgs& a, const LdsCfg& c) {
  const int64_t rpw = 64 >> c.log2g;
  const int64_t waves = (a.N + rpw - 1) / rpw;
  const int wpg = lds_wpg(c, a.M);
  return (waves + wpg - 1) / wpg;
}

template <int FMT>
int64_t gemv_argmax_parts_fmt(const GemvArgs& a) {
  LdsCfg c;
  return argmax_fusable<FMT>(a, &c) ? fused_parts(a, c) : 0;
}

template <int FMT>
int gemv_argmax_fmt(const GemvArgs& a, int32_t* out, void* ws) {
  LdsCfg c;
  if (!argmax_fusable<FMT>(a, &c)) {
    int err = launch_gemv(a);
    if (err) return err;
    return launch_argmax(a.y, a.N, a.M, out, ws, a.stream);
  }
  Best* part = static_cast<Best*>(ws);
  const int err = launch_lds_mt<FMT, 1>(a, 0, c, part);
  if (err) return err;
  return launch_argmax_final(part, (int)fused_parts(a, c), a.M, out, a.stream);
}

}  // namespace

int64_t gemv_argmax_fused_parts(const GemvArgs& a) {
  switch (a.fmt) {
    case KQ_Q8_0: return gemv_argmax_parts_fmt<F_Q8_0>(a);
    case KQ_Q4_0: return gemv_argmax_parts_fmt<F_Q4_0>(a);
    case KQ_Q5_0: return gemv_argmax_parts_fmt<F_Q5_0>(a);
    case KQ_Q5_1: return gemv_argmax_parts_fmt<F_Q5_1>(a);
    default: return gemv_argmax_parts_fmt<F_AFFINE4>(a);
  }
}

int launch_gemv_argmax(const GemvArgs& a, int32_t* out, void* ws) {
  switch (a.fmt) {
    case KQ_Q8_0: return gemv_argmax_fmt<F_Q8_0>(a, out, ws);
    case KQ_Q4_0: return gemv_argmax_fmt<F_Q4_0>(a, out, ws);
    case KQ_Q5_0: return gemv_argmax_fmt<F_Q5_0>(a, out, ws);
    case KQ_Q5_1: return gemv_argmax_fmt<F_Q5_1>(a, out, ws);
    default: return gemv_argmax_fmt<F_AFFINE4>(a, out, ws);
  }
}

// ------------------------------------------------- allocation-free argmax
// Device memory for the partial argmax results of kq_gemv_argmax_noalloc,
// for callers that cannot allocate. Each device holds its own copy, at its own
// address, until the process ends. In host code the name is not a device
// address: kernels get the address hipGetSymbolAddress returns for the current
// device (noalloc_scratch below). Calls on one device share it, so calls that
// overlap in time on one device race. Every slot a call reads was written
// earlier in that call, so nothing needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[KQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};
}  // namespace

int noalloc_scratch(void** ptr) {
  int dev = -1;
  int err = (int)hipGetDevice(&dev);
  if (err) return err;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = (int)hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err) return err;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

int launch_gemv_argmax_noalloc(const GemvArgs& a, int32_t* out) {
  void* ws = nullptr;
  const int err = noalloc_scratch(&ws);
  if (err) return err;
  return launch_gemv_argmax(a, out, ws);
}

int launch_gemv_invariant(const GemvArgs& a) {
  switch (a.fmt) {
    case KQ_Q8_0: return dispatch_invariant<F_Q8_0>(a);
    case KQ_Q4_0: return dispatch_invariant<F_Q4_0>(a);
    case KQ_Q5_0: return dispatch_invariant<F_Q5_0>(a);
    case KQ_Q5_1: return dispatch_invariant<F_Q5_1>(a);
    default: return dispatch_invariant<F_AFFINE4>(a);
  }
}

}  // namespace kq
