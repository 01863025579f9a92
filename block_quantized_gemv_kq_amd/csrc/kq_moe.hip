// kq_moe.hip — routed-expert (mixture-of-experts) decode GEMVs for gfx950.
//
// A mixture of experts uses only a few experts per token (kinfer page,
// "Models bigger than the machine": 10 of 512; Kinetic docs, "What makes it
// fast": experts in use stay on the GPU), so only the routed experts' weights
// are read, and each distinct expert is read once per call for all of the
// tokens routed to it.
//
// Grid: (row tiles, M * top_k route slots). The workgroup of slot p handles
// expert e = ids[p] only if no earlier slot names e; it then gathers every
// slot routed to e (on the device, no host synchronisation) and runs the
// VALU tile over them as the activation columns, so e's rows stream once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_dev.h"
#include "kq_internal.h"

namespace kqd {

constexpr int MOE_MAX_SLOTS = 64 * 64;  // M * top_k upper bound
constexpr int MOE_COLS = 4;             // activation columns per VALU pass

// Returns the number of slots routed to ids[p] (0 if an earlier slot owns the
// expert). Slot indices are written to s_list in increasing order.
__device__ int gather_expert_slots(const int32_t* __restrict__ ids, int p, int P, int* s_list,
                                   int* s_cnt) {
  const int e = ids[p];
  int dup = 0;
  for (int q = threadIdx.x; q < p; q += 256) dup |= (ids[q] == e);   // 256-thread workgroups
  dup = __syncthreads_or(dup);
  if (dup) return 0;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int cnt = 0;
    for (int base = p; base < P; base += 64) {
      const int q = base + lane;
      const bool hit = q < P && ids[q] == e;
      const uint64_t mask = __ballot(hit);
      if (hit) s_list[cnt + __popcll(mask & ((1ull << lane) - 1ull))] = q;
      cnt += __popcll(mask);
    }
    if (lane == 0) *s_cnt = cnt;
  }
  __syncthreads();
  return *s_cnt;
}

// Per-slot GEMV outputs y_slot[p][n] for the rows of this wave's tile.
template <int FMT, int MT, int R>
__device__ __forceinline__ void moe_cols(rsrc_t rs, uint32_t row_bytes, int units, int log2g,
                                         const uint16_t* __restrict__ x, const int* list, int c0,
                                         int K, int top_k, int x_per_slot, float* __restrict__ y_slot,
                                         int64_t N, int64_t row_base) {
  const uint16_t* xc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int p = list[c0 + m];
    const int64_t xrow = x_per_slot ? p : p / top_k;
    xc[m] = x + xrow * K;
  }
  float acc[R][MT];
  valu_tile<FMT, MT, R>(rs, row_bytes, units, log2g, xc, acc);
  const int lane = threadIdx.x & 63;
  const int G = 1 << log2g, rpw = 64 >> log2g;
  if ((lane & (G - 1)) == 0) {
    const int rho = lane >> log2g;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row_base + rho + rpw * r;
      if (row < N) {
#pragma unroll
        for (int m = 0; m < MT; ++m) y_slot[(int64_t)list[c0 + m] * N + row] = acc[r][m];
      }
    }
  }
}

template <int FMT, int R>
__global__ __launch_bounds__(256) void k_moe_valu(const uint8_t* __restrict__ W,
                                                  const uint16_t* __restrict__ x,
                                                  const int32_t* __restrict__ ids,
                                                  float* __restrict__ y_slot, int N, int K, int M,
                                                  int top_k, int n_experts, int x_per_slot,
                                                  int log2g, int64_t expert_bytes) {
  __shared__ int s_list[MOE_MAX_SLOTS];
  __shared__ int s_cnt;
  const int P = M * top_k;
  const int p = blockIdx.y;
  const int cnt = gather_expert_slots(ids, p, P, s_list, &s_cnt);
  if (cnt == 0) return;
  const int e = ids[p];
  const int rpw = 64 >> log2g;
  const int tile_rows = rpw * R;
  const int wave = blockIdx.x * 4 + wave_id();
  const int64_t row_base = (int64_t)wave * tile_rows;
  if (row_base >= N) return;
  if (e < 0 || e >= n_experts) {  // precondition violated: read nothing, flag with NaN
    const int lane = threadIdx.x & 63;
    for (int c = 0; c < cnt; ++c)
      for (int r = lane; r < tile_rows; r += 64)
        if (row_base + r < N) y_slot[(int64_t)s_list[c] * N + row_base + r] = __builtin_nanf("");
    return;
  }
  const uint32_t row_bytes = (uint32_t)(K / 32) * Fmt<FMT>::BB;
  const int valid = (int)min<int64_t>(tile_rows, N - row_base);
  const uint8_t* We = W + (int64_t)e * expert_bytes;
  const rsrc_t rs = make_rsrc(We + row_base * row_bytes, (uint32_t)valid * row_bytes);
  const int units = K / (32 * Fmt<FMT>::UB);
  for (int c0 = 0; c0 < cnt; c0 += MOE_COLS) {
    const int mt = cnt - c0 < MOE_COLS ? cnt - c0 : MOE_COLS;
    switch (mt) {
      case 1: moe_cols<FMT, 1, R>(rs, row_bytes, units, log2g, x, s_list, c0, K, top_k, x_per_slot, y_slot, N, row_base); break;
      case 2: moe_cols<FMT, 2, R>(rs, row_bytes, units, log2g, x, s_list, c0, K, top_k, x_per_slot, y_slot, N, row_base); break;
      case 3: moe_cols<FMT, 3, R>(rs, row_bytes, units, log2g, x, s_list, c0, K, top_k, x_per_slot, y_slot, N, row_base); break;
      default: moe_cols<FMT, 4, R>(rs, row_bytes, units, log2g, x, s_list, c0, K, top_k, x_per_slot, y_slot, N, row_base); break;
    }
  }
}

// Gate and up rows of one expert in the same pass, SwiGLU in registers:
// h[p][n] = fp16(silu(gate_n . x) * (up_n . x)), silu(z) = z / (1 + e^-z).
template <int FMT, int MT, int R>
__device__ __forceinline__ void gate_up_cols(rsrc_t rg, rsrc_t ru, uint32_t row_bytes, int units,
                                             int log2g, const uint16_t* __restrict__ x,
                                             const int* list, int c0, int K, int top_k,
                                             uint16_t* __restrict__ h, int64_t N, int64_t row_base) {
  const uint16_t* xc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xc[m] = x + (int64_t)(list[c0 + m] / top_k) * K;
  float g[R][MT], u[R][MT];
  valu_tile<FMT, MT, R>(rg, row_bytes, units, log2g, xc, g);
  valu_tile<FMT, MT, R>(ru, row_bytes, units, log2g, xc, u);
  const int lane = threadIdx.x & 63;
  const int G = 1 << log2g, rpw = 64 >> log2g;
  if ((lane & (G - 1)) == 0) {
    const int rho = lane >> log2g;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row_base + rho + rpw * r;
      if (row < N) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float z = g[r][m];
          const float hv = z / (1.0f + __expf(-z)) * u[r][m];
          h[(int64_t)list[c0 + m] * N + row] = (uint16_t)f2h_bits(hv);
        }
      }
    }
  }
}

template <int FMT, int R>
__global__ __launch_bounds__(256) void k_moe_gate_up(const uint8_t* __restrict__ Wg,
                                                     const uint8_t* __restrict__ Wu,
                                                     const uint16_t* __restrict__ x,
                                                     const int32_t* __restrict__ ids,
                                                     uint16_t* __restrict__ h, int N, int K, int M,
                                                     int top_k, int n_experts, int log2g,
                                                     int64_t expert_bytes) {
  __shared__ int s_list[MOE_MAX_SLOTS];
  __shared__ int s_cnt;
  const int P = M * top_k;
  const int p = blockIdx.y;
  const int cnt = gather_expert_slots(ids, p, P, s_list, &s_cnt);
  if (cnt == 0) return;
  const int e = ids[p];
  const int rpw = 64 >> log2g;
  const int tile_rows = rpw * R;
  const int wave = blockIdx.x * 4 + wave_id();
  const int64_t row_base = (int64_t)wave * tile_rows;
  if (row_base >= N) return;
  if (e < 0 || e >= n_experts) {
    const int lane = threadIdx.x & 63;
    const uint16_t nan16 = 0x7e00;
    for (int c = 0; c < cnt; ++c)
      for (int r = lane; r < tile_rows; r += 64)
        if (row_base + r < N) h[(int64_t)s_list[c] * N + row_base + r] = nan16;
    return;
  }
  const uint32_t row_bytes = (uint32_t)(K / 32) * Fmt<FMT>::BB;
  const int valid = (int)min<int64_t>(tile_rows, N - row_base);
  const int64_t off = (int64_t)e * expert_bytes + row_base * row_bytes;
  const rsrc_t rg = make_rsrc(Wg + off, (uint32_t)valid * row_bytes);
  const rsrc_t ru = make_rsrc(Wu + off, (uint32_t)valid * row_bytes);
  const int units = K / (32 * Fmt<FMT>::UB);
  for (int c0 = 0; c0 < cnt; c0 += MOE_COLS) {
    const int mt = cnt - c0 < MOE_COLS ? cnt - c0 : MOE_COLS;
    switch (mt) {
      case 1: gate_up_cols<FMT, 1, R>(rg, ru, row_bytes, units, log2g, x, s_list, c0, K, top_k, h, N, row_base); break;
      case 2: gate_up_cols<FMT, 2, R>(rg, ru, row_bytes, units, log2g, x, s_list, c0, K, top_k, h, N, row_base); break;
      case 3: gate_up_cols<FMT, 3, R>(rg, ru, row_bytes, units, log2g, x, s_list, c0, K, top_k, h, N, row_base); break;
      default: gate_up_cols<FMT, 4, R>(rg, ru, row_bytes, units, log2g, x, s_list, c0, K, top_k, h, N, row_base); break;
    }
  }
}

// Routed-expert GEMV with the tokens' activations staged in LDS (rows of
// whole load units). Grid (row tiles, M * top_k route slots); the workgroup
// of slot p owns expert e = ids[p] when no earlier slot names e, and serves
// every slot routed to e. The route ids are read once into LDS; then, in this
// order: the activations of the first (up to MOE_COLS) routed tokens into
// registers, this wave's weight loads (G lanes per row, ITERS units each),
// the activations into LDS with their block sums, and the products through
// LDS. More tokens on one expert take further passes, which reload the
// weights (by then in L2). GATE_UP: W0 = gate, W1 = up of the same rows, and
// the output is h = fp16(silu(gate . x) * (up . x)); otherwise W0 alone and
// fp32 per-slot outputs. Dynamic LDS: MOE_COLS columns of x and their block
// sums, then the ids and the gathered slot list (P ints each), then a 16-byte
// idle slot. K <= 256 * MOE_XCH * 8 / MOE_COLS.
constexpr int MOE_XCH = 4;   // 16-byte x pieces per thread per pass

template <int FMT, int ITERS, bool GATE_UP>
__global__ __launch_bounds__(256) void k_moe_lds(const uint8_t* __restrict__ W0, const uint8_t* __restrict__ W1,
                                                const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
                                                void* __restrict__ out, int N, int K, int M, int top_k,
                                                int n_experts, int x_per_slot, int log2g, int64_t expert_bytes) {
  extern __shared__ u32x4 x_lds4[];
  uint32_t* xl = reinterpret_cast<uint32_t*>(x_lds4);
  const int kdw = K / 2;
  const int nblk = K / 32;
  constexpr int UP = 4 * Fmt<FMT>::UB;   // x staged with an idle piece after each load unit
  const int xdw = 4 * xrun_pieces<UP>(MOE_COLS * (K / 8));
  float* xs = reinterpret_cast<float*>(xl + xdw);
  int* s_ids = reinterpret_cast<int*>(xs + MOE_COLS * nblk * 2);
  const int P = M * top_k;
  int* s_list = s_ids + P;
  __shared__ int s_cnt;
  const int p = blockIdx.y;
  // 1. routing: ids into LDS, then the owner test and the gather from LDS
  for (int q = threadIdx.x; q < P; q += 256) s_ids[q] = ids[q];
  __syncthreads();
  const int e = s_ids[p];
  int dup = 0;
  for (int q = threadIdx.x; q < p; q += 256) dup |= (s_ids[q] == e);
  if (__syncthreads_or(dup)) return;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int cnt = 0;
    for (int base = p; base < P; base += 64) {
      const int q = base + lane;
      const bool hit = q < P && s_ids[q] == e;
      const uint64_t mask = __ballot(hit);
      if (hit) s_list[cnt + __popcll(mask & ((1ull << lane) - 1ull))] = q;
      cnt += __popcll(mask);
    }
    if (lane == 0) s_cnt = cnt;
  }
  __syncthreads();
  const int cnt = s_cnt;
  const int lane = threadIdx.x & 63;
  const int G = 1 << log2g;
  const int rpw = 64 >> log2g;
  const int64_t row_base = (int64_t)(blockIdx.x * 4 + wave_id()) * rpw;
  const int rho = lane >> log2g, g = lane & (G - 1);
  if (e < 0 || e >= n_experts) {   // precondition violated: read nothing, flag with NaN
    if (g == 0 && row_base + rho < N) {
      for (int c = 0; c < cnt; ++c) {
        if constexpr (GATE_UP) static_cast<uint16_t*>(out)[(int64_t)s_list[c] * N + row_base + rho] = 0x7e00;
        else static_cast<float*>(out)[(int64_t)s_list[c] * N + row_base + rho] = __builtin_nanf("");
      }
    }
    return;
  }
  const uint32_t row_bytes = (uint32_t)nblk * Fmt<FMT>::BB;
  const int valid = row_base < N ? (int)min<int64_t>(rpw, N - row_base) : 0;
  const int64_t off = (int64_t)e * expert_bytes + (valid ? row_base * row_bytes : 0);
  const rsrc_t r0 = make_rsrc(W0 + off, (uint32_t)valid * row_bytes);
  const rsrc_t r1 = make_rsrc((GATE_UP ? W1 : W0) + off, (uint32_t)valid * row_bytes);
  const uint32_t roff = (uint32_t)rho * row_bytes;
  const int units = K / (32 * Fmt<FMT>::UB);
  const int kq8 = K / 8;
  const int xrows = (GATE_UP || !x_per_slot) ? M : P;
  const rsrc_t xsrc = make_rsrc(x, (uint32_t)xrows * (uint32_t)K * 2u);
  // a 16-byte slot after the slot list for pieces past the x area
  const int idle = (int)(((uint32_t)(xdw + MOE_COLS * nblk * 2 + 2 * P) * 4u + 15u) / 16u);
  for (int c0 = 0; c0 < cnt; c0 += MOE_COLS) {
    const int mt = cnt - c0 < MOE_COLS ? cnt - c0 : MOE_COLS;
    if (c0 > 0) __syncthreads();   // the previous pass has finished reading LDS
    // x of this pass's tokens, then the weights (so writing x waits for x alone).
    // The stores below are unconditional: a load used only inside a branch
    // would be moved behind the weight loads, and writing x would then wait
    // for them too. Loads a whole wave would make past the pass's x are not
    // issued (a wave-uniform test): they would still occupy the address unit.
    u32x4 xr[MOE_XCH];
    const int wave_i0 = wave_id() * 64;
#pragma unroll
    for (int c = 0; c < MOE_XCH; ++c) {
      const int i = (int)threadIdx.x + 256 * c;
      const int m = i / kq8, k8 = i - m * kq8;
      const int q = s_list[c0 + (m < mt ? m : 0)];
      const uint32_t xrow = (uint32_t)((GATE_UP || !x_per_slot) ? q / top_k : q);
      xr[c] = wave_i0 + 256 * c < mt * kq8 ? ld128(xsrc, m < mt ? (xrow * (uint32_t)kq8 + (uint32_t)k8) * 16u : OOB)
                                           : u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_sched_barrier(0);
    Loaded<FMT, ITERS> w0, w1;
    issue_units<FMT, ITERS>(r0, roff, g, G, units, w0);
    if constexpr (GATE_UP) issue_units<FMT, ITERS>(r1, roff, g, G, units, w1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < MOE_XCH; ++c) {
      const int i = (int)threadIdx.x + 256 * c;
      x_lds4[i < MOE_COLS * kq8 ? xphys<UP>(i) : idle] = xr[c];   // unused pieces land past the x of this pass
    }
    __syncthreads();
    block_sums_to_lds<UP>(xl, kdw, mt, xs, 256);
    __syncthreads();
    float a0[MOE_COLS], a1[MOE_COLS];
#pragma unroll
    for (int m = 0; m < MOE_COLS; ++m) a0[m] = a1[m] = 0.0f;
    switch (mt) {
#define KQ_MOE_CONSUME(MTV)                                                                                  \
  case MTV: {                                                                                                \
    float b0[MTV], b1[MTV];                                                                                  \
    for (int m = 0; m < MTV; ++m) b0[m] = b1[m] = 0.0f;                                                      \
    consume_units<FMT, MTV, ITERS, true>(w0, xl, xs, kdw, g, G, units, b0);                                  \
    if constexpr (GATE_UP) consume_units<FMT, MTV, ITERS, true>(w1, xl, xs, kdw, g, G, units, b1);           \
    group_reduce<MTV>(b0, G);                                                                                \
    if constexpr (GATE_UP) group_reduce<MTV>(b1, G);                                                         \
    for (int m = 0; m < MTV; ++m) { a0[m] = b0[m]; a1[m] = b1[m]; }                                          \
    break;                                                                                                   \
  }
      KQ_MOE_CONSUME(1)
      KQ_MOE_CONSUME(2)
      KQ_MOE_CONSUME(3)
      default: KQ_MOE_CONSUME(4)
#undef KQ_MOE_CONSUME
    }
    if (g == 0 && rho < valid) {
      for (int m = 0; m < mt; ++m) {
        const int64_t o = (int64_t)s_list[c0 + m] * N + row_base + rho;
        if constexpr (GATE_UP) {
          const float z = a0[m];
          static_cast<uint16_t*>(out)[o] = (uint16_t)f2h_bits(z / (1.0f + __expf(-z)) * a1[m]);
        } else {
          static_cast<float*>(out)[o] = a0[m];
        }
      }
    }
  }
}

// One token (M = 1): gate|up + SwiGLU with the routing off the weights' path.
// Grid and lane layout as k_moe_lds (row tiles x top_k slots, G lanes per
// row). The workgroup of slot p reads its expert id e with a scalar load,
// issues the token's activation loads, then its gate and up weight loads,
// and only then checks (scalar loads of the earlier slots' ids) whether an
// earlier slot names e: then it stops, and that slot's workgroup writes h for
// every slot routed to e. A router gives one token distinct experts, so the
// early weight loads are normally all used. The sums are those of k_moe_lds
// for one column (the same h bits). Dynamic LDS: x (K fp16), its block sums,
// a 16-byte idle slot. K <= 256 * 8 * XCH, top_k <= 16, expert_bytes < 2^31.
typedef const __attribute__((address_space(4))) int32_t* const_id_ptr;

template <int FMT, int ITERS, int XCH, int NIDS>
__global__ __launch_bounds__(256) void k_moe_gate_up_one(const uint8_t* __restrict__ Wg,
                                                        const uint8_t* __restrict__ Wu,
                                                        const uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ ids,
                                                        uint16_t* __restrict__ h, int expert_bytes, int N, int K,
                                                        int top_k, int n_experts, int log2g) {
  extern __shared__ u32x4 x_lds4[];
  uint32_t* xl = reinterpret_cast<uint32_t*>(x_lds4);
  const int kdw = K / 2;
  const int nblk = K / 32;
  constexpr int UP = 4 * Fmt<FMT>::UB;   // x staged with an idle piece after each load unit
  const int xdw = 4 * xrun_pieces<UP>(K / 8);
  float* xs = reinterpret_cast<float*>(xl + xdw);
  const int p = blockIdx.y;
  // the token's activations: registers, ahead of the weights
  const int kq8 = K / 8;
  const rsrc_t xsrc = make_rsrc(x, (uint32_t)K * 2u);
  u32x4 xr[XCH];
  const int wave_i0 = wave_id() * 64;
#pragma unroll
  for (int c = 0; c < XCH; ++c) {   // (loads a whole wave would make past x are not issued)
    const int i = (int)threadIdx.x + 256 * c;
    xr[c] = wave_i0 + 256 * c < kq8 ? ld128(xsrc, i < kq8 ? (uint32_t)i * 16u : OOB) : u32x4{0u, 0u, 0u, 0u};
  }
  __builtin_amdgcn_sched_barrier(0);
  // every slot's id in one round of scalar loads (NIDS >= top_k of them,
  // indexes clamped into the table), this slot's picked out by selects
  const const_id_ptr sid = (const_id_ptr)ids;
  int idv[NIDS];
#pragma unroll
  for (int q = 0; q < NIDS; ++q) idv[q] = sid[q < top_k ? q : top_k - 1];
  int e = idv[0];
#pragma unroll
  for (int q = 1; q < NIDS; ++q) e = q == p ? idv[q] : e;
  const bool ok = e >= 0 && e < n_experts;   // else read nothing, write NaN
  const int lane = threadIdx.x & 63;
  const int G = 1 << log2g;
  const int rpw = 64 >> log2g;
  const int64_t row_base = (int64_t)(blockIdx.x * 4 + wave_id()) * rpw;
  const int rho = lane >> log2g, g = lane & (G - 1);
  const uint32_t row_bytes = (uint32_t)nblk * Fmt<FMT>::BB;
  const int rows = row_base < N ? (int)min<int64_t>(rpw, N - row_base) : 0;
  const int valid = ok ? rows : 0;
  const int64_t off = valid ? (int64_t)e * expert_bytes + row_base * row_bytes : 0;
  const rsrc_t r0 = make_rsrc(Wg + off, (uint32_t)valid * row_bytes);
  const rsrc_t r1 = make_rsrc(Wu + off, (uint32_t)valid * row_bytes);
  const uint32_t roff = (uint32_t)rho * row_bytes;
  const int units = K / (32 * Fmt<FMT>::UB);
  Loaded<FMT, ITERS> w0, w1;
  issue_units<FMT, ITERS>(r0, roff, g, G, units, w0);
  issue_units<FMT, ITERS>(r1, roff, g, G, units, w1);
  __builtin_amdgcn_sched_barrier(0);
  // an earlier slot with the same expert serves this one
  bool dup = false;
#pragma unroll
  for (int q = 0; q < NIDS; ++q) dup |= q < p && idv[q] == e;
  if (dup) return;   // uniform over the workgroup
  const int idle = (xdw + nblk * 2 + 3) / 4;
#pragma unroll
  for (int c = 0; c < XCH; ++c) {
    const int i = (int)threadIdx.x + 256 * c;
    x_lds4[i < kq8 ? xphys<UP>(i) : idle] = xr[c];   // unused pieces land in the idle slot
  }
  __syncthreads();
  block_sums_to_lds<UP>(xl, kdw, 1, xs, 256);
  __syncthreads();
  float b0[1] = {0.0f}, b1[1] = {0.0f};
  consume_units<FMT, 1, ITERS, true>(w0, xl, xs, kdw, g, G, units, b0);
  consume_units<FMT, 1, ITERS, true>(w1, xl, xs, kdw, g, G, units, b1);
  group_reduce<1>(b0, G);
  group_reduce<1>(b1, G);
  if (g == 0 && rho < rows) {
    const float z = b0[0];
    const uint16_t hv = ok ? (uint16_t)f2h_bits(z / (1.0f + __expf(-z)) * b1[0]) : (uint16_t)0x7e00;
#pragma unroll
    for (int q = 0; q < NIDS; ++q)
      if (q >= p && q < top_k && idv[q] == e) h[(int64_t)q * N + row_base + rho] = hv;
  }
}

// One token (M = 1), weighted: the down projection of every routed slot and
// their weighted sum in one launch. Workgroup = top_k waves over the same rpw
// rows; wave j computes slot j exactly as k_moe_lds does for one column (x of
// the slot staged in LDS with its block sums, the same lane groups and units),
// leaves its row results in LDS, and the first wave adds them in slot order as
// k_weighted_slot_sum does, so y has the same bits as the three-kernel path.
// An id outside [0, n_experts) makes that slot's result, and so y, NaN.
// Dynamic LDS: per slot the x row (K fp16) and its block sums (K/32 x 2 fp32),
// then top_k x rpw fp32 slot results.
template <int FMT, int ITERS>
__global__ __launch_bounds__(1024) void k_moe_down_sum(const uint8_t* __restrict__ W, const uint16_t* __restrict__ x,
                                                      const int32_t* __restrict__ ids, int expert_bytes, int N, int K,
                                                      int n_experts, int log2g, int x_per_slot, int top_k,
                                                      const float* __restrict__ rw, float* __restrict__ y) {
  extern __shared__ u32x4 x_lds4[];
  const int lane = threadIdx.x & 63;
  const int j = wave_id();                       // this wave's slot
  const int kdw = K / 2, nblk = K / 32;
  constexpr int UP = 4 * Fmt<FMT>::UB;           // x staged with an idle piece after each load unit
  const int xdw = 4 * xrun_pieces<UP>(K / 8);
  const int slot_dw = xdw + nblk * 2;            // x dwords + block sums of one slot
  uint32_t* xl = reinterpret_cast<uint32_t*>(x_lds4) + (int64_t)j * slot_dw;
  float* xs = reinterpret_cast<float*>(xl + xdw);
  float* s_y = reinterpret_cast<float*>(reinterpret_cast<uint32_t*>(x_lds4) + (int64_t)top_k * slot_dw);
  const int G = 1 << log2g;
  const int rpw = 64 >> log2g;
  const int64_t row_base = (int64_t)blockIdx.x * rpw;
  const int rho = lane >> log2g, g = lane & (G - 1);
  const int valid = row_base < N ? (int)min<int64_t>(rpw, N - row_base) : 0;
  const int kq8 = K / 8;
  // x of this slot into registers (it does not depend on the route id), then
  // the id (a scalar load; the arguments it needs are in preloaded
  // registers), then the weights, then x into LDS
  const rsrc_t xsrc = make_rsrc(x + (int64_t)(x_per_slot ? j : 0) * K, (uint32_t)K * 2u);
  u32x4 xr[MOE_XCH];
#pragma unroll
  for (int c = 0; c < MOE_XCH; ++c) {
    const int i = lane + 64 * c;
    xr[c] = ld128(xsrc, i < kq8 ? (uint32_t)i * 16u : OOB);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int e = ((const_id_ptr)ids)[j];
  const bool e_ok = e >= 0 && e < n_experts;
  const uint32_t row_bytes = (uint32_t)nblk * Fmt<FMT>::BB;
  const int64_t off = (int64_t)(e_ok ? e : 0) * expert_bytes + (valid ? row_base * row_bytes : 0);
  const rsrc_t rs = make_rsrc(W + off, e_ok ? (uint32_t)valid * row_bytes : 0u);
  const uint32_t roff = (uint32_t)rho * row_bytes;
  const int units = K / (32 * Fmt<FMT>::UB);
  Loaded<FMT, ITERS> w;
  issue_units<FMT, ITERS>(rs, roff, g, G, units, w);
  __builtin_amdgcn_sched_barrier(0);
  u32x4* xl4 = reinterpret_cast<u32x4*>(xl);
#pragma unroll
  for (int c = 0; c < MOE_XCH; ++c) {
    const int i = lane + 64 * c;
    if (i < kq8) xl4[xphys<UP>(i)] = xr[c];
  }
  __syncthreads();
  // block sums of this slot's x (as block_sums_to_lds for one column)
  for (int h = lane; h < kdw / 8; h += 64) {
    const u32x4* q = reinterpret_cast<const u32x4*>(xl) + xphys<UP>(2 * h);
    const u32x4 a = q[0], c = q[1];
    float v = 0.0f;
    v = dot2(a.x, ONES, v); v = dot2(a.y, ONES, v); v = dot2(a.z, ONES, v); v = dot2(a.w, ONES, v);
    v = dot2(c.x, ONES, v); v = dot2(c.y, ONES, v); v = dot2(c.z, ONES, v); v = dot2(c.w, ONES, v);
    xs[h] = v;
  }
  __syncthreads();
  float acc[1] = {0.0f};
  consume_units<FMT, 1, ITERS, true>(w, xl, xs, kdw, g, G, units, acc);
  group_reduce<1>(acc, G);
  if (g == 0 && rho < valid) s_y[j * rpw + rho] = e_ok ? acc[0] : __builtin_nanf("");
  __syncthreads();
  if (j == 0 && g == 0 && rho < valid) {
    float t = 0.0f;
    for (int q = 0; q < top_k; ++q) t = __builtin_fmaf(rw[q], s_y[q * rpw + rho], t);
    y[row_base + rho] = t;
  }
}

// Generic routed kernel for rows that are only 2-byte aligned (Q4_0/Q8_0 with
// an odd number of blocks per row): one wave per (row, slot), per-block loads.
template <int FMT>
__global__ __launch_bounds__(256) void k_moe_generic(const uint8_t* __restrict__ W,
                                                     const uint16_t* __restrict__ x,
                                                     const int32_t* __restrict__ ids,
                                                     float* __restrict__ y_slot, int N, int K,
                                                     int top_k, int n_experts, int x_per_slot,
                                                     int64_t expert_bytes) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  const int p = blockIdx.y;
  if (row >= N) return;
  const int e = ids[p];
  if (e < 0 || e >= n_experts) {
    if (lane == 0) y_slot[(int64_t)p * N + row] = __builtin_nanf("");
    return;
  }
  const int nb = K / 32;
  const int64_t row_bytes = (int64_t)nb * Fmt<FMT>::BB;
  const uint8_t* Wr = W + (int64_t)e * expert_bytes + row * row_bytes;
  const uint16_t* xr = x + (int64_t)(x_per_slot ? p : p / top_k) * K;
  float acc = 0.0f;
  for (int b = lane; b < nb; b += 64) {
    const uint16_t* blk = reinterpret_cast<const uint16_t*>(Wr + (int64_t)b * Fmt<FMT>::BB);
    const uint16_t* xb = xr + b * 32;
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
        const int q[4] = {(int)(two & 15), (int)((two >> 4) & 15), (int)((two >> 8) & 15), (int)((two >> 12) & 15)};
        const int el[4] = {2 * j, 2 * j + 16, 2 * j + 1, 2 * j + 17};
        for (int i = 0; i < 4; ++i) {
          const float w = FMT == F_AFFINE4 ? __builtin_fmaf(s, (float)q[i], bias) : s * (float)(q[i] - 8);
          acc = __builtin_fmaf(w, h2f(xb[el[i]]), acc);
        }
      }
    }
  }
  acc = group_sum(acc, 64);
  if (lane == 0) y_slot[(int64_t)p * N + row] = acc;
}

}  // namespace kqd

namespace kq {

using namespace kqd;

namespace {

int ilog2(int v) {
  int l = 0;
  while ((1 << (l + 1)) <= v) ++l;
  return l;
}

// Expert matrices are small (a few MB), so prefer many waves: G near units/4,
// one row per lane.
int moe_log2g(int units) {
  int G = 1 << ilog2(units / 4 > 0 ? units / 4 : 1);
  G = G < 4 ? 4 : (G > 64 ? 64 : G);
  return ilog2(G);
}

// The LDS-staged kernel: rows of whole units, and MOE_COLS tokens' x within
// 256 threads x MOE_XCH pieces.
bool moe_lds_fits(int64_t K) { return (int64_t)MOE_COLS * (K / 8) <= 256 * MOE_XCH; }

// G lanes per row giving each lane about 128 bytes of weights (at most 5
// units; the larger G on a tie).
template <int FMT>
int moe_lds_log2g(int units) {
  constexpr int UBYTES = Fmt<FMT>::BB * Fmt<FMT>::UB;
  int best = -1, G = 64;
  for (int g = 64; g >= 1; g >>= 1) {
    const int it = (units + g - 1) / g;
    if (it > 5) break;
    const int dev = it * UBYTES > 128 ? it * UBYTES - 128 : 128 - it * UBYTES;
    if (best < 0 || dev < best) {
      best = dev;
      G = g;
    }
  }
  return ilog2(G);
}

// Few routed slots (one token): widen the lane groups (fewer rows per wave,
// fewer units per lane) while the per-slot grid of 4-wave workgroups is below
// MOE_MIN_WG, so the weights of 8 experts are spread over more CUs. The rule
// depends on the slot count, not on which slots are duplicates, so the fused
// one-token down kernel and the per-slot kernel pick the same G (the same
// per-row sums, bit for bit). The moe_min_wg tuning override replaces the
// threshold (0 keeps the byte-per-lane choice).
constexpr int MOE_MIN_WG = 512;

template <int FMT>
int moe_slot_log2g(int units, int64_t N, int P) {
  int log2g = moe_lds_log2g<FMT>(units);
  const int tv = tune(TUNE_MOE_MIN_WG);
  const int64_t min_wg = tv != TUNE_UNSET ? tv : MOE_MIN_WG;
  while (log2g < 6 && ((units + (1 << log2g) - 1) >> log2g) > 1) {
    const int64_t rpw = 64 >> log2g;
    const int64_t wg = ((N + rpw - 1) / rpw + 3) / 4 * P;
    if (wg >= min_wg) break;
    ++log2g;
  }
  return log2g;
}

template <int FMT, bool GATE_UP>
int launch_moe_lds(const uint8_t* W0, const uint8_t* W1, const uint16_t* x, const int32_t* ids, void* out, int64_t N,
                   int64_t K, int M, int top_k, int n_experts, int x_per_slot, int64_t eb, hipStream_t stream) {
  const int units = (int)(K / (32 * Fmt<FMT>::UB));
  const int log2g = moe_slot_log2g<FMT>(units, N, M * top_k);
  const int iters = (units + (1 << log2g) - 1) >> log2g;
  const int64_t rpw = 64 >> log2g;
  const int64_t waves = (N + rpw - 1) / rpw;
  const int P = M * top_k;
  const dim3 grid((unsigned)((waves + 3) / 4), (unsigned)P), block(256);
  const size_t lds = (size_t)16 * xrun_pieces<4 * Fmt<FMT>::UB>((int)(MOE_COLS * K / 8)) +
                     (size_t)MOE_COLS * (K / 32) * 8 + (size_t)2 * P * 4 + 32;
  dispatch_log(GATE_UP ? "k_moe_lds(gate|up+swiglu)" : "k_moe_lds", FMT, N, K, M, grid.x, grid.y, 256, lds,
               "G=%d units/lane=%d slots=%d", 1 << log2g, iters, P);
#define KQ_MOE_LAUNCH(IT)                                                                                       \
  hipLaunchKernelGGL((k_moe_lds<FMT, IT, GATE_UP>), grid, block, lds, stream, W0, W1, x, ids, out, (int)N, (int)K, \
                     M, top_k, n_experts, x_per_slot, log2g, eb)
  switch (iters) {
    case 1: KQ_MOE_LAUNCH(1); break;
    case 2: KQ_MOE_LAUNCH(2); break;
    case 3: KQ_MOE_LAUNCH(3); break;
    case 4: KQ_MOE_LAUNCH(4); break;
    default: KQ_MOE_LAUNCH(5); break;
  }
#undef KQ_MOE_LAUNCH
  return (int)hipGetLastError();
}

template <int FMT>
int moe_dispatch(const MoeArgs& a) {
  const int64_t eb = a.N * (a.K / 32) * Fmt<FMT>::BB;
  const int P = a.M * a.top_k;
  if (a.K % (32 * Fmt<FMT>::UB) != 0) {
    const dim3 grid((unsigned)((a.N + 3) / 4), (unsigned)P), block(256);
    hipLaunchKernelGGL((k_moe_generic<FMT>), grid, block, 0, a.stream, a.W, a.x, a.ids, a.y_slot,
                       (int)a.N, (int)a.K, a.top_k, a.n_experts, a.x_per_slot, eb);
    return (int)hipGetLastError();
  }
  const int units = (int)(a.K / (32 * Fmt<FMT>::UB));
  if (moe_lds_fits(a.K)) return launch_moe_lds<FMT, false>(a.W, nullptr, a.x, a.ids, a.y_slot, a.N, a.K, a.M,
                                                            a.top_k, a.n_experts, a.x_per_slot, eb, a.stream);
  const int log2g = moe_log2g(units);
  const int64_t tile = 64 >> log2g;
  const int64_t waves = (a.N + tile - 1) / tile;
  const dim3 grid((unsigned)((waves + 3) / 4), (unsigned)P), block(256);
  hipLaunchKernelGGL((k_moe_valu<FMT, 1>), grid, block, 0, a.stream, a.W, a.x, a.ids, a.y_slot,
                     (int)a.N, (int)a.K, a.M, a.top_k, a.n_experts, a.x_per_slot, log2g, eb);
  return (int)hipGetLastError();
}

// LDS bytes of k_moe_gate_up_one: x (padded), its block sums, an idle slot.
template <int FMT>
int64_t moe_one_lds_bytes(int64_t hidden) {
  return 16 * (int64_t)xrun_pieces<4 * Fmt<FMT>::UB>((int)(hidden / 8)) + (hidden / 32) * 8 + 32;
}

template <int FMT, int XCH, int NIDS>
int launch_moe_gate_up_one(const MoeGateUpArgs& a, int64_t eb) {
  const int units = (int)(a.hidden / (32 * Fmt<FMT>::UB));
  const int log2g = moe_slot_log2g<FMT>(units, a.inter, a.top_k);
  const int iters = (units + (1 << log2g) - 1) >> log2g;
  const int64_t rpw = 64 >> log2g;
  const int64_t waves = (a.inter + rpw - 1) / rpw;
  const dim3 grid((unsigned)((waves + 3) / 4), (unsigned)a.top_k), block(256);
  const size_t lds = moe_one_lds_bytes<FMT>(a.hidden);
  dispatch_log("k_moe_gate_up_one", FMT, a.inter, a.hidden, 1, grid.x, grid.y, 256, lds, "G=%d units/lane=%d slots=%d",
               1 << log2g, iters, a.top_k);
#define KQ_MOE_ONE(IT)                                                                                        \
  hipLaunchKernelGGL((k_moe_gate_up_one<FMT, IT, XCH, NIDS>), grid, block, lds, a.stream, a.Wg, a.Wu, a.x, a.ids, a.h, \
                     (int)eb, (int)a.inter, (int)a.hidden, a.top_k, a.n_experts, log2g)
  switch (iters) {
    case 1: KQ_MOE_ONE(1); break;
    case 2: KQ_MOE_ONE(2); break;
    case 3: KQ_MOE_ONE(3); break;
    case 4: KQ_MOE_ONE(4); break;
    default: KQ_MOE_ONE(5); break;
  }
#undef KQ_MOE_ONE
  return (int)hipGetLastError();
}

template <int FMT>
int gate_up_dispatch(const MoeGateUpArgs& a) {
  const int64_t eb = a.inter * (a.hidden / 32) * Fmt<FMT>::BB;
  const int P = a.M * a.top_k;
  const int units = (int)(a.hidden / (32 * Fmt<FMT>::UB));
  // one token: the routing-off-the-path kernel (the moe_one tuning override,
  // 0, forces the general kernel)
  if (a.M == 1 && a.top_k <= 16 && a.hidden % (32 * Fmt<FMT>::UB) == 0 && tune(TUNE_MOE_ONE) != 0 &&
      eb <= INT32_MAX && moe_one_lds_bytes<FMT>(a.hidden) <= 64 * 1024) {
    if (a.hidden / 8 <= 256)
      return a.top_k <= 8 ? launch_moe_gate_up_one<FMT, 1, 8>(a, eb) : launch_moe_gate_up_one<FMT, 1, 16>(a, eb);
    if (a.hidden / 8 <= 1024)
      return a.top_k <= 8 ? launch_moe_gate_up_one<FMT, 4, 8>(a, eb) : launch_moe_gate_up_one<FMT, 4, 16>(a, eb);
  }
  if (moe_lds_fits(a.hidden))
    return launch_moe_lds<FMT, true>(a.Wg, a.Wu, a.x, a.ids, a.h, a.inter, a.hidden, a.M, a.top_k, a.n_experts, 0,
                                     eb, a.stream);
  const int log2g = moe_log2g(units);
  const int64_t tile = 64 >> log2g;
  const int64_t waves = (a.inter + tile - 1) / tile;
  const dim3 grid((unsigned)((waves + 3) / 4), (unsigned)P), block(256);
  hipLaunchKernelGGL((k_moe_gate_up<FMT, 1>), grid, block, 0, a.stream, a.Wg, a.Wu, a.x, a.ids, a.h,
                     (int)a.inter, (int)a.hidden, a.M, a.top_k, a.n_experts, log2g, eb);
  return (int)hipGetLastError();
}

template <int FMT>
int launch_moe_down_sum_fmt(const MoeArgs& a, const float* rw, float* y) {
  const int64_t eb = a.N * (a.K / 32) * Fmt<FMT>::BB;
  const int units = (int)(a.K / (32 * Fmt<FMT>::UB));
  const int log2g = moe_slot_log2g<FMT>(units, a.N, a.M * a.top_k);
  const int iters = (units + (1 << log2g) - 1) >> log2g;
  const int64_t rpw = 64 >> log2g;
  const dim3 grid((unsigned)((a.N + rpw - 1) / rpw)), block((unsigned)(64 * a.top_k));
  const size_t lds = (size_t)a.top_k * ((size_t)16 * xrun_pieces<4 * Fmt<FMT>::UB>((int)(a.K / 8)) +
                                         (size_t)(a.K / 32) * 8) + (size_t)a.top_k * rpw * 4;
  dispatch_log("k_moe_down_sum", FMT, a.N, a.K, a.M, grid.x, 1, block.x, lds, "G=%d units/lane=%d top_k=%d",
               1 << log2g, iters, a.top_k);
#define KQ_MOE_DS(IT)                                                                                          \
  hipLaunchKernelGGL((k_moe_down_sum<FMT, IT>), grid, block, lds, a.stream, a.W, a.x, a.ids, (int)eb, (int)a.N,    \
                     (int)a.K, a.n_experts, log2g, a.x_per_slot, a.top_k, rw, y)
  switch (iters) {
    case 1: KQ_MOE_DS(1); break;
    case 2: KQ_MOE_DS(2); break;
    case 3: KQ_MOE_DS(3); break;
    case 4: KQ_MOE_DS(4); break;
    default: KQ_MOE_DS(5); break;
  }
#undef KQ_MOE_DS
  return (int)hipGetLastError();
}

}  // namespace

bool moe_down_sum_applies(const MoeArgs& a) {
  const int ub = (a.fmt == KQ_AFFINE4_G32 || a.fmt == KQ_Q5_1) ? 1 : 2;   // blocks per load unit
  return a.M == 1 && a.top_k >= 1 && a.top_k <= 16 && a.K % (32 * ub) == 0 && moe_lds_fits(a.K) &&
         a.K / 8 <= 64 * MOE_XCH && a.N * (a.K / 32) * 34 <= INT32_MAX;   // expert bytes as an int
}

int launch_moe_down_sum(const MoeArgs& a, const float* route_w, float* y) {
  switch (a.fmt) {
    case KQ_Q8_0: return launch_moe_down_sum_fmt<F_Q8_0>(a, route_w, y);
    case KQ_Q4_0: return launch_moe_down_sum_fmt<F_Q4_0>(a, route_w, y);
    case KQ_Q5_0: return launch_moe_down_sum_fmt<F_Q5_0>(a, route_w, y);
    case KQ_Q5_1: return launch_moe_down_sum_fmt<F_Q5_1>(a, route_w, y);
    default: return launch_moe_down_sum_fmt<F_AFFINE4>(a, route_w, y);
  }
}

int launch_moe_gemv(const MoeArgs& a) {
  switch (a.fmt) {
    case KQ_Q8_0: return moe_dispatch<F_Q8_0>(a);
    case KQ_Q4_0: return moe_dispatch<F_Q4_0>(a);
    case KQ_Q5_0: return moe_dispatch<F_Q5_0>(a);
    case KQ_Q5_1: return moe_dispatch<F_Q5_1>(a);
    default: return moe_dispatch<F_AFFINE4>(a);
  }
}

int launch_moe_gate_up_swiglu(const MoeGateUpArgs& a) {
  switch (a.fmt) {
    case KQ_Q8_0: return gate_up_dispatch<F_Q8_0>(a);
    case KQ_Q4_0: return gate_up_dispatch<F_Q4_0>(a);
    case KQ_Q5_0: return gate_up_dispatch<F_Q5_0>(a);
    case KQ_Q5_1: return gate_up_dispatch<F_Q5_1>(a);
    default: return gate_up_dispatch<F_AFFINE4>(a);
  }
}

}  // namespace kq
