// kq_misc.hip — small kernels around the GEMVs: the fixed-order weighted sum
// of routed-expert outputs, and the greedy argmax over a vocabulary-sized
// output layer (Kinetic docs, "What makes it fast": choosing the next token
// reads an output layer of up to a quarter of a million rows).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_dev.h"
#include "kq_internal.h"

namespace kqd {

// y[m][n] = sum_j w[m][j] * ys[m][j][n], accumulated in slot order j = 0..top_k-1.
__global__ __launch_bounds__(256) void k_weighted_slot_sum(const float* __restrict__ ys,
                                                           const float* __restrict__ w,
                                                           float* __restrict__ y, int64_t N,
                                                           int top_k) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= N) return;
  const float* base = ys + (int64_t)m * top_k * N + n;
  const float* wm = w + (int64_t)m * top_k;
  float acc = 0.0f;
  int j = 0;
  for (; j + 8 <= top_k; j += 8) {   // eight independent loads in flight, then the sums in order
    float v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = base[(int64_t)(j + t) * N];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc = __builtin_fmaf(wm[j + t], v[t], acc);
  }
  for (; j < top_k; ++j) acc = __builtin_fmaf(wm[j], base[(int64_t)j * N], acc);
  y[(int64_t)m * N + n] = acc;
}


template <int NT>
__device__ __forceinline__ Best block_best(Best b, Best* s_red) {
  for (int off = 32; off > 0; off >>= 1) {
    Best o{__shfl_xor(b.v, off, 64), __shfl_xor(b.i, off, 64)};
    b = better(b, o);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) s_red[wave] = b;
  __syncthreads();
  if (threadIdx.x == 0) {
    Best r = s_red[0];
    for (int w = 1; w < NT / 64; ++w) r = better(r, s_red[w]);
    s_red[0] = r;
  }
  __syncthreads();
  return s_red[0];
}

constexpr int ARGMAX_CHUNK = 2048;  // 8 values per thread: many workgroups per column

__global__ __launch_bounds__(256) void k_argmax_partial(const float* __restrict__ y, int64_t N,
                                                        Best* __restrict__ part, int nparts) {
  __shared__ Best s_red[4];
  const int m = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * ARGMAX_CHUNK;
  const int64_t c1 = c0 + ARGMAX_CHUNK < N ? c0 + ARGMAX_CHUNK : N;
  const float* row = y + (int64_t)m * N;
  Best b{-__builtin_inff(), INT32_MAX};
  int64_t i = c0 + threadIdx.x;
  for (; i + 7 * 256 < c1; i += 8 * 256) {   // eight loads in flight, then the comparisons in order
    float v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = row[i + t * 256];
#pragma unroll
    for (int t = 0; t < 8; ++t) b = better(b, Best{v[t], (int32_t)(i + t * 256)});
  }
  for (; i < c1; i += 256) b = better(b, Best{row[i], (int32_t)i});
  b = block_best<256>(b, s_red);
  if (threadIdx.x == 0) part[(int64_t)m * nparts + blockIdx.x] = b;
}

// NT threads (the workgroup size as a constant: reading it at run time would
// put a scalar load of the dispatch arguments ahead of the first loads).
template <int NT>
__global__ __launch_bounds__(NT) void k_argmax_final(const Best* __restrict__ part, int nparts,
                                                     int32_t* __restrict__ out) {
  __shared__ Best s_red[16];
  const int m = blockIdx.x;
  const Best* p = part + (int64_t)m * nparts;
  Best b{-__builtin_inff(), INT32_MAX};
  constexpr int nt = NT;
  int i = threadIdx.x;
  for (; i + 3 * nt < nparts; i += 4 * nt) {   // four loads in flight per thread
    const Best a0 = p[i], a1 = p[i + nt], a2 = p[i + 2 * nt], a3 = p[i + 3 * nt];
    b = better(better(b, a0), better(better(a1, a2), a3));
  }
  for (; i < nparts; i += nt) b = better(b, p[i]);
  b = block_best<NT>(b, s_red);
  if (threadIdx.x == 0) out[m] = b.i == INT32_MAX ? 0 : b.i;
}

}  // namespace kqd

namespace kq {

using namespace kqd;

int launch_weighted_slot_sum(const float* ys, const float* w, float* y, int64_t N, int M, int top_k,
                             hipStream_t stream) {
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)M), block(256);
  hipLaunchKernelGGL(k_weighted_slot_sum, grid, block, 0, stream, ys, w, y, N, top_k);
  return (int)hipGetLastError();
}

int64_t argmax_partials(int64_t N) { return (N + ARGMAX_CHUNK - 1) / ARGMAX_CHUNK; }

int launch_argmax_final(const void* part, int nparts, int M, int32_t* out, hipStream_t stream) {
  if (nparts >= 4096)
    hipLaunchKernelGGL(k_argmax_final<1024>, dim3((unsigned)M), dim3(1024), 0, stream,
                       static_cast<const Best*>(part), nparts, out);
  else
    hipLaunchKernelGGL(k_argmax_final<256>, dim3((unsigned)M), dim3(256), 0, stream,
                       static_cast<const Best*>(part), nparts, out);
  return (int)hipGetLastError();
}

int launch_argmax(const float* y, int64_t N, int M, int32_t* out, void* ws, hipStream_t stream) {
  const int nparts = (int)argmax_partials(N);
  Best* part = static_cast<Best*>(ws);
  dispatch_log("k_argmax_partial+final", -1, N, 0, M, (unsigned)nparts, (unsigned)M, 256, 0, "two passes");
  hipLaunchKernelGGL(k_argmax_partial, dim3((unsigned)nparts, (unsigned)M), dim3(256), 0, stream, y, N,
                     part, nparts);
  int err = (int)hipGetLastError();
  if (err) return err;
  hipLaunchKernelGGL(k_argmax_final<256>, dim3((unsigned)M), dim3(256), 0, stream, part, nparts, out);
  return (int)hipGetLastError();
}

}  // namespace kq
