// kq_probe.hip — measurement only (libkq_probe.so, loaded by the benchmark,
// never by the GEMV library): a read-only streaming kernel that gives the
// rate at which this GPU can read a buffer of a given size in one launch,
// the ceiling any one-launch-per-matrix GEMV is compared against.
//
// Each workgroup reads one contiguous chunk of 256 * 16 * PER bytes: thread t
// issues all PER of its 16-byte buffer loads (pieces i * 256 + t of the chunk,
// the same load the GEMV kernels use) before it uses any, folds them with XOR,
// and stores the word only if it equals a value the caller passes (never met
// for the benchmark's data), so no load is dead and nothing is written: no
// barrier, no reduction, no tail beyond the loads. Loads past the end read zero.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int PER>
__global__ __launch_bounds__(256) void k_stream_read(const uint8_t* __restrict__ p, uint32_t bytes,
                                                     uint32_t* __restrict__ sink, uint32_t match) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, (int)bytes, 0x00020000);
  const uint32_t base = blockIdx.x * (256u * 16u * PER) + threadIdx.x * 16u;
  u32x4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, base + (uint32_t)i * 4096u, 0, 0);
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (acc == match) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Read `bytes` (< 4 GiB - 1 MiB, a multiple of 16) at device address p once,
// `per` (1, 2, 4, 8 or 16) 16-byte loads per thread, 256 threads per
// workgroup; sink: device uint32 [ceil(bytes / (4096 * per))], written only
// where a workgroup's XOR of its loads equals 0x9e3779b9. Returns the number
// of workgroups launched, or a negative value on a bad argument.
int kq_probe_stream_read(const void* p, int64_t bytes, uint32_t* sink, int per, void* stream) {
  if (!p || !sink || bytes <= 0 || bytes % 16 || bytes >= ((int64_t)1 << 32) - (1 << 20)) return -1;
  const int64_t chunk = 4096LL * per;
  const unsigned wg = (unsigned)((bytes + chunk - 1) / chunk);
  hipStream_t s = (hipStream_t)stream;
  const uint8_t* b = static_cast<const uint8_t*>(p);
  const uint32_t n = (uint32_t)bytes;
  switch (per) {
    case 1: hipLaunchKernelGGL(k_stream_read<1>, dim3(wg), dim3(256), 0, s, b, n, sink, 0x9e3779b9u); break;
    case 2: hipLaunchKernelGGL(k_stream_read<2>, dim3(wg), dim3(256), 0, s, b, n, sink, 0x9e3779b9u); break;
    case 4: hipLaunchKernelGGL(k_stream_read<4>, dim3(wg), dim3(256), 0, s, b, n, sink, 0x9e3779b9u); break;
    case 8: hipLaunchKernelGGL(k_stream_read<8>, dim3(wg), dim3(256), 0, s, b, n, sink, 0x9e3779b9u); break;
    case 16: hipLaunchKernelGGL(k_stream_read<16>, dim3(wg), dim3(256), 0, s, b, n, sink, 0x9e3779b9u); break;
    default: return -1;
  }
  const int err = (int)hipGetLastError();
  return err ? -err : (int)wg;
}

}  // extern "C"
