// kq_stack.hip — a chain of dependent M = 1 GEMVs (one decode token through a
// dense stack) in ONE persistent launch.
//
// A decode step is hundreds of small GPU kernels, and recording it once and
// replaying it with one call per token removes the launch cost (Kinetic docs,
// "What makes it fast", the paragraph on recording the step). On MI355X even a
// replayed graph pays ~1.6 us between dependent kernels, and every kernel
// ramps up and drains, so a 4B-shaped layer (four GEMVs of 6.5-31 MB) cannot
// stream near the HBM rate as separate launches. Here all stages run in one
// grid that stays resident:
//   * each workgroup (one per CU) owns an equal, contiguous share of stage s's
//     rows and walks it in rounds (every wave takes 64/G rows per round, G
//     lanes per row), two rounds in flight in registers;
//   * a workgroup that finishes its share arrives at a device-wide barrier for
//     s; before stage s+1 reads its activations it waits until all workgroups
//     arrived (so x of stage s+1 may be y of stage s);
//   * weights do not depend on activations, so the first two stage-(s+1)
//     rounds of a workgroup are loaded into registers BEFORE it waits: HBM
//     keeps streaming across the barrier.
// Waits are bounded: a workgroup that waits too long sets an error word and
// goes on, so the grid always drains.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_dev.h"
#include "kq_internal.h"

namespace kqd {

using kq::StackStage;

constexpr int STACK_ITERS_NIB = 5;   // affine4 / Q4_0 units per lane per tile
constexpr int STACK_ITERS_Q8 = 2;    // Q8_0 (34-byte blocks, 2 per unit)
// Waves per workgroup (one workgroup per CU): 16 when only affine4 stages
// are present (the kernel then fits 128 VGPRs, 4 waves per SIMD), else 8.
template <int FMASK> struct StackWaves { static constexpr int v = FMASK == (1 << F_AFFINE4) ? 16 : 8; };
constexpr uint32_t SPIN_LIMIT = 1u << 22;

// Barrier words: one 128-byte line each, so arrivals on different counters
// never share a line. Per stage: STACK_GROUPS group counters, one total
// counter, STACK_GROUPS release flags. Then a "done" line and an error line.
constexpr int LINE_WORDS = 32;
constexpr int STACK_GROUPS = 8;      // one per XCD (workgroups are dealt to XCDs round-robin)
constexpr int LINES_PER_STAGE = 2 * STACK_GROUPS + 1;

// Register buffer for one tile's weights, sized for the largest format in use.
template <int FMASK>
struct RawSize {
  static constexpr int a4 = (FMASK & (1 << F_AFFINE4)) ? STACK_ITERS_NIB * Fmt<F_AFFINE4>::UDW : 1;
  static constexpr int q4 = (FMASK & (1 << F_Q4_0)) ? STACK_ITERS_NIB * Fmt<F_Q4_0>::UDW : 1;
  static constexpr int q8 = (FMASK & (1 << F_Q8_0)) ? STACK_ITERS_Q8 * Fmt<F_Q8_0>::UDW : 1;
  static constexpr int m1 = a4 > q4 ? a4 : q4;
  static constexpr int v = m1 > q8 ? m1 : q8;
};

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every vector memory operation this wave issued has completed
// (stores acknowledged); also a compiler barrier for memory.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Rows of stage d owned by workgroup b of nb: [r0, r1).
__device__ __forceinline__ void share(const StackStage& d, int b, int nb, int64_t& r0, int64_t& r1) {
  r0 = d.N * b / nb;
  r1 = d.N * (b + 1) / nb;
}

// Round k of a workgroup's share: wave w takes rows r0 + (k * WAVES + w) * rpw, rpw of them.
template <int FMASK>
__device__ __forceinline__ void issue_round(const StackStage& d, int64_t r0, int64_t r1, int k, uint32_t* raw) {
  constexpr int WAVES = StackWaves<FMASK>::v;
  const int lane = threadIdx.x & 63;
  const int G = 1 << d.log2g, rpw = 64 >> d.log2g;
  const uint32_t row_bytes = (uint32_t)(d.K / 32) * (uint32_t)d.block_bytes;
  const int64_t row_base = r0 + ((int64_t)k * WAVES + wave_id()) * rpw;
  const int valid = row_base < r1 ? (int)min<int64_t>(rpw, r1 - row_base) : 0;
  const rsrc_t rs = make_rsrc(d.W + (valid ? row_base * row_bytes : 0), (uint32_t)valid * row_bytes);
  const uint32_t roff = (uint32_t)(lane >> d.log2g) * row_bytes;
  const int g = lane & (G - 1);
  if ((FMASK & (1 << F_AFFINE4)) && d.fmt == F_AFFINE4)
    issue_units_raw<F_AFFINE4, STACK_ITERS_NIB>(rs, roff, g, G, d.units, raw);
  else if ((FMASK & (1 << F_Q4_0)) && d.fmt == F_Q4_0)
    issue_units_raw<F_Q4_0, STACK_ITERS_NIB>(rs, roff, g, G, d.units, raw);
  else if ((FMASK & (1 << F_Q8_0)) && d.fmt == F_Q8_0)
    issue_units_raw<F_Q8_0, STACK_ITERS_Q8>(rs, roff, g, G, d.units, raw);
}

// Outputs go straight to the device coherence point (agent-scope stores), so
// workgroups on other XCDs read them after the barrier without cache flushes.
template <int FMASK>
__device__ __forceinline__ void finish_round(const StackStage& d, int64_t r0, int64_t r1, int k,
                                             const uint32_t* raw, const uint32_t* xl, const float* xs) {
  constexpr int WAVES = StackWaves<FMASK>::v;
  const int lane = threadIdx.x & 63;
  const int G = 1 << d.log2g, rpw = 64 >> d.log2g;
  const int64_t row_base = r0 + ((int64_t)k * WAVES + wave_id()) * rpw;
  if (row_base >= r1) return;   // wave-uniform: this wave has no rows in round k
  const int g = lane & (G - 1), rho = lane >> d.log2g;
  float acc[1] = {0.0f};
  if ((FMASK & (1 << F_AFFINE4)) && d.fmt == F_AFFINE4)
    acc[0] = consume_units_raw<F_AFFINE4, STACK_ITERS_NIB>(raw, xl, xs, g, G, d.units);
  else if ((FMASK & (1 << F_Q4_0)) && d.fmt == F_Q4_0)
    acc[0] = consume_units_raw<F_Q4_0, STACK_ITERS_NIB>(raw, xl, xs, g, G, d.units);
  else if ((FMASK & (1 << F_Q8_0)) && d.fmt == F_Q8_0)
    acc[0] = consume_units_raw<F_Q8_0, STACK_ITERS_Q8>(raw, xl, xs, g, G, d.units);
  group_reduce<1>(acc, G);
  const int64_t row = row_base + rho;
  if (g == 0 && row < r1) {
    __hip_atomic_store(d.y + row, acc[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d.y16)
      __hip_atomic_store(d.y16 + row, (uint16_t)f2h_bits(acc[0]), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Copy x (K fp16) into LDS with loads that read the device coherence point
// (a previous stage may just have written it from another XCD).
__device__ __forceinline__ void stage_x_coherent(const uint16_t* x, uint32_t* xl, int n16) {
  constexpr int SC1 = 16;   // cache-policy bit: device-scope coherent load
  for (int i = threadIdx.x; i < n16; i += blockDim.x) {
    const int wave_first = i - (int)(threadIdx.x & 63);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(reinterpret_cast<const u32x4*>(x) + i),
                                     (lds_void_t*)(xl + 4 * wave_first), 16, 0, SC1);
  }
}

// Arrival at the barrier of stage s: per-XCD-group counter, the last of a
// group adds to the total, the last group raises every group's flag.
__device__ __forceinline__ void stage_arrive(uint32_t* st_lines, int nb) {
  wait_vmem();              // this wave's outputs are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const int g = blockIdx.x % STACK_GROUPS;
    const int gsize = nb / STACK_GROUPS + (g < nb % STACK_GROUPS ? 1 : 0);
    const int ngroups = nb < STACK_GROUPS ? nb : STACK_GROUPS;
    if (add_dev(st_lines + g * LINE_WORDS, 1u) == (uint32_t)gsize - 1) {
      if (add_dev(st_lines + STACK_GROUPS * LINE_WORDS, 1u) == (uint32_t)ngroups - 1) {
        for (int k = 0; k < ngroups; ++k) st_dev(st_lines + (STACK_GROUPS + 1 + k) * LINE_WORDS, 1u);
      }
    }
  }
}

__device__ __forceinline__ void stage_wait(const uint32_t* st_lines, uint32_t* err) {
  if (threadIdx.x == 0) {
    const uint32_t* flag = st_lines + (STACK_GROUPS + 1 + blockIdx.x % STACK_GROUPS) * LINE_WORDS;
    uint32_t spins = 0;
    while (ld_dev(flag) == 0) {
      if (++spins > SPIN_LIMIT) {
        add_dev(err, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// Rounds of stage d for a share of r1 - r0 rows.
template <int FMASK>
__device__ __forceinline__ int rounds_of(const StackStage& d, int64_t r0, int64_t r1) {
  const int64_t per = (int64_t)StackWaves<FMASK>::v * (64 >> d.log2g);
  return (int)((r1 - r0 + per - 1) / per);
}

template <int FMASK>
__device__ __forceinline__ void issue_first_two(const StackStage& d, int b, int nb, uint32_t* A, uint32_t* B) {
  int64_t r0, r1;
  share(d, b, nb, r0, r1);
  const int n = rounds_of<FMASK>(d, r0, r1);
  if (n > 0) issue_round<FMASK>(d, r0, r1, 0, A);
  if (n > 1) issue_round<FMASK>(d, r0, r1, 1, B);
}

template <int FMASK>
__global__ __launch_bounds__(64 * StackWaves<FMASK>::v) void k_stack(
    const StackStage* __restrict__ stages, int n_stages, uint32_t* __restrict__ sync) {
  extern __shared__ u32x4 lds4[];
  uint32_t* xl = reinterpret_cast<uint32_t*>(lds4);
  uint32_t* done = sync + (size_t)n_stages * LINES_PER_STAGE * LINE_WORDS;
  uint32_t* err = done + LINE_WORDS;
  __shared__ int s_last;
  const int nb = gridDim.x, b = blockIdx.x;
  // Two rounds in flight: round k of a stage lives in A when k is even, B
  // when odd; after consuming round k its buffer takes round k + 2.
  uint32_t A[RawSize<FMASK>::v], B[RawSize<FMASK>::v];

  issue_first_two<FMASK>(stages[0], b, nb, A, B);
  for (int s = 0; s < n_stages; ++s) {
    const StackStage d = stages[s];
    uint32_t* lines = sync + (size_t)s * LINES_PER_STAGE * LINE_WORDS;
    if (s > 0) stage_wait(lines - LINES_PER_STAGE * LINE_WORDS, err);
    int64_t r0, r1;
    share(d, b, nb, r0, r1);
    const int n = rounds_of<FMASK>(d, r0, r1);
    if (n > 0) {
      const int kdw = d.K / 2;
      float* xs = reinterpret_cast<float*>(xl + kdw);
      stage_x_coherent(d.x, xl, d.K / 8);
      __syncthreads();
      block_sums_to_lds(xl, kdw, 1, xs);
      __syncthreads();
      for (int k = 0; k < n; ++k) {
        if ((k & 1) == 0) {
          finish_round<FMASK>(d, r0, r1, k, A, xl, xs);
          if (k + 2 < n) issue_round<FMASK>(d, r0, r1, k + 2, A);
        } else {
          finish_round<FMASK>(d, r0, r1, k, B, xl, xs);
          if (k + 2 < n) issue_round<FMASK>(d, r0, r1, k + 2, B);
        }
      }
    }
    stage_arrive(lines, nb);
    // the next stage's first two rounds stream in while the barrier completes
    if (s + 1 < n_stages) issue_first_two<FMASK>(stages[s + 1], b, nb, A, B);
  }
  // The last workgroup out clears the barrier words for the next launch:
  // every workgroup has passed all of its waits once `done` reaches nb.
  __syncthreads();
  if (threadIdx.x == 0) s_last = add_dev(done, 1u) == (uint32_t)nb - 1;
  __syncthreads();
  if (s_last) {
    const int words = n_stages * LINES_PER_STAGE * LINE_WORDS;
    for (int i = threadIdx.x; i < words; i += blockDim.x) st_dev(sync + i, 0u);
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0) st_dev(done, 0u);
  }
}

}  // namespace kqd

namespace kq {

using namespace kqd;

int stack_iters(int fmt) { return fmt == KQ_Q8_0 ? STACK_ITERS_Q8 : STACK_ITERS_NIB; }
int stack_waves(int fmask) { return fmask == (1 << F_AFFINE4) ? StackWaves<4>::v : StackWaves<1>::v; }
int64_t stack_sync_words(int n_stages) { return ((int64_t)n_stages * LINES_PER_STAGE + 2) * LINE_WORDS; }
int64_t stack_error_word(int n_stages) { return ((int64_t)n_stages * LINES_PER_STAGE + 1) * LINE_WORDS; }

int stack_device_info(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  return (int)e;
}

int copy_to_device(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  hipError_t e = hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return (int)e;
}

int read_from_device(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  hipError_t e = hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return (int)e;
}

namespace {

template <int FMASK>
int launch_stack_mask(const StackStage* stages, int n_stages, uint32_t* sync, int kmax,
                      hipStream_t stream) {
  static int cached_blocks[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return (int)hipErrorInvalidDevice;
  const size_t lds = (size_t)kmax * 2 + (size_t)(kmax / 32) * 8;  // x + block sums
  int& nb = cached_blocks[dev & 63];
  if (nb == 0) {
    int cus = 0, per_cu = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stack<FMASK>,
                                                     64 * StackWaves<FMASK>::v, 64 * 1024);
    if (e != hipSuccess) return (int)e;
    // Every workgroup must be resident at once (they wait on each other):
    // one per CU, and only if the occupancy calculation allows it.
    if (per_cu < 1) return (int)hipErrorLaunchOutOfResources;
    nb = cus;
  }
  hipLaunchKernelGGL((k_stack<FMASK>), dim3((unsigned)nb), dim3(64 * StackWaves<FMASK>::v), lds, stream,
                     stages, n_stages, sync);
  return (int)hipGetLastError();
}

}  // namespace

int launch_stack(const StackStage* stages, int n_stages, uint32_t* sync, int fmask, int kmax,
                 hipStream_t stream) {
  switch (fmask) {
    case 1: return launch_stack_mask<1>(stages, n_stages, sync, kmax, stream);
    case 2: return launch_stack_mask<2>(stages, n_stages, sync, kmax, stream);
    case 3: return launch_stack_mask<3>(stages, n_stages, sync, kmax, stream);
    case 4: return launch_stack_mask<4>(stages, n_stages, sync, kmax, stream);
    case 5: return launch_stack_mask<5>(stages, n_stages, sync, kmax, stream);
    case 6: return launch_stack_mask<6>(stages, n_stages, sync, kmax, stream);
    default: return launch_stack_mask<7>(stages, n_stages, sync, kmax, stream);
  }
}

}  // namespace kq
