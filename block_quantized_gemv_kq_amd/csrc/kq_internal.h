// kq_internal.h — declarations shared by the C-ABI layer, the host packer
// and the kernel launchers. Not part of the public interface.
#pragma once

#include <stdint.h>

#include "../../include/kq.h"

typedef struct ihipStream_t* hipStream_t;

namespace kq {

// ---- host packer (kq_pack.cpp)
int64_t block_bytes(int fmt);
int pack(int fmt, const float* W, int64_t N, int64_t K, void* out, int n_threads);
int unpack(int fmt, const void* packed, int64_t N, int64_t K, float* W);
uint16_t f32_to_f16_bits(float f);
float f16_bits_to_f32(uint16_t h);

// ---- launchers (kernels in *.hip). Each returns 0 or a HIP error code.
// Arguments are validated by the C-ABI layer before these are called.

struct GemvArgs {
  int fmt;
  const uint8_t* W;
  const uint16_t* x;
  float* y;
  int64_t N;
  int64_t K;
  int M;
  hipStream_t stream;
};
int launch_gemv(const GemvArgs& a);
int launch_gemv_mfma(const GemvArgs& a);

struct MoeArgs {
  int fmt;
  const uint8_t* W;         // [E][N][K/32] blocks
  const uint16_t* x;        // [M][K] or [M][top_k][K]
  const int32_t* ids;       // [M][top_k]
  float* y_slot;            // [M][top_k][N] per-slot outputs
  int64_t N;
  int64_t K;
  int M;
  int top_k;
  int n_experts;
  int x_per_slot;
  hipStream_t stream;
};
int launch_moe_gemv(const MoeArgs& a);

struct MoeGateUpArgs {
  int fmt;
  const uint8_t* Wg;        // [E][inter][hidden/32]
  const uint8_t* Wu;
  const uint16_t* x;        // [M][hidden]
  const int32_t* ids;
  uint16_t* h;              // [M][top_k][inter] fp16 bits
  int64_t inter;
  int64_t hidden;
  int M;
  int top_k;
  int n_experts;
  hipStream_t stream;
};
int launch_moe_gate_up_swiglu(const MoeGateUpArgs& a);

// y[m][n] = sum_j w[m][j] * ys[m][j][n], slot order.
int launch_weighted_slot_sum(const float* ys, const float* w, float* y, int64_t N, int M,
                             int top_k, hipStream_t stream);

// One stage of a persistent GEMV chain (M = 1), as the kernel reads it.
struct StackStage {
  const uint8_t* W;
  const uint16_t* x;
  float* y;
  uint16_t* y16;   // optional fp16 copy of y
  int64_t N;
  int32_t K;
  int32_t fmt;
  int32_t block_bytes;
  int32_t log2g;   // lanes per row = 2^log2g; a wave takes 64 >> log2g rows per round
  int32_t tiles;   // unused (0)
  int32_t units;   // load units per row (1 block for affine4, 2 for Q4_0/Q8_0)
};
int stack_iters(int fmt);
int stack_waves(int fmask);
int64_t stack_sync_words(int n_stages);
int64_t stack_error_word(int n_stages);
int launch_stack(const StackStage* stages, int n_stages, uint32_t* sync, int fmask, int kmax,
                 hipStream_t stream);
int stack_device_info(int* cus);
int copy_to_device(void* dst, const void* src, int64_t bytes, hipStream_t stream);
int read_from_device(void* dst, const void* src, int64_t bytes, hipStream_t stream);

int64_t argmax_partials(int64_t N);
int launch_argmax(const float* y, int64_t N, int M, int32_t* out, void* ws, hipStream_t stream);

const char* hip_error_string(int err);

}  // namespace kq
