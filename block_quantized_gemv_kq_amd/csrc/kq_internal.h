// kq_internal.h — declarations shared by the C-ABI layer, the host packer
// and the kernel launchers. Not part of the public interface.
#pragma once

#include <stdint.h>

#include "../../include/kq.h"

typedef struct ihipStream_t* hipStream_t;

namespace kq {

// ---- tuning overrides (kq_set_tuning). Every default is the measured
// choice; an override forces another kernel or configuration so that tests
// can reach each path at small shapes and sweeps can compare them. The
// environment is never read.
enum TuneKey {
  TUNE_FORCE_PATH,       // 'g' generic, 'v' register-x VALU, 'l' LDS VALU, 'm' matrix cores
  TUNE_VALU_G,           // lanes per row of the VALU kernels
  TUNE_VALU_R,           // rows per lane of the register-x kernel
  TUNE_LDS_WPG,          // waves per workgroup of the one-column LDS kernel
  TUNE_MFMA_VARIANT,     // MfmaVariant below
  TUNE_MFMA_S,           // waves per tile (split-K teams kernel)
  TUNE_MFMA_R,           // tiles per workgroup (split-K teams kernel)
  TUNE_MFMA_WAVES,       // wave count below which the teams kernel doubles S
  TUNE_MFMA_XF,          // teams kernel, x through registers: 1 x written first, 0 weights first
  TUNE_MFMA_PERS_TPW,    // persistent kernel: tiles per wave
  TUNE_MFMA_PERS_WAVES,  // persistent kernel: waves per workgroup
  TUNE_MFMA_CHUNK_L2CG,  // chunked kernel: log2 of groups per chunk
  TUNE_MOE_UNFUSED,      // 1: one-token MoE down + weighted sum as two kernels
  TUNE_MOE_MIN_WG,       // routed-expert kernels: widen lane groups below this many workgroups
  TUNE_MOE_ONE,          // 0: one-token gate|up through the general routed-expert kernel
  TUNE_MFMA_SPLIT,       // K splits of the teams kernel when a workspace is given (1: none)
  TUNE_SL_G,             // lanes per row of the Shortlist bound kernel
  TUNE_LOG,              // 1: one line per kernel launch on stderr (the dispatch log)
  TUNE_LDS_XDMA,         // 1: the one-column LDS kernel copies x by DMA even where registers would do
  TUNE_MFMA_XDMA,        // teams kernel: 1 x by DMA, column-major; 0 through registers
  TUNE_COUNT
};
enum MfmaVariant { MV_PERS = 1, MV_TEAMS, MV_TEAMS_SX, MV_CHUNK, MV_CHUNK_WHOLE, MV_CHUNK_SPLIT, MV_DIRECT };
constexpr int TUNE_UNSET = -0x7fffffff;
// The override of `k`, or TUNE_UNSET.
int tune(TuneKey k);
// Compute units of the current device (looked up once per device).
int device_cus();
// Dispatch log: when the log override is 1, one line on stderr per kernel
// launch: kernel, format, shape, grid, workgroup size, LDS bytes and the
// configuration the dispatcher chose (free text).
void dispatch_log(const char* kernel, int fmt, int64_t N, int64_t K, int M, unsigned gx, unsigned gy,
                  unsigned block, size_t lds, const char* cfg_fmt, ...);

// ---- host packer (kq_pack.cpp)
int64_t block_bytes(int fmt);
int pack(int fmt, const float* W, int64_t N, int64_t K, void* out, int n_threads);
int unpack(int fmt, const void* packed, int64_t N, int64_t K, float* W);
uint16_t f32_to_f16_bits(float f);
float f16_bits_to_f32(uint16_t h);
// Shortlist bound copy of a Q8_0 matrix (K a multiple of 256).
int64_t shortlist_copy_bytes(int64_t N, int64_t K);
int shortlist_pack(const void* q8, int64_t N, int64_t K, void* out, int n_threads);

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
  void* ws = nullptr;        // caller's workspace for K-split partial sums (kq_gemv_ws), or none
  int64_t ws_bytes = 0;
};
// Workspace bytes the matrix-core path would use for a K split of this call
// (0: no split).
int64_t gemv_split_bytes(const GemvArgs& a);
int launch_gemv(const GemvArgs& a);
int launch_gemv_invariant(const GemvArgs& a);
// GEMV then the argmax of every column (out: device int32 [M]); ws holds the
// partials (gemv_argmax_fused_parts(a) per column when fused, else kq_argmax's).
int launch_gemv_argmax(const GemvArgs& a, int32_t* out, void* ws);
int64_t gemv_argmax_fused_parts(const GemvArgs& a);
// The same with the partials in the library's static scratch array of the
// current device (KQ_NOALLOC_SCRATCH_BYTES; the caller checks the size).
int launch_gemv_argmax_noalloc(const GemvArgs& a, int32_t* out);
int launch_gemv_mfma(const GemvArgs& a);
// Per-row configuration of the one-column GEMV kernel for a Q8_0 matrix of
// this shape: lanes per row (log2), units per lane, passes. A row computed
// with it has the bits kq_gemv gives that row.
struct RowCfg {
  int log2g, iters, passes;
};
RowCfg q8_row_cfg(int64_t N, int64_t K);

// Shortlist argmax over a Q8_0 output layer (one column).
struct ShortlistArgs {
  const uint8_t* W;     // Q8_0 matrix
  const uint8_t* Wc;    // its bound copy
  const uint16_t* x;
  int64_t N;
  int64_t K;
  void* ws;
  int32_t* out;         // device int32 [1]
  int32_t* kept;        // device int32 [1] or null: rows scored exactly
  hipStream_t stream;
};
int64_t shortlist_workspace_bytes(int64_t N, int64_t K);
int launch_shortlist_argmax(const ShortlistArgs& a);
// The matrix-core GEMV with every configuration chosen from N and K alone
// (batch-invariant columns).
int launch_gemv_mfma_invariant(const GemvArgs& a);

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
// One token, weighted: per-slot outputs and their slot-order weighted sum in
// one launch (same bits as launch_moe_gemv + launch_weighted_slot_sum);
// moe_down_sum_applies tells whether the shape allows it.
bool moe_down_sum_applies(const MoeArgs& a);
int launch_moe_down_sum(const MoeArgs& a, const float* route_w, float* y);

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

// The persistent chain's workgroup shape: STACK_CWAVES compute waves and one
// control wave; STACK_NT compute lanes.
constexpr int STACK_CWAVES = 11;
constexpr int STACK_NT = 64 * STACK_CWAVES;

// One stage of a persistent GEMV chain (M = 1), as the kernel reads it (128 B).
// The plan fixes the number of workgroups nb (one per CU): workgroup b owns
// rows [b*rows_per + min(b, rows_rem), ...), rows_per + (b < rows_rem) of them.
// Within a workgroup, G = 2^log2g lanes share a row; lane group gamma of the
// STACK_NT / G groups takes rows gamma, gamma + groups, ... and lane g of it
// units g, g + G, ... of each row: kpr = ceil(upr / G) steps per row.
struct StackStage {
  const uint8_t* W;
  const uint16_t* x;       // activations from outside the chain (ll_in == nullptr)
  float* y;
  uint16_t* y16;           // optional fp16 copy of y
  uint32_t* ll_out;        // tagged fp16 outputs that later stages read, or nullptr
  const uint32_t* ll_in;   // the K tagged words holding x, or nullptr
  int32_t N;
  int32_t K;
  int32_t fmt;
  int32_t upr;             // load units per row (1 block for affine4, 2 for Q4_0/Q8_0)
  int32_t row_bytes;
  int32_t rows_per;        // N / nb
  int32_t rows_rem;        // N % nb
  int32_t log2g;           // lanes per row = 2^log2g
  int32_t kpr;             // steps per row = ceil(upr / G)
  int32_t dep;             // stage whose outputs ll_in points into, or -1
  int32_t ll_out_stride;   // words between the replicas of ll_out
  int32_t ll_in_stride;    // words between the replicas of ll_in
  int32_t pad[8];
};
static_assert(sizeof(StackStage) == 128, "stage descriptor is 128 bytes");

// Limits of the persistent chain and the layout of its sync words (32-bit
// words after the stage descriptors; each has a 128-byte line of its own).
constexpr int STACK_MAX_WG = 1024;          // workgroups (CUs) a plan can span
constexpr int STACK_MAX_SHARE_ROWS = 4096;  // rows of one stage per workgroup
constexpr int STACK_MAX_K = 16384;          // inputs per row
// Copies of each tagged output: workgroup b reads copy b % STACK_LL_COPIES, so
// each copy is read by a fraction of the grid instead of all of it.
constexpr int STACK_LL_COPIES = 8;
constexpr int64_t STACK_ERR_WORD = 0;
constexpr int64_t STACK_EPOCH_WORD = 32;                         // + 32 * workgroup
constexpr int64_t STACK_HINT_WORD = 32 + 32 * STACK_MAX_WG;      // + 32 * workgroup
constexpr int64_t STACK_SYNC_WORDS = 32 + 2 * 32 * STACK_MAX_WG;
// Lanes per row for a stage of `rows_max` rows per workgroup and `upr` units
// per row: the G in {4, ..., 64} with the fewest steps per lane.
int stack_log2g(int64_t rows_max, int upr);
int64_t stack_lds_bytes(int kmax);
int launch_stack(const StackStage* stages, int n_stages, uint32_t* sync, int fmask, int nb, int kmax,
                 hipStream_t stream);
int stack_device_info(int* cus);
int copy_to_device(void* dst, const void* src, int64_t bytes, hipStream_t stream);
int read_from_device(void* dst, const void* src, int64_t bytes, hipStream_t stream);

int64_t argmax_partials(int64_t N);
int launch_argmax(const float* y, int64_t N, int M, int32_t* out, void* ws, hipStream_t stream);
int launch_argmax_final(const void* part, int nparts, int M, int32_t* out, hipStream_t stream);

const char* hip_error_string(int err);

}  // namespace kq
