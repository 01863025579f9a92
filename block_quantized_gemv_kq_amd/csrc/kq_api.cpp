// kq_api.cpp — the C ABI: argument checks (all on the host, before any HIP
// call), thread-local error messages, and dispatch to the kernel launchers.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <vector>

#include "kq_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return KQ_OK;
}

bool valid_fmt(int fmt) {
  return fmt == KQ_Q8_0 || fmt == KQ_Q4_0 || fmt == KQ_AFFINE4_G32 || fmt == KQ_Q5_0 || fmt == KQ_Q5_1;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_fmt_k(int fmt, int64_t K) {
  if (!valid_fmt(fmt)) return fail(KQ_ERR_FORMAT, "unknown format %d", fmt);
  if (K <= 0 || K % 32 != 0 || K > KQ_MAX_K)
    return fail(KQ_ERR_SHAPE, "K=%lld must be a positive multiple of 32 and <= %d", (long long)K, KQ_MAX_K);
  return KQ_OK;
}

int check_n(int64_t N, const char* what) {
  if (N < 0 || N > KQ_MAX_N) return fail(KQ_ERR_ARG, "%s=%lld out of range", what, (long long)N);
  return KQ_OK;
}

// Overrides stored as value + 1, so the zero-initialised table means "none set".
std::atomic<int> g_tune[kq::TUNE_COUNT] = {};

struct TuneName {
  const char* name;
  kq::TuneKey key;
};
const TuneName kTuneNames[] = {
    {"force_path", kq::TUNE_FORCE_PATH},         {"valu_g", kq::TUNE_VALU_G},
    {"valu_r", kq::TUNE_VALU_R},                 {"lds_wpg", kq::TUNE_LDS_WPG},
    {"mfma_variant", kq::TUNE_MFMA_VARIANT},     {"mfma_s", kq::TUNE_MFMA_S},
    {"mfma_r", kq::TUNE_MFMA_R},                 {"mfma_waves", kq::TUNE_MFMA_WAVES},
    {"mfma_xf", kq::TUNE_MFMA_XF},               {"mfma_pers_tpw", kq::TUNE_MFMA_PERS_TPW},
    {"mfma_chunk_l2cg", kq::TUNE_MFMA_CHUNK_L2CG}, {"moe_unfused", kq::TUNE_MOE_UNFUSED},
    {"moe_min_wg", kq::TUNE_MOE_MIN_WG},          {"log", kq::TUNE_LOG},
    {"mfma_pers_waves", kq::TUNE_MFMA_PERS_WAVES}, {"moe_one", kq::TUNE_MOE_ONE},
    {"mfma_split", kq::TUNE_MFMA_SPLIT},         {"sl_g", kq::TUNE_SL_G},
    {"mfma_xdma", kq::TUNE_MFMA_XDMA},           {"lds_xdma", kq::TUNE_LDS_XDMA},
};

// Parse a tuning value: force_path and mfma_variant take names, the others integers.
bool parse_tune(kq::TuneKey key, const char* v, int* out) {
  if (key == kq::TUNE_FORCE_PATH) {
    if (strlen(v) != 1 || !strchr("gvlm", v[0])) return false;
    *out = v[0];
    return true;
  }
  if (key == kq::TUNE_MFMA_VARIANT) {
    static const char* names[] = {"pers", "teams", "teams_sx", "chunk", "chunk_whole", "chunk_split", "direct"};
    for (int i = 0; i < 7; ++i)
      if (!strcmp(v, names[i])) {
        *out = kq::MV_PERS + i;
        return true;
      }
    return false;
  }
  char* end = nullptr;
  const long n = strtol(v, &end, 10);
  if (end == v || *end != '\0' || n < 0 || n > 1 << 20) return false;
  *out = (int)n;
  return true;
}

int hip_status(int err, const char* where) {
  if (err == 0) return ok();
  return fail(KQ_ERR_HIP, "%s: HIP error %d (%s)", where, err, kq::hip_error_string(err));
}

}  // namespace

namespace kq {
int tune(TuneKey k) {
  const int v = g_tune[k].load(std::memory_order_relaxed);
  return v == 0 ? TUNE_UNSET : v - 1;
}

void dispatch_log(const char* kernel, int fmt, int64_t N, int64_t K, int M, unsigned gx, unsigned gy,
                  unsigned block, size_t lds, const char* cfg_fmt, ...) {
  if (tune(TUNE_LOG) != 1) return;
  static const char* names[] = {"q8_0", "q4_0", "affine4", "q5_0", "q5_1"};
  char cfg[256];
  va_list ap;
  va_start(ap, cfg_fmt);
  vsnprintf(cfg, sizeof(cfg), cfg_fmt, ap);
  va_end(ap);
  fprintf(stderr, "kq: %s fmt=%s N=%lld K=%lld M=%d grid=(%u,%u) block=%u lds=%zu %s\n", kernel,
          fmt >= 0 && fmt < 5 ? names[fmt] : "-", (long long)N, (long long)K, M, gx, gy, block, lds, cfg);
}
}  // namespace kq

extern "C" {

int kq_version(void) { return KQ_VERSION; }

const char* kq_status_string(int status) {
  switch (status) {
    case KQ_OK: return "KQ_OK";
    case KQ_ERR_ARG: return "KQ_ERR_ARG";
    case KQ_ERR_FORMAT: return "KQ_ERR_FORMAT";
    case KQ_ERR_SHAPE: return "KQ_ERR_SHAPE";
    case KQ_ERR_ALIGN: return "KQ_ERR_ALIGN";
    case KQ_ERR_RANGE: return "KQ_ERR_RANGE";
    case KQ_ERR_HIP: return "KQ_ERR_HIP";
    default: return "KQ_ERR_UNKNOWN";
  }
}

const char* kq_last_error(void) { return g_err; }

int kq_set_tuning(const char* name, const char* value) {
  if (!name) {
    for (auto& t : g_tune) t.store(0, std::memory_order_relaxed);
    return ok();
  }
  for (const TuneName& t : kTuneNames) {
    if (strcmp(t.name, name)) continue;
    if (!value || !value[0]) {
      g_tune[t.key].store(0, std::memory_order_relaxed);
      return ok();
    }
    int v;
    if (!parse_tune(t.key, value, &v)) return fail(KQ_ERR_ARG, "kq_set_tuning: bad value '%s' for %s", value, name);
    g_tune[t.key].store(v + 1, std::memory_order_relaxed);
    return ok();
  }
  return fail(KQ_ERR_ARG, "kq_set_tuning: unknown name '%s'", name);
}

int64_t kq_block_bytes(int fmt) {
  if (!valid_fmt(fmt)) return fail(KQ_ERR_FORMAT, "unknown format %d", fmt);
  return kq::block_bytes(fmt);
}

int64_t kq_packed_bytes(int fmt, int64_t N, int64_t K) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  return N * (K / 32) * kq::block_bytes(fmt);
}

int kq_pack(int fmt, const float* W, int64_t N, int64_t K, void* out, int n_threads) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  if (N > 0 && (!W || !out)) return fail(KQ_ERR_ARG, "kq_pack: null pointer");
  st = kq::pack(fmt, W, N, K, out, n_threads);
  if (st == KQ_ERR_RANGE)
    return fail(st, "kq_pack: non-finite weight, or a scale/bias that overflows fp16");
  return st ? st : ok();
}

int kq_unpack(int fmt, const void* packed, int64_t N, int64_t K, float* W_out) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  if (N > 0 && (!packed || !W_out)) return fail(KQ_ERR_ARG, "kq_unpack: null pointer");
  return kq::unpack(fmt, packed, N, K, W_out) ? KQ_ERR_ARG : ok();
}

int kq_f32_to_f16(const float* in, uint16_t* out, int64_t n) {
  if (n < 0 || (n > 0 && (!in || !out))) return fail(KQ_ERR_ARG, "kq_f32_to_f16: bad arguments");
  for (int64_t i = 0; i < n; ++i) out[i] = kq::f32_to_f16_bits(in[i]);
  return ok();
}

int kq_gemv(int fmt, const void* W, const uint16_t* x, float* y, int64_t N, int64_t K, int M,
            void* stream) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  if (M < 0 || M > KQ_MAX_M) return fail(KQ_ERR_ARG, "M=%d must be in [0, %d]", M, KQ_MAX_M);
  if (M == 0 || N == 0) return ok();
  if (!W || !x || !y) return fail(KQ_ERR_ARG, "kq_gemv: null pointer");
  if (!aligned(W, 4) || !aligned(y, 4)) return fail(KQ_ERR_ALIGN, "kq_gemv: W and y must be 4-byte aligned");
  if (!aligned(x, 16)) return fail(KQ_ERR_ALIGN, "kq_gemv: x must be 16-byte aligned");
  kq::GemvArgs a{fmt, static_cast<const uint8_t*>(W), x, y, N, K, M, static_cast<hipStream_t>(stream)};
  return hip_status(kq::launch_gemv(a), "kq_gemv");
}

int64_t kq_gemv_workspace_bytes(int fmt, int64_t N, int64_t K, int M) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  if (M < 0 || M > KQ_MAX_M) return fail(KQ_ERR_ARG, "M=%d must be in [0, %d]", M, KQ_MAX_M);
  kq::GemvArgs a{fmt, nullptr, nullptr, nullptr, N, K, M, nullptr};
  return kq::gemv_split_bytes(a);
}

int kq_gemv_ws(int fmt, const void* W, const uint16_t* x, float* y, int64_t N, int64_t K, int M, void* workspace,
               int64_t workspace_bytes, void* stream) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  if (M < 0 || M > KQ_MAX_M) return fail(KQ_ERR_ARG, "M=%d must be in [0, %d]", M, KQ_MAX_M);
  if (M == 0 || N == 0) return ok();
  if (!W || !x || !y) return fail(KQ_ERR_ARG, "kq_gemv_ws: null pointer");
  if (!aligned(W, 4) || !aligned(y, 4)) return fail(KQ_ERR_ALIGN, "kq_gemv_ws: W and y must be 4-byte aligned");
  if (!aligned(x, 16)) return fail(KQ_ERR_ALIGN, "kq_gemv_ws: x must be 16-byte aligned");
  if (workspace_bytes < 0) return fail(KQ_ERR_ARG, "kq_gemv_ws: negative workspace size");
  kq::GemvArgs a{fmt, static_cast<const uint8_t*>(W), x, y, N, K, M, static_cast<hipStream_t>(stream)};
  const int64_t need = kq::gemv_split_bytes(a);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(KQ_ERR_ARG, "kq_gemv_ws: workspace of %lld bytes needed", (long long)need);
    if (!aligned(workspace, 16)) return fail(KQ_ERR_ALIGN, "kq_gemv_ws: workspace must be 16-byte aligned");
    a.ws = workspace;
    a.ws_bytes = workspace_bytes;
  }
  return hip_status(kq::launch_gemv(a), "kq_gemv_ws");
}

int kq_gemv_invariant(int fmt, const void* W, const uint16_t* x, float* y, int64_t N, int64_t K, int M,
                      void* stream) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  if (M < 0 || M > KQ_MAX_M) return fail(KQ_ERR_ARG, "M=%d must be in [0, %d]", M, KQ_MAX_M);
  if (M == 0 || N == 0) return ok();
  if (!W || !x || !y) return fail(KQ_ERR_ARG, "kq_gemv_invariant: null pointer");
  if (!aligned(W, 4) || !aligned(y, 4))
    return fail(KQ_ERR_ALIGN, "kq_gemv_invariant: W and y must be 4-byte aligned");
  if (!aligned(x, 16)) return fail(KQ_ERR_ALIGN, "kq_gemv_invariant: x must be 16-byte aligned");
  kq::GemvArgs a{fmt, static_cast<const uint8_t*>(W), x, y, N, K, M, static_cast<hipStream_t>(stream)};
  return hip_status(kq::launch_gemv_invariant(a), "kq_gemv_invariant");
}

int64_t kq_moe_gemv_workspace_bytes(int64_t N, int M, int top_k, int weighted) {
  if (N < 0 || M < 0 || top_k < 0) return fail(KQ_ERR_ARG, "negative size");
  if (!weighted) return 0;
  return (int64_t)M * top_k * N * 4;
}

static int check_moe_common(int fmt, const void* Wexp, int64_t N, int64_t K, int M, int top_k,
                            int n_experts) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  if (M < 0 || M > KQ_MAX_M) return fail(KQ_ERR_ARG, "M=%d must be in [0, %d]", M, KQ_MAX_M);
  if (n_experts < 1) return fail(KQ_ERR_ARG, "n_experts=%d must be >= 1", n_experts);
  if (top_k < 1 || top_k > n_experts || top_k > 64)
    return fail(KQ_ERR_ARG, "top_k=%d must be in [1, min(n_experts, 64)]", top_k);
  const int64_t per = N * (K / 32) * kq::block_bytes(fmt);
  if (per > 0 && n_experts > INT64_MAX / per) return fail(KQ_ERR_ARG, "expert table too large");
  if (!aligned(Wexp, 4)) return fail(KQ_ERR_ALIGN, "expert weights must be 4-byte aligned");
  return KQ_OK;
}

int kq_moe_gemv(int fmt, const void* W_experts, const uint16_t* x, const int32_t* route_ids,
                const float* route_w, float* y, int64_t N, int64_t K, int M, int top_k,
                int n_experts, int x_per_slot, void* workspace, int64_t workspace_bytes,
                void* stream) {
  int st = check_moe_common(fmt, W_experts, N, K, M, top_k, n_experts);
  if (st) return st;
  if (x_per_slot != 0 && x_per_slot != 1) return fail(KQ_ERR_ARG, "x_per_slot must be 0 or 1");
  if (M == 0 || N == 0) return ok();
  if (!W_experts || !x || !route_ids || !y) return fail(KQ_ERR_ARG, "kq_moe_gemv: null pointer");
  if (!aligned(x, 16)) return fail(KQ_ERR_ALIGN, "kq_moe_gemv: x must be 16-byte aligned");
  if (!aligned(y, 4) || !aligned(route_ids, 4) || (route_w && !aligned(route_w, 4)))
    return fail(KQ_ERR_ALIGN, "kq_moe_gemv: y, route_ids, route_w must be 4-byte aligned");
  const int64_t need = kq_moe_gemv_workspace_bytes(N, M, top_k, route_w != nullptr);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(KQ_ERR_ARG, "kq_moe_gemv: workspace of %lld bytes needed", (long long)need);
    if (!aligned(workspace, 16)) return fail(KQ_ERR_ALIGN, "kq_moe_gemv: workspace must be 16-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* slots = route_w ? static_cast<float*>(workspace) : y;
  kq::MoeArgs a{fmt, static_cast<const uint8_t*>(W_experts), x, route_ids, slots, N, K, M, top_k,
                n_experts, x_per_slot, s};
  if (route_w && kq::moe_down_sum_applies(a) && kq::tune(kq::TUNE_MOE_UNFUSED) != 1)
    return hip_status(kq::launch_moe_down_sum(a, route_w, y), "kq_moe_gemv");
  int err = kq::launch_moe_gemv(a);
  if (!err && route_w) err = kq::launch_weighted_slot_sum(slots, route_w, y, N, M, top_k, s);
  return hip_status(err, "kq_moe_gemv");
}

int64_t kq_moe_ffn_workspace_bytes(int64_t hidden, int64_t inter, int M, int top_k) {
  if (hidden < 0 || inter < 0 || M < 0 || top_k < 0) return fail(KQ_ERR_ARG, "negative size");
  const int64_t h_bytes = ((int64_t)M * top_k * inter * 2 + 255) / 256 * 256;
  return h_bytes + (int64_t)M * top_k * hidden * 4;
}

int kq_moe_ffn(int fmt, const void* W_gate, const void* W_up, const void* W_down, const uint16_t* x,
               const int32_t* route_ids, const float* route_w, float* y, uint16_t* h_out,
               int64_t hidden, int64_t inter, int M, int top_k, int n_experts, void* workspace,
               int64_t workspace_bytes, void* stream) {
  int st = check_moe_common(fmt, W_gate, inter, hidden, M, top_k, n_experts);
  if (st) return st;
  if ((st = check_moe_common(fmt, W_down, hidden, inter, M, top_k, n_experts))) return st;
  if (!aligned(W_up, 4)) return fail(KQ_ERR_ALIGN, "W_up must be 4-byte aligned");
  if (fmt != KQ_AFFINE4_G32 && fmt != KQ_Q5_1 && hidden % 64 != 0)
    return fail(KQ_ERR_SHAPE, "kq_moe_ffn: Q8_0/Q4_0/Q5_0 need hidden %% 64 == 0");
  if (M == 0 || hidden == 0 || inter == 0) return ok();
  if (!W_gate || !W_up || !W_down || !x || !route_ids || !route_w || !y)
    return fail(KQ_ERR_ARG, "kq_moe_ffn: null pointer");
  if (!aligned(x, 16)) return fail(KQ_ERR_ALIGN, "kq_moe_ffn: x must be 16-byte aligned");
  if (!aligned(y, 4) || !aligned(route_ids, 4) || !aligned(route_w, 4))
    return fail(KQ_ERR_ALIGN, "kq_moe_ffn: y, route_ids, route_w must be 4-byte aligned");
  if (h_out && !aligned(h_out, 16)) return fail(KQ_ERR_ALIGN, "kq_moe_ffn: h_out must be 16-byte aligned");
  const int64_t need = kq_moe_ffn_workspace_bytes(hidden, inter, M, top_k);
  if (!workspace || workspace_bytes < need)
    return fail(KQ_ERR_ARG, "kq_moe_ffn: workspace of %lld bytes needed", (long long)need);
  if (!aligned(workspace, 16)) return fail(KQ_ERR_ALIGN, "kq_moe_ffn: workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t h_bytes = ((int64_t)M * top_k * inter * 2 + 255) / 256 * 256;
  uint16_t* h = h_out ? h_out : static_cast<uint16_t*>(workspace);
  float* slots = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + h_bytes);
  kq::MoeGateUpArgs g{fmt, static_cast<const uint8_t*>(W_gate), static_cast<const uint8_t*>(W_up),
                      x, route_ids, h, inter, hidden, M, top_k, n_experts, s};
  int err = kq::launch_moe_gate_up_swiglu(g);
  if (err) return hip_status(err, "kq_moe_ffn");
  kq::MoeArgs d{fmt, static_cast<const uint8_t*>(W_down), h, route_ids, slots, hidden, inter, M,
                top_k, n_experts, 1, s};
  if (kq::moe_down_sum_applies(d) && kq::tune(kq::TUNE_MOE_UNFUSED) != 1)
    return hip_status(kq::launch_moe_down_sum(d, route_w, y), "kq_moe_ffn");
  err = kq::launch_moe_gemv(d);
  if (!err) err = kq::launch_weighted_slot_sum(slots, route_w, y, hidden, M, top_k, s);
  return hip_status(err, "kq_moe_ffn");
}

static int64_t stack_descs_bytes(int n) {
  return ((int64_t)n * (int64_t)sizeof(kq::StackStage) + 255) / 256 * 256;
}

namespace {

struct Range {
  uintptr_t lo, hi;   // [lo, hi)
  bool overlaps(const Range& o) const { return lo < o.hi && o.lo < hi; }
  bool contains(const Range& o) const { return lo <= o.lo && o.hi <= hi; }
};

// The dataflow of a chain: for each stage, the earlier stage whose fp16
// output holds its x (or -1) and the element offset of x in it; plus the
// layout of the tagged buffers in the plan. Checks the stage fields and that
// no stage writes memory that another stage reads or writes (the kernel runs
// stages concurrently across workgroups, so only the x-in-an-earlier-y16
// pattern has a defined order).
struct ChainLayout {
  std::vector<int> dep;
  std::vector<int64_t> dep_off;     // elements
  std::vector<int64_t> ll_word;     // first tagged word of a stage's outputs, or -1
  std::vector<int64_t> ll_stride;   // words between the copies of a stage's outputs
  int64_t ll_words = 0;
};

int check_stages(const kq_stage* stages, int n, ChainLayout& L) {
  if (n < 1 || n > KQ_STACK_MAX_STAGES)
    return fail(KQ_ERR_ARG, "n_stages=%d must be in [1, %d]", n, KQ_STACK_MAX_STAGES);
  if (!stages) return fail(KQ_ERR_ARG, "stages is null");
  for (int i = 0; i < n; ++i) {
    const kq_stage& s = stages[i];
    int st = check_fmt_k(s.fmt, s.K);
    if (st) return fail(st, "stage %d: %s", i, kq_last_error());
    if (s.fmt == KQ_Q5_0 || s.fmt == KQ_Q5_1)
      return fail(KQ_ERR_FORMAT, "stage %d: the persistent chain takes Q8_0, Q4_0 and affine4 only", i);
    if (s.reserved != 0) return fail(KQ_ERR_ARG, "stage %d: reserved must be 0", i);
    if (s.N < 1 || s.N > KQ_MAX_N) return fail(KQ_ERR_ARG, "stage %d: N=%lld out of range", i, (long long)s.N);
    if (!s.W || !s.x || !s.y) return fail(KQ_ERR_ARG, "stage %d: null pointer", i);
    if (!aligned(s.W, 4) || !aligned(s.y, 4) || !aligned(s.x, 16) || (s.y16 && !aligned(s.y16, 2)))
      return fail(KQ_ERR_ALIGN, "stage %d: W, y need 4-byte, x 16-byte, y16 2-byte alignment", i);
    const int ub = s.fmt == KQ_AFFINE4_G32 ? 1 : 2;
    if (s.K % (32 * ub) != 0) return fail(KQ_ERR_SHAPE, "stage %d: K must be a multiple of %d", i, 32 * ub);
    if (s.K > kq::STACK_MAX_K)
      return fail(KQ_ERR_SHAPE, "stage %d: K=%lld exceeds %d for the stacked kernel", i, (long long)s.K,
                  kq::STACK_MAX_K);
  }
  std::vector<Range> xr(n), yr(n), hr(n);
  for (int i = 0; i < n; ++i) {
    const kq_stage& s = stages[i];
    const uintptr_t x = reinterpret_cast<uintptr_t>(s.x), y = reinterpret_cast<uintptr_t>(s.y);
    const uintptr_t h = reinterpret_cast<uintptr_t>(s.y16);
    xr[i] = {x, x + (uintptr_t)s.K * 2};
    yr[i] = {y, y + (uintptr_t)s.N * 4};
    hr[i] = s.y16 ? Range{h, h + (uintptr_t)s.N * 2} : Range{0, 0};
  }
  L.dep.assign(n, -1);
  L.dep_off.assign(n, 0);
  L.ll_word.assign(n, -1);
  L.ll_stride.assign(n, 0);
  for (int i = 0; i < n; ++i) {
    if (stages[i].y16 && yr[i].overlaps(hr[i])) return fail(KQ_ERR_ARG, "stage %d: y and y16 overlap", i);
    for (int j = 0; j < n; ++j) {
      if (j == i) continue;
      if (yr[i].overlaps(yr[j]) || (stages[j].y16 && yr[i].overlaps(hr[j])) ||
          (stages[i].y16 && stages[j].y16 && hr[i].overlaps(hr[j])))
        return fail(KQ_ERR_ARG, "stages %d and %d write overlapping outputs", i, j);
    }
    for (int j = 0; j < n; ++j) {
      if (xr[i].overlaps(yr[j]))
        return fail(KQ_ERR_ARG, "stage %d reads x from the fp32 output of stage %d", i, j);
      if (!stages[j].y16 || !xr[i].overlaps(hr[j])) continue;
      if (j >= i)
        return fail(KQ_ERR_ARG, "stage %d reads x from the fp16 output of stage %d, which is not earlier", i, j);
      if (!hr[j].contains(xr[i]))
        return fail(KQ_ERR_ARG, "stage %d: x only partly inside the fp16 output of stage %d", i, j);
      const int64_t off = (int64_t)(xr[i].lo - hr[j].lo) / 2;
      if (off % 4 != 0)
        return fail(KQ_ERR_ALIGN, "stage %d: x starts at element %lld of stage %d's y16 (need a multiple of 4)", i,
                    (long long)off, j);
      L.dep[i] = j;
      L.dep_off[i] = off;
    }
  }
  for (int i = 0; i < n; ++i) {
    if (L.dep[i] >= 0 && L.ll_word[L.dep[i]] < 0) {
      // STACK_LL_COPIES copies, each a 256-byte aligned run
      const int64_t run = (stages[L.dep[i]].N + 63) / 64 * 64;
      L.ll_word[L.dep[i]] = L.ll_words;
      L.ll_stride[L.dep[i]] = run;
      L.ll_words += run * kq::STACK_LL_COPIES;
    }
  }
  return KQ_OK;
}

int64_t plan_bytes(int n, const ChainLayout& L) {
  return stack_descs_bytes(n) + kq::STACK_SYNC_WORDS * 4 + L.ll_words * 4;
}

}  // namespace

int64_t kq_stack_plan_bytes(const kq_stage* stages, int n_stages) {
  ChainLayout L;
  int st = check_stages(stages, n_stages, L);
  if (st) return st;
  return plan_bytes(n_stages, L);
}

int kq_stack_plan(const kq_stage* stages, int n_stages, void* plan, int64_t plan_bytes_given,
                  kq_stack_info* info, void* stream) {
  if (!plan || !info) return fail(KQ_ERR_ARG, "kq_stack_plan: null pointer");
  ChainLayout L;
  int st = check_stages(stages, n_stages, L);
  if (st) return st;
  const int64_t need = plan_bytes(n_stages, L);
  if (plan_bytes_given < need) return fail(KQ_ERR_ARG, "kq_stack_plan: plan of %lld bytes needed", (long long)need);
  if (!aligned(plan, 256)) return fail(KQ_ERR_ALIGN, "kq_stack_plan: plan must be 256-byte aligned");
  int cus = 0;
  int err = kq::stack_device_info(&cus);
  if (err) return hip_status(err, "kq_stack_plan");
  if (cus < 1 || cus > kq::STACK_MAX_WG) return fail(KQ_ERR_HIP, "kq_stack_plan: %d compute units", cus);
  for (int i = 0; i < n_stages; ++i) {
    if ((stages[i].N + cus - 1) / cus > kq::STACK_MAX_SHARE_ROWS)
      return fail(KQ_ERR_SHAPE, "stage %d: N=%lld exceeds %lld rows (%d per compute unit)", i,
                  (long long)stages[i].N, (long long)cus * kq::STACK_MAX_SHARE_ROWS,
                  kq::STACK_MAX_SHARE_ROWS);
  }
  int fmask = 0, kmax = 0;
  for (int i = 0; i < n_stages; ++i) {
    fmask |= 1 << stages[i].fmt;
    if (stages[i].K > kmax) kmax = (int)stages[i].K;
  }
  uint8_t* base = static_cast<uint8_t*>(plan);
  uint32_t* ll = reinterpret_cast<uint32_t*>(base + stack_descs_bytes(n_stages) + kq::STACK_SYNC_WORDS * 4);
  std::vector<kq::StackStage> d((size_t)n_stages);
  for (int i = 0; i < n_stages; ++i) {
    const kq_stage& s = stages[i];
    const int ub = s.fmt == KQ_AFFINE4_G32 ? 1 : 2;
    kq::StackStage& o = d[(size_t)i];
    memset(&o, 0, sizeof(o));
    o.W = static_cast<const uint8_t*>(s.W);
    o.x = s.x;
    o.y = s.y;
    o.y16 = s.y16;
    o.ll_out = L.ll_word[i] >= 0 ? ll + L.ll_word[i] : nullptr;
    o.ll_in = L.dep[i] >= 0 ? ll + L.ll_word[L.dep[i]] + L.dep_off[i] : nullptr;
    o.N = (int32_t)s.N;
    o.K = (int32_t)s.K;
    o.fmt = s.fmt;
    o.upr = (int32_t)(s.K / (32 * ub));
    o.row_bytes = (int32_t)((s.K / 32) * kq::block_bytes(s.fmt));
    o.rows_per = (int32_t)(s.N / cus);
    o.rows_rem = (int32_t)(s.N % cus);
    o.log2g = kq::stack_log2g((s.N + cus - 1) / cus, o.upr);
    o.kpr = (o.upr + (1 << o.log2g) - 1) >> o.log2g;
    o.dep = L.dep[i];
    o.ll_out_stride = (int32_t)L.ll_stride[i];
    o.ll_in_stride = L.dep[i] >= 0 ? (int32_t)L.ll_stride[L.dep[i]] : 0;
  }
  // descriptors, then the sync words and tagged buffers: all zero (no error,
  // epoch 0, no tag; a zero word carries tag 0, which no stage of epoch 0 uses)
  std::vector<uint8_t> host((size_t)need, 0);
  memcpy(host.data(), d.data(), d.size() * sizeof(kq::StackStage));
  err = kq::copy_to_device(plan, host.data(), need, static_cast<hipStream_t>(stream));
  if (err) return hip_status(err, "kq_stack_plan");
  info->n_stages = n_stages;
  info->fmt_mask = fmask;
  info->k_max = kmax;
  info->workgroups = cus;
  return ok();
}

int kq_stack_run(const void* plan, const kq_stack_info* info, void* stream) {
  if (!plan || !info) return fail(KQ_ERR_ARG, "kq_stack_run: null pointer");
  if (info->n_stages < 1 || info->n_stages > KQ_STACK_MAX_STAGES || info->fmt_mask < 1 ||
      info->fmt_mask > 7 || info->k_max < 32 || info->k_max > kq::STACK_MAX_K ||
      info->workgroups < 1 || info->workgroups > kq::STACK_MAX_WG)
    return fail(KQ_ERR_ARG, "kq_stack_run: info was not filled by kq_stack_plan");
  int cus = 0;
  int err = kq::stack_device_info(&cus);
  if (err) return hip_status(err, "kq_stack_run");
  if (cus != info->workgroups)
    return fail(KQ_ERR_ARG, "kq_stack_run: plan made for %d compute units, device has %d", info->workgroups, cus);
  const kq::StackStage* st = static_cast<const kq::StackStage*>(plan);
  uint32_t* sync = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(const_cast<void*>(plan)) +
                                               stack_descs_bytes(info->n_stages));
  return hip_status(kq::launch_stack(st, info->n_stages, sync, info->fmt_mask, info->workgroups,
                                     info->k_max, static_cast<hipStream_t>(stream)),
                    "kq_stack_run");
}

int kq_stack_status(const void* plan, const kq_stack_info* info, int* error, void* stream) {
  if (!plan || !info || !error) return fail(KQ_ERR_ARG, "kq_stack_status: null pointer");
  if (info->n_stages < 1 || info->n_stages > KQ_STACK_MAX_STAGES)
    return fail(KQ_ERR_ARG, "kq_stack_status: info was not filled by kq_stack_plan");
  const uint32_t* sync = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(plan) +
                                                           stack_descs_bytes(info->n_stages));
  uint32_t word = 0;
  int err = kq::read_from_device(&word, sync + kq::STACK_ERR_WORD, 4, static_cast<hipStream_t>(stream));
  if (err) return hip_status(err, "kq_stack_status");
  *error = (int)word;
  return ok();
}

int64_t kq_gemv_argmax_workspace_bytes(int fmt, int64_t N, int64_t K, int M) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  if (M < 0 || M > KQ_MAX_M) return fail(KQ_ERR_ARG, "M=%d must be in [0, %d]", M, KQ_MAX_M);
  if (N > KQ_MAX_N) return fail(KQ_ERR_ARG, "N=%lld out of range", (long long)N);
  kq::GemvArgs a{fmt, nullptr, nullptr, nullptr, N, K, M, nullptr};
  const int64_t fused = (int64_t)M * kq::gemv_argmax_fused_parts(a) * 8;
  const int64_t plain = (int64_t)M * kq::argmax_partials(N) * 8;
  return fused > plain ? fused : plain;
}

int kq_gemv_argmax(int fmt, const void* W, const uint16_t* x, float* y, int64_t N, int64_t K, int M,
                   int32_t* out, void* workspace, int64_t workspace_bytes, void* stream) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  if (N < 1 || N > KQ_MAX_N) return fail(KQ_ERR_ARG, "kq_gemv_argmax: N=%lld out of range", (long long)N);
  if (M < 0 || M > KQ_MAX_M) return fail(KQ_ERR_ARG, "M=%d must be in [0, %d]", M, KQ_MAX_M);
  if (M == 0) return ok();
  if (!W || !x || !y || !out) return fail(KQ_ERR_ARG, "kq_gemv_argmax: null pointer");
  if (!aligned(W, 4) || !aligned(y, 4) || !aligned(out, 4))
    return fail(KQ_ERR_ALIGN, "kq_gemv_argmax: W, y and out must be 4-byte aligned");
  if (!aligned(x, 16)) return fail(KQ_ERR_ALIGN, "kq_gemv_argmax: x must be 16-byte aligned");
  const int64_t need = kq_gemv_argmax_workspace_bytes(fmt, N, K, M);
  if (need < 0) return (int)need;
  if (!workspace || workspace_bytes < need)
    return fail(KQ_ERR_ARG, "kq_gemv_argmax: workspace of %lld bytes needed", (long long)need);
  if (!aligned(workspace, 8)) return fail(KQ_ERR_ALIGN, "kq_gemv_argmax: workspace must be 8-byte aligned");
  kq::GemvArgs a{fmt, static_cast<const uint8_t*>(W), x, y, N, K, M, static_cast<hipStream_t>(stream)};
  return hip_status(kq::launch_gemv_argmax(a, out, workspace), "kq_gemv_argmax");
}

int kq_gemv_argmax_noalloc(int fmt, const void* W, const uint16_t* x, float* y, int64_t N, int64_t K, int M,
                           int32_t* out, void* stream) {
  int st = check_fmt_k(fmt, K);
  if (st) return st;
  if ((st = check_n(N, "N"))) return st;
  if (N < 1 || N > KQ_MAX_N) return fail(KQ_ERR_ARG, "kq_gemv_argmax_noalloc: N=%lld out of range", (long long)N);
  if (M < 0 || M > KQ_MAX_M) return fail(KQ_ERR_ARG, "M=%d must be in [0, %d]", M, KQ_MAX_M);
  if (M == 0) return ok();
  if (!W || !x || !y || !out) return fail(KQ_ERR_ARG, "kq_gemv_argmax_noalloc: null pointer");
  if (!aligned(W, 4) || !aligned(y, 4) || !aligned(out, 4))
    return fail(KQ_ERR_ALIGN, "kq_gemv_argmax_noalloc: W, y and out must be 4-byte aligned");
  if (!aligned(x, 16)) return fail(KQ_ERR_ALIGN, "kq_gemv_argmax_noalloc: x must be 16-byte aligned");
  const int64_t need = kq_gemv_argmax_workspace_bytes(fmt, N, K, M);
  if (need < 0) return (int)need;
  if (need > KQ_NOALLOC_SCRATCH_BYTES)
    return fail(KQ_ERR_ARG, "kq_gemv_argmax_noalloc: this shape needs %lld bytes of partials, more than the "
                "%d-byte static scratch; use kq_gemv_argmax with a workspace", (long long)need,
                KQ_NOALLOC_SCRATCH_BYTES);
  kq::GemvArgs a{fmt, static_cast<const uint8_t*>(W), x, y, N, K, M, static_cast<hipStream_t>(stream)};
  return hip_status(kq::launch_gemv_argmax_noalloc(a, out), "kq_gemv_argmax_noalloc");
}

int64_t kq_argmax_workspace_bytes(int64_t N, int M) {
  if (N < 0 || M < 0) return fail(KQ_ERR_ARG, "negative size");
  return (int64_t)M * kq::argmax_partials(N) * 8;
}

int kq_argmax(const float* y, int64_t N, int M, int32_t* out, void* workspace,
              int64_t workspace_bytes, void* stream) {
  if (N < 1 || N > KQ_MAX_N) return fail(KQ_ERR_ARG, "kq_argmax: N=%lld out of range", (long long)N);
  if (M < 0 || M > KQ_MAX_M) return fail(KQ_ERR_ARG, "kq_argmax: M=%d out of range", M);
  if (M == 0) return ok();
  if (!y || !out) return fail(KQ_ERR_ARG, "kq_argmax: null pointer");
  if (!aligned(y, 4) || !aligned(out, 4)) return fail(KQ_ERR_ALIGN, "kq_argmax: y and out must be 4-byte aligned");
  const int64_t need = kq_argmax_workspace_bytes(N, M);
  if (!workspace || workspace_bytes < need)
    return fail(KQ_ERR_ARG, "kq_argmax: workspace of %lld bytes needed", (long long)need);
  if (!aligned(workspace, 8)) return fail(KQ_ERR_ALIGN, "kq_argmax: workspace must be 8-byte aligned");
  return hip_status(kq::launch_argmax(y, N, M, out, workspace, static_cast<hipStream_t>(stream)),
                    "kq_argmax");
}

// ------------------------------------------------------------- Shortlist
namespace {
// Shapes the Shortlist path takes: K a multiple of 256 up to KQ_SHORTLIST_MAX_K
// (x and its block sums fit one workgroup's LDS), the Q8_0 matrix and its
// bound copy each below 2 GiB (32-bit buffer offsets with room for the
// out-of-range marker).
int check_shortlist_shape(int64_t N, int64_t K, const char* who) {
  if (N < 1 || N > KQ_MAX_N) return fail(KQ_ERR_ARG, "%s: N=%lld out of range", who, (long long)N);
  if (K <= 0 || K % 256 != 0 || K > KQ_SHORTLIST_MAX_K)
    return fail(KQ_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 256 and <= %d", who, (long long)K,
                KQ_SHORTLIST_MAX_K);
  const int64_t limit = (int64_t)1 << 31;
  if (N * (K / 32) * 34 >= limit || kq::shortlist_copy_bytes(N, K) >= limit)
    return fail(KQ_ERR_SHAPE, "%s: the matrix or its bound copy reaches 2 GiB", who);
  return KQ_OK;
}
}  // namespace

int64_t kq_shortlist_copy_bytes(int64_t N, int64_t K) {
  const int st = check_shortlist_shape(N, K, "kq_shortlist_copy_bytes");
  if (st) return st;
  return kq::shortlist_copy_bytes(N, K);
}

int kq_shortlist_pack(const void* q8_packed, int64_t N, int64_t K, void* out, int n_threads) {
  int st = check_shortlist_shape(N, K, "kq_shortlist_pack");
  if (st) return st;
  if (!q8_packed || !out) return fail(KQ_ERR_ARG, "kq_shortlist_pack: null pointer");
  st = kq::shortlist_pack(q8_packed, N, K, out, n_threads);
  if (st) return fail(st, "kq_shortlist_pack: a block scale is infinite or NaN");
  return ok();
}

int64_t kq_shortlist_workspace_bytes(int64_t N, int64_t K) {
  const int st = check_shortlist_shape(N, K, "kq_shortlist_workspace_bytes");
  if (st) return st;
  return kq::shortlist_workspace_bytes(N, K);
}

int kq_shortlist_argmax(const void* W, const void* W_copy, const uint16_t* x, int64_t N, int64_t K,
                        void* workspace, int64_t workspace_bytes, int32_t* out, int32_t* kept, void* stream) {
  int st = check_shortlist_shape(N, K, "kq_shortlist_argmax");
  if (st) return st;
  if (!W || !W_copy || !x || !out) return fail(KQ_ERR_ARG, "kq_shortlist_argmax: null pointer");
  if (!aligned(W, 16) || !aligned(W_copy, 16) || !aligned(x, 16))
    return fail(KQ_ERR_ALIGN, "kq_shortlist_argmax: W, W_copy and x must be 16-byte aligned");
  if (!aligned(out, 4) || (kept && !aligned(kept, 4)))
    return fail(KQ_ERR_ALIGN, "kq_shortlist_argmax: out and kept must be 4-byte aligned");
  const int64_t need = kq::shortlist_workspace_bytes(N, K);
  if (!workspace || workspace_bytes < need)
    return fail(KQ_ERR_ARG, "kq_shortlist_argmax: workspace of %lld bytes needed", (long long)need);
  if (!aligned(workspace, 256)) return fail(KQ_ERR_ALIGN, "kq_shortlist_argmax: workspace must be 256-byte aligned");
  kq::ShortlistArgs a{static_cast<const uint8_t*>(W), static_cast<const uint8_t*>(W_copy), x, N, K, workspace,
                      out, kept, static_cast<hipStream_t>(stream)};
  return hip_status(kq::launch_shortlist_argmax(a), "kq_shortlist_argmax");
}

}  // extern "C"
