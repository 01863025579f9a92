/*
 * kq.h — block-quantized decode GEMV for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels for the memory-bound decode step of
 * LLM inference: dequantize-and-multiply of block-quantized weights against a
 * few activation columns, and the routed-expert (mixture-of-experts) variant.
 *
 * Where the operation comes from (page title, section):
 *  - Kinetic docs, "What makes it fast": generating a token reads every weight
 *    of a dense model once, so decode is bound by memory bandwidth; guessed
 *    tokens are checked "in one pass over the weights" (M columns share one
 *    weight pass); up to four requests share every pass; choosing the next
 *    token reads an output layer of up to a quarter of a million rows; a
 *    mixture of experts keeps only the experts in use busy.
 *  - Kipp README, "How fast" (footnote to the 4-bit row): affine4 gs32 stores
 *    a scale and a bias per 32 weights, Q4_0 only a scale.
 *  - Kapitsa README, "What's new" and "How it works": a verify pass checks 8
 *    rows (draft-tree candidates); three requests can share one verify pass.
 *  - kinfer page, "Models bigger than the machine": a mixture of experts uses
 *    a few experts per token (10 of 512), so only those weights are read.
 *
 * Block formats (32 weights per block along K; a packed row is K/32 blocks
 * back to back, a packed matrix is its N rows back to back, no padding):
 *   KQ_Q8_0        34 B: fp16 d, 32 x int8 q;            w' = d*q
 *   KQ_Q4_0        18 B: fp16 d, 16 B nibbles;            w' = d*(q-8)
 *   KQ_AFFINE4_G32 20 B: fp16 s, fp16 b, 16 B nibbles;    w' = s*q + b
 *   KQ_Q5_0        22 B: fp16 d, 4 B fifth bits, 16 B nibbles;          w' = d*(q-16)
 *   KQ_Q5_1        24 B: fp16 d, fp16 m, 4 B fifth bits, 16 B nibbles;  w' = d*q + m
 * KQ_Q4_1 names the affine4 gs32 block: the scale-and-minimum 4-bit format
 * (Kinetic docs, "Supported models" list Q4_1 but print no layout; read as
 * Q5_1 with four bits, it is this block, 15 steps from the minimum).
 * fp16 values are little-endian; in the nibble areas element j sits in the
 * low nibble of byte j and element j+16 in the high nibble (the low four bits
 * of q in the 5-bit formats, whose bit 4 of q_j is bit j of the little-endian
 * 32-bit word after the scale(s)).
 *
 * Conventions for every call:
 *  - Return 0 (KQ_OK) or a negative kq_status. kq_last_error() gives a
 *    thread-local message for the last failure on the calling thread.
 *  - All argument checks run on the host before any HIP call; a call that
 *    fails them touches no memory and launches nothing.
 *  - "device" pointers are HIP device memory of the current device; "host"
 *    pointers are ordinary CPU memory. The caller owns every buffer; the
 *    library keeps no pointer after a call returns and allocates nothing.
 *  - GPU calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream) and never synchronise. Faults inside a kernel surface at
 *    the caller's next synchronisation of that stream.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef KQ_H_
#define KQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KQ_VERSION 100  /* 1.0.0 */

typedef enum kq_format {
  KQ_Q8_0 = 0,
  KQ_Q4_0 = 1,
  KQ_AFFINE4_G32 = 2,
  KQ_Q5_0 = 3,
  KQ_Q5_1 = 4,
  KQ_Q4_1 = KQ_AFFINE4_G32
} kq_format;

typedef enum kq_status {
  KQ_OK = 0,
  KQ_ERR_ARG = -1,     /* null pointer, negative or too large size, bad M/top_k */
  KQ_ERR_FORMAT = -2,  /* unknown kq_format */
  KQ_ERR_SHAPE = -3,   /* K <= 0 or K % 32 != 0, or K beyond KQ_MAX_K */
  KQ_ERR_ALIGN = -4,   /* pointer misaligned (see each call) */
  KQ_ERR_RANGE = -5,   /* kq_pack: non-finite weight, or scale/bias overflows fp16 */
  KQ_ERR_HIP = -6      /* HIP launch/runtime error (message in kq_last_error) */
} kq_status;

#define KQ_MAX_M 64            /* activation columns per call */
#define KQ_MAX_K (1 << 20)     /* inputs per row */
#define KQ_MAX_N 0x7fffffff    /* output rows per call */

/* Library version (KQ_VERSION of the built library). */
int kq_version(void);

/* Human-readable name of a kq_status value. Never NULL. */
const char* kq_status_string(int status);

/* Message describing the last failure on this thread ("" if none). */
const char* kq_last_error(void);

/* Bytes per 32-weight block of `fmt` (34, 18, 20, 22, 24), or a negative kq_status. */
int64_t kq_block_bytes(int fmt);

/* Bytes of a packed N x K matrix: N * (K/32) * kq_block_bytes(fmt).
 * Returns a negative kq_status for a bad format, N < 0 or a bad K. */
int64_t kq_packed_bytes(int fmt, int64_t N, int64_t K);

/* kq_pack — quantize a row-major fp32 matrix W[N][K] (host) into packed blocks
 * written to `out` (host, kq_packed_bytes(fmt,N,K) bytes). The formats are
 * those the pages name: Q8_0 and Q4_0 among the GGUF weight formats (Kinetic
 * docs, "Supported models"; its quantize command writes them), affine4 gs32 as
 * the scale-and-bias 4-bit scheme beside scale-only Q4_0 (Kipp README, "How
 * fast", footnote to the 4-bit row). The pages print no block layout or
 * quantizer formula; the steps below are the reading this library takes.
 * Per block of 32 consecutive weights w_j of one row (all arithmetic IEEE fp32
 * with round-to-nearest-even; fp16() rounds to nearest even, keeping
 * subnormals; round() is round-half-away-from-zero; q uses the STORED fp16
 * scale/bias):
 *   Q8_0:    d = fp16(max|w_j| / 127); q_j = clamp(round(w_j/d), -127, 127), 0 if d == 0
 *   Q4_0:    m = w_i at the first i maximising |w_i|; d = fp16(m / -8);
 *            q_j = clamp(round(w_j/d) + 8, 0, 15), 8 if d == 0
 *   AFFINE4: lo/hi = min/max w_j (first index on ties); s = fp16((hi-lo)/15),
 *            b = fp16(lo); q_j = clamp(round((w_j-b)/s), 0, 15), 0 if s == 0
 *   Q5_0:    as Q4_0 with d = fp16(m / -16); q_j = clamp(round(w_j/d) + 16, 0, 31), 16 if d == 0
 *   Q5_1:    as AFFINE4 with d = fp16((hi-lo)/31), m = fp16(lo);
 *            q_j = clamp(round((w_j-m)/d), 0, 31), 0 if d == 0
 * The bytes are identical to those of the library's CPU reference.
 * Errors: KQ_ERR_ARG (null, N < 0), KQ_ERR_FORMAT, KQ_ERR_SHAPE,
 * KQ_ERR_RANGE (non-finite weight, or a scale/bias that is infinite in fp16;
 * `out` is then left partly written). Uses up to `n_threads` host threads
 * (<= 0: one per hardware thread, capped at 64). */
int kq_pack(int fmt, const float* W, int64_t N, int64_t K, void* out, int n_threads);

/* kq_unpack — dequantize packed blocks (host) to fp32 W_out[N][K] (host), the
 * inverse view of kq_pack's formats (Kinetic docs, "Supported models"; Kipp
 * README, "How fast", footnote to the 4-bit row):
 * w' as above, computed in fp32 (exact for Q8_0 and Q4_0; affine4 is
 * s*q + b rounded once, exact unless s and b differ by more than 2^13 in scale). */
int kq_unpack(int fmt, const void* packed, int64_t N, int64_t K, float* W_out);

/* kq_gemv — y[m][n] = sum_k w'[n][k] * x[m][k] for m < M, n < N: the decode
 * step's weight pass (Kinetic docs, "What makes it fast": a token reads every
 * weight once; several guessed tokens, or up to four requests, share one pass
 * over the weights, so M columns ride on one read of W; Kapitsa README, "How it
 * works": a verify pass checks 8 rows, and "What's new": three requests share
 * one verify pass, M = 48 here).
 *   W: device, packed N x K matrix (kq_pack layout), 4-byte aligned.
 *   x: device, fp16 bits [M][K] (column m contiguous), 16-byte aligned.
 *   y: device, fp32 [M][N], 4-byte aligned; overwritten, never accumulated.
 * Every weight byte is read once per call whatever M is.
 * Accumulation is fp32;
 * results are run-to-run deterministic (fixed reduction order, no atomics).
 * M == 0 or N == 0 is a valid empty call. 1 <= M <= KQ_MAX_M.
 * Errors: KQ_ERR_ARG, KQ_ERR_FORMAT, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_HIP. */
int kq_gemv(int fmt, const void* W, const uint16_t* x, float* y,
            int64_t N, int64_t K, int M, void* stream);

/* kq_gemv_ws — kq_gemv with a caller-owned workspace, so that outputs with
 * few rows and long rows at verify widths (Kinetic docs, "What makes it
 * fast": several guessed tokens checked in one pass over the weights) can
 * split K across workgroups: each stages the activations of its part of K
 * only, and a second kernel adds the partial results in split order (the
 * result is deterministic; its bits may differ from kq_gemv's by the
 * summation order, within the same tolerance).
 *   workspace: device, 16-byte aligned, at least kq_gemv_workspace_bytes(fmt,
 *     N, K, M) bytes; may be NULL when that is 0 (then the call is kq_gemv).
 *     Its contents are scratch: nothing is kept between calls, and calls that
 *     share one workspace must not overlap.
 * Other arguments as kq_gemv.
 * Errors: as kq_gemv, and KQ_ERR_ARG (workspace missing or too small),
 * KQ_ERR_ALIGN (workspace not 16-byte aligned). */
int kq_gemv_ws(int fmt, const void* W, const uint16_t* x, float* y, int64_t N, int64_t K, int M,
               void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes kq_gemv_ws needs for this call shape (M * N * 4 per K
 * split), 0 when it does not split; or a negative error code (KQ_ERR_FORMAT,
 * KQ_ERR_SHAPE, KQ_ERR_ARG). */
int64_t kq_gemv_workspace_bytes(int fmt, int64_t N, int64_t K, int M);

/* kq_gemv_invariant — the product of kq_gemv, batch-invariant: column m of y
 * has the same bits as kq_gemv_invariant returns for column m alone (M = 1),
 * whatever M is (Kinetic docs, "What makes it fast": every row of a batch is
 * summed in the order that token would be summed on its own, so checking
 * eight guesses at once gives the bits of plain decoding). It runs the
 * matrix-core kernels with every launch configuration chosen from N and K
 * alone, for every M including 1: columns go 8 at a time through the split-K
 * kernel (the weights are read once per 8 columns) and 16 at a time through
 * the others (vocabulary-sized outputs, long rows); rows of 2-byte-aligned
 * blocks (an odd number of Q4_0/Q8_0 blocks) take a generic kernel. Its bits
 * differ from kq_gemv's (another summation order), both within the same
 * tolerance. Arguments, layout, ownership, determinism and errors as kq_gemv. */
int kq_gemv_invariant(int fmt, const void* W, const uint16_t* x, float* y,
                      int64_t N, int64_t K, int M, void* stream);

/* Workspace bytes kq_moe_gemv needs (0 when route_w is NULL). */
int64_t kq_moe_gemv_workspace_bytes(int64_t N, int M, int top_k, int weighted);

/* kq_moe_gemv — routed-expert GEMV for M decode tokens with top_k slots each:
 * only the experts a token is routed to are read (kinfer page, "Models bigger
 * than the machine": a few experts of many per token; Kinetic docs, "What makes
 * it fast": a mixture of experts keeps only the experts in use busy).
 *   W_experts: device, n_experts packed N x K matrices back to back (expert e
 *              starts at e * kq_packed_bytes(fmt, N, K)), 4-byte aligned.
 *   x: device fp16 bits; x_per_slot == 0: [M][K] (every slot of token m reads
 *      x[m]); x_per_slot == 1: [M][top_k][K] (slot j reads x[m][j]). 16-B aligned.
 *   route_ids: device int32 [M][top_k]; ids must lie in [0, n_experts).
 *      An id outside that range reads nothing and yields NaN outputs for its slot.
 *   route_w: device fp32 [M][top_k] or NULL.
 *   y: device fp32. route_w == NULL: per-slot outputs y[M][top_k][N].
 *      route_w != NULL: y[M][N] = sum_j route_w[m][j] * (W_{id[m][j]} x_{m,j}),
 *      summed in slot order j = 0..top_k-1.
 *   workspace: device, kq_moe_gemv_workspace_bytes(N, M, top_k, route_w != NULL)
 *      bytes, 16-B aligned (may be NULL when that size is 0).
 * Each distinct expert's weights are read once per call, for all the tokens
 * routed to it (found on the device; no host synchronisation).
 * Errors: KQ_ERR_ARG (incl. top_k not in [1, n_experts], small workspace),
 * KQ_ERR_FORMAT, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_HIP. */
int kq_moe_gemv(int fmt, const void* W_experts, const uint16_t* x,
                const int32_t* route_ids, const float* route_w, float* y,
                int64_t N, int64_t K, int M, int top_k, int n_experts, int x_per_slot,
                void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes kq_moe_ffn needs. */
int64_t kq_moe_ffn_workspace_bytes(int64_t hidden, int64_t inter, int M, int top_k);

/* kq_moe_ffn — the routed-expert FFN of M decode tokens (kinfer page, "Models
 * bigger than the machine"; Kinetic docs, "What makes it fast": only the
 * experts in use are read). The pages do not name the operation between the
 * gate/up and down projections; the gated SiLU below is the reading taken:
 *   for token m, slot j, expert e = route_ids[m][j]:
 *     g = Gate_e x_m, u = Up_e x_m            (inter outputs each)
 *     h = fp16(silu(g) * u), silu(z) = z / (1 + e^-z) in fp32
 *   y[m] = sum_j route_w[m][j] * (Down_e h)    (hidden outputs, slot order)
 *   W_gate, W_up: device, n_experts packed inter x hidden matrices back to back.
 *   W_down: device, n_experts packed hidden x inter matrices back to back.
 *   x: device fp16 [M][hidden]; y: device fp32 [M][hidden]; route_* as above
 *   (route_w must not be NULL). Gate and up rows of one expert are read in
 *   the same pass and SwiGLU is applied in registers.
 *   h_out: optional device fp16 [M][top_k][inter] copy of h (NULL: not kept).
 *   workspace: kq_moe_ffn_workspace_bytes(hidden, inter, M, top_k) bytes, 16-B aligned.
 * Errors: as kq_moe_gemv; KQ_ERR_SHAPE also when hidden % 64 != 0 for Q8_0/Q4_0. */
int kq_moe_ffn(int fmt, const void* W_gate, const void* W_up, const void* W_down,
               const uint16_t* x, const int32_t* route_ids, const float* route_w,
               float* y, uint16_t* h_out, int64_t hidden, int64_t inter,
               int M, int top_k, int n_experts,
               void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes kq_argmax needs. */
int64_t kq_argmax_workspace_bytes(int64_t N, int M);

/* kq_argmax — (Kinetic docs, "What makes it fast": choosing the next token
 * reads an output layer of up to a quarter of a million rows, and no speed-up
 * changes the answer) for each column m < M of y (device fp32 [M][N]), the index of
 * its largest value; the lowest index wins ties; NaN never wins (all-NaN
 * columns give 0). Written to out (device int32 [M]). This is the greedy
 * next-token choice over a vocabulary-sized output layer.
 * Errors: KQ_ERR_ARG, KQ_ERR_ALIGN, KQ_ERR_HIP. */
int kq_argmax(const float* y, int64_t N, int M, int32_t* out,
              void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes kq_gemv_argmax needs for this shape (< 0: the error of an
 * invalid shape). */
int64_t kq_gemv_argmax_workspace_bytes(int fmt, int64_t N, int64_t K, int M);

/* kq_gemv_argmax — kq_gemv, then kq_argmax of every column: y as kq_gemv
 * writes it, and out[m] (device int32 [M]) the index of column m's largest
 * value with kq_argmax's rules. The argmax is the output layer's greedy
 * next-token choice (Kinetic docs, "What makes it fast": choosing the next
 * token reads an output layer of up to a quarter of a million rows, and the
 * choice is exact). For one column on rows of whole units, the GEMV kernel
 * itself leaves each workgroup's best (value, row) in the workspace and one
 * small kernel picks the winner, instead of two kernels over y.
 * workspace: device, >= kq_gemv_argmax_workspace_bytes, 8-byte aligned,
 * caller-owned, no initial contents. Arguments otherwise as kq_gemv; out is
 * 4-byte aligned. Errors: those of kq_gemv, KQ_ERR_ARG (N < 1, workspace). */
int kq_gemv_argmax(int fmt, const void* W, const uint16_t* x, float* y,
                   int64_t N, int64_t K, int M, int32_t* out,
                   void* workspace, int64_t workspace_bytes, void* stream);

/* kq_gemv_argmax_noalloc — for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): kq_gemv_argmax with no workspace argument. The argmax partials
 * go to a static device array of KQ_NOALLOC_SCRATCH_BYTES that the library
 * holds on each device it runs on until the process ends; the call allocates
 * nothing. y and out are as kq_gemv_argmax writes them, bit for bit. Every
 * call on one device shares that array: calls that overlap in time on one
 * device (other streams, other threads) race and must be serialised by the
 * caller. Errors: those of kq_gemv_argmax, and KQ_ERR_ARG when the shape
 * needs more than KQ_NOALLOC_SCRATCH_BYTES of partials
 * (kq_gemv_argmax_workspace_bytes tells; 151936 rows need 76 KB at M = 1). */
#define KQ_NOALLOC_SCRATCH_BYTES (1 << 20)
int kq_gemv_argmax_noalloc(int fmt, const void* W, const uint16_t* x, float* y,
                           int64_t N, int64_t K, int M, int32_t* out, void* stream);

/* ---- Shortlist: an exact argmax that scores only the rows that can win ----
 * Kinetic docs, "What makes it fast" (the Shortlist paragraph): choosing the
 * next token reads an output layer with up to a quarter of a million rows; a
 * small copy of the layer bounds every row's score, and exact scores are
 * computed only for the rows whose bound still lets them win. The pages give
 * no copy or bound; this library's reading, for a Q8_0 layer (w' = d q):
 *
 * Each int8 quant splits as q = 8 (v - 16) + ql, v = floor(q / 8) + 16 (0..31),
 * ql = q - 8 (v - 16) (0..7). The bound copy of an N x K Q8_0 matrix (K a
 * multiple of 256, nb = K / 32) holds per row 22 nb bytes in three planes,
 * rows back to back: the nb fp16 block scales d (bit copies, little-endian);
 * nb little-endian uint32 words whose bit j is bit 4 of v_j; nb blocks of 16
 * nibble bytes, byte j = (v_j & 15) | (v_{j+16} & 15) << 4. After the N rows:
 * N little-endian fp32 E_n, the least fp32 with E_n^2 >= the sum over the
 * row's blocks of d^2 (ql_j - 3.5)^2 (computed exactly). 65 % of the Q8_0
 * bytes plus 4 per row.
 *
 * For one fp16 column x, per row n (real arithmetic): yhat = sum_b d_b (8
 * sum_j (v_j - 16) x_j + 3.5 sum_j x_j) differs from the exact score y by at
 * most E_n ||x||_2 (Cauchy-Schwarz on the error d (ql - 3.5)). On the device,
 * u_n = yhat + r + s and l_n = yhat - r - s with r = E_n ||x||_2 and
 * s = T/4 + r/256 + 2^-80, T = sum_b |d_b| sum_j |x_j|. s covers the fp32
 * rounding of yhat and of the exact score: each fp32 step rounds once (a
 * pair-dot step at most twice), on intermediates of at most
 * 8 (1055 + 1040) |d_b| sum|x| per block for yhat and (1279 + 1152) |d_b| sum|x|
 * for the exact score, plus running sums of at most 128 T and 127 T over at
 * most 2 K/32 + 6 steps: below 0.05 T together for K <= 16384. The row c
 * with the largest l is scored exactly (tau); rows with u_n < tau score below
 * row c and are skipped; every other row is scored exactly and the largest
 * wins (lowest index on ties, NaN never wins). */

/* Bytes of the bound copy of an N x K Q8_0 matrix (< 0: the error of an
 * invalid shape: K not a positive multiple of 256 or above
 * KQ_SHORTLIST_MAX_K, N out of range, or the matrix or copy reaching 2 GiB). */
#define KQ_SHORTLIST_MAX_K 16384
int64_t kq_shortlist_copy_bytes(int64_t N, int64_t K);

/* kq_shortlist_pack — host: the bound copy (above) of the packed Q8_0 matrix
 * q8_packed (host, kq_packed_bytes(KQ_Q8_0, N, K) bytes) into out (host,
 * kq_shortlist_copy_bytes(N, K) bytes). n_threads as kq_pack. The bytes are
 * fixed by the definition above.
 * Errors: the shape errors of kq_shortlist_copy_bytes, KQ_ERR_ARG (null
 * pointer), KQ_ERR_RANGE (a block scale is infinite or NaN). */
int kq_shortlist_pack(const void* q8_packed, int64_t N, int64_t K, void* out, int n_threads);

/* Workspace bytes kq_shortlist_argmax needs (< 0: invalid shape). About
 * 4 N + 12 N / 256 + 8 N / rows-per-workgroup bytes. */
int64_t kq_shortlist_workspace_bytes(int64_t N, int64_t K);

/* kq_shortlist_argmax — the index of the largest of the N scores W x of one
 * fp16 column x (device, K halves, 16-B aligned), through the bound copy
 * W_copy (device, kq_shortlist_pack's bytes, 16-B aligned) of the Q8_0
 * matrix W (device, 16-B aligned): out[0] (device int32) is the index
 * kq_gemv_argmax gives for (KQ_Q8_0, W, x, N, K, M = 1) — the rows it scores
 * exactly have the bits kq_gemv gives them, and every other row is shown to
 * score below one of them. kept (device int32, or NULL) receives the number
 * of rows scored exactly. y is not written. Four kernels on `stream`, no
 * host synchronisation, no allocation: the workspace (device,
 * kq_shortlist_workspace_bytes, 256-B aligned, caller-owned, no initial
 * contents) holds the bounds and partial results; calls sharing a workspace
 * must not overlap in time. It reads 65 % of W's bytes plus the rows it
 * scores exactly: on seeded N(0, 0.02) weights with a standard normal x,
 * about 3 % of a 151936-row layer.
 * Errors: the shape errors of kq_shortlist_copy_bytes, KQ_ERR_ARG (null
 * pointer, small workspace), KQ_ERR_ALIGN, KQ_ERR_HIP. */
int kq_shortlist_argmax(const void* W, const void* W_copy, const uint16_t* x, int64_t N, int64_t K,
                        void* workspace, int64_t workspace_bytes, int32_t* out, int32_t* kept,
                        void* stream);

/* ---- A chain of dependent M = 1 GEMVs in one persistent launch ----------
 * Kinetic docs, "What makes it fast": a decode step is hundreds of small GPU
 * kernels, recorded once and replayed with one call per token. kq_stack_run
 * goes further: the whole chain (e.g. every projection of every layer of a
 * dense model, then its output layer) is ONE kernel launch, and each stage's
 * weights stream in while earlier stages finish: weights never depend on
 * activations.
 *
 * Dataflow: a stage whose x lies inside the y16 (fp16 output) of an EARLIER
 * stage waits for exactly those values of that launch; that is how a chain
 * is expressed (stages[s].x = stages[s-1].y16, or any 4-element-aligned run
 * of it, e.g. the q part of a fused q|k|v output). Any other x is read as it
 * is at the start of the launch, and stages that do not depend on each other
 * may run at the same time. So that this is well defined, kq_stack_plan
 * rejects (KQ_ERR_ARG) stages whose outputs (y, y16) overlap each other,
 * and an x that overlaps any y, a later (or the same) stage's y16, or only
 * part of an earlier stage's y16. */
typedef struct kq_stage {
  int32_t fmt;          /* kq_format */
  int32_t reserved;     /* must be 0 */
  const void* W;        /* device, packed N x K (kq_pack layout), 4-byte aligned */
  const uint16_t* x;    /* device, fp16 bits [K], 16-byte aligned */
  float* y;             /* device, fp32 [N], 4-byte aligned; overwritten */
  int64_t N;            /* 1 <= N <= 4096 * (compute units of the device) */
  int64_t K;            /* multiple of 32 (of 64 for Q8_0/Q4_0), at most 16384 */
  uint16_t* y16;        /* device or NULL: also store fp16(y) (round to nearest
                           even), 2-byte aligned, so a later stage can read it as x */
} kq_stage;

/* Filled by kq_stack_plan, passed to kq_stack_run (host memory). */
typedef struct kq_stack_info {
  int32_t n_stages;
  int32_t fmt_mask;
  int32_t k_max;
  int32_t workgroups;   /* one per compute unit of the device the plan was made on */
} kq_stack_info;

#define KQ_STACK_MAX_STAGES 4096

/* Device bytes of a plan for these stages (the plan holds the stage
 * descriptors, per-workgroup sync words and a tagged copy of every fp16
 * output that a later stage reads). Checks the stages as kq_stack_plan does
 * (host only) and returns a negative kq_status if they are not valid. */
int64_t kq_stack_plan_bytes(const kq_stage* stages, int n_stages);

/* kq_stack_plan — validate `stages` (host array of n_stages) and write the
 * device-side plan (`plan`: device, kq_stack_plan_bytes bytes, 256-byte
 * aligned) plus `info` (host). Copies over `stream` and synchronises it: call
 * it once at set-up, not inside graph capture. The plan stays valid while the
 * buffers it names do, on the device it was made on (kq_stack_run checks the
 * compute-unit count). Errors: KQ_ERR_ARG (also the overlaps above),
 * KQ_ERR_FORMAT (also Q5_0 and Q5_1: the chain takes the other three formats),
 * KQ_ERR_SHAPE (also K > 16384, or N above 4096 rows per
 * compute unit), KQ_ERR_ALIGN (also an x starting at an element of an earlier
 * y16 that is not a multiple of 4), KQ_ERR_HIP. */
int kq_stack_plan(const kq_stage* stages, int n_stages, void* plan, int64_t plan_bytes,
                  kq_stack_info* info, void* stream);

/* kq_stack_run — run every stage of a plan in one launch on `stream`
 * (asynchronous; may be captured in a graph). Results are deterministic run
 * to run, bit for bit, and each output is within the kq_gemv tolerance of the
 * exact value. Runs on one plan must not overlap in time (they share its sync
 * words). The grid (one workgroup per CU) needs every CU free; a wait that
 * exceeds its spin limit counts in the plan's error word (kq_stack_status;
 * sticky until the next kq_stack_plan) and lets the launch finish instead of
 * hanging; outputs of such a run are undefined. The plan needs no reset
 * between runs (each run advances epochs stored in the plan), so a captured
 * graph can replay it with nothing else in the graph. */
int kq_stack_run(const void* plan, const kq_stack_info* info, void* stream);

/* kq_stack_status — synchronise `stream`, then read the plan's error word
 * into *error (0: every wait completed). */
int kq_stack_status(const void* plan, const kq_stack_info* info, int* error, void* stream);

/* kq_set_tuning — tests and tuning sweeps only: force a kernel or a launch
 * configuration that the library would not choose by itself, so that every
 * path can be reached at small shapes. Results change by at most the
 * floating-point summation order (every path meets the kq_gemv tolerance).
 * Process-wide; the environment is never read. name NULL clears every
 * override; value NULL or "" clears one. Names and values:
 *   force_path       "g" generic, "v" register-x VALU, "l" LDS VALU, "m" matrix cores
 *   mfma_variant     "pers", "teams", "teams_sx", "chunk", "chunk_whole",
 *                    "chunk_split", "direct"
 *   valu_g, valu_r, lds_wpg, mfma_s, mfma_r, mfma_waves, mfma_xf,
 *   mfma_pers_tpw, mfma_pers_waves, mfma_chunk_l2cg, moe_unfused,
 *   moe_min_wg, moe_one, mfma_split, sl_g, mfma_xdma,
 *   lds_xdma                                                  (decimal integers)
 *   log              "1": one line per kernel launch on stderr (kernel, format,
 *                    shape, grid, workgroup, LDS bytes, chosen configuration)
 * Errors: KQ_ERR_ARG (unknown name or malformed value). Not synchronised
 * with calls running on other threads. */
int kq_set_tuning(const char* name, const char* value);

/* Test hook: convert n fp32 values (host) to fp16 bits (host) with the
 * packer's own round-to-nearest-even conversion. */
int kq_f32_to_f16(const float* in, uint16_t* out, int64_t n);

#ifdef __cplusplus
}
#endif
#endif /* KQ_H_ */
