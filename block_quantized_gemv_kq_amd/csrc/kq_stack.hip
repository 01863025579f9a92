// kq_stack.hip — a chain of dependent M = 1 GEMVs (one decode token through a
// dense stack) in ONE persistent launch.
//
// A decode step is hundreds of small GPU kernels, and recording it once and
// replaying it with one call per token removes the launch cost (Kinetic docs,
// "What makes it fast", the paragraph on recording the step). On MI355X a
// replayed graph still pays for every kernel's ramp-up and drain, and a
// 4B-shaped layer is four GEMVs of only 6.5-31 MB, so separate launches stream
// far below the HBM rate. Here the whole chain is one grid, one workgroup per
// CU, and each workgroup keeps HBM busy across stage boundaries:
//
//  * 11 COMPUTE waves only stream weights and multiply. Weights never depend
//    on activations, so each wave keeps a ring of three register slots of
//    packed weights in flight that runs ahead across stages; a slot is
//    refilled with a later round (of this stage or a later one) as soon as
//    it is consumed. These waves issue no other vector memory operation, so
//    waiting for a slot never waits for an activation or an output.
//  * 1 CONTROL wave does everything that touches activations, outputs and
//    other workgroups: it brings x of each stage into LDS, sums the compute
//    waves' per-unit partial dot products into rows in a fixed order, and
//    writes the outputs.
//
// Work split: a workgroup owns a contiguous share of stage s's rows, i.e. a
// contiguous run of U load units (1 affine4 block, or 2 Q4_0/Q8_0 blocks). Let
// S = (704 / upr) * upr, the largest multiple of the row length that fits the
// 704 compute lanes. Lane t < S takes units t, t + S, t + 2S, ...: all in the
// same column t mod upr, so the lane holds that column's activations in
// registers for the whole stage, and each load instruction of a wave covers
// consecutive units. Each unit's partial goes to LDS; the control wave sums
// each row's partials in unit order (deterministic run to run).
//
// Dataflow between stages without barriers: a stage whose x lies in an
// earlier stage's fp16 output reads it from that stage's tagged buffer, in
// which every element is one 32-bit word {fp16 value, 16-bit tag}; the tag
// names the producing stage and the launch (epoch * (n + 1) + s + 1), so one
// device-coherent store publishes value and readiness together. A consumer
// copies the words into LDS and copies again only the 16-byte chunks whose
// tags are not yet current: one memory round trip after the last producer's
// store, instead of a grid barrier (arrive, gather, release) per stage. Each
// workgroup keeps its own epoch word and advances it at the end of a launch,
// so nothing is reset between runs and a captured graph replays as is. Every
// wait is bounded: a wait that times out counts in the error word and the
// workgroup goes on, so the grid always drains.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_dev.h"
#include "kq_internal.h"

namespace kqd {

using kq::StackStage;

constexpr int CWAVES = kq::STACK_CWAVES;    // compute waves per workgroup
constexpr int NT = kq::STACK_NT;            // compute lanes per workgroup
constexpr int SLOT_DW = 20;                 // dwords per lane per register slot
constexpr int PART_N = 4 * NT;              // partials of one round (largest CU)
constexpr int LINE = 32;                    // words per sync line (128 bytes)
constexpr int YROWS = kq::STACK_MAX_SHARE_ROWS;
constexpr uint32_t SPIN_LIMIT = 1u << 20;

// Load units per compute lane per round: one slot (SLOT_DW dwords).
template <int FMT> struct ChainCU;
template <> struct ChainCU<F_AFFINE4> { static constexpr int v = 4; };   // 4 x 5 dw
template <> struct ChainCU<F_Q4_0> { static constexpr int v = 2; };      // 2 x 9 dw
template <> struct ChainCU<F_Q8_0> { static constexpr int v = 1; };      // 1 x 17 dw

__device__ __forceinline__ int cu_of(int fmt) { return fmt == F_AFFINE4 ? 4 : (fmt == F_Q4_0 ? 2 : 1); }

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every vector memory operation this wave issued has completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Stage descriptors are written by the host before the launch and never
// change during it: read them through the constant address space (scalar
// loads). A vector load here would be a VMEM operation in the compute waves
// and break their explicit vmcnt accounting.
typedef const __attribute__((address_space(4))) uint32_t* const_word_ptr;
__device__ __forceinline__ StackStage load_stage(const StackStage* st, int s) {
  const const_word_ptr p = (const_word_ptr)(st + __builtin_amdgcn_readfirstlane(s));
  uint32_t w[sizeof(StackStage) / 4];
#pragma unroll
  for (int i = 0; i < (int)(sizeof(StackStage) / 4); ++i) w[i] = p[i];
  StackStage d;
  __builtin_memcpy(&d, w, sizeof(StackStage));
  return d;
}

// A workgroup's share of a stage: rows [r0, r0 + rows), U units, rounds.
struct Share {
  int r0, rows, U, rounds;
};

__device__ __forceinline__ Share share_of(const StackStage& d, int b) {
  Share s;
  s.rows = d.rows_per + (b < d.rows_rem ? 1 : 0);
  s.r0 = b * d.rows_per + (b < d.rows_rem ? b : d.rows_rem);
  s.U = s.rows * d.upr;
  const int per = cu_of(d.fmt) * d.stride;
  s.rounds = (s.U + per - 1) / per;
  return s;
}

// ------------------------------------------------------------ compute waves

// One register slot: four pieces of 20 bytes, piece i = a 16-byte load (v[i],
// dwords 5i..5i+3) and a 4-byte load (e[i], dword 5i+4). Piece i of a round
// holds bytes 20*p .. 20*p+19 of unit i >> log2ppu, p = i & (ppu - 1), so a
// unit's bytes land in consecutive slot dwords: affine4 unit u (20 B) at dword
// 5u, Q4_0 unit u (36 B) at dword 10u, the Q8_0 unit (68 B) at dword 0. The
// load sequence is the same for every format; pieces past the share read 0.
struct Slot {
  u32x4 v[4];
  uint32_t e[4];
};

// Weight loads are inline assembly so that the compiler can neither sink them
// to their use (which would serialize the ring) nor count them: each round is
// exactly 8 load instructions and the consumer waits with an explicit vmcnt.
__device__ __forceinline__ void asm_load_piece(u32x4& v, uint32_t& e, uint32_t off, u32x4 rs) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(off), "s"(rs));
  asm volatile("buffer_load_dword %0, %1, %2, 0 offen offset:16" : "=v"(e) : "v"(off), "s"(rs));
}

// Wait until the oldest of the three slots in flight has landed (the two
// younger slots, 16 loads, may still be pending). The slot's registers are
// operands, so no use of them can be scheduled before the wait.
__device__ __forceinline__ void wait_oldest_slot(Slot& s) {
  asm volatile("s_waitcnt vmcnt(16)"
               : "+v"(s.v[0]), "+v"(s.v[1]), "+v"(s.v[2]), "+v"(s.v[3]), "+v"(s.e[0]), "+v"(s.e[1]),
                 "+v"(s.e[2]), "+v"(s.e[3]));
}

__device__ __forceinline__ void slot_dwords(const Slot& s, uint32_t (&D)[SLOT_DW]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    D[5 * i] = s.v[i].x;
    D[5 * i + 1] = s.v[i].y;
    D[5 * i + 2] = s.v[i].z;
    D[5 * i + 3] = s.v[i].w;
    D[5 * i + 4] = s.e[i];
  }
}

// Raw buffer descriptor over [base, base + bytes): loads past the end read 0.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);   // stride 0
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = (uint32_t)RSRC_FLAGS;
  return r;
}

// Where the next weight round to load comes from.
struct IssueCursor {
  int s, j, rounds, U, cu, stride, log2ppu, ubytes;
  u32x4 rs;
};

// Move to the first stage >= c.s that has work for this workgroup.
__device__ __forceinline__ void seek_stage(IssueCursor& c, const StackStage* st, int n, int b) {
  for (; c.s < n; ++c.s) {
    const StackStage d = load_stage(st, c.s);
    const Share sh = share_of(d, b);
    if (sh.rounds > 0) {
      c.j = 0;
      c.rounds = sh.rounds;
      c.U = sh.U;
      c.cu = cu_of(d.fmt);
      c.stride = d.stride;
      c.log2ppu = d.fmt == F_AFFINE4 ? 0 : (d.fmt == F_Q4_0 ? 1 : 2);
      c.ubytes = d.fmt == F_AFFINE4 ? 20 : (d.fmt == F_Q4_0 ? 36 : 68);
      c.rs = rsrc_words(d.W + (int64_t)sh.r0 * d.row_bytes, (uint32_t)sh.rows * (uint32_t)d.row_bytes);
      return;
    }
  }
}

// Load the cursor's round into slot `sl` (zeros once the chain is exhausted,
// and for lanes t >= stride) and advance the cursor. Always exactly 8 load
// instructions.
__device__ __forceinline__ void issue_next(Slot& sl, IssueCursor& c, const StackStage* st, int n, int b,
                                           int t) {
  const bool live = c.s < n && t < c.stride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = i >> c.log2ppu, p = i & ((1 << c.log2ppu) - 1);
    const int v = t + (c.j * c.cu + u) * c.stride;
    const uint32_t off = live && v < c.U ? (uint32_t)v * (uint32_t)c.ubytes + 20u * (uint32_t)p : OOB;
    asm_load_piece(sl.v[i], sl.e[i], off, c.rs);
  }
  if (c.s < n && ++c.j >= c.rounds) {
    ++c.s;
    seek_stage(c, st, n, b);
  }
}

// Dot product of one load unit (dwords D) with this lane's activations: X
// holds the unit's 16*UB activation dwords, SX its 2*UB half-block sums.
template <int FMT>
__device__ __forceinline__ float unit_partial(const uint32_t* D, const uint32_t (&X)[32], const float (&SX)[4]) {
  uint32_t A[16];
  if constexpr (FMT == F_AFFINE4) {
    const uint32_t nib[4] = {D[1], D[2], D[3], D[4]};
    unpack_nibbles_split(nib, A);
    return block_dot_split<F_AFFINE4>(A, X, SX[0], SX[1], h2f(D[0]), h2f(D[0] >> 16), 0.0f);
  } else if constexpr (FMT == F_Q4_0) {
    // block a: d at bytes 0-1, nibbles 2-17; block b: d at 18-19, nibbles 20-35
    const uint32_t na[4] = {alignbyte2(D[1], D[0]), alignbyte2(D[2], D[1]), alignbyte2(D[3], D[2]),
                            alignbyte2(D[4], D[3])};
    unpack_nibbles_split(na, A);
    const float acc = block_dot_split<F_Q4_0>(A, X, SX[0], SX[1], h2f(D[0]), 0.0f, 0.0f);
    const uint32_t nb[4] = {D[5], D[6], D[7], D[8]};
    unpack_nibbles_split(nb, A);
    return block_dot_split<F_Q4_0>(A, X + 16, SX[2], SX[3], h2f(D[4] >> 16), 0.0f, acc);
  } else {
    // block a: d at bytes 0-1, quants 2-33; block b: d at 34-35, quants 36-67
    uint32_t qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = alignbyte2(D[i + 1], D[i]);
    unpack_int8(qv, A);
    const float acc = block_dot_split<F_Q8_0>(A, X, SX[0], SX[1], h2f(D[0]), 0.0f, 0.0f);
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = D[9 + i];
    unpack_int8(qv, A);
    return block_dot_split<F_Q8_0>(A, X + 16, SX[2], SX[3], h2f(D[8] >> 16), 0.0f, acc);
  }
}

template <int FMT>
__device__ __forceinline__ void consume_fmt(const uint32_t (&raw)[SLOT_DW], const StackStage& d, int U,
                                            int j, int t, const uint32_t (&X)[32], const float (&SX)[4],
                                            float* part) {
  constexpr int CU = ChainCU<FMT>::v;
  constexpr int UDW = SLOT_DW / CU;   // slot dwords per unit (see Slot)
#pragma unroll
  for (int i = 0; i < CU; ++i) {
    const int v = t + (j * CU + i) * d.stride;
    if (t < d.stride && v < U) part[i * d.stride + t] = unit_partial<FMT>(raw + i * UDW, X, SX);
    // one unit at a time: interleaving units would hold several units'
    // dequantized weights at once and spill the slots
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int FMASK>
__device__ __forceinline__ void consume(Slot& sl, const StackStage& d, int U, int j, int t,
                                        const uint32_t (&X)[32], const float (&SX)[4], float* part) {
  wait_oldest_slot(sl);
  uint32_t raw[SLOT_DW];
  slot_dwords(sl, raw);
  if ((FMASK & (1 << F_AFFINE4)) && d.fmt == F_AFFINE4) consume_fmt<F_AFFINE4>(raw, d, U, j, t, X, SX, part);
  else if ((FMASK & (1 << F_Q4_0)) && d.fmt == F_Q4_0) consume_fmt<F_Q4_0>(raw, d, U, j, t, X, SX, part);
  else if ((FMASK & (1 << F_Q8_0)) && d.fmt == F_Q8_0) consume_fmt<F_Q8_0>(raw, d, U, j, t, X, SX, part);
}

// Consumption side of the round sequence: stage s, round j of its `rounds`.
struct ConsCursor {
  int s, j, rounds;
  StackStage d;
  Share sh;
};

// This lane's activations for stage d: its column's 16*UB dwords of x from
// LDS and their half-block sums (lanes t >= stride have no column).
__device__ __forceinline__ void load_column(const StackStage& d, int t, const uint32_t* xl, uint32_t (&X)[32],
                                            float (&SX)[4]) {
  const int ub = d.fmt == F_AFFINE4 ? 1 : 2;
  const int col = t < d.stride ? t % d.upr : 0;
  const u32x4* p = reinterpret_cast<const u32x4*>(xl + col * 16 * ub);
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const u32x4 w = v < 4 * ub ? p[v] : u32x4{0u, 0u, 0u, 0u};
    X[4 * v] = w.x;
    X[4 * v + 1] = w.y;
    X[4 * v + 2] = w.z;
    X[4 * v + 3] = w.w;
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot2(X[8 * h + i], ONES, s);
    SX[h] = s;
  }
}

// Move to the next round, entering stages (one workgroup barrier each, after
// which their x is in LDS) until one has work. False once every stage is done.
__device__ __forceinline__ bool next_round(ConsCursor& c, const StackStage* st, int n, int b, int t,
                                           const uint32_t* xl, uint32_t (&X)[32], float (&SX)[4]) {
  while (c.j >= c.rounds) {
    if (++c.s >= n) return false;
    c.d = load_stage(st, c.s);
    c.sh = share_of(c.d, b);
    c.rounds = c.sh.rounds;
    c.j = 0;
    __syncthreads();   // x of stage s is in LDS
    if (c.rounds > 0) load_column(c.d, t, xl, X, SX);
  }
  return true;
}

// The slots rotate A -> B -> C in code order, so the slot consumed is always
// the one loaded longest ago.
template <int FMASK>
__device__ __forceinline__ void compute_wave(const StackStage* st, int n, int b, const uint32_t* xl,
                                             float* part) {
  const int t = threadIdx.x;   // 0 .. NT-1
  Slot A, B, C;
  IssueCursor ic;
  ic.s = 0;
  ic.j = ic.rounds = ic.U = ic.cu = ic.stride = ic.log2ppu = ic.ubytes = 0;
  ic.rs = rsrc_words(st, 0u);   // empty range: every load reads zero
  seek_stage(ic, st, n, b);
  issue_next(A, ic, st, n, b, t);
  issue_next(B, ic, st, n, b, t);
  issue_next(C, ic, st, n, b, t);
  ConsCursor cc;
  cc.s = -1;
  cc.j = cc.rounds = 0;
  uint32_t X[32];
  float SX[4];
  int q = 0;
  for (;;) {
    if (!next_round(cc, st, n, b, t, xl, X, SX)) break;
    consume<FMASK>(A, cc.d, cc.sh.U, cc.j, t, X, SX, part + (q & 1) * PART_N);
    issue_next(A, ic, st, n, b, t);
    ++q;
    ++cc.j;
    __syncthreads();   // partials of this round are in LDS
    if (!next_round(cc, st, n, b, t, xl, X, SX)) break;
    consume<FMASK>(B, cc.d, cc.sh.U, cc.j, t, X, SX, part + (q & 1) * PART_N);
    issue_next(B, ic, st, n, b, t);
    ++q;
    ++cc.j;
    __syncthreads();
    if (!next_round(cc, st, n, b, t, xl, X, SX)) break;
    consume<FMASK>(C, cc.d, cc.sh.U, cc.j, t, X, SX, part + (q & 1) * PART_N);
    issue_next(C, ic, st, n, b, t);
    ++q;
    ++cc.j;
    __syncthreads();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load outlives the wave
}

// ------------------------------------------------------------- control wave

// Sum the partials of one round into the share's row accumulators: units
// [R0, R1) of the share, partial of unit u at part[u - R0]. Lanes split rows
// (L lanes per row, L a power of two); each lane sums a contiguous run in unit
// order with four interleaved accumulators, then the L lanes combine by a
// fixed butterfly. The order depends only on the shapes: deterministic.
__device__ __forceinline__ void reduce_round(const float* part, float* yacc, int R0, int R1, int upr,
                                             int lane) {
  const int rA = R0 / upr, rB = (R1 - 1) / upr;
  const int nrows = rB - rA + 1;
  int log2l = 0;
  while (log2l < 6 && (nrows << (log2l + 1)) <= 64) ++log2l;
  const int L = 1 << log2l, rpp = 64 >> log2l;
  for (int base = 0; base < nrows; base += rpp) {
    const int rr = base + (lane >> log2l), sub = lane & (L - 1);
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    if (rr < nrows) {
      const int r = rA + rr;
      const int a = max(R0, r * upr), e = min(R1, (r + 1) * upr);
      const int chunk = (e - a + L - 1) >> log2l;
      const int u0 = a + sub * chunk, u1 = min(e, u0 + chunk);
      const float* p = part - R0;
      int u = u0;
      for (; u + 4 <= u1; u += 4) {
        s0 += p[u];
        s1 += p[u + 1];
        s2 += p[u + 2];
        s3 += p[u + 3];
      }
      for (; u < u1; ++u) s0 += p[u];
    }
    float sum = (s0 + s1) + (s2 + s3);
    for (int o = 1; o < L; o <<= 1) sum += __shfl_xor(sum, o, 64);
    if (rr < nrows && sub == 0) yacc[rA + rr] += sum;
  }
}

constexpr int SC1 = 16;   // cache-policy bit: device-scope coherent access

// Copy x (K fp16, from outside the chain) into LDS.
__device__ __forceinline__ void stage_x(const uint16_t* x, int K, uint32_t* xl, int lane) {
  const int n16 = K / 8;
  for (int i = lane; i < n16; i += 64) {
    __builtin_amdgcn_global_load_lds((glb_void_t*)(reinterpret_cast<const u32x4*>(x) + i),
                                     (lds_void_t*)(xl + 4 * (i - lane)), 16, 0, SC1);
  }
  wait_vmem();
}

// Copy the K tagged words at `src` into LDS x as fp16, once every word carries
// `tag`. Chunk i (words 4i..4i+3) of lane i % 64 is fetched (LDS DMA, at the
// device coherence point) into the staging area; chunks whose four tags are
// current are unpacked into x, the others are fetched again. False if the wait
// timed out (x then holds whatever had arrived).
__device__ __forceinline__ bool ingest_tagged(const uint32_t* src, int K, uint32_t tag, uint32_t* xl,
                                              uint32_t* stg, uint32_t* err, int lane, bool broken) {
  const int nch = K / 4;
  const int rounds = (nch + 63) / 64;
  uint64_t pend = 0;
  for (int k = 0; k < rounds; ++k)
    if (64 * k + lane < nch) pend |= 1ull << k;
  uint32_t spins = 0;
  for (;;) {
    for (int k = 0; k < rounds; ++k) {
      if ((pend >> k) & 1ull)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(src + 4 * (64 * k + lane)),
                                         (lds_void_t*)(stg + 4 * 64 * k), 16, 0, SC1);
    }
    wait_vmem();
    for (int k = 0; k < rounds; ++k) {
      if ((pend >> k) & 1ull) {
        const int i = 64 * k + lane;
        const u32x4 w = *reinterpret_cast<const u32x4*>(stg + 4 * i);
        if ((w.x >> 16) == tag && (w.y >> 16) == tag && (w.z >> 16) == tag && (w.w >> 16) == tag) {
          uint32_t* o = xl + 2 * i;
          o[0] = perm(w.y, w.x, 0x05040100u);   // fp16 of words 4i, 4i+1
          o[1] = perm(w.w, w.z, 0x05040100u);
          pend &= ~(1ull << k);
        }
      }
    }
    if (!__any(pend != 0)) return true;
    if (broken || ++spins > SPIN_LIMIT) {
      if (!broken && lane == 0) add_dev(err, 1u);
      return false;
    }
  }
}

__device__ __forceinline__ void control_wave(const StackStage* st, int n, uint32_t* sync, int b, uint32_t* xl,
                                             uint32_t* stg, const float* part, float* yacc) {
  const int lane = threadIdx.x & 63;
  uint32_t* err = sync + kq::STACK_ERR_WORD;
  uint32_t* epoch_word = sync + kq::STACK_EPOCH_WORD + (int64_t)b * LINE;
  for (int r = lane; r < YROWS; r += 64) yacc[r] = 0.0f;
  const uint32_t epoch = ld_dev(epoch_word);
  const uint32_t tag_base = epoch * (uint32_t)(n + 1) + 1u;   // tag of stage s: (tag_base + s) mod 2^16
  bool broken = false;
  int q = 0;
  for (int s = 0; s < n; ++s) {
    const StackStage d = load_stage(st, s);
    const Share sh = share_of(d, b);
    if (sh.rounds > 0) {
      if (d.ll_in) {
        const uint32_t tag = (tag_base + (uint32_t)d.dep) & 0xffffu;
        if (!ingest_tagged(d.ll_in, d.K, tag, xl, stg, err, lane, broken)) broken = true;
      } else {
        stage_x(d.x, d.K, xl, lane);
      }
    }
    __syncthreads();   // x of stage s is in LDS
    const int per = cu_of(d.fmt) * d.stride;
    for (int j = 0; j < sh.rounds; ++j) {
      __syncthreads();   // the compute waves' partials of round j are in LDS
      const int R0 = j * per;
      reduce_round(part + (q & 1) * PART_N, yacc, R0, min(sh.U, R0 + per), d.upr, lane);
      ++q;
    }
    // Outputs: y and y16 with ordinary stores (read after the launch); the
    // tagged copy for later stages with device-coherent stores, value and tag
    // in one word, so a reader on any XCD sees both or neither.
    const uint32_t out_tag = ((tag_base + (uint32_t)s) & 0xffffu) << 16;
    for (int r = lane; r < sh.rows; r += 64) {
      const float v = yacc[r];
      yacc[r] = 0.0f;
      const int64_t row = sh.r0 + r;
      d.y[row] = v;
      const uint32_t h = f2h_bits(v);
      if (d.y16) d.y16[row] = (uint16_t)h;
      if (d.ll_out) st_dev(d.ll_out + row, h | out_tag);
    }
  }
  wait_vmem();
  if (lane == 0) st_dev(epoch_word, epoch + 1u);
}

template <int FMASK>
__global__ __launch_bounds__(64 * (CWAVES + 1)) void k_stack(const StackStage* __restrict__ st, int n,
                                                            uint32_t* __restrict__ sync, int kmax) {
  extern __shared__ u32x4 lds4[];
  uint32_t* xl = reinterpret_cast<uint32_t*>(lds4);   // x: kmax/2 dwords
  uint32_t* stg = xl + kmax / 2;                        // tagged words: kmax
  float* part = reinterpret_cast<float*>(stg + kmax);   // 2 x PART_N
  float* yacc = part + 2 * PART_N;                      // YROWS
  const int b = blockIdx.x;
  if (wave_id() == CWAVES)
    control_wave(st, n, sync, b, xl, stg, part, yacc);
  else
    compute_wave<FMASK>(st, n, b, xl, part);
}

}  // namespace kqd

namespace kq {

using namespace kqd;

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

int64_t stack_lds_bytes(int kmax) {
  return ((int64_t)kmax / 2 + kmax + 2 * PART_N + YROWS) * 4;
}

namespace {

template <int FMASK>
int launch_stack_mask(const StackStage* stages, int n_stages, uint32_t* sync, int nb, int kmax,
                      hipStream_t stream) {
  const size_t lds = (size_t)stack_lds_bytes(kmax);
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stack<FMASK>, 64 * (CWAVES + 1), lds);
  if (e != hipSuccess) return (int)e;
  if (per_cu < 1) return (int)hipErrorLaunchOutOfResources;
  hipLaunchKernelGGL((k_stack<FMASK>), dim3((unsigned)nb), dim3(64 * (CWAVES + 1)), lds, stream, stages,
                     n_stages, sync, kmax);
  return (int)hipGetLastError();
}

}  // namespace

int launch_stack(const StackStage* stages, int n_stages, uint32_t* sync, int fmask, int nb, int kmax,
                 hipStream_t stream) {
  switch (fmask) {
    case 1: return launch_stack_mask<1>(stages, n_stages, sync, nb, kmax, stream);
    case 2: return launch_stack_mask<2>(stages, n_stages, sync, nb, kmax, stream);
    case 3: return launch_stack_mask<3>(stages, n_stages, sync, nb, kmax, stream);
    case 4: return launch_stack_mask<4>(stages, n_stages, sync, nb, kmax, stream);
    case 5: return launch_stack_mask<5>(stages, n_stages, sync, nb, kmax, stream);
    case 6: return launch_stack_mask<6>(stages, n_stages, sync, nb, kmax, stream);
    default: return launch_stack_mask<7>(stages, n_stages, sync, nb, kmax, stream);
  }
}

}  // namespace kq
