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
//    other workgroups: it brings x of each stage into LDS with its per-block
//    sums, and writes the outputs the compute waves leave in LDS.
//
// Work split: a workgroup owns a contiguous share of stage s's rows. Within
// it, G lanes share a row (G in 4..64, chosen per stage so that the busiest
// lane has the fewest steps): lane group gamma takes rows gamma, gamma +
// groups, ... and lane g of it units g, g + G, ... of each row (a unit is one
// affine4 block or two Q4_0/Q8_0 blocks), accumulating in a register; the G
// lanes combine a finished row by a fixed butterfly (deterministic run to
// run). The activations of a stage sit in LDS with their 16-byte pieces
// rotated per column, so that the G consecutive columns one instruction reads
// fall in different banks. A wave's load instruction covers G consecutive
// units of each of its 64/G rows.
//
// Dataflow between stages without barriers: a stage whose x lies in an
// earlier stage's fp16 output reads it from that stage's tagged buffer, in
// which every element is one 32-bit word {fp16 value, 16-bit tag}; the tag
// names the producing stage and the launch (epoch * (n + 1) + s + 1), so one
// device-coherent store publishes value and readiness together. Producers
// also raise a per-workgroup hint word after each stage; a consumer polls the
// hints (one small round trip) and then copies the tagged words, copying
// again only chunks whose tags are not yet current. Each workgroup keeps its
// own epoch word and advances it at the end of a launch, so nothing is reset
// between runs and a captured graph replays as is. Every wait is bounded: a
// wait that times out counts in the error word and the workgroup goes on, so
// the grid always drains.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_dev.h"
#include "kq_internal.h"

namespace kqd {

using kq::StackStage;

constexpr int CWAVES = kq::STACK_CWAVES;    // compute waves per workgroup
constexpr int SLOT_DW = 20;                 // dwords per lane per register slot
constexpr int LINE = 32;                    // words per sync line (128 bytes)
constexpr uint32_t SPIN_LIMIT = 1u << 20;
constexpr int SC1 = 16;                     // cache-policy bit: device-scope coherent access

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

// A workgroup's share of a stage: rows [r0, r0 + rows).
struct Share {
  int r0, rows;
};

__device__ __forceinline__ Share share_of(const StackStage& d, int b) {
  Share s;
  s.rows = d.rows_per + (b < d.rows_rem ? 1 : 0);
  s.r0 = b * d.rows_per + (b < d.rows_rem ? b : d.rows_rem);
  return s;
}

// Lane groups of a stage: `groups` groups of G = 2^log2g lanes; wave w holds
// groups w*gpw .. w*gpw + gpw - 1 (gpw = 64 / G).
__device__ __forceinline__ int groups_of(int log2g) { return CWAVES << (6 - log2g); }

// Steps of wave w in a stage with `rows` rows in this workgroup: its first
// group has the most rows (ceil((rows - gamma0) / groups)), each kpr steps.
__device__ __forceinline__ int wave_steps(const StackStage& d, int rows, int w) {
  const int groups = groups_of(d.log2g);
  const int gamma0 = w << (6 - d.log2g);
  const int mcount = rows > gamma0 ? (rows - gamma0 + groups - 1) / groups : 0;
  return mcount * d.kpr;
}

// ------------------------------------------------------------ compute waves

// One register slot: four pieces of 20 bytes, piece i = a 16-byte load (v[i],
// dwords 5i..5i+3) and a 4-byte load (e[i], dword 5i+4). Piece i of a round
// holds bytes 20*p .. 20*p+19 of step i >> log2ppu's unit, p = i & (ppu - 1),
// so a unit's bytes land in consecutive slot dwords: affine4 unit u (20 B) at
// dword 5u, Q4_0 unit u (36 B) at dword 10u, the Q8_0 unit (68 B) at dword 0.
// The load sequence is the same for every format; invalid pieces read 0.
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

// Step position (row slot m, unit slot k) of a lane group walking a stage:
// unit g + G*k of row gamma + groups*m; k runs over kpr per row.
__device__ __forceinline__ void step_advance(int& m, int& k, int kpr) {
  if (++k == kpr) {
    k = 0;
    ++m;
  }
}

// Where the next weight round of this wave comes from.
struct IssueCursor {
  int s, j, rounds, m, k;
  int rows, upr, kpr, log2g, cu, log2ppu, ubytes;
  u32x4 rs;
};

// Move to the first stage >= c.s in which this wave has work.
__device__ __forceinline__ void seek_stage(IssueCursor& c, const StackStage* st, int n, int b, int w) {
  for (; c.s < n; ++c.s) {
    const StackStage d = load_stage(st, c.s);
    const Share sh = share_of(d, b);
    const int cu = cu_of(d.fmt);
    const int rounds = (wave_steps(d, sh.rows, w) + cu - 1) / cu;
    if (rounds > 0) {
      c.j = c.m = c.k = 0;
      c.rounds = rounds;
      c.rows = sh.rows;
      c.upr = d.upr;
      c.kpr = d.kpr;
      c.log2g = d.log2g;
      c.cu = cu;
      c.log2ppu = d.fmt == F_AFFINE4 ? 0 : (d.fmt == F_Q4_0 ? 1 : 2);
      c.ubytes = d.fmt == F_AFFINE4 ? 20 : (d.fmt == F_Q4_0 ? 36 : 68);
      c.rs = rsrc_words(d.W + (int64_t)sh.r0 * d.row_bytes, (uint32_t)sh.rows * (uint32_t)d.row_bytes);
      return;
    }
  }
}

// Load the cursor's round into slot `sl` (zeros once the chain is exhausted
// and for steps past a lane group's rows) and advance the cursor. Always
// exactly 8 load instructions.
__device__ __forceinline__ void issue_next(Slot& sl, IssueCursor& c, const StackStage* st, int n, int b, int w,
                                           int lane) {
  const bool live = c.s < n;
  // positions of the round's steps 0..3 and of the step after the round
  int ms[5], ks[5];
  ms[0] = c.m;
  ks[0] = c.k;
#pragma unroll
  for (int u = 1; u < 5; ++u) {
    ms[u] = ms[u - 1];
    ks[u] = ks[u - 1];
    step_advance(ms[u], ks[u], live ? c.kpr : 1);
  }
  const int gamma = (w << (6 - c.log2g)) + (lane >> c.log2g);
  const int g = lane & ((1 << c.log2g) - 1);
  const int groups = groups_of(c.log2g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = i >> c.log2ppu, p = i & ((1 << c.log2ppu) - 1);
    const int row = gamma + groups * ms[u];
    const int unit = g + (ks[u] << c.log2g);
    const bool ok = live && row < c.rows && unit < c.upr;
    const uint32_t off = ok ? (uint32_t)(row * c.upr + unit) * (uint32_t)c.ubytes + 20u * (uint32_t)p : OOB;
    asm_load_piece(sl.v[i], sl.e[i], off, c.rs);
  }
  if (live) {
    c.m = c.cu == 4 ? ms[4] : (c.cu == 2 ? ms[2] : ms[1]);
    c.k = c.cu == 4 ? ks[4] : (c.cu == 2 ? ks[2] : ks[1]);
    if (++c.j >= c.rounds) {
      ++c.s;
      seek_stage(c, st, n, b, w);
    }
  }
}

// Activations of column c (16*UB dwords) from the rotated LDS layout: piece p
// of column c is quad c*P + ((p + rot(c)) mod P), P = 4*UB pieces per column,
// rot(c) = c >> 1 for P = 4 and c for P = 8.
template <int UB>
__device__ __forceinline__ void load_x_col(const uint32_t* xl, int c, uint32_t (&X)[32]) {
  constexpr int P = 4 * UB;
  const int rot = UB == 1 ? (c >> 1) : c;
  const u32x4* q = reinterpret_cast<const u32x4*>(xl) + c * P;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const u32x4 t = q[(p + rot) & (P - 1)];
    X[4 * p] = t.x;
    X[4 * p + 1] = t.y;
    X[4 * p + 2] = t.z;
    X[4 * p + 3] = t.w;
  }
}

// Dot product of one load unit (dwords D) with its activations: X holds the
// unit's 16*UB activation dwords, SX its 2*UB half-block sums.
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

// Consumption side: stage s, round j of this wave's `rounds`, at step (m, k);
// acc is the lane's running sum of its current row.
struct ConsCursor {
  int s, j, rounds, m, k, rows;
  StackStage d;
};

template <int FMT>
__device__ __forceinline__ void consume_fmt(const uint32_t (&raw)[SLOT_DW], ConsCursor& c, int w, int lane,
                                            const uint32_t* xl, const float* xs, float* yacc, float& acc) {
  constexpr int CU = ChainCU<FMT>::v, UB = Fmt<FMT>::UB;
  constexpr int UDW = SLOT_DW / CU;   // slot dwords per unit (see Slot)
  const int log2g = c.d.log2g;
  const int gamma = (w << (6 - log2g)) + (lane >> log2g);
  const int g = lane & ((1 << log2g) - 1);
  const int groups = groups_of(log2g);
#pragma unroll
  for (int i = 0; i < CU; ++i) {
    const int row = gamma + groups * c.m;
    const int unit = g + (c.k << log2g);
    if (row < c.rows && unit < c.d.upr) {
      uint32_t X[32];
      float SX[4];
      load_x_col<UB>(xl, unit, X);
#pragma unroll
      for (int h = 0; h < 2 * UB; ++h) SX[h] = xs[unit * 2 * UB + h];
      acc += unit_partial<FMT>(raw + i * UDW, X, SX);
    }
    if (c.k == c.d.kpr - 1) {   // the group's row is complete (uniform over the wave)
      acc = group_sum(acc, 1 << log2g);
      if (g == 0 && row < c.rows) yacc[row] = acc;
      acc = 0.0f;
    }
    step_advance(c.m, c.k, c.d.kpr);
    // one unit at a time: interleaving units would hold several units'
    // activations and dequantized weights at once and spill the slots
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int FMASK>
__device__ __forceinline__ void consume(Slot& sl, ConsCursor& c, int w, int lane, const uint32_t* xl,
                                        const float* xs, float* yacc, float& acc) {
  wait_oldest_slot(sl);
  uint32_t raw[SLOT_DW];
  slot_dwords(sl, raw);
  const int fmt = c.d.fmt;
  if ((FMASK & (1 << F_AFFINE4)) && fmt == F_AFFINE4) consume_fmt<F_AFFINE4>(raw, c, w, lane, xl, xs, yacc, acc);
  else if ((FMASK & (1 << F_Q4_0)) && fmt == F_Q4_0) consume_fmt<F_Q4_0>(raw, c, w, lane, xl, xs, yacc, acc);
  else if ((FMASK & (1 << F_Q8_0)) && fmt == F_Q8_0) consume_fmt<F_Q8_0>(raw, c, w, lane, xl, xs, yacc, acc);
}

// Move to the next round, passing stage boundaries: every stage, with or
// without work for this wave, is one barrier after its x is in LDS and one
// after its rows are in yacc. False once every stage is done.
__device__ __forceinline__ bool next_round(ConsCursor& c, const StackStage* st, int n, int b, int w, float& acc) {
  while (c.j >= c.rounds) {
    if (c.s >= 0) __syncthreads();   // stage s done: its rows are in yacc
    if (++c.s >= n) return false;
    c.d = load_stage(st, c.s);
    const Share sh = share_of(c.d, b);
    c.rows = sh.rows;
    const int cu = cu_of(c.d.fmt);
    c.rounds = (wave_steps(c.d, sh.rows, w) + cu - 1) / cu;
    c.j = c.m = c.k = 0;
    acc = 0.0f;
    __syncthreads();   // x of stage s and its sums are in LDS
  }
  return true;
}

// The slots rotate A -> B -> C in code order, so the slot consumed is always
// the one loaded longest ago.
template <int FMASK>
__device__ __forceinline__ void compute_wave(const StackStage* st, int n, int b, const uint32_t* xl,
                                             const float* xs, float* yacc) {
  const int w = wave_id(), lane = threadIdx.x & 63;
  Slot A, B, C;
  IssueCursor ic;
  ic.s = ic.j = ic.rounds = ic.m = ic.k = 0;
  ic.rows = ic.upr = ic.kpr = ic.log2g = ic.cu = ic.log2ppu = ic.ubytes = 0;
  ic.rs = rsrc_words(st, 0u);   // empty range: every load reads zero
  seek_stage(ic, st, n, b, w);
  issue_next(A, ic, st, n, b, w, lane);
  issue_next(B, ic, st, n, b, w, lane);
  issue_next(C, ic, st, n, b, w, lane);
  ConsCursor cc;
  cc.s = -1;
  cc.j = cc.rounds = cc.m = cc.k = cc.rows = 0;
  float acc = 0.0f;
  for (;;) {
    if (!next_round(cc, st, n, b, w, acc)) break;
    consume<FMASK>(A, cc, w, lane, xl, xs, yacc, acc);
    issue_next(A, ic, st, n, b, w, lane);
    ++cc.j;
    if (!next_round(cc, st, n, b, w, acc)) break;
    consume<FMASK>(B, cc, w, lane, xl, xs, yacc, acc);
    issue_next(B, ic, st, n, b, w, lane);
    ++cc.j;
    if (!next_round(cc, st, n, b, w, acc)) break;
    consume<FMASK>(C, cc, w, lane, xl, xs, yacc, acc);
    issue_next(C, ic, st, n, b, w, lane);
    ++cc.j;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load outlives the wave
}

// ------------------------------------------------------------- control wave

// Copy `n16` 16-byte chunks from `src` (global) to `stg` (LDS), reading at the
// device coherence point; chunk i lands at stg + 4i dwords.
__device__ __forceinline__ void dma_chunks(const void* src, int n16, uint32_t* stg, int lane) {
  for (int i = lane; i < n16; i += 64) {
    __builtin_amdgcn_global_load_lds((glb_void_t*)(reinterpret_cast<const u32x4*>(src) + i),
                                     (lds_void_t*)(stg + 4 * (i - lane)), 16, 0, SC1);
  }
  wait_vmem();
}

// Bring the K tagged words at `src` into the staging area, once every word
// carries `tag`: all chunks first, then only the chunks not yet current, with
// a short pause between passes. False if the wait timed out.
__device__ __forceinline__ bool fetch_tagged(const uint32_t* src, int K, uint32_t tag, uint32_t* stg,
                                             uint32_t* err, int lane, bool broken) {
  const int nch = K / 4;   // 16-byte chunks of 4 words
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
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + 4 * (64 * k + lane));
        if ((v.x >> 16) == tag && (v.y >> 16) == tag && (v.z >> 16) == tag && (v.w >> 16) == tag)
          pend &= ~(1ull << k);
      }
    }
    if (!__any(pend != 0)) return true;
    if (broken || ++spins > SPIN_LIMIT) {
      if (!broken && lane == 0) add_dev(err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Wait until every workgroup's hint word has reached `tag32` (it finished the
// stage with that tag). One batched round trip per poll. False on timeout.
__device__ __forceinline__ bool wait_hints(const uint32_t* hint, int nb, uint32_t tag32, uint32_t* err, int lane) {
  const rsrc_t hs = make_rsrc(hint, (uint32_t)nb * LINE * 4u);
  uint32_t spins = 0;
  for (;;) {
    // plain loads at the device coherence point (SC1), which the compiler may
    // batch; the memory clobber makes each poll load again
    asm volatile("" ::: "memory");
    bool behind = false;
#pragma unroll
    for (int k = 0; k < kq::STACK_MAX_WG / 64; ++k) {
      const int i = lane + 64 * k;
      const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(hs, (uint32_t)i * LINE * 4u, 0, SC1);
      behind |= i < nb && (int32_t)(v - tag32) < 0;
    }
    if (!__any(behind)) return true;
    if (++spins > SPIN_LIMIT) {
      if (lane == 0) add_dev(err, 1u);
      return false;
    }
  }
}

// Turn the staged x (plain fp16, or tagged words) into the rotated LDS layout
// (see load_x_col) and form the half-block sums xs[h] of elements 16h..16h+15.
__device__ __forceinline__ void place_x(const uint32_t* stg, bool tagged, int K, int ub, uint32_t* xl, float* xs,
                                        int lane) {
  const int P = 4 * ub;
  u32x4* xq = reinterpret_cast<u32x4*>(xl);
  for (int h = lane; h < K / 16; h += 64) {
    float sum = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int Q = 2 * h + half;   // quad of x: elements 8Q .. 8Q+7
      u32x4 v;
      if (tagged) {
        const u32x4* t = reinterpret_cast<const u32x4*>(stg + 8 * Q);
        const u32x4 a = t[0], c = t[1];
        v.x = perm(a.y, a.x, 0x05040100u);   // fp16 of words 8Q, 8Q+1
        v.y = perm(a.w, a.z, 0x05040100u);
        v.z = perm(c.y, c.x, 0x05040100u);
        v.w = perm(c.w, c.z, 0x05040100u);
      } else {
        v = *reinterpret_cast<const u32x4*>(stg + 4 * Q);
      }
      sum = dot2(v.x, ONES, sum);
      sum = dot2(v.y, ONES, sum);
      sum = dot2(v.z, ONES, sum);
      sum = dot2(v.w, ONES, sum);
      const int c = Q / P, p = Q - c * P;
      const int rot = ub == 1 ? (c >> 1) : c;
      xq[c * P + ((p + rot) & (P - 1))] = v;
    }
    xs[h] = sum;
  }
}

__device__ __forceinline__ void control_wave(const StackStage* st, int n, uint32_t* sync, int b, int nb,
                                             uint32_t* xl, float* xs, uint32_t* stg, const float* yacc) {
  const int lane = threadIdx.x & 63;
  uint32_t* err = sync + kq::STACK_ERR_WORD;
  uint32_t* epoch_word = sync + kq::STACK_EPOCH_WORD + (int64_t)b * LINE;
  uint32_t* hints = sync + kq::STACK_HINT_WORD;
  const uint32_t epoch = ld_dev(epoch_word);
  const uint32_t tag_base = epoch * (uint32_t)(n + 1) + 1u;   // tag of stage s: tag_base + s
  bool broken = false;
  for (int s = 0; s < n; ++s) {
    const StackStage d = load_stage(st, s);
    const Share sh = share_of(d, b);
    if (sh.rows > 0) {
      const int ub = d.fmt == F_AFFINE4 ? 1 : 2;
      if (d.ll_in) {
        const uint32_t dep_tag = tag_base + (uint32_t)d.dep;
        if (!broken && !wait_hints(hints, nb, dep_tag, err, lane)) broken = true;
        const uint32_t* src = d.ll_in + (int64_t)(b % kq::STACK_LL_COPIES) * d.ll_in_stride;
        if (!fetch_tagged(src, d.K, dep_tag & 0xffffu, stg, err, lane, broken)) broken = true;
        place_x(stg, true, d.K, ub, xl, xs, lane);
      } else {
        dma_chunks(d.x, d.K / 8, stg, lane);
        place_x(stg, false, d.K, ub, xl, xs, lane);
      }
    }
    __syncthreads();   // x of stage s is in LDS
    __syncthreads();   // the compute waves have left every row of the share in yacc
    // Outputs: y and y16 with ordinary stores (read after the launch); the
    // tagged copy for later stages with device-coherent stores, value and tag
    // in one word, so a reader on any XCD sees both or neither; then the hint.
    const uint32_t out_tag = ((tag_base + (uint32_t)s) & 0xffffu) << 16;
    for (int r = lane; r < sh.rows; r += 64) {
      const float v = yacc[r];
      const int64_t row = sh.r0 + r;
      d.y[row] = v;
      const uint32_t h = f2h_bits(v);
      if (d.y16) d.y16[row] = (uint16_t)h;
      if (d.ll_out) {
#pragma unroll
        for (int c = 0; c < kq::STACK_LL_COPIES; ++c) st_dev(d.ll_out + (int64_t)c * d.ll_out_stride + row, h | out_tag);
      }
    }
    if (lane == 0) st_dev(hints + (int64_t)b * LINE, tag_base + (uint32_t)s);
  }
  wait_vmem();
  if (lane == 0) st_dev(epoch_word, epoch + 1u);
}

template <int FMASK>
__global__ __launch_bounds__(64 * (CWAVES + 1)) void k_stack(const StackStage* __restrict__ st, int n,
                                                            uint32_t* __restrict__ sync, int kmax) {
  extern __shared__ u32x4 lds4[];
  uint32_t* xl = reinterpret_cast<uint32_t*>(lds4);      // x, rotated: kmax/2 dwords
  float* xs = reinterpret_cast<float*>(xl + kmax / 2);     // half-block sums: kmax/16
  uint32_t* stg = reinterpret_cast<uint32_t*>(xs + kmax / 16);   // staging: kmax dwords
  float* yacc = reinterpret_cast<float*>(stg + kmax);      // rows of the share
  const int b = blockIdx.x;
  if (wave_id() == CWAVES)
    control_wave(st, n, sync, b, gridDim.x, xl, xs, stg, yacc);
  else
    compute_wave<FMASK>(st, n, b, xl, xs, yacc);
}

}  // namespace kqd

namespace kq {

using namespace kqd;

int stack_log2g(int64_t rows_max, int upr) {
  int best = 2;
  int64_t best_steps = -1;
  for (int l = 2; l <= 6; ++l) {
    const int64_t groups = (int64_t)STACK_CWAVES << (6 - l);
    const int64_t steps = (rows_max + groups - 1) / groups * ((upr + (1 << l) - 1) >> l);
    if (best_steps < 0 || steps < best_steps) {
      best = l;
      best_steps = steps;
    }
  }
  return best;
}

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
  return ((int64_t)kmax / 2 + kmax / 16 + kmax + STACK_MAX_SHARE_ROWS) * 4;
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
