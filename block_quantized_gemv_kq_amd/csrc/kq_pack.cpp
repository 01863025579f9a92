// kq_pack.cpp — host-side block-format packer and unpacker.
//
// Encodes fp32 weight rows into Q8_0, Q4_0, affine4 gs32, Q5_0 and Q5_1
// blocks (the block definitions are in include/kq.h). The 4-bit formats are
// the two the Kipp README, "How fast" contrasts: affine4 carries a bias term,
// Q4_0 is scale-only; Q5_0 and Q5_1 are the same two schemes with a fifth bit
// (Kinetic docs, "Supported models" list them among the GGUF weights). Kinetic docs, "Switching from llama.cpp" describe a quantizer
// that writes fixed bytes per format; this packer writes the bytes fixed by
// those definitions (byte equality with any other tool is not claimed).
//
// Built with -ffp-contract=off: every step is a single IEEE fp32 operation
// with round-to-nearest-even, so the bytes are reproducible.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <thread>
#include <vector>

#include "kq_internal.h"

namespace kq {

// fp32 -> fp16 bits, round to nearest even, subnormals kept, overflow to inf.
uint16_t f32_to_f16_bits(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) {                    // inf or NaN
    return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? (0x0200u | ((ax >> 13) & 0x3ffu)) : 0u));
  }
  const uint32_t e = ax >> 23;                // biased fp32 exponent
  if (e >= 113) {                             // |f| >= 2^-14: normal fp16 (or overflow)
    uint32_t h = ((e - 112) << 10) | ((ax >> 13) & 0x3ffu);
    const uint32_t rem = ax & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;   // carry may reach inf
    if (h >= 0x7c00u) h = 0x7c00u;
    return (uint16_t)(sign | h);
  }
  if (e < 102) return (uint16_t)sign;         // |f| < 2^-25: rounds to zero
  // subnormal: value = m * 2^(e-150), unit 2^-24 -> k = m >> (126 - e), RNE
  const uint32_t m = (ax & 0x7fffffu) | 0x800000u;
  const int shift = 126 - (int)e;             // 14..24
  uint32_t k = m >> shift;
  const uint32_t rem = m & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (k & 1u))) k += 1;
  return (uint16_t)(sign | k);                // k == 0x400 is the smallest normal
}

float f16_bits_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1fu;
  const uint32_t m = h & 0x3ffu;
  uint32_t x;
  if (e == 0x1f) {
    x = sign | 0x7f800000u | (m << 13);
  } else if (e == 0) {
    // subnormal or zero: m * 2^-24, exact in fp32
    const float v = (float)m * 5.9604644775390625e-08f;
    memcpy(&x, &v, 4);
    x |= sign;
  } else {
    x = sign | ((e + 112) << 23) | (m << 13);
  }
  float f;
  memcpy(&f, &x, 4);
  return f;
}

namespace {

inline float round_half_away(float v) { return std::round(v); }  // C round(): half away from zero

inline bool finite16(uint16_t h) { return (h & 0x7c00u) != 0x7c00u; }

inline void put16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xff);
  p[1] = (uint8_t)(v >> 8);
}

// One block of 32 weights -> bytes. Returns false on a range error.
bool pack_q8_0(const float* w, uint8_t* out) {
  float a = 0.0f;
  for (int j = 0; j < 32; ++j) a = std::max(a, std::fabs(w[j]));
  const uint16_t dh = f32_to_f16_bits(a / 127.0f);
  if (!finite16(dh)) return false;
  const float d = f16_bits_to_f32(dh);
  put16(out, dh);
  for (int j = 0; j < 32; ++j) {
    int q = 0;
    if (d != 0.0f) {
      const float r = round_half_away(w[j] / d);
      q = (int)std::min(127.0f, std::max(-127.0f, r));
    }
    out[2 + j] = (uint8_t)(int8_t)q;
  }
  return true;
}

bool pack_q4_0(const float* w, uint8_t* out) {
  int istar = 0;
  float amax = std::fabs(w[0]);
  for (int j = 1; j < 32; ++j) {
    const float a = std::fabs(w[j]);
    if (a > amax) { amax = a; istar = j; }     // strict: first index wins ties
  }
  const uint16_t dh = f32_to_f16_bits(w[istar] / -8.0f);
  if (!finite16(dh)) return false;
  const float d = f16_bits_to_f32(dh);
  put16(out, dh);
  uint8_t q[32];
  for (int j = 0; j < 32; ++j) {
    int v = 8;
    if (d != 0.0f) {
      const float r = round_half_away(w[j] / d) + 8.0f;
      v = (int)std::min(15.0f, std::max(0.0f, r));
    }
    q[j] = (uint8_t)v;
  }
  for (int j = 0; j < 16; ++j) out[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
  return true;
}

bool pack_affine4(const float* w, uint8_t* out) {
  float lo = w[0], hi = w[0];
  for (int j = 1; j < 32; ++j) {               // strict: first index wins ties
    if (w[j] < lo) lo = w[j];
    if (w[j] > hi) hi = w[j];
  }
  const float range = hi - lo;
  const uint16_t sh = f32_to_f16_bits(range / 15.0f);
  const uint16_t bh = f32_to_f16_bits(lo);
  if (!finite16(sh) || !finite16(bh)) return false;
  const float s = f16_bits_to_f32(sh);
  const float b = f16_bits_to_f32(bh);
  put16(out, sh);
  put16(out + 2, bh);
  uint8_t q[32];
  for (int j = 0; j < 32; ++j) {
    int v = 0;
    if (s != 0.0f) {
      const float diff = w[j] - b;
      const float r = round_half_away(diff / s);
      v = (int)std::min(15.0f, std::max(0.0f, r));
    }
    q[j] = (uint8_t)v;
  }
  for (int j = 0; j < 16; ++j) out[4 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
  return true;
}

// The 5-bit formats: bit 4 of q_j in bit j of a little-endian word, the low
// four bits as nibbles (element j low, j + 16 high), after the scale(s).
void put_q5_bits(const uint8_t (&q)[32], uint8_t* out) {
  uint32_t hbits = 0;
  for (int j = 0; j < 32; ++j) hbits |= (uint32_t)((q[j] >> 4) & 1u) << j;
  for (int i = 0; i < 4; ++i) out[i] = (uint8_t)(hbits >> (8 * i));
  for (int j = 0; j < 16; ++j) out[4 + j] = (uint8_t)((q[j] & 15) | ((q[j + 16] & 15) << 4));
}

bool pack_q5_0(const float* w, uint8_t* out) {
  int istar = 0;
  float amax = std::fabs(w[0]);
  for (int j = 1; j < 32; ++j) {
    const float a = std::fabs(w[j]);
    if (a > amax) { amax = a; istar = j; }     // strict: first index wins ties
  }
  const uint16_t dh = f32_to_f16_bits(w[istar] / -16.0f);
  if (!finite16(dh)) return false;
  const float d = f16_bits_to_f32(dh);
  put16(out, dh);
  uint8_t q[32];
  for (int j = 0; j < 32; ++j) {
    int v = 16;
    if (d != 0.0f) {
      const float r = round_half_away(w[j] / d) + 16.0f;
      v = (int)std::min(31.0f, std::max(0.0f, r));
    }
    q[j] = (uint8_t)v;
  }
  put_q5_bits(q, out + 2);
  return true;
}

bool pack_q5_1(const float* w, uint8_t* out) {
  float lo = w[0], hi = w[0];
  for (int j = 1; j < 32; ++j) {               // strict: first index wins ties
    if (w[j] < lo) lo = w[j];
    if (w[j] > hi) hi = w[j];
  }
  const float range = hi - lo;
  const uint16_t dh = f32_to_f16_bits(range / 31.0f);
  const uint16_t mh = f32_to_f16_bits(lo);
  if (!finite16(dh) || !finite16(mh)) return false;
  const float d = f16_bits_to_f32(dh);
  const float m = f16_bits_to_f32(mh);
  put16(out, dh);
  put16(out + 2, mh);
  uint8_t q[32];
  for (int j = 0; j < 32; ++j) {
    int v = 0;
    if (d != 0.0f) {
      const float diff = w[j] - m;
      const float r = round_half_away(diff / d);
      v = (int)std::min(31.0f, std::max(0.0f, r));
    }
    q[j] = (uint8_t)v;
  }
  put_q5_bits(q, out + 4);
  return true;
}

bool pack_block(int fmt, const float* w, uint8_t* out) {
  switch (fmt) {
    case KQ_Q8_0: return pack_q8_0(w, out);
    case KQ_Q4_0: return pack_q4_0(w, out);
    case KQ_AFFINE4_G32: return pack_affine4(w, out);
    case KQ_Q5_0: return pack_q5_0(w, out);
    default: return pack_q5_1(w, out);
  }
}

bool pack_rows(int fmt, const float* W, int64_t r0, int64_t r1, int64_t K, uint8_t* out) {
  const int64_t nb = K / 32;
  const int64_t bb = block_bytes(fmt);
  for (int64_t r = r0; r < r1; ++r) {
    const float* wr = W + r * K;
    uint8_t* orow = out + r * nb * bb;
    for (int64_t b = 0; b < nb; ++b) {
      const float* w = wr + b * 32;
      for (int j = 0; j < 32; ++j)
        if (!std::isfinite(w[j])) return false;
      if (!pack_block(fmt, w, orow + b * bb)) return false;
    }
  }
  return true;
}

}  // namespace

int64_t block_bytes(int fmt) {
  switch (fmt) {
    case KQ_Q8_0: return 34;
    case KQ_Q4_0: return 18;
    case KQ_AFFINE4_G32: return 20;
    case KQ_Q5_0: return 22;
    case KQ_Q5_1: return 24;
    default: return -1;
  }
}

int pack(int fmt, const float* W, int64_t N, int64_t K, void* out, int n_threads) {
  uint8_t* o = static_cast<uint8_t*>(out);
  if (N == 0) return KQ_OK;
  int nt = n_threads;
  if (nt <= 0) nt = (int)std::min<unsigned>(64u, std::max(1u, std::thread::hardware_concurrency()));
  const int64_t work = N * K;
  if (work < (1 << 20)) nt = 1;
  nt = (int)std::min<int64_t>(nt, N);
  if (nt <= 1) return pack_rows(fmt, W, 0, N, K, o) ? KQ_OK : KQ_ERR_RANGE;
  std::vector<std::thread> th;
  std::vector<char> ok(nt, 1);
  for (int t = 0; t < nt; ++t) {
    const int64_t r0 = N * t / nt, r1 = N * (t + 1) / nt;
    th.emplace_back([=, &ok] { ok[t] = pack_rows(fmt, W, r0, r1, K, o) ? 1 : 0; });
  }
  for (auto& t : th) t.join();
  for (char c : ok)
    if (!c) return KQ_ERR_RANGE;
  return KQ_OK;
}

int unpack(int fmt, const void* packed, int64_t N, int64_t K, float* W) {
  const uint8_t* p = static_cast<const uint8_t*>(packed);
  const int64_t nb = K / 32;
  const int64_t bb = block_bytes(fmt);
  for (int64_t r = 0; r < N; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* blk = p + (r * nb + b) * bb;
      float* w = W + r * K + b * 32;
      const uint16_t h0 = (uint16_t)(blk[0] | (blk[1] << 8));
      if (fmt == KQ_Q8_0) {
        const float d = f16_bits_to_f32(h0);
        for (int j = 0; j < 32; ++j) w[j] = d * (float)(int8_t)blk[2 + j];
      } else if (fmt == KQ_Q4_0) {
        const float d = f16_bits_to_f32(h0);
        for (int j = 0; j < 16; ++j) {
          w[j] = d * (float)((blk[2 + j] & 15) - 8);
          w[j + 16] = d * (float)((blk[2 + j] >> 4) - 8);
        }
      } else if (fmt == KQ_Q5_0 || fmt == KQ_Q5_1) {
        const float d = f16_bits_to_f32(h0);
        const int hb = fmt == KQ_Q5_0 ? 2 : 4;   // fifth-bit word offset
        const float m = fmt == KQ_Q5_1 ? f16_bits_to_f32((uint16_t)(blk[2] | (blk[3] << 8))) : 0.0f;
        const uint32_t hbits = (uint32_t)blk[hb] | ((uint32_t)blk[hb + 1] << 8) | ((uint32_t)blk[hb + 2] << 16) |
                               ((uint32_t)blk[hb + 3] << 24);
        for (int j = 0; j < 32; ++j) {
          const uint8_t nib = blk[hb + 4 + (j & 15)];
          const int q = (j < 16 ? (nib & 15) : (nib >> 4)) | (int)(((hbits >> j) & 1u) << 4);
          w[j] = fmt == KQ_Q5_0 ? d * (float)(q - 16) : std::fma(d, (float)q, m);
        }
      } else {
        const float s = f16_bits_to_f32(h0);
        const float bias = f16_bits_to_f32((uint16_t)(blk[2] | (blk[3] << 8)));
        for (int j = 0; j < 16; ++j) {
          w[j] = std::fma(s, (float)(blk[4 + j] & 15), bias);
          w[j + 16] = std::fma(s, (float)(blk[4 + j] >> 4), bias);
        }
      }
    }
  }
  return KQ_OK;
}

// ------------------------------------------------------- Shortlist bound copy
// From the bytes of a Q8_0 matrix (K a multiple of 256), the bound copy the
// Shortlist argmax reads instead of the full layer (Kinetic docs, "What makes
// it fast": a small copy bounds every row's score). Each int8 quant q splits
// as q = 8 (v - 16) + ql with v = floor(q / 8) + 16 (0..31) and ql = q & 7; per
// row the copy keeps the block scales, v as Q5_0-style fifth-bit words and
// nibbles, and E, the least fp32 with E^2 >= S = sum_b d_b^2 sum_j (ql_j - 3.5)^2
// (the squared 2-norm of the row's error when ql is replaced by 3.5). S is
// formed exactly in integers: with |d| = M 2^e (M < 2^11, e in -24..5 from
// the fp16 bits) and Q = sum_j (2 ql_j - 7)^2 (< 2^11), 4 S 2^48 is the sum of
// M^2 Q 2^(2e + 48), each term below 2^91.
namespace {

typedef unsigned __int128 u128;

// fp16 magnitude as M * 2^e; false for inf/NaN.
bool f16_mant_exp(uint16_t h, uint32_t* M, int* e) {
  const uint32_t ex = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  if (ex == 0x1f) return false;
  if (ex == 0) {
    *M = m;
    *e = -24;
  } else {
    *M = m | 0x400u;
    *e = (int)ex - 25;
  }
  return true;
}

// Is f^2 >= S, with S = s4 * 2^-50 (s4 as above)? f >= 0 finite fp32.
bool square_covers(float f, u128 s4) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint32_t ex = (x >> 23) & 0xffu;
  const uint64_t F = ex ? ((x & 0x7fffffu) | 0x800000u) : (x & 0x7fffffu);
  const int G = ex ? (int)ex - 150 : -149;            // f = F 2^G
  const u128 F2 = (u128)F * F;                         // < 2^48
  const int sh = 2 * G + 50;                           // f^2 2^50 = F2 2^sh
  if (F2 == 0) return s4 == 0;
  if (sh >= 0) {
    if (sh > 79) return true;                          // F2 2^sh >= 2^79 > any s4 here
    return (F2 << sh) >= s4;
  }
  const int k = -sh;
  if (k >= 128) return s4 == 0;
  if (s4 >> (127 - k)) return false;                   // s4 2^k >= 2^127 > F2
  return F2 >= (s4 << k);
}

float norm_up(u128 s4) {
  if (s4 == 0) return 0.0f;
  const double S = std::ldexp((double)s4, -50);
  float f = (float)std::sqrt(S);
  while (!square_covers(f, s4)) f = std::nextafter(f, INFINITY);
  while (f > 0.0f && square_covers(std::nextafter(f, 0.0f), s4)) f = std::nextafter(f, 0.0f);
  return f;
}

bool shortlist_rows(const uint8_t* q8, int64_t r0, int64_t r1, int64_t K, int64_t N, uint8_t* out) {
  const int64_t nb = K / 32;
  const int64_t rb = 22 * nb;
  float* E = reinterpret_cast<float*>(out + N * rb);
  for (int64_t r = r0; r < r1; ++r) {
    uint8_t* dpl = out + r * rb;
    uint8_t* fpl = dpl + 2 * nb;
    uint8_t* npl = dpl + 6 * nb;
    u128 s4 = 0;
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* blk = q8 + (r * nb + b) * 34;
      const uint16_t h = (uint16_t)(blk[0] | (blk[1] << 8));
      uint32_t M;
      int e;
      if (!f16_mant_exp(h, &M, &e)) return false;
      dpl[2 * b] = blk[0];
      dpl[2 * b + 1] = blk[1];
      uint32_t word = 0, Q = 0;
      uint8_t v[32];
      for (int j = 0; j < 32; ++j) {
        const int q = (int8_t)blk[2 + j];
        const int hi = q >> 3;                     // arithmetic shift: floor(q / 8)
        v[j] = (uint8_t)(hi + 16);
        const int ql = q - 8 * hi;
        Q += (uint32_t)((2 * ql - 7) * (2 * ql - 7));
        word |= (uint32_t)((v[j] >> 4) & 1u) << j;
      }
      for (int i = 0; i < 4; ++i) fpl[4 * b + i] = (uint8_t)(word >> (8 * i));
      for (int j = 0; j < 16; ++j) npl[16 * b + j] = (uint8_t)((v[j] & 15u) | ((v[j + 16] & 15u) << 4));
      s4 += ((u128)((uint64_t)M * M) * Q) << (2 * e + 48);
    }
    const float f = norm_up(s4);
    memcpy(E + r, &f, 4);
  }
  return true;
}

}  // namespace

int64_t shortlist_copy_bytes(int64_t N, int64_t K) { return N * (22 * (K / 32) + 4); }

int shortlist_pack(const void* q8, int64_t N, int64_t K, void* out, int n_threads) {
  const uint8_t* p = static_cast<const uint8_t*>(q8);
  uint8_t* o = static_cast<uint8_t*>(out);
  int nt = n_threads;
  if (nt <= 0) nt = (int)std::min<unsigned>(64u, std::max(1u, std::thread::hardware_concurrency()));
  if (N * K < (1 << 20)) nt = 1;
  nt = (int)std::min<int64_t>(nt, N);
  if (nt <= 1) return shortlist_rows(p, 0, N, K, N, o) ? KQ_OK : KQ_ERR_RANGE;
  std::vector<std::thread> th;
  std::vector<char> ok(nt, 1);
  for (int t = 0; t < nt; ++t) {
    const int64_t r0 = N * t / nt, r1 = N * (t + 1) / nt;
    th.emplace_back([=, &ok] { ok[t] = shortlist_rows(p, r0, r1, K, N, o) ? 1 : 0; });
  }
  for (auto& t : th) t.join();
  for (char c : ok)
    if (!c) return KQ_ERR_RANGE;
  return KQ_OK;
}

}  // namespace kq
