// blake2b.hpp - BLAKE2b compression for gfx950 device code (RFC 7693,
// Saarinen and Aumasson, 2015): 12 rounds of the G mixing function over a
// 16-word state, unkeyed, 32-byte digests. A thread holds the state and the
// message block in registers; the message schedule is a compile-time table,
// so the fully unrolled rounds index registers only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t B2_IV_H[8] = {0x6a09e667f3bcc908ull, 0xbb67ae8584caa73bull, 0x3c6ef372fe94f82bull,
                                 0xa54ff53a5f1d36f1ull, 0x510e527fade682d1ull, 0x9b05688c2b3e6c1full,
                                 0x1f83d9abfb41bd6bull, 0x5be0cd19137e2179ull};
constexpr unsigned char B2_SIGMA[12][16] = {
    {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15}, {14, 10, 4, 8, 9, 15, 13, 6, 1, 12, 0, 2, 11, 7, 5, 3},
    {11, 8, 12, 0, 5, 2, 15, 13, 10, 14, 3, 6, 7, 1, 9, 4}, {7, 9, 3, 1, 13, 12, 11, 14, 2, 6, 5, 10, 4, 0, 15, 8},
    {9, 0, 5, 7, 2, 4, 10, 15, 14, 1, 11, 12, 6, 8, 3, 13}, {2, 12, 6, 10, 0, 11, 8, 3, 4, 13, 7, 5, 15, 14, 1, 9},
    {12, 5, 1, 15, 14, 13, 4, 10, 0, 7, 6, 3, 9, 2, 8, 11}, {13, 11, 7, 14, 12, 1, 3, 9, 5, 0, 15, 4, 8, 6, 2, 10},
    {6, 15, 14, 9, 11, 3, 0, 8, 12, 2, 13, 7, 1, 4, 10, 5}, {10, 2, 8, 4, 7, 6, 1, 5, 15, 11, 9, 14, 3, 12, 13, 0},
    {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15}, {14, 10, 4, 8, 9, 15, 13, 6, 1, 12, 0, 2, 11, 7, 5, 3}};

// 64-bit rotation right by a constant, as two 32-bit funnel shifts
// (v_alignbit_b32): the 64-bit shift-and-or form costs three to four ops.
template <int N>
__device__ __forceinline__ uint64_t rotr64(uint64_t x) {
  const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  uint32_t rl, rh;
  if constexpr (N == 32) {
    rl = hi;
    rh = lo;
  } else if constexpr (N < 32) {
    rl = __builtin_amdgcn_alignbit(hi, lo, N);
    rh = __builtin_amdgcn_alignbit(lo, hi, N);
  } else {
    rl = __builtin_amdgcn_alignbit(lo, hi, N - 32);
    rh = __builtin_amdgcn_alignbit(hi, lo, N - 32);
  }
  return ((uint64_t)rh << 32) | rl;
}

__device__ __forceinline__ void b2_g(uint64_t& a, uint64_t& b, uint64_t& c, uint64_t& d, uint64_t x, uint64_t y) {
  a = a + b + x;
  d = rotr64<32>(d ^ a);
  c = c + d;
  b = rotr64<24>(b ^ c);
  a = a + b + y;
  d = rotr64<16>(d ^ a);
  c = c + d;
  b = rotr64<63>(b ^ c);
}

// h <- compress(h, m, t, last)
__device__ __forceinline__ void b2_compress(uint64_t (&h)[8], const uint64_t (&m)[16], uint64_t t, bool last) {
  uint64_t v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = h[i];
    v[i + 8] = B2_IV_H[i];
  }
  v[12] ^= t;  // byte counter (messages here are far below 2^64 bytes)
  if (last) v[14] = ~v[14];
#pragma unroll
  for (int r = 0; r < 12; ++r) {
    const unsigned char* s = B2_SIGMA[r];
    b2_g(v[0], v[4], v[8], v[12], m[s[0]], m[s[1]]);
    b2_g(v[1], v[5], v[9], v[13], m[s[2]], m[s[3]]);
    b2_g(v[2], v[6], v[10], v[14], m[s[4]], m[s[5]]);
    b2_g(v[3], v[7], v[11], v[15], m[s[6]], m[s[7]]);
    b2_g(v[0], v[5], v[10], v[15], m[s[8]], m[s[9]]);
    b2_g(v[1], v[6], v[11], v[12], m[s[10]], m[s[11]]);
    b2_g(v[2], v[7], v[8], v[13], m[s[12]], m[s[13]]);
    b2_g(v[3], v[4], v[9], v[14], m[s[14]], m[s[15]]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] ^= v[i] ^ v[i + 8];
}

// ---- one compression spread over the 4 lanes of a quad
// Lane k of the quad holds column k of the working state (v[k], v[4+k],
// v[8+k], v[12+k]) and the chaining words h[k], h[4+k]; the message block is
// in LDS. The column step is one G per lane; for the diagonal step lane k
// takes b, c, d from columns k+1, k+2, k+3 (quad permutes) and returns them
// afterwards. A lane's four message words of round r are m[sigma_r[2k]],
// m[sigma_r[2k+1]] (column step) and m[sigma_r[8+2k]], m[sigma_r[9+2k]]
// (diagonal step): their indices, four nibbles per round, are packed into six
// words per lane (B2Q_SIG). About 2.6 times fewer instructions per lane than
// one lane's whole compression, so a chain of dependent compressions (the
// levels near a Merkle root) waits that much less per step.
struct B2QSig {
  uint32_t w[4][6];
};
constexpr B2QSig b2q_sig() {
  B2QSig t{};
  for (int k = 0; k < 4; ++k)
    for (int r = 0; r < 12; ++r) {
      const unsigned char* s = B2_SIGMA[r];
      const uint32_t v = s[2 * k] | (s[2 * k + 1] << 4) | (s[8 + 2 * k] << 8) | (s[9 + 2 * k] << 12);
      t.w[k][r / 2] |= v << (16 * (r % 2));
    }
  return t;
}
constexpr B2QSig B2Q_SIG = b2q_sig();

// lane k of its quad takes lane (k + ROT) mod 4's value
template <int ROT>
__device__ __forceinline__ uint64_t quad_rot(uint64_t x) {
  constexpr int CTRL = ((0 + ROT) & 3) | (((1 + ROT) & 3) << 2) | (((2 + ROT) & 3) << 4) | (((3 + ROT) & 3) << 6);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t quad_pick(int k, uint64_t a0, uint64_t a1, uint64_t a2, uint64_t a3) {
  return k == 0 ? a0 : (k == 1 ? a1 : (k == 2 ? a2 : a3));
}

// (h0, h1) = (h[k], h[4+k]) <- compress(h, m, t, last) for lane k of a quad;
// m: the block's 16 words (LDS); every lane of the quad must take part.
__device__ __forceinline__ void b2q_compress(uint64_t& h0, uint64_t& h1, const uint64_t* m, uint64_t t, bool last,
                                             int k) {
  uint32_t sg[6];
#pragma unroll
  for (int w = 0; w < 6; ++w)
    sg[w] = k == 0 ? B2Q_SIG.w[0][w] : (k == 1 ? B2Q_SIG.w[1][w] : (k == 2 ? B2Q_SIG.w[2][w] : B2Q_SIG.w[3][w]));
  uint64_t a = h0, b = h1;
  uint64_t c = quad_pick(k, B2_IV_H[0], B2_IV_H[1], B2_IV_H[2], B2_IV_H[3]);
  uint64_t d = quad_pick(k, B2_IV_H[4] ^ t, B2_IV_H[5], last ? ~B2_IV_H[6] : B2_IV_H[6], B2_IV_H[7]);
#pragma unroll
  for (int r = 0; r < 12; ++r) {
    const uint32_t ix = sg[r / 2] >> (16 * (r % 2));
    const uint64_t x0 = m[ix & 15], y0 = m[(ix >> 4) & 15], x1 = m[(ix >> 8) & 15], y1 = m[(ix >> 12) & 15];
    b2_g(a, b, c, d, x0, y0);
    b = quad_rot<1>(b);
    c = quad_rot<2>(c);
    d = quad_rot<3>(d);
    b2_g(a, b, c, d, x1, y1);
    b = quad_rot<3>(b);
    c = quad_rot<2>(c);
    d = quad_rot<1>(d);
  }
  h0 ^= a ^ c;
  h1 ^= b ^ d;
}

// lane k's chaining words (h[k], h[4+k]) of an unkeyed 32-byte digest before its first block
__device__ __forceinline__ void b2q_init32(int k, uint64_t& h0, uint64_t& h1) {
  h0 = quad_pick(k, B2_IV_H[0] ^ 0x01010020ull, B2_IV_H[1], B2_IV_H[2], B2_IV_H[3]);
  h1 = quad_pick(k, B2_IV_H[4], B2_IV_H[5], B2_IV_H[6], B2_IV_H[7]);
}

// parameter block of an unkeyed 32-byte digest: h0 ^= 0x01010000 | 32
__device__ __forceinline__ void b2_init32(uint64_t (&h)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = B2_IV_H[i];
  h[0] ^= 0x01010020ull;
}

}  // namespace
