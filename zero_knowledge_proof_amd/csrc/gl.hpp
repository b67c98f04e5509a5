// gl.hpp - Goldilocks field arithmetic for gfx950 device code.
//
// p = 2^64 - 2^32 + 1 ("How fast can FlashProve go", §3.1 names this field).
// Elements are canonical uint64_t in [0, p). gfx950 has no 64x64-bit
// multiplier, so a product is built from 32-bit partial products
// (v_mad_u64_u32) and reduced with 2^64 = 2^32 - 1 and 2^96 = -1 (mod p); the
// same page's §4 (footnote 20) notes that this costs several 32-bit multiplies.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gl {

constexpr uint64_t P = 0xFFFFFFFF00000001ull;
constexpr uint64_t EPS = 0xFFFFFFFFull;  // 2^64 mod p = 2^32 - 1

__device__ __forceinline__ uint64_t canon(uint64_t a) { return a >= P ? a - P : a; }

__device__ __forceinline__ uint64_t add(uint64_t a, uint64_t b) {
  uint64_t s = a + b;
  // a + b < 2p: on a carry the true sum is s + 2^64 = s + EPS (mod p), and
  // s + EPS cannot carry again.
  s += (s < a) ? EPS : 0;
  return canon(s);
}

__device__ __forceinline__ uint64_t sub(uint64_t a, uint64_t b) {
  uint64_t d = a - b;
  // on a borrow d = a - b + 2^64; a - b + p = d - EPS (no further borrow).
  d -= (a < b) ? EPS : 0;
  return d;
}

// 128-bit value (hi:lo) reduced mod p. hi = h0 + 2^32 h1:
// x = lo + 2^64 h0 + 2^96 h1 = lo + EPS*h0 - h1 (mod p). The corrections take
// the carry and borrow flags of the 64-bit adds; h0 * EPS = h0 2^32 - h0 is
// formed with 32-bit subtracts rather than a multiply.
__device__ __forceinline__ uint64_t reduce128(uint64_t lo, uint64_t hi) {
  const uint32_t h0 = (uint32_t)hi, h1 = (uint32_t)(hi >> 32);
  unsigned long long bor, carry, b2;
  uint64_t t = __builtin_subcll(lo, (uint64_t)h1, 0ull, &bor);
  t -= bor ? EPS : 0;  // lo - h1 + p after a borrow; t >= 2^64 - 2^32 then, so no new borrow
  unsigned int b0;
  const uint32_t ulo = __builtin_subc(0u, h0, 0u, &b0);
  const uint64_t u = ((uint64_t)(h0 - b0) << 32) | ulo;  // h0 * (2^32 - 1)
  uint64_t s = __builtin_addcll(t, u, 0ull, &carry);
  s += carry ? EPS : 0;  // after a carry s < u < 2^64 - 2^32, so s + EPS fits
  const uint64_t d = __builtin_subcll(s, P, 0ull, &b2);
  return b2 ? s : d;
}

// Schoolbook product of the 32-bit halves; every partial sum below fits in
// 64 bits (a0 b1 + (a0 b0 >> 32) <= (2^32 - 1) 2^32, likewise for the others),
// so no carry has to be tracked.
__device__ __forceinline__ uint64_t mul(uint64_t a, uint64_t b) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
  const uint32_t b0 = (uint32_t)b, b1 = (uint32_t)(b >> 32);
  const uint64_t p00 = (uint64_t)a0 * b0;
  const uint64_t t1 = (uint64_t)a0 * b1 + (p00 >> 32);
  const uint64_t t2 = (uint64_t)a1 * b0 + (uint32_t)t1;
  const uint64_t hi = (uint64_t)a1 * b1 + (t1 >> 32) + (t2 >> 32);
  const uint64_t lo = (t2 << 32) | (uint32_t)p00;
  return reduce128(lo, hi);
}

// a * c for a small non-negative integer c < 2^32.
__device__ __forceinline__ uint64_t mul_small(uint64_t a, uint32_t c) {
  uint64_t lo_part = (uint64_t)(uint32_t)a * c;
  uint64_t hi_part = (a >> 32) * (uint64_t)c;
  uint64_t lo = lo_part + (hi_part << 32);
  uint64_t hi = (hi_part >> 32) + ((lo < lo_part) ? 1 : 0);
  return reduce128(lo, hi);
}

// The field element of a signed 64-bit integer (v < 0 maps to v + p).
__device__ __forceinline__ uint64_t from_i64(int64_t v) {
  if (v >= 0) return canon((uint64_t)v);
  uint64_t m = (uint64_t)(-(v + 1)) + 1;  // |v| without overflow
  m = canon(m);
  return m ? P - m : 0;
}

// Degree-2 polynomial given by its values at 0, 1, 2, evaluated at x
// (Lagrange form on the nodes 0, 1, 2).
__device__ __forceinline__ uint64_t eval_deg2(uint64_t g0, uint64_t g1, uint64_t g2, uint64_t x) {
  constexpr uint64_t INV2 = 0x7FFFFFFF80000001ull;
  uint64_t xm1 = sub(x, 1), xm2 = sub(x, 2);
  uint64_t l0 = mul(mul(xm1, xm2), INV2);
  uint64_t l1 = mul(x, xm2);
  uint64_t l2 = mul(mul(x, xm1), INV2);
  return add(sub(mul(g0, l0), mul(g1, l1)), mul(g2, l2));
}

}  // namespace gl
