// ext.hpp - arithmetic in the quadratic extension F_p[u]/(u^2 - 7) of
// Goldilocks ("How fast can FlashProve go", §4 footnote 20: the protocol's
// challenges and the arithmetic that meets them live in an extension of the
// base field). 7 generates F_p*, so it is not a square and u^2 - 7 is
// irreducible; x = a + u b multiplies as (a c + 7 b d) + u (a d + b c).
#pragma once
#include "gl.hpp"

namespace fpx {

struct E2 {
  uint64_t a, b;  // a + u b, both canonical
};
__device__ __forceinline__ E2 e2_add(E2 x, E2 y) { return E2{gl::add(x.a, y.a), gl::add(x.b, y.b)}; }
__device__ __forceinline__ E2 e2_sub(E2 x, E2 y) { return E2{gl::sub(x.a, y.a), gl::sub(x.b, y.b)}; }
__device__ __forceinline__ E2 e2_mul(E2 x, E2 y) {
  return E2{gl::add(gl::mul(x.a, y.a), gl::mul_small(gl::mul(x.b, y.b), 7u)),
            gl::add(gl::mul(x.a, y.b), gl::mul(x.b, y.a))};
}
__device__ __forceinline__ E2 e2_lerp(E2 x0, E2 x1, E2 r) { return e2_add(x0, e2_mul(r, e2_sub(x1, x0))); }
__device__ __forceinline__ uint64_t canon(uint64_t w) { return w >= gl::P ? w - gl::P : w; }

// eq(r, k) = prod_j (bit j of k ? r_j : 1 - r_j) over n coordinates read by
// coord(j) (extension elements).
template <typename F>
__device__ __forceinline__ E2 eq_at(F coord, int n, int64_t k) {
  E2 e{1, 0};
  for (int j = 0; j < n; ++j) {
    const E2 rj = coord(j);
    e = e2_mul(e, ((k >> j) & 1) ? rj : e2_sub(E2{1, 0}, rj));
  }
  return e;
}

}  // namespace fpx
