// eq.hpp - one workgroup's block of an eq table, E[k] = eq(r, k) =
// prod_j (k_j ? r_j : 1 - r_j) ("How fast can FlashProve go", §2: the
// weights of a table's folded row). Shared by the eq-table launch and by the
// witness launch, which builds a proof's eq tables in spare workgroups while
// its GEMM runs.
#pragma once
#include "common.hpp"
#include "gl.hpp"

namespace eqk {

constexpr int EQ_MAX_MID = 6;

// Entries [blk 2^(8+nm), (blk+1) 2^(8+nm)) of the n-variable table (nm mid
// variables, nm <= EQ_MAX_MID, nm = 0 when n <= 8), by 256 threads. The
// challenges and their complements are staged in LDS once; each thread takes
// the product over its entries' low 8 variables (its lane) as a balanced tree
// (depth 3, no barriers); up to 2^nm threads form the product over the
// variables above them (the mid variables that differ between a thread's
// entries, times the high ones, the same for the whole workgroup), and every
// entry is then one multiply.
__device__ __forceinline__ void eq_block(const fp_elem* __restrict__ r, int n, fp_elem* __restrict__ E, int64_t blk,
                                         int nm) {
  __shared__ uint64_t f[2][FP_MAX_N];      // f[1][j] = r_j, f[0][j] = 1 - r_j
  __shared__ uint64_t mh[1 << EQ_MAX_MID];  // product over variables 8 .. n-1 for mid bits k
  const int tid = threadIdx.x;
  const int nl = n < 8 ? n : 8;  // low variables: the lane
  const int hb = 8 + nm;         // first high variable
  if (tid < n) {
    const uint64_t rj = r[tid];
    f[1][tid] = rj;
    f[0][tid] = gl::sub(1, rj);
  }
  __syncthreads();
  const int64_t base = blk << hb;
  if (tid < (1 << nm)) {
    // mid variables from k = tid, high ones from the block (four interleaved
    // partial products keep the chains short)
    uint64_t hp[4] = {1, 1, 1, 1};
#pragma unroll
    for (int j = 8; j < FP_MAX_N; ++j)
      if (j < n) hp[j & 3] = gl::mul(hp[j & 3], f[j < hb ? (tid >> (j - 8)) & 1 : (base >> j) & 1][j]);
    mh[tid] = gl::mul(gl::mul(hp[0], hp[1]), gl::mul(hp[2], hp[3]));
  }
  // the product over the lane's low variables as a balanced tree (factors of
  // absent variables are 1)
  uint64_t lf[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) lf[j] = (j < nl) ? f[(tid >> j) & 1][j] : 1;
  const uint64_t low = gl::mul(gl::mul(gl::mul(lf[0], lf[1]), gl::mul(lf[2], lf[3])),
                               gl::mul(gl::mul(lf[4], lf[5]), gl::mul(lf[6], lf[7])));
  __syncthreads();
  if (tid < (1 << nl)) {
    if (n <= 8) {
      E[base + tid] = low;
    } else {
      for (int k = 0; k < (1 << nm); ++k) E[base + ((int64_t)k << 8) + tid] = gl::mul(low, mh[k]);
    }
  }
}

}  // namespace eqk
