// eq.hip - eq-table expansion: E[k] = eq(r, k) = prod_j (k_j ? r_j : 1 - r_j).
//
// "How fast can FlashProve go", §2: a table's folded row is the weighted sum
// of its rows; these are the weights. A workgroup writes 256 entries, or 4096
// for tables of at least 2^16:
// the challenges and their complements are staged in LDS once; each thread
// takes the product over its entries' low 8 variables (its lane) as a
// balanced tree (depth 3, no barriers); up to 16 threads form the product over
// the variables above them (the 4 "mid" variables that differ between a
// thread's 16 entries, times the high ones, the same for the whole workgroup),
// and every entry is then one multiply, so large tables are written at memory
// speed.
#include "common.hpp"
#include "gl.hpp"

namespace {

struct EqJob {
  const fp_elem* r;
  fp_elem* E;
  int32_t n;
  int32_t block_start;
};
constexpr int EQ_INLINE = 48;  // descriptors carried in one launch's arguments
struct EqList {
  EqJob j[EQ_INLINE];
  int32_t count;
};

// Mid variables of an n-variable table: 4 (4096 entries per workgroup) once
// the table has at least 2^16 entries, none below (256 per workgroup, more
// workgroups for the small, latency-bound tables).
__host__ __device__ constexpr int eq_mid(int n) { return n >= 16 ? 4 : 0; }

__device__ __forceinline__ void eq_block(const fp_elem* __restrict__ r, int n, fp_elem* __restrict__ E,
                                         int64_t blk) {
  __shared__ uint64_t f[2][FP_MAX_N];  // f[1][j] = r_j, f[0][j] = 1 - r_j
  __shared__ uint64_t mh[16];          // product over variables 8 .. n-1 for mid bits k
  const int tid = threadIdx.x;
  const int nl = n < 8 ? n : 8;  // low variables: the lane
  const int nm = eq_mid(n);      // mid variables: k
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

__global__ __launch_bounds__(256) void eq_kernel(EqList jl) {
  int k = 0;
#pragma unroll 1
  for (int q = 1; q < jl.count; ++q)
    if (jl.j[q].block_start <= (int)blockIdx.x) k = q;
  const EqJob& j = jl.j[k];
  eq_block(j.r, j.n, j.E, (int)blockIdx.x - j.block_start);
}

inline int64_t eq_blocks(int n) { return n <= 8 ? 1 : (int64_t)1 << (n - 8 - eq_mid(n)); }

}  // namespace

namespace fpi {

int launch_eq_list(int32_t count, const fp_eq_desc* d, hipStream_t st) {
  EqList jl{};
  int64_t blocks = 0;
  for (int32_t i = 0; i <= count; ++i) {
    const bool flush = (i == count) || jl.count == EQ_INLINE || blocks + eq_blocks(d[i].n) > 0x7FFFFFFF;
    if (flush && jl.count > 0) {
      hipLaunchKernelGGL(eq_kernel, dim3((unsigned)blocks), dim3(256), 0, st, jl);
      int rc = check_launch("eq_kernel");
      if (rc) return rc;
      jl = EqList{};
      blocks = 0;
    }
    if (i == count) break;
    jl.j[jl.count++] = EqJob{d[i].r, d[i].E, d[i].n, (int32_t)blocks};
    blocks += eq_blocks(d[i].n);
  }
  return FP_OK;
}

int launch_eq(const fp_elem* r, int32_t n, fp_elem* E, hipStream_t st) {
  fp_eq_desc d{r, n, E};
  return launch_eq_list(1, &d, st);
}

size_t eq_batched_ws(int32_t count) {
  (void)count;
  return 0;
}

}  // namespace fpi

extern "C" int fp_eq_table(const fp_elem* r, int32_t n, fp_elem* E, hipStream_t stream) {
  if (n < 0 || n > FP_MAX_N) return fpi::fail(FP_ESHAPE, "fp_eq_table: n=%d outside [0, %d]", n, FP_MAX_N);
  if (!E || (n > 0 && !r)) return fpi::fail(FP_EARG, "fp_eq_table: null pointer");
  int rc = fpi::launch_eq(r, n, E, stream);
  return rc ? rc : fpi::ok();
}

extern "C" size_t fp_eq_table_batched_workspace(int32_t count) { return fpi::eq_batched_ws(count); }

extern "C" int fp_eq_table_batched(int32_t count, const fp_eq_desc* descs, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (count < 0) return fpi::fail(FP_EARG, "fp_eq_table_batched: count < 0");
  if (count == 0) return fpi::ok();
  if (!descs) return fpi::fail(FP_EARG, "fp_eq_table_batched: null descs");
  for (int32_t i = 0; i < count; ++i) {
    if (descs[i].n < 0 || descs[i].n > FP_MAX_N)
      return fpi::fail(FP_ESHAPE, "fp_eq_table_batched: desc %d has n=%d outside [0, %d]", i, descs[i].n, FP_MAX_N);
    if (!descs[i].E || (descs[i].n > 0 && !descs[i].r))
      return fpi::fail(FP_EARG, "fp_eq_table_batched: desc %d has a null pointer", i);
  }
  int rc = fpi::launch_eq_list(count, descs, stream);
  return rc ? rc : fpi::ok();
}
