// eq.hip - eq-table expansion: E[k] = eq(r, k) = prod_j (k_j ? r_j : 1 - r_j).
//
// "How fast can FlashProve go", §2: a table's folded row is the weighted sum
// of its rows; these are the weights. A workgroup writes 256 entries: the
// challenges and their complements are staged in LDS once, each thread takes
// the product over its entry's low 8 variables as a balanced tree (depth 3, no
// barriers), and multiplies it by the product over the high variables, which
// is the same for the whole workgroup.
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

__device__ __forceinline__ void eq_block(const fp_elem* __restrict__ r, int n, fp_elem* __restrict__ E,
                                         int64_t blk) {
  __shared__ uint64_t f[2][FP_MAX_N];  // f[1][j] = r_j, f[0][j] = 1 - r_j
  const int tid = threadIdx.x;
  const int nl = n < 8 ? n : 8;
  if (tid < n) {
    const uint64_t rj = r[tid];
    f[1][tid] = rj;
    f[0][tid] = gl::sub(1, rj);
  }
  __syncthreads();
  const int64_t base = blk << 8;
  // entry base + tid: the product over its low variables as a balanced tree
  // (factors of absent variables are 1) ...
  uint64_t lf[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) lf[j] = (j < nl) ? f[(tid >> j) & 1][j] : 1;
  const uint64_t low = gl::mul(gl::mul(gl::mul(lf[0], lf[1]), gl::mul(lf[2], lf[3])),
                               gl::mul(gl::mul(lf[4], lf[5]), gl::mul(lf[6], lf[7])));
  // ... times the product over the high variables, the same for the whole
  // block (four interleaved partial products keep the chains short)
  uint64_t hpart[4] = {1, 1, 1, 1};
#pragma unroll
  for (int j = 8; j < FP_MAX_N; ++j)
    if (j < n) hpart[j & 3] = gl::mul(hpart[j & 3], f[(base >> j) & 1][j]);
  if (tid < (1 << nl))
    E[base + tid] = (n > 8) ? gl::mul(low, gl::mul(gl::mul(hpart[0], hpart[1]), gl::mul(hpart[2], hpart[3]))) : low;
}

__global__ __launch_bounds__(256) void eq_kernel(EqList jl) {
  int k = 0;
#pragma unroll 1
  for (int q = 1; q < jl.count; ++q)
    if (jl.j[q].block_start <= (int)blockIdx.x) k = q;
  const EqJob& j = jl.j[k];
  eq_block(j.r, j.n, j.E, (int)blockIdx.x - j.block_start);
}

inline int64_t eq_blocks(int n) { return n <= 8 ? 1 : (int64_t)1 << (n - 8); }

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
