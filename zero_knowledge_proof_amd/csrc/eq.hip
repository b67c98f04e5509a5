// eq.hip - eq-table expansion: E[k] = eq(r, k) = prod_j (k_j ? r_j : 1 - r_j).
//
// "How fast can FlashProve go", §2: a table's folded row is the weighted sum
// of its rows; these are the weights. One launch takes a list of tables; a
// workgroup writes 256 entries (eqk::eq_block), or 4096 for tables of at least
// 2^16, so large tables are written at memory speed.
#include "common.hpp"
#include "eq.hpp"
#include "gl.hpp"

namespace {

struct EqJob {
  const fp_elem* r;
  fp_elem* E;
  int32_t n;
  int32_t block_start;
};
// descriptors carried in one launch's arguments (the MoE block's ~370 tables
// of a step in three launches instead of eight)
constexpr int EQ_INLINE = 160;
struct EqList {
  EqJob j[EQ_INLINE];
  int32_t count;
};
static_assert(sizeof(EqList) <= 4096, "an eq list travels in the kernel arguments");

// Mid variables of an n-variable table: 4 (4096 entries per workgroup) once
// the table has at least 2^16 entries, none below (256 per workgroup, more
// workgroups for the small, latency-bound tables).
__host__ __device__ constexpr int eq_mid(int n) { return n >= 16 ? 4 : 0; }

__global__ __launch_bounds__(256) void eq_kernel(EqList jl) {
  // the last job whose first workgroup is at or before this one (binary search)
  int lo = 0, hi = jl.count - 1;
#pragma unroll 1
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (jl.j[mid].block_start <= (int)blockIdx.x) lo = mid;
    else hi = mid - 1;
  }
  const EqJob& j = jl.j[lo];
  eqk::eq_block(j.r, j.n, j.E, (int)blockIdx.x - j.block_start, eq_mid(j.n));
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
