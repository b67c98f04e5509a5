// api.hip - error reporting and host-only entry points of libfp.
#include <string.h>

#include <vector>

#include "common.hpp"

namespace {
thread_local char g_msg[512] = "";
}

namespace fpi {

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_msg[0] = 0;
  return FP_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FP_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return FP_OK;
}

}  // namespace fpi

extern "C" const char* fp_last_error(void) { return g_msg; }

// MoE grouping plan ("How fast can FlashProve go", §2: each token goes to one
// of the routed experts). Counting sort by expert; stable, so tokens stay in
// ascending order within a group.
extern "C" int fp_moe_plan(const int32_t* route, int32_t T, int32_t n_experts, int32_t* counts, int32_t* offsets,
                           int32_t* perm) {
  if (T < 0 || n_experts < 1) return fpi::fail(FP_EARG, "fp_moe_plan: T=%d n_experts=%d", T, n_experts);
  if ((T > 0 && (!route || !perm)) || !counts || !offsets) return fpi::fail(FP_EARG, "fp_moe_plan: null pointer");
  for (int32_t e = 0; e < n_experts; ++e) counts[e] = 0;
  for (int32_t t = 0; t < T; ++t) {
    if (route[t] < 0 || route[t] >= n_experts)
      return fpi::fail(FP_EARG, "fp_moe_plan: route[%d]=%d outside [0, %d)", t, route[t], n_experts);
    ++counts[route[t]];
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < n_experts; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> fill(offsets, offsets + n_experts);
  for (int32_t t = 0; t < T; ++t) perm[fill[route[t]]++] = t;
  return fpi::ok();
}

namespace {
__global__ __launch_bounds__(256) void gather_rows_kernel(const int8_t* __restrict__ X, int64_t ldx,
                                                          const int32_t* __restrict__ perm, int32_t cols,
                                                          int8_t* __restrict__ Xg, int vec) {
  const int row = blockIdx.x;
  const int8_t* src = X + (int64_t)perm[row] * ldx;
  int8_t* dst = Xg + (int64_t)row * cols;
  if (vec) {
    for (int c = threadIdx.x * 16; c < cols; c += 256 * 16) *(uint4*)(dst + c) = *(const uint4*)(src + c);
  } else {
    for (int c = threadIdx.x; c < cols; c += 256) dst[c] = src[c];
  }
}
}  // namespace

extern "C" int fp_gather_rows(const int8_t* X, int64_t ldx, const int32_t* perm, int32_t n_rows, int32_t cols,
                              int8_t* Xg, hipStream_t stream) {
  if (n_rows < 0 || cols < 0 || ldx < cols) return fpi::fail(FP_EARG, "fp_gather_rows: bad sizes");
  if (n_rows == 0 || cols == 0) return fpi::ok();
  if (!X || !perm || !Xg) return fpi::fail(FP_EARG, "fp_gather_rows: null pointer");
  const int vec = ((cols & 15) == 0) && ((ldx & 15) == 0) && ((((uintptr_t)X) & 15) == 0) &&
                  ((((uintptr_t)Xg) & 15) == 0);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(n_rows), dim3(256), 0, stream, X, ldx, perm, cols, Xg, vec);
  int rc = fpi::check_launch("gather_rows_kernel");
  return rc ? rc : fpi::ok();
}
