// common.hpp - internal helpers shared by the libfp translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "fp.h"

namespace fpi {

// Sets the thread-local message and returns `code`.
int fail(int code, const char* fmt, ...);
// Clears the message; returns FP_OK.
int ok();
// Checks hipGetLastError() after a launch.
int check_launch(const char* what);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Limb folds on the matrix cores. With digit rows D [N, K] (N = 8 R: row
// 8 j + l holds the signed byte digits of request j's weights, limb l) and a
// transposed int8 matrix Xt [T, K], writes for every request j and column t
//   part[s psplit + j ldp + t] = sum_l 2^(8l) sum_{k in chunk s} D[8j+l, k] Xt[t, k]
//                                (+ 128 colsum[t] sum_l 2^(8l) in chunk 0)   mod p,
// the reduction over [0, K) cut into ksplit chunks of kchunk (a multiple of the
// tile's K step; at most 2^16, which keeps each int32 limb sum exact).
constexpr int32_t SPLITK_MAX_CHUNK = 65536;
struct SplitK {
  int32_t ksplit;  // chunks
  int32_t kchunk;  // reduction length per chunk
};
// Split for T tokens, reduction length K and N digit rows.
SplitK splitk_plan(int32_t T, int32_t K, int32_t N);
int witness_fold_splitk(const int8_t* Xt, int64_t ldx, const int8_t* D, int64_t ldd, int32_t T, int32_t K, int32_t N,
                        const int32_t* colsum, const SplitK& p, uint64_t* part, int64_t ldp, int64_t psplit,
                        hipStream_t st);
// The same with the digit rows in the packed-weight layout (Dp, written as
// fp_witness_pack_weights lays out N rows of reduction length K: 1 KiB
// fragments, zero past N and K) on the packed-weight kernel, for which Xt's
// rows must be 16-byte aligned (ldx % 16 == 0); chunks from splitk_plan_packed.
constexpr int PACK_BK = 64;  // K block of the packed layout
SplitK splitk_plan_packed(int32_t T, int32_t K, int32_t N);
size_t packed_rows_bytes(int32_t N, int32_t K);
int witness_fold_splitk_packed(const int8_t* Xt, int64_t ldx, const int8_t* Dp, int32_t T, int32_t K, int32_t N,
                               const int32_t* colsum, const SplitK& p, uint64_t* part, int64_t ldp, int64_t psplit,
                               hipStream_t st);

// Wave64 reductions of a 64-bit value held as two 32-bit halves.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((int)(uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Cross-lane moves of a 64-bit value inside a row of 16 lanes (DPP).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

// v of the lane d above this one (wave64 shuffle).
__device__ __forceinline__ uint64_t shfl_down_u64(uint64_t v, int d) {
  const uint32_t lo = (uint32_t)__shfl_down((int)(uint32_t)v, d, 64);
  const uint32_t hi = (uint32_t)__shfl_down((int)(uint32_t)(v >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

}  // namespace fpi
#include "gl.hpp"
namespace fpi {

// Field sum over the 64 lanes of a wave (every lane active), returned to all
// lanes: DPP butterflies inside each row of 16, then the four row sums.
__device__ __forceinline__ uint64_t wave_total(uint64_t v) {
  v = gl::add(v, dpp_u64<DPP_XOR1>(v));
  v = gl::add(v, dpp_u64<DPP_XOR2>(v));
  v = gl::add(v, dpp_u64<DPP_HALF_MIRROR>(v));
  v = gl::add(v, dpp_u64<DPP_MIRROR>(v));  // every lane: its row's sum
  const uint64_t a = readlane_u64(v, 0), b = readlane_u64(v, 16);
  const uint64_t c = readlane_u64(v, 32), d = readlane_u64(v, 48);
  return gl::add(gl::add(a, b), gl::add(c, d));
}

// --- launchers implemented in the .hip files (no validation inside) -------
int launch_eq(const fp_elem* r, int32_t n, fp_elem* E, hipStream_t st);
int launch_eq_list(int32_t count, const fp_eq_desc* descs_host, hipStream_t st);
size_t eq_batched_ws(int32_t count);

}  // namespace fpi
