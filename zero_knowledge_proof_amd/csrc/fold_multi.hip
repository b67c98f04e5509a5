// fold_multi.hip - folded rows of one int8 weight matrix for many eq vectors.
//
// out[j, k] = sum_t E_j[t] M[t, k] for requests j < R ("How fast can FlashProve
// go", §2.1: each request of a batch commits the folded row of the weight table,
// its request vector, before one shared opening; §4 counts one pass over the
// weights per request for the matmul sum-checks). Folding R requests one by one
// streams M from HBM R times. Here M is read once per launch and the fold
// becomes an int8 matrix product on the MFMA units:
//
//   E_j[t] = sum_l 2^(8l) e_jl[t],   e_jl[t] the bytes of E_j[t] (0..255)
//   a_jl[t] = e_jl[t] - 128          (a signed byte)
//   sum_t e_jl[t] M[t,k] = sum_t a_jl[t] M[t,k] + 128 c[k],   c[k] = sum_t M[t,k]
//
// The digit rows D[8j + l, t] = a_jl[t] (int8 [8R, rows]) take the weight
// operand's place in the witness GEMM and the transposed matrix Mt[k, t] =
// M[t, k] the token operand's, so each lane ends with the 8 limb sums of one
// request at one column k in its own registers, and the GEMM's epilogue
// reduces them to  sum_l 2^(8l) limb_l + 128 c[k] sum_l 2^(8l)  mod p.
// The reduction over t is split into chunks so that a few requests still fill
// the chip; a small kernel adds the chunks' field values. Mt and c depend on M
// only: the weights are prepared once and reused by every batch of requests.
#include "common.hpp"
#include "gl.hpp"

namespace {

constexpr int TP = 64;  // transpose tile (rows x columns)

// Mt[k, t] = M[t, k] through a 64 x 64 byte tile in LDS.
__global__ __launch_bounds__(256) void transpose_kernel(const int8_t* __restrict__ M, int64_t ld, int32_t rows,
                                                        int32_t cols, int8_t* __restrict__ Mt, int64_t ldt,
                                                        int32_t tiles_c) {
  __shared__ int8_t tile[TP][TP + 4];
  const int tid = threadIdx.x;
  const int t0 = (blockIdx.x / tiles_c) * TP, k0 = (blockIdx.x % tiles_c) * TP;
  const int x = tid & 63, y = tid >> 6;
#pragma unroll
  for (int i = 0; i < TP / 4; ++i) {
    const int t = t0 + y + 4 * i, k = k0 + x;
    tile[y + 4 * i][x] = (t < rows && k < cols) ? M[(int64_t)t * ld + k] : (int8_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TP / 4; ++i) {
    const int k = k0 + y + 4 * i, t = t0 + x;
    if (k < cols && t < rows) Mt[(int64_t)k * ldt + t] = tile[x][y + 4 * i];
  }
}

// c[k] = sum_t Mt[k, t], one wave per k.
__global__ __launch_bounds__(256) void colsum_kernel(const int8_t* __restrict__ Mt, int64_t ldt, int32_t rows,
                                                     int32_t cols, int32_t* __restrict__ c) {
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (k >= cols) return;
  const int8_t* row = Mt + (int64_t)k * ldt;
  int s = 0;
  for (int t = lane; t < rows; t += 64) s += row[t];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (lane == 0) c[k] = s;
}

// A[8j + l, t] = byte_l(E_j[t]) - 128 for t < rows, 0 for rows <= t < ldA.
// One thread per (j, 4 consecutive t): 32 bytes in, one dword into each of 8 rows.
__global__ __launch_bounds__(256) void digits_kernel(const uint64_t* __restrict__ E, int64_t lde, int32_t rows,
                                                     int32_t R, int8_t* __restrict__ A, int64_t ldA) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = ldA / 4;
  const int64_t j = q / per;
  if (j >= R) return;
  const int t = (int)(q - j * per) * 4;
  uint64_t e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = (t + i < rows) ? E[j * lde + t + i] : 0;
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t b = (t + i < rows) ? (((uint32_t)(e[i] >> (8 * l)) & 0xFF) ^ 0x80u) : 0u;  // byte - 128
      w |= b << (8 * i);
    }
    *(uint32_t*)(A + (8 * j + l) * ldA + t) = w;
  }
}

// The same digits in the packed-weight layout: fragment (b, c, q) of 1 KiB at
// ((b nkb + c) 2 + q) 1024, lane u holding row 32 b + u % 32 at k = 64 c +
// 32 (u / 32) + 16 q + 0..15; zero past `rows` and for rows past 8 R (the
// rest of the last 32-row block). One wave per fragment, so each wave writes
// its 1 KiB in one piece; the 8 lanes of a request's limbs read the same 16
// weights (from L1 after the first).
__global__ __launch_bounds__(256) void digits_packed_kernel(const uint64_t* __restrict__ E, int64_t lde, int32_t rows,
                                                            int32_t R, int32_t nrb, int32_t nkb,
                                                            int8_t* __restrict__ Dp) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int64_t f = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (f >= (int64_t)nrb * nkb * 2) return;
  const int u = threadIdx.x & 63;
  const int qq = (int)(f & 1);
  const int64_t bc = f >> 1;
  const int c = (int)(bc % nkb);
  const int64_t row = 32 * (bc / nkb) + (u & 31);
  const int64_t j = row >> 3;
  const int l = (int)(row & 7);
  const int k0 = 64 * c + 32 * (u >> 5) + 16 * qq;
  uint32_t w[4] = {0, 0, 0, 0};
  if (j < R) {
    const uint64_t* e = E + j * lde;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (k0 + i < rows) w[i >> 2] |= ((((uint32_t)(e[k0 + i] >> (8 * l))) & 0xFF) ^ 0x80u) << (8 * (i & 3));  // byte - 128
  }
  *(u32x4*)(Dp + f * 1024 + u * 16) = u32x4{w[0], w[1], w[2], w[3]};
}

// out[j, k] = sum_s part[s][j, k] for k0 <= k < cols (nothing added when
// nsum = 0), and 0 for cols <= k < cols_pad.
__global__ __launch_bounds__(256) void finish_kernel(const uint64_t* __restrict__ part, int64_t psplit, int32_t nsum,
                                                     int32_t k0, int32_t cols, int32_t cols_pad,
                                                     uint64_t* __restrict__ out, int64_t ldo) {
  const int j = blockIdx.y;
  const int k = k0 + blockIdx.x * 256 + threadIdx.x;
  if (k >= cols_pad) return;
  uint64_t v = 0;
  if (k < cols) {
    const uint64_t* q = part + (int64_t)j * cols + k;
#pragma unroll 8
    for (int s = 0; s < nsum; ++s) v = gl::add(v, q[(int64_t)s * psplit]);
  }
  out[(int64_t)j * ldo + k] = v;
}

struct Layout {
  fpi::SplitK p;
  bool packed;      // digit rows in the packed-weight layout (the packed-weight kernel)
  int64_t ldA;      // row-major digit matrix leading dimension (bytes)
  size_t a_bytes;   // digit matrix
  size_t z_bytes;   // field values of the reduction chunks (none without a split)
};

// From 16 requests (128 digit rows) on, the digit rows fill the packed-weight
// kernel's 256-row tiles well enough for its faster loop; fewer stay on the
// row-major kernel's 128-row tiles.
constexpr int32_t PACKED_MIN_R = 16;

Layout layout(int32_t rows, int32_t cols, int32_t R) {
  Layout L{};
  L.packed = R >= PACKED_MIN_R;
  L.p = L.packed ? fpi::splitk_plan_packed(cols, rows, 8 * R) : fpi::splitk_plan(cols, rows, 8 * R);
  L.ldA = (int64_t)fpi::align_up((size_t)(rows > 0 ? rows : 1), 16);
  L.a_bytes = L.packed ? fpi::align_up(fpi::packed_rows_bytes(8 * R, rows > 0 ? rows : 1), 256)
                       : fpi::align_up((size_t)(8 * (int64_t)R) * (size_t)L.ldA, 256);
  L.z_bytes = L.p.ksplit > 1 ? fpi::align_up((size_t)L.p.ksplit * (size_t)R * (size_t)cols * 8, 256) : 0;
  return L;
}

}  // namespace

extern "C" int fp_fold_weights_prepare(const int8_t* M, int64_t ld, int32_t rows, int32_t cols, int8_t* Mt,
                                       int64_t ldt, int32_t* colsum, hipStream_t stream) {
  const char* fn = "fp_fold_weights_prepare";
  if (rows < 0 || cols < 0) return fpi::fail(FP_EARG, "%s: negative size", fn);
  if (rows > FP_MAX_FOLD_ROWS) return fpi::fail(FP_ESHAPE, "%s: rows=%d > %d", fn, rows, FP_MAX_FOLD_ROWS);
  if (ld < cols) return fpi::fail(FP_ESHAPE, "%s: ld < cols", fn);
  if (ldt < rows || (ldt & 15)) return fpi::fail(FP_ESHAPE, "%s: ldt=%lld must be >= rows and a multiple of 16", fn,
                                                (long long)ldt);
  if (cols == 0) return fpi::ok();
  if (!colsum || (rows > 0 && (!M || !Mt))) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  if ((((uintptr_t)Mt) & 15) != 0) return fpi::fail(FP_EARG, "%s: Mt must be 16-byte aligned", fn);
  if (rows > 0) {
    const int tiles_c = (cols + TP - 1) / TP;
    const int64_t blocks = (int64_t)((rows + TP - 1) / TP) * tiles_c;
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, M, ld, rows, cols, Mt, ldt,
                       tiles_c);
    int rc = fpi::check_launch("transpose_kernel");
    if (rc) return rc;
  }
  hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((cols + 3) / 4)), dim3(256), 0, stream, Mt, ldt, rows, cols,
                     colsum);
  int rc = fpi::check_launch("colsum_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" size_t fp_fold_matrix_multi_workspace(int32_t rows, int32_t cols, int32_t R) {
  if (rows < 0 || cols < 0 || R <= 0) return 0;
  const Layout L = layout(rows, cols, R);
  return L.a_bytes + L.z_bytes;
}

extern "C" int fp_fold_matrix_multi(const int8_t* Mt, int64_t ldt, const int32_t* colsum, int32_t rows, int32_t cols,
                                    int32_t R, const fp_elem* E, int64_t lde, fp_elem* out, int64_t ldo,
                                    int32_t cols_pad, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "fp_fold_matrix_multi";
  if (rows < 0 || cols < 0 || R < 0) return fpi::fail(FP_EARG, "%s: negative size", fn);
  if (R > FP_MAX_REQUESTS) return fpi::fail(FP_ESHAPE, "%s: R=%d > %d", fn, R, FP_MAX_REQUESTS);
  if (rows > FP_MAX_FOLD_ROWS) return fpi::fail(FP_ESHAPE, "%s: rows=%d > %d", fn, rows, FP_MAX_FOLD_ROWS);
  if (cols_pad < cols) return fpi::fail(FP_ESHAPE, "%s: cols_pad < cols", fn);
  if (ldt < rows || (ldt & 15)) return fpi::fail(FP_ESHAPE, "%s: ldt must be >= rows and a multiple of 16", fn);
  if (lde < rows || ldo < cols_pad) return fpi::fail(FP_ESHAPE, "%s: lde < rows or ldo < cols_pad", fn);
  if (R == 0 || cols_pad == 0) return fpi::ok();
  if (!out) return fpi::fail(FP_EARG, "%s: null out", fn);
  if (cols > 0 && (!colsum || (rows > 0 && (!Mt || !E)))) return fpi::fail(FP_EARG, "%s: null input", fn);
  if (cols > 0 && rows > 0 && (((uintptr_t)Mt) & 15)) return fpi::fail(FP_EARG, "%s: Mt must be 16-byte aligned", fn);
  const Layout L = layout(rows, cols, R);
  const bool gemm = cols > 0 && rows > 0;
  int32_t nsum = 0, k0 = 0;
  uint64_t* part = nullptr;
  int64_t psplit = 0;
  if (gemm) {
    if (!ws || ws_bytes < L.a_bytes + L.z_bytes)
      return fpi::fail(FP_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, L.a_bytes + L.z_bytes);
    if (((uintptr_t)ws) & 255) return fpi::fail(FP_EARG, "%s: workspace must be 256-byte aligned", fn);
    int8_t* A = (int8_t*)ws;
    int rc;
    if (L.packed) {
      const int32_t nkb = (rows + fpi::PACK_BK - 1) / fpi::PACK_BK;
      const int32_t nrb = (8 * R + 31) / 32;
      const int64_t frags = (int64_t)nrb * nkb * 2;
      hipLaunchKernelGGL(digits_packed_kernel, dim3((unsigned)((frags + 3) / 4)), dim3(256), 0, stream, E, lde, rows, R,
                         nrb, nkb, A);
      rc = fpi::check_launch("digits_packed_kernel");
    } else {
      const int64_t threads = (int64_t)R * (L.ldA / 4);
      hipLaunchKernelGGL(digits_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, E, lde, rows,
                         R, A, L.ldA);
      rc = fpi::check_launch("digits_kernel");
    }
    if (rc) return rc;
    auto gemm_into = [&](uint64_t* dst, int64_t ldp, int64_t ps) {
      return L.packed ? fpi::witness_fold_splitk_packed(Mt, ldt, A, cols, rows, 8 * R, colsum, L.p, dst, ldp, ps, stream)
                      : fpi::witness_fold_splitk(Mt, ldt, A, L.ldA, cols, rows, 8 * R, colsum, L.p, dst, ldp, ps, stream);
    };
    if (L.p.ksplit > 1) {  // chunks into the workspace, added below
      part = (uint64_t*)((char*)ws + L.a_bytes);
      psplit = (int64_t)R * cols;
      nsum = L.p.ksplit;
      rc = gemm_into(part, cols, psplit);
    } else {  // straight into out; only the padding is left
      k0 = cols;
      rc = gemm_into(out, ldo, 0);
    }
    if (rc) return rc;
  }
  // rows == 0: every fold is 0
  if (cols_pad > k0) {
    hipLaunchKernelGGL(finish_kernel, dim3((unsigned)((cols_pad - k0 + 255) / 256), (unsigned)R), dim3(256), 0, stream,
                       part, psplit, nsum, k0, cols, cols_pad, out, ldo);
    int rc = fpi::check_launch("finish_kernel");
    if (rc) return rc;
  }
  return fpi::ok();
}
