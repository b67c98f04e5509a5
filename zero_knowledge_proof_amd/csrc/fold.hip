// fold.hip - folded rows of integer matrices and MLE evaluation.
//
// out[k] = sum_t E[t] M[t, k] ("How fast can FlashProve go", §2: the folded
// row is the eq-weighted sum of all of a table's rows; §4 counts this as one of
// the three passes over the weights, the one "for the matmuls' sum-checks").
//
// The pass is bound by HBM bandwidth only if the inner loop stays within a few
// vector ops per byte, so no Goldilocks multiply runs per matrix entry. Instead
// the field weight E[t] (< 2^64) is split into 8 unsigned bytes e_l[t] and the
// entry is offset to an unsigned byte u = m + 128 (int8) or to four unsigned
// bytes of m + 2^31 (int32). Then
//     sum_t E[t] m[t,k] = sum_l 2^(8l) sum_t e_l[t] u[t,k]  -  off * sum_t E[t]
// where every inner sum is an exact integer built with v_dot4_u32_u8 over four
// rows at a time (each product of two bytes, four per instruction). A thread
// reads one dword (int8: 4 columns) or one dwordx4 (int32: 4 columns) per row,
// transposes 4 rows x 4 bytes with v_perm_b32 so that each dword holds one
// column's 4 rows, and accumulates into u32 limb sums. The field reduction
// happens once per column per block. Rows are split over row-chunk blocks whose
// per-column partial field values are summed by a second, small kernel (or,
// for an MLE, weighted by the column eq table and summed per block).
#include <vector>

#include "common.hpp"
#include "gl.hpp"

namespace {

constexpr int FT = 256;        // threads per block
constexpr int FCT = 64;        // column threads (one wave wide)
constexpr int FRG = FT / FCT;  // row groups (waves)
constexpr int FCOLS = FCT * 4; // columns per block
constexpr int FMAX_CHUNK = 1024;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct FoldJob {
  const void* M;
  int64_t ld;
  fp_elem* dst;         // partials [n_chunks][cols] (or out when n_chunks == 1 and not MLE)
  const fp_elem* E;     // row weights
  const fp_elem* Ecol;  // MLE column weights (nullptr for a plain fold)
  int32_t rows, cols, cols_pad;
  int32_t chunk_rows, n_chunks, n_colblk;
  int32_t block_start;
  int32_t direct;       // 1: single chunk, write out[] directly incl. zero tail
};

struct JobList {
  const FoldJob* dev;  // device array (batched) or nullptr
  int32_t count;
  FoldJob one;
};

__device__ __forceinline__ FoldJob find_job(const JobList& jl, int b) {
  if (!jl.dev) return jl.one;
  int lo = 0, hi = jl.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (jl.dev[mid].block_start <= b) lo = mid; else hi = mid - 1;
  }
  return jl.dev[lo];
}

// 4x4 byte transpose: w[c] byte i = v[i] byte c.
__device__ __forceinline__ void transpose4(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3, uint32_t& w0,
                                           uint32_t& w1, uint32_t& w2, uint32_t& w3) {
  // v_perm_b32(S0, S1, sel): byte i of the result is byte sel_i of {S0:S1},
  // S1 being bytes 0..3.
  const uint32_t a_lo = __builtin_amdgcn_perm(v1, v0, 0x05010400u);  // v0[0] v1[0] v0[1] v1[1]
  const uint32_t a_hi = __builtin_amdgcn_perm(v1, v0, 0x07030602u);  // v0[2] v1[2] v0[3] v1[3]
  const uint32_t b_lo = __builtin_amdgcn_perm(v3, v2, 0x05010400u);
  const uint32_t b_hi = __builtin_amdgcn_perm(v3, v2, 0x07030602u);
  w0 = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);
  w1 = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);
  w2 = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);
  w3 = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);
}

__device__ __forceinline__ uint32_t udot4(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_udot4(a, b, c, false);
}

// 128-bit accumulate of v << sh (v < 2^32, sh < 96).
__device__ __forceinline__ void acc128(uint64_t& lo, uint64_t& hi, uint32_t v, int sh) {
  uint64_t plo, phi;
  if (sh == 0) { plo = v; phi = 0; }
  else if (sh < 64) { plo = (uint64_t)v << sh; phi = (sh > 32) ? ((uint64_t)v >> (64 - sh)) : 0; }
  else { plo = 0; phi = (uint64_t)v << (sh - 64); }
  const uint64_t nlo = lo + plo;
  hi += phi + (nlo < lo ? 1 : 0);
  lo = nlo;
}

// Row-chunk x column-block kernel. EB = element bytes (1: int8, 4: int32).
template <int EB>
__global__ __launch_bounds__(FT) void fold_rows_kernel(JobList jl) {
  constexpr int NL = (EB == 1) ? 8 : 11;  // limb accumulators per column
  // LDS: E digits for the chunk (8 dwords per 4-row group), reused for the
  // cross-wave reduction (3 waves x 64 threads x 4 cols x NL u32).
  constexpr int DIG_WORDS = FMAX_CHUNK / 4 * 8;
  constexpr int RED_WORDS = (FRG - 1) * FCT * 4 * NL;
  constexpr int LDS_WORDS = DIG_WORDS > RED_WORDS ? DIG_WORDS : RED_WORDS;
  __shared__ __align__(16) uint32_t lds[LDS_WORDS];
  __shared__ uint64_t esum_part[FT / 64];

  const FoldJob job = find_job(jl, blockIdx.x);
  const int lb = blockIdx.x - job.block_start;
  const int chunk = lb / job.n_colblk;
  const int colblk = lb - chunk * job.n_colblk;
  const int tid = threadIdx.x;
  const int ct = tid % FCT, rg = tid / FCT;
  const int row0 = chunk * job.chunk_rows;
  const int nrows = min(job.chunk_rows, job.rows - row0);
  const int ngroups = (nrows + 3) >> 2;

  // ---- prologue: digits of E for this chunk and the chunk's sum of E ----
  uint64_t esum = 0;
  for (int g = tid; g < ngroups; g += FT) {
    uint32_t dg[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g + i;
      const uint64_t e = (t < nrows) ? job.E[row0 + t] : 0;
      esum = gl::add(esum, e);
#pragma unroll
      for (int l = 0; l < 8; ++l) dg[l] |= (uint32_t)((e >> (8 * l)) & 0xFF) << (8 * i);
    }
#pragma unroll
    for (int l = 0; l < 8; ++l) lds[g * 8 + l] = dg[l];
  }
  // block sum of esum
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) esum = gl::add(esum, fpi::shfl_xor_u64(esum, m));
  if ((tid & 63) == 0) esum_part[tid >> 6] = esum;
  __syncthreads();

  // ---- main loop ----
  const int c0 = colblk * FCOLS + 4 * ct;
  const bool full_cols = (c0 + 4 <= job.cols);
  uint32_t acc[4][NL];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int l = 0; l < NL; ++l) acc[c][l] = 0;

  if (c0 < job.cols) {
    if constexpr (EB == 1) {
      const int8_t* base = (const int8_t*)job.M + (int64_t)row0 * job.ld + c0;
      const bool vec = full_cols && ((job.ld & 3) == 0) && ((((uintptr_t)job.M) & 3) == 0);
      for (int g = rg; g < ngroups; g += FRG) {
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * g + i;
          const int8_t* p = base + (int64_t)t * job.ld;
          if (t < nrows && vec) {
            v[i] = __builtin_nontemporal_load((const uint32_t*)p);
          } else if (t < nrows) {
            uint32_t w = 0;
            for (int c = 0; c < 4; ++c)
              if (c0 + c < job.cols) w |= (uint32_t)(uint8_t)p[c] << (8 * c);
            v[i] = w;
          } else {
            v[i] = 0;
          }
        }
        uint32_t w[4];
        transpose4(v[0], v[1], v[2], v[3], w[0], w[1], w[2], w[3]);
        const uint4 d0 = *(const uint4*)&lds[g * 8];
        const uint4 d1 = *(const uint4*)&lds[g * 8 + 4];
        const uint32_t dg[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t u = w[c] ^ 0x80808080u;  // m + 128 per byte
#pragma unroll
          for (int l = 0; l < 8; ++l) acc[c][l] = udot4(u, dg[l], acc[c][l]);
        }
      }
    } else {
      const int32_t* base = (const int32_t*)job.M + (int64_t)row0 * job.ld + c0;
      const bool vec = full_cols && ((job.ld & 3) == 0) && ((((uintptr_t)job.M) & 15) == 0);
      for (int g = rg; g < ngroups; g += FRG) {
        uint32_t v[4][4];  // [row][col]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * g + i;
          const int32_t* p = base + (int64_t)t * job.ld;
          if (t < nrows && vec) {
            const u32x4 q = __builtin_nontemporal_load((const u32x4*)p);
            v[i][0] = q[0]; v[i][1] = q[1]; v[i][2] = q[2]; v[i][3] = q[3];
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) v[i][c] = (t < nrows && c0 + c < job.cols) ? (uint32_t)p[c] : 0x80000000u;
          }
        }
        const uint4 d0 = *(const uint4*)&lds[g * 8];
        const uint4 d1 = *(const uint4*)&lds[g * 8 + 4];
        const uint32_t dg[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t pl[4];  // byte planes of this column's 4 rows
          transpose4(v[0][c], v[1][c], v[2][c], v[3][c], pl[0], pl[1], pl[2], pl[3]);
          pl[3] ^= 0x80808080u;  // m + 2^31 as an unsigned 32-bit value
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int l = 0; l < 8; ++l) acc[c][b + l] = udot4(pl[b], dg[l], acc[c][b + l]);
        }
      }
    }
  }

  // ---- cross-wave reduction (exact u32 sums: chunk_rows <= 1024) ----
  __syncthreads();  // digits no longer needed
  if (rg > 0) {
    uint32_t* dst = &lds[((rg - 1) * FCT + ct) * 4 * NL];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int l = 0; l < NL; ++l) dst[c * NL + l] = acc[c][l];
  }
  __syncthreads();
  if (rg != 0) return;
#pragma unroll
  for (int w = 0; w < FRG - 1; ++w) {
    const uint32_t* src = &lds[(w * FCT + ct) * 4 * NL];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int l = 0; l < NL; ++l) acc[c][l] += src[c * NL + l];
  }
  uint64_t es = 0;
#pragma unroll
  for (int w = 0; w < FT / 64; ++w) es = gl::add(es, esum_part[w]);
  // offset correction: off * sum E, off = 128 (int8) or 2^31 (int32)
  const uint64_t corr = gl::mul_small(es, EB == 1 ? 128u : 0x80000000u);

  uint64_t vals[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint64_t lo = 0, hi = 0;
#pragma unroll
    for (int l = 0; l < NL; ++l) acc128(lo, hi, acc[c][l], 8 * l);
    vals[c] = gl::sub(gl::reduce128(lo, hi), corr);
  }

  if (job.Ecol) {
    // MLE: weight each column by its eq value, one field sum per block.
    uint64_t s = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c0 + c < job.cols) s = gl::add(s, gl::mul(vals[c], job.Ecol[c0 + c]));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s = gl::add(s, fpi::shfl_xor_u64(s, m));
    if (ct == 0) job.dst[lb] = s;
    return;
  }
  if (job.direct) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = c0 + c;
      if (col < job.cols) job.dst[col] = vals[c];
      else if (col < job.cols_pad) job.dst[col] = 0;
    }
  } else {
    fp_elem* dst = job.dst + (int64_t)chunk * job.cols;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c0 + c < job.cols) dst[c0 + c] = vals[c];
  }
}

// Sum of the row-chunk partials per column, zero tail up to cols_pad.
struct SumJob {
  const fp_elem* part;
  fp_elem* out;
  int32_t cols, cols_pad, n_chunks;
  int32_t block_start;
};
struct SumList {
  const SumJob* dev;
  int32_t count;
  SumJob one;
};

__global__ __launch_bounds__(256) void fold_sum_kernel(SumList sl) {
  SumJob j;
  if (!sl.dev) {
    j = sl.one;
  } else {
    int lo = 0, hi = sl.count - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sl.dev[mid].block_start <= (int)blockIdx.x) lo = mid; else hi = mid - 1;
    }
    j = sl.dev[lo];
  }
  const int col = (blockIdx.x - j.block_start) * 256 + threadIdx.x;
  if (col >= j.cols_pad) return;
  uint64_t s = 0;
  if (col < j.cols)
    for (int c = 0; c < j.n_chunks; ++c) s = gl::add(s, j.part[(int64_t)c * j.cols + col]);
  j.out[col] = s;
}

// Final sum of per-block MLE partials (one block).
__global__ __launch_bounds__(1024) void sum_partials_kernel(const fp_elem* __restrict__ part, int n,
                                                            fp_elem* __restrict__ out) {
  __shared__ uint64_t wsum[16];
  uint64_t s = 0;
  for (int i = threadIdx.x; i < n; i += 1024) s = gl::add(s, part[i]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s = gl::add(s, fpi::shfl_xor_u64(s, m));
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
    for (int w = 0; w < 16; ++w) t = gl::add(t, wsum[w]);
    out[0] = t;
  }
}

// ---- planning ------------------------------------------------------------
struct Plan {
  int32_t chunk_rows, n_chunks, n_colblk;
};

Plan plan_fold(int32_t rows, int32_t cols, bool mle) {
  Plan p;
  p.n_colblk = (cols + FCOLS - 1) / FCOLS;
  const int target_blocks = 2048;
  int want_chunks = (target_blocks + p.n_colblk - 1) / p.n_colblk;
  int cr = (rows + want_chunks - 1) / want_chunks;
  cr = (cr + 15) / 16 * 16;
  const int min_cr = mle ? 32 : 256;
  if (cr < min_cr) cr = min_cr;
  if (cr > FMAX_CHUNK) cr = FMAX_CHUNK;
  if (cr >= rows) cr = (rows + 3) / 4 * 4;
  if (cr < 4) cr = 4;
  p.chunk_rows = cr;
  p.n_chunks = (rows + cr - 1) / cr;
  if (p.n_chunks < 1) p.n_chunks = 1;
  return p;
}

size_t fold_ws_one(int32_t rows, int32_t cols) {
  if (rows <= 0) return 0;
  const Plan p = plan_fold(rows, cols, false);
  return p.n_chunks > 1 ? fpi::align_up((size_t)p.n_chunks * (size_t)cols * 8, 256) : 0;
}

int launch_fold_rows(int eb, const JobList& jl, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return FP_OK;
  if (eb == 1) hipLaunchKernelGGL(fold_rows_kernel<1>, dim3((unsigned)blocks), dim3(FT), 0, st, jl);
  else hipLaunchKernelGGL(fold_rows_kernel<4>, dim3((unsigned)blocks), dim3(FT), 0, st, jl);
  return fpi::check_launch("fold_rows_kernel");
}

int zero_fill(fp_elem* out, int32_t n, hipStream_t st) {
  if (n <= 0) return FP_OK;
  SumList sl{nullptr, 1, SumJob{nullptr, out, 0, n, 0, 0}};
  hipLaunchKernelGGL(fold_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, sl);
  return fpi::check_launch("fold_sum_kernel");
}

int validate_fold(const char* fn, fp_dtype dt, const void* M, int64_t ld, int32_t rows, int32_t cols,
                  const fp_elem* E, fp_elem* out, int32_t cols_pad) {
  if (dt != FP_I8 && dt != FP_I32) return fpi::fail(FP_EARG, "%s: unknown dtype %d", fn, (int)dt);
  if (rows < 0 || cols < 0 || cols_pad < cols) return fpi::fail(FP_ESHAPE, "%s: bad sizes rows=%d cols=%d cols_pad=%d", fn, rows, cols, cols_pad);
  if (ld < cols) return fpi::fail(FP_ESHAPE, "%s: ld=%lld < cols=%d", fn, (long long)ld, cols);
  if (!out && cols_pad > 0) return fpi::fail(FP_EARG, "%s: null out", fn);
  if (rows > 0 && cols > 0 && (!M || !E)) return fpi::fail(FP_EARG, "%s: null M or E", fn);
  return FP_OK;
}

}  // namespace

extern "C" size_t fp_fold_matrix_workspace(fp_dtype dt, int32_t rows, int32_t cols) {
  (void)dt;
  return fold_ws_one(rows, cols);
}

extern "C" int fp_fold_matrix(fp_dtype dt, const void* M, int64_t ld, int32_t rows, int32_t cols, const fp_elem* E,
                              fp_elem* out, int32_t cols_pad, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = validate_fold("fp_fold_matrix", dt, M, ld, rows, cols, E, out, cols_pad);
  if (rc) return rc;
  if (rows == 0 || cols == 0) {
    rc = zero_fill(out, cols_pad, stream);
    return rc ? rc : fpi::ok();
  }
  const size_t need = fold_ws_one(rows, cols);
  if (ws_bytes < need || (need && !ws)) return fpi::fail(FP_EWORKSPACE, "fp_fold_matrix: workspace %zu < %zu", ws_bytes, need);
  const Plan p = plan_fold(rows, cols, false);
  FoldJob j{};
  j.M = M; j.ld = ld; j.E = E; j.Ecol = nullptr;
  j.rows = rows; j.cols = cols; j.cols_pad = cols_pad;
  j.chunk_rows = p.chunk_rows; j.n_chunks = p.n_chunks; j.block_start = 0;
  if (p.n_chunks == 1) {
    j.direct = 1; j.dst = out;
    j.n_colblk = (cols_pad + FCOLS - 1) / FCOLS;
    rc = launch_fold_rows(dt == FP_I8 ? 1 : 4, JobList{nullptr, 1, j}, j.n_colblk, stream);
    return rc ? rc : fpi::ok();
  }
  j.direct = 0; j.dst = (fp_elem*)ws; j.n_colblk = p.n_colblk;
  rc = launch_fold_rows(dt == FP_I8 ? 1 : 4, JobList{nullptr, 1, j}, (int64_t)p.n_chunks * p.n_colblk, stream);
  if (rc) return rc;
  SumList sl{nullptr, 1, SumJob{(const fp_elem*)ws, out, cols, cols_pad, p.n_chunks, 0}};
  hipLaunchKernelGGL(fold_sum_kernel, dim3((unsigned)((cols_pad + 255) / 256)), dim3(256), 0, stream, sl);
  rc = fpi::check_launch("fold_sum_kernel");
  return rc ? rc : fpi::ok();
}

// ---- batched folds ---------------------------------------------------------
// Workspace layout: [FoldJob x count][SumJob x count][partials...]
extern "C" size_t fp_fold_matrix_batched_workspace(fp_dtype dt, int32_t count, const fp_fold_desc* d) {
  (void)dt;
  size_t s = fpi::align_up(sizeof(FoldJob) * (size_t)count, 256) + fpi::align_up(sizeof(SumJob) * (size_t)count, 256);
  for (int32_t i = 0; i < count; ++i) s += fold_ws_one(d[i].rows, d[i].cols);
  return s;
}

extern "C" int fp_fold_matrix_batched(fp_dtype dt, int32_t count, const fp_fold_desc* d, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  if (count < 0) return fpi::fail(FP_EARG, "fp_fold_matrix_batched: count < 0");
  if (count == 0) return fpi::ok();
  if (!d) return fpi::fail(FP_EARG, "fp_fold_matrix_batched: null descs");
  for (int32_t i = 0; i < count; ++i) {
    int rc = validate_fold("fp_fold_matrix_batched", dt, d[i].M, d[i].ld, d[i].rows, d[i].cols, d[i].E, d[i].out,
                           d[i].cols_pad);
    if (rc) return rc;
  }
  const size_t need = fp_fold_matrix_batched_workspace(dt, count, d);
  if (!ws || ws_bytes < need) return fpi::fail(FP_EWORKSPACE, "fp_fold_matrix_batched: workspace %zu < %zu", ws_bytes, need);
  char* w = (char*)ws;
  FoldJob* djobs = (FoldJob*)w;
  w += fpi::align_up(sizeof(FoldJob) * (size_t)count, 256);
  SumJob* dsums = (SumJob*)w;
  w += fpi::align_up(sizeof(SumJob) * (size_t)count, 256);
  std::vector<FoldJob> jobs;
  std::vector<SumJob> sums;
  int64_t blocks = 0, sblocks = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (d[i].rows == 0 || d[i].cols == 0) {
      if (d[i].cols_pad > 0) {
        sums.push_back(SumJob{nullptr, d[i].out, 0, d[i].cols_pad, 0, (int32_t)sblocks});
        sblocks += (d[i].cols_pad + 255) / 256;
      }
      continue;
    }
    const Plan p = plan_fold(d[i].rows, d[i].cols, false);
    FoldJob j{};
    j.M = d[i].M; j.ld = d[i].ld; j.E = d[i].E; j.Ecol = nullptr;
    j.rows = d[i].rows; j.cols = d[i].cols; j.cols_pad = d[i].cols_pad;
    j.chunk_rows = p.chunk_rows; j.n_chunks = p.n_chunks; j.block_start = (int32_t)blocks;
    if (p.n_chunks == 1) {
      j.direct = 1; j.dst = d[i].out; j.n_colblk = (d[i].cols_pad + FCOLS - 1) / FCOLS;
    } else {
      j.direct = 0; j.dst = (fp_elem*)w; j.n_colblk = p.n_colblk;
      sums.push_back(SumJob{(const fp_elem*)w, d[i].out, d[i].cols, d[i].cols_pad, p.n_chunks, (int32_t)sblocks});
      sblocks += (d[i].cols_pad + 255) / 256;
      w += fold_ws_one(d[i].rows, d[i].cols);
    }
    blocks += (int64_t)j.n_chunks * j.n_colblk;
    jobs.push_back(j);
  }
  if (blocks > 0x7FFFFFFF || sblocks > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "fp_fold_matrix_batched: too many blocks");
  hipError_t e;
  if (!jobs.empty()) {
    e = hipMemcpyAsync(djobs, jobs.data(), sizeof(FoldJob) * jobs.size(), hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return fpi::fail(FP_EHIP, "fp_fold_matrix_batched: copy: %s", hipGetErrorString(e));
    int rc = launch_fold_rows(dt == FP_I8 ? 1 : 4, JobList{djobs, (int32_t)jobs.size(), FoldJob{}}, blocks, stream);
    if (rc) return rc;
  }
  if (!sums.empty()) {
    e = hipMemcpyAsync(dsums, sums.data(), sizeof(SumJob) * sums.size(), hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return fpi::fail(FP_EHIP, "fp_fold_matrix_batched: copy: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(fold_sum_kernel, dim3((unsigned)sblocks), dim3(256), 0, stream,
                       SumList{dsums, (int32_t)sums.size(), SumJob{}});
    int rc = fpi::check_launch("fold_sum_kernel");
    if (rc) return rc;
  }
  return fpi::ok();
}

// ---- MLE -------------------------------------------------------------------
// Workspace: [E_rows: 2^n_rows][E_cols: 2^n_cols][block partials]
extern "C" size_t fp_mle_eval_workspace(fp_dtype dt, int32_t rows, int32_t cols, int32_t n_rows, int32_t n_cols) {
  (void)dt;
  if (n_rows < 0 || n_cols < 0 || n_rows > FP_MAX_N || n_cols > FP_MAX_N) return 0;
  const Plan p = plan_fold(rows > 0 ? rows : 1, cols > 0 ? cols : 1, true);
  return fpi::align_up(((size_t)8) << n_rows, 256) + fpi::align_up(((size_t)8) << n_cols, 256) +
         fpi::align_up((size_t)p.n_chunks * p.n_colblk * 8, 256);
}

extern "C" int fp_mle_eval(fp_dtype dt, const void* M, int64_t ld, int32_t rows, int32_t cols, const fp_elem* r_rows,
                           int32_t n_rows, const fp_elem* r_cols, int32_t n_cols, fp_elem* out, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (dt != FP_I8 && dt != FP_I32) return fpi::fail(FP_EARG, "fp_mle_eval: unknown dtype %d", (int)dt);
  if (n_rows < 0 || n_cols < 0 || n_rows > 24 || n_cols > 24)
    return fpi::fail(FP_ESHAPE, "fp_mle_eval: n_rows=%d n_cols=%d outside [0, 24]", n_rows, n_cols);
  if (rows < 0 || cols < 0 || (int64_t)rows > ((int64_t)1 << n_rows) || (int64_t)cols > ((int64_t)1 << n_cols))
    return fpi::fail(FP_ESHAPE, "fp_mle_eval: [%d, %d] does not fit [2^%d, 2^%d]", rows, cols, n_rows, n_cols);
  if (ld < cols) return fpi::fail(FP_ESHAPE, "fp_mle_eval: ld < cols");
  if (!out || (rows > 0 && cols > 0 && !M) || (n_rows > 0 && !r_rows) || (n_cols > 0 && !r_cols))
    return fpi::fail(FP_EARG, "fp_mle_eval: null pointer");
  const size_t need = fp_mle_eval_workspace(dt, rows, cols, n_rows, n_cols);
  if (!ws || ws_bytes < need) return fpi::fail(FP_EWORKSPACE, "fp_mle_eval: workspace %zu < %zu", ws_bytes, need);
  if (rows == 0 || cols == 0) {
    int rc = zero_fill(out, 1, stream);
    return rc ? rc : fpi::ok();
  }
  char* w = (char*)ws;
  fp_elem* Er = (fp_elem*)w;
  w += fpi::align_up(((size_t)8) << n_rows, 256);
  fp_elem* Ec = (fp_elem*)w;
  w += fpi::align_up(((size_t)8) << n_cols, 256);
  fp_elem* part = (fp_elem*)w;
  int rc = fpi::launch_eq(r_rows, n_rows, Er, stream);
  if (rc) return rc;
  rc = fpi::launch_eq(r_cols, n_cols, Ec, stream);
  if (rc) return rc;
  const Plan p = plan_fold(rows, cols, true);
  FoldJob j{};
  j.M = M; j.ld = ld; j.E = Er; j.Ecol = Ec; j.dst = part;
  j.rows = rows; j.cols = cols; j.cols_pad = cols;
  j.chunk_rows = p.chunk_rows; j.n_chunks = p.n_chunks; j.n_colblk = p.n_colblk; j.block_start = 0; j.direct = 0;
  const int64_t blocks = (int64_t)p.n_chunks * p.n_colblk;
  rc = launch_fold_rows(dt == FP_I8 ? 1 : 4, JobList{nullptr, 1, j}, blocks, stream);
  if (rc) return rc;
  hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(1024), 0, stream, (const fp_elem*)part, (int)blocks, out);
  rc = fpi::check_launch("sum_partials_kernel");
  return rc ? rc : fpi::ok();
}

// ---- batched claims from eq tables -------------------------------------------
// out_j = sum_t sum_c E_rows_j[t] E_cols_j[c] M_j[t, c]: the fold kernel in MLE
// mode gives one partial per workgroup; one workgroup per claim sums them.
namespace {
struct ClaimSum {
  const fp_elem* part;
  fp_elem* out;
  int32_t n;
};

__global__ __launch_bounds__(1024) void claim_sum_kernel(const ClaimSum* __restrict__ jobs) {
  const ClaimSum j = jobs[blockIdx.x];
  __shared__ uint64_t wsum[16];
  uint64_t s = 0;
  for (int i = threadIdx.x; i < j.n; i += 1024) s = gl::add(s, j.part[i]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s = gl::add(s, fpi::shfl_xor_u64(s, m));
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
    for (int w = 0; w < 16; ++w) t = gl::add(t, wsum[w]);
    j.out[0] = t;
  }
}

size_t claim_ws(int32_t count, const fp_claim_desc* d) {
  size_t s = fpi::align_up(sizeof(FoldJob) * (size_t)count, 256) + fpi::align_up(sizeof(ClaimSum) * (size_t)count, 256);
  size_t parts = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (d[i].rows <= 0 || d[i].cols <= 0) continue;
    const Plan p = plan_fold(d[i].rows, d[i].cols, true);
    parts += (size_t)p.n_chunks * p.n_colblk;
  }
  return s + fpi::align_up(parts * 8, 256);
}
}  // namespace

extern "C" size_t fp_claim_eval_batched_workspace(fp_dtype dt, int32_t count, const fp_claim_desc* descs) {
  (void)dt;
  if (count <= 0 || !descs) return 0;
  return claim_ws(count, descs);
}

extern "C" int fp_claim_eval_batched(fp_dtype dt, int32_t count, const fp_claim_desc* d, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  if (dt != FP_I8 && dt != FP_I32) return fpi::fail(FP_EARG, "fp_claim_eval_batched: unknown dtype %d", (int)dt);
  if (count < 0) return fpi::fail(FP_EARG, "fp_claim_eval_batched: count < 0");
  if (count == 0) return fpi::ok();
  if (!d) return fpi::fail(FP_EARG, "fp_claim_eval_batched: null descs");
  for (int32_t i = 0; i < count; ++i) {
    if (d[i].rows < 0 || d[i].cols < 0 || d[i].ld < d[i].cols)
      return fpi::fail(FP_ESHAPE, "fp_claim_eval_batched: desc %d has bad sizes", i);
    if (!d[i].out || (d[i].rows > 0 && d[i].cols > 0 && (!d[i].M || !d[i].E_rows || !d[i].E_cols)))
      return fpi::fail(FP_EARG, "fp_claim_eval_batched: desc %d has a null pointer", i);
  }
  const size_t need = claim_ws(count, d);
  if (!ws || ws_bytes < need) return fpi::fail(FP_EWORKSPACE, "fp_claim_eval_batched: workspace %zu < %zu", ws_bytes, need);
  char* w = (char*)ws;
  FoldJob* djobs = (FoldJob*)w;
  w += fpi::align_up(sizeof(FoldJob) * (size_t)count, 256);
  ClaimSum* dsums = (ClaimSum*)w;
  w += fpi::align_up(sizeof(ClaimSum) * (size_t)count, 256);
  fp_elem* part = (fp_elem*)w;
  std::vector<FoldJob> jobs;
  std::vector<ClaimSum> sums;
  int64_t blocks = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (d[i].rows == 0 || d[i].cols == 0) {
      sums.push_back(ClaimSum{part, d[i].out, 0});
      continue;
    }
    const Plan p = plan_fold(d[i].rows, d[i].cols, true);
    FoldJob j{};
    j.M = d[i].M; j.ld = d[i].ld; j.E = d[i].E_rows; j.Ecol = d[i].E_cols;
    j.dst = part + blocks;
    j.rows = d[i].rows; j.cols = d[i].cols; j.cols_pad = d[i].cols;
    j.chunk_rows = p.chunk_rows; j.n_chunks = p.n_chunks; j.n_colblk = p.n_colblk;
    j.block_start = (int32_t)blocks; j.direct = 0;
    const int64_t nb = (int64_t)p.n_chunks * p.n_colblk;
    sums.push_back(ClaimSum{part + blocks, d[i].out, (int32_t)nb});
    blocks += nb;
    jobs.push_back(j);
  }
  if (blocks > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "fp_claim_eval_batched: too many blocks");
  hipError_t e;
  if (!jobs.empty()) {
    e = hipMemcpyAsync(djobs, jobs.data(), sizeof(FoldJob) * jobs.size(), hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return fpi::fail(FP_EHIP, "fp_claim_eval_batched: copy: %s", hipGetErrorString(e));
    int rc = launch_fold_rows(dt == FP_I8 ? 1 : 4, JobList{djobs, (int32_t)jobs.size(), FoldJob{}}, blocks, stream);
    if (rc) return rc;
  }
  e = hipMemcpyAsync(dsums, sums.data(), sizeof(ClaimSum) * sums.size(), hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fpi::fail(FP_EHIP, "fp_claim_eval_batched: copy: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(claim_sum_kernel, dim3((unsigned)sums.size()), dim3(1024), 0, stream, (const ClaimSum*)dsums);
  int rc = fpi::check_launch("claim_sum_kernel");
  return rc ? rc : fpi::ok();
}
