// fold.hip - folded rows of integer matrices, and matmul claims.
//
// out[k] = sum_t E[t] M[t, k] ("How fast can FlashProve go", §2: the folded
// row is the eq-weighted sum of all of a table's rows; §4 counts this as one of
// the three passes over the weights, the one "for the matmuls' sum-checks").
//
// The pass is bound by HBM bandwidth only if the inner loop stays within a few
// vector ops per byte, so no Goldilocks multiply runs per matrix entry. The
// field weight E[t] (< 2^64) is split into 8 unsigned bytes e_l[t] and each
// entry is offset to unsigned bytes: u = m + 128 (int8) or the four bytes of
// m + 2^31 (int32). Then
//     sum_t E[t] m[t,k] = sum_l 2^(8l) sum_t e_l[t] u[t,k]  -  off * sum_t E[t]
// where every inner sum is an exact integer built with v_dot4_u32_u8 over four
// rows at a time. A thread reads one dword (int8: 4 columns) or one dwordx4
// (int32: 4 columns) per row, transposes 4 rows x 4 bytes with v_perm_b32 so
// that each dword holds one column's 4 rows, and accumulates u32 limb sums
// (exact: a workgroup covers at most 1024 rows). The field reduction happens
// once per column per workgroup.
//
// Rows are split into chunks, one workgroup per (chunk, 256-column strip)
// (the workgroup code is in fold.hpp). Each workgroup stores its per-column
// field values, and a second small kernel adds the chunks per column (16 chunk
// lanes per column, so the adds are not one long dependent chain). For a
// claim, each workgroup weights its columns with the column eq table and
// stores one value; one workgroup per claim then adds them. The two kernels
// need no atomics and no cross-XCD fences. (The fused layer-step launch in
// witness.hip runs the same workgroups in fold.hpp's arrival mode instead.)
#include <vector>

#include "common.hpp"
#include "fold.hpp"
#include "gl.hpp"

namespace {

using namespace foldk;
constexpr int INLINE = 32;  // jobs carried in one launch's arguments (kernel arguments <= 4 KB)

struct JobList {
  FoldJob j[INLINE];
  int32_t count;
};
static_assert(sizeof(JobList) <= 4096, "a job list travels in the kernel arguments");

// Every job of the list, int8 or int32, folds or claims, in one launch.
__global__ __launch_bounds__(FT) void fold_rows_kernel(JobList jl) {
  __shared__ __align__(16) uint32_t lds[LDS_WORDS];
  __shared__ uint64_t gsum[MAXG_ALL];
  const FoldJob& job = jl.j[find_job(jl.j, jl.count, blockIdx.x)];
  fold_block<false>(job, (int)blockIdx.x - job.block_start, lds, gsum);
}

// ---- cross-chunk sums ----------------------------------------------------------
// fold: out[c] = sum_chunk part[chunk][c] for c < cols, 0 up to cols_pad.
//   A workgroup covers 16 columns with 16 chunk lanes each.
// claim: out[0] = sum_i part[i] over the claim's workgroup values.
struct SumJob {
  const fp_elem* part;
  fp_elem* out;
  int32_t cols, cols_pad, n_chunks;  // claim: cols = 0, n_chunks = number of values
  int32_t claim;
  int32_t block_start;
};
struct SumList {
  SumJob j[INLINE];
  int32_t count;
};

__global__ __launch_bounds__(256) void fold_sum_kernel(SumList sl) {
  __shared__ uint64_t red[256];
  const SumJob& j = sl.j[find_job(sl.j, sl.count, blockIdx.x)];
  const int lb = blockIdx.x - j.block_start;
  const int tid = threadIdx.x;
  uint64_t s = 0;
  if (j.claim) {
    for (int i = tid; i < j.n_chunks; i += 256) s = gl::add(s, j.part[i]);
    red[tid] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
      if (tid < w) red[tid] = gl::add(red[tid], red[tid + w]);
      __syncthreads();
    }
    if (tid == 0) j.out[0] = red[0];
    return;
  }
  const int cl = tid & 15, lane_ch = tid >> 4;
  const int col = lb * 16 + cl;
  if (col < j.cols) {
    for (int ch = lane_ch; ch < j.n_chunks; ch += 16) s = gl::add(s, j.part[(int64_t)ch * j.cols + col]);
  }
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w >= 16; w >>= 1) {
    if (tid < w) red[tid] = gl::add(red[tid], red[tid + w]);
    __syncthreads();
  }
  if (tid < 16 && col < j.cols_pad) j.out[col] = red[tid];
}

// ---- planning ------------------------------------------------------------
int launch_list(const JobList& jl, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return FP_OK;
  if (blocks > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "fold: too many workgroups");
  hipLaunchKernelGGL(fold_rows_kernel, dim3((unsigned)blocks), dim3(FT), 0, st, jl);
  return fpi::check_launch("fold_rows_kernel");
}

// Zero-fill of an output without data (empty matrix): padding strips only.
int zero_only(fp_elem* out, int32_t n, hipStream_t st) {
  if (n <= 0) return FP_OK;
  JobList jl{};
  FoldJob& j = jl.j[0];
  j.out = out;
  j.cols = 0;
  j.cols_pad = n;
  j.n_chunks = 1;
  j.n_strips = 0;
  j.n_pad_strips = (n + FCOLS - 1) / FCOLS;
  j.eb = 1;
  jl.count = 1;
  return launch_list(jl, j.n_pad_strips, st);
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

// A fold or claim job before planning.
struct Item {
  FoldJob j;
  bool claim;
};

void add_folds(std::vector<Item>& v, fp_dtype dt, int32_t count, const fp_fold_desc* d) {
  for (int32_t i = 0; i < count; ++i) {
    Item it{};
    FoldJob& j = it.j;
    j.M = d[i].M; j.ld = d[i].ld; j.E = d[i].E; j.Ecol = nullptr; j.out = d[i].out;
    j.rows = d[i].rows; j.cols = d[i].cols; j.cols_pad = d[i].cols_pad;
    j.eb = dt == FP_I8 ? 1 : 4;
    it.claim = false;
    v.push_back(it);
  }
}

void add_claims(std::vector<Item>& v, fp_dtype dt, int32_t count, const fp_claim_desc* d) {
  for (int32_t i = 0; i < count; ++i) {
    Item it{};
    FoldJob& j = it.j;
    j.M = d[i].M; j.ld = d[i].ld; j.E = d[i].E_rows; j.Ecol = d[i].E_cols; j.out = d[i].out;
    j.rows = d[i].rows; j.cols = d[i].cols; j.cols_pad = d[i].cols;
    j.eb = dt == FP_I8 ? 1 : 4;
    it.claim = true;
    v.push_back(it);
  }
}

// Workgroups per job: about 256 (one per compute unit), except that a launch
// of int8 folds alone aims at about 512 in all (two per compute unit), shared
// by its jobs in proportion to their rows. The up-projection's folds of X and
// W: 17.3 us with 512 for W, 19.0 with 256, 18.5 with 768, 19.4 with 1024 (more
// chunks lengthen the cross-chunk sums); with the claim of its Z beside them,
// 22.6 us at 256 per job against 23.0 with 512 for the folds; the seven-map
// layer's 28 extension folds: 0.111 ms at 256 per job, 0.128 with 512 each.
int64_t fold_rows_only(const std::vector<Item>& v) {  // rows of a launch of int8 folds alone, else 0
  int64_t rows = 0;
  for (const Item& x : v) {
    if (x.claim || x.j.eb != 1) return 0;
    if (x.j.rows > 0 && x.j.cols > 0) rows += x.j.rows;
  }
  return rows;
}
int job_target(int64_t launch_rows, const Item& it) {
  const int64_t t = launch_rows > 0 ? 512 * (int64_t)it.j.rows / launch_rows : 256;
  return t > 256 ? (int)t : 256;
}

// Workspace: the partials of every job, back to back.
size_t items_ws(const std::vector<Item>& v) {
  size_t parts = 0;
  const int64_t lr = fold_rows_only(v);
  for (const Item& it : v) {
    if (it.j.rows <= 0 || it.j.cols <= 0) continue;
    parts += plan_job(it.j.rows, it.j.cols, it.j.cols_pad, it.j.eb, it.claim, false, job_target(lr, it)).part_bytes;
  }
  return parts;
}

// Enqueue the jobs, INLINE at a time: one fold launch and (when needed) one
// cross-chunk sum launch per INLINE jobs.
int run_items(std::vector<Item>& v, char* ws, hipStream_t st) {
  char* parts = ws;
  JobList jl{};
  SumList sl{};
  int64_t blocks = 0, sblocks = 0;
  const int64_t lr = fold_rows_only(v);
  auto flush = [&]() -> int {
    int rc = launch_list(jl, blocks, st);
    if (!rc && sblocks > 0) {
      hipLaunchKernelGGL(fold_sum_kernel, dim3((unsigned)sblocks), dim3(256), 0, st, sl);
      rc = fpi::check_launch("fold_sum_kernel");
    }
    jl = JobList{};
    sl = SumList{};
    blocks = sblocks = 0;
    return rc;
  };
  for (Item& it : v) {
    FoldJob j = it.j;
    const bool claim = it.claim;
    const int eb = j.eb;
    if (j.rows <= 0 || j.cols <= 0) {
      // empty matrix: zero output
      int rc = claim ? zero_only(j.out, 1, st) : zero_only(j.out, j.cols_pad, st);
      if (rc) return rc;
      continue;
    }
    const int64_t span = (int64_t)j.ld * eb * (j.rows < FMAX_CHUNK ? j.rows : FMAX_CHUNK);
    if (span > 0x7FFFFFFF)
      return fpi::fail(FP_ESHAPE, "fold: row stride %lld x %d rows exceeds 2^31 bytes", (long long)j.ld, FMAX_CHUNK);
    const uintptr_t align = eb == 1 ? 3 : 15;
    j.vec = (j.cols % 4 == 0) && (j.ld % 4 == 0) && (((uintptr_t)j.M & align) == 0);
    const Plan p = plan_job(j.rows, j.cols, j.cols_pad, eb, claim, false, job_target(lr, it));
    j.chunk_rows = p.chunk_rows;
    j.n_chunks = p.n_chunks;
    j.n_strips = p.n_strips;
    j.n_pad_strips = p.n_pad_strips;
    j.part = p.part_bytes ? (fp_elem*)parts : nullptr;
    parts += p.part_bytes;
    if (jl.count == INLINE || blocks + p.blocks > 0x7FFFFFFF) {
      int rc = flush();
      if (rc) return rc;
    }
    j.block_start = (int32_t)blocks;
    jl.j[jl.count++] = j;
    blocks += p.blocks;
    if (p.sum_blocks) {
      SumJob sj{};
      sj.part = j.part;
      sj.out = j.out;
      sj.claim = claim ? 1 : 0;
      sj.cols = claim ? 0 : j.cols;
      sj.cols_pad = claim ? 1 : j.cols_pad;
      sj.n_chunks = claim ? (int32_t)(p.n_chunks * p.n_strips * FRG) : p.n_chunks;
      sj.block_start = (int32_t)sblocks;
      sl.j[sl.count++] = sj;
      sblocks += p.sum_blocks;
    }
  }
  return jl.count ? flush() : FP_OK;
}

int validate_claims(const char* fn, fp_dtype dt, int32_t count, const fp_claim_desc* d) {
  if (dt != FP_I8 && dt != FP_I32) return fpi::fail(FP_EARG, "%s: unknown dtype %d", fn, (int)dt);
  if (count < 0) return fpi::fail(FP_EARG, "%s: count < 0", fn);
  if (count > 0 && !d) return fpi::fail(FP_EARG, "%s: null descs", fn);
  for (int32_t i = 0; i < count; ++i) {
    if (d[i].rows < 0 || d[i].cols < 0 || d[i].ld < d[i].cols)
      return fpi::fail(FP_ESHAPE, "%s: desc %d has bad sizes", fn, i);
    if (!d[i].out || (d[i].rows > 0 && d[i].cols > 0 && (!d[i].M || !d[i].E_rows || !d[i].E_cols)))
      return fpi::fail(FP_EARG, "%s: desc %d has a null pointer", fn, i);
  }
  return FP_OK;
}

int validate_folds(const char* fn, fp_dtype dt, int32_t count, const fp_fold_desc* d) {
  if (count < 0) return fpi::fail(FP_EARG, "%s: count < 0", fn);
  if (count > 0 && !d) return fpi::fail(FP_EARG, "%s: null descs", fn);
  for (int32_t i = 0; i < count; ++i) {
    if (d[i].E2 || d[i].out2)
      return fpi::fail(FP_EARG, "%s: fold %d has a second weight vector (the step launches' folds only)", fn, i);
    int rc = validate_fold(fn, dt, d[i].M, d[i].ld, d[i].rows, d[i].cols, d[i].E, d[i].out, d[i].cols_pad);
    if (rc) return rc;
  }
  return FP_OK;
}

}  // namespace

extern "C" size_t fp_fold_matrix_workspace(fp_dtype dt, int32_t rows, int32_t cols) {
  fp_fold_desc d{nullptr, cols, rows, cols, cols, nullptr, nullptr, nullptr, nullptr};
  return fp_fold_matrix_batched_workspace(dt, 1, &d);
}

extern "C" int fp_fold_matrix(fp_dtype dt, const void* M, int64_t ld, int32_t rows, int32_t cols, const fp_elem* E,
                              fp_elem* out, int32_t cols_pad, void* ws, size_t ws_bytes, hipStream_t stream) {
  fp_fold_desc d{M, ld, rows, cols, cols_pad, E, out, nullptr, nullptr};
  return fp_fold_matrix_batched(dt, 1, &d, ws, ws_bytes, stream);
}

extern "C" size_t fp_fold_matrix_batched_workspace(fp_dtype dt, int32_t count, const fp_fold_desc* d) {
  return fp_fold_claim_batched_workspace(dt, count, d, FP_I32, 0, nullptr);
}

extern "C" int fp_fold_matrix_batched(fp_dtype dt, int32_t count, const fp_fold_desc* d, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  return fp_fold_claim_batched(dt, count, d, FP_I32, 0, nullptr, ws, ws_bytes, stream);
}

extern "C" size_t fp_claim_eval_batched_workspace(fp_dtype dt, int32_t count, const fp_claim_desc* d) {
  return fp_fold_claim_batched_workspace(FP_I8, 0, nullptr, dt, count, d);
}

extern "C" int fp_claim_eval_batched(fp_dtype dt, int32_t count, const fp_claim_desc* d, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  return fp_fold_claim_batched(FP_I8, 0, nullptr, dt, count, d, ws, ws_bytes, stream);
}

extern "C" size_t fp_fold_claim_batched_workspace(fp_dtype fold_dt, int32_t n_fold, const fp_fold_desc* folds,
                                                  fp_dtype claim_dt, int32_t n_claim, const fp_claim_desc* claims) {
  std::vector<Item> v;
  if (n_fold > 0 && folds) add_folds(v, fold_dt, n_fold, folds);
  if (n_claim > 0 && claims) add_claims(v, claim_dt, n_claim, claims);
  return items_ws(v);
}

extern "C" int fp_fold_claim_batched(fp_dtype fold_dt, int32_t n_fold, const fp_fold_desc* folds, fp_dtype claim_dt,
                                     int32_t n_claim, const fp_claim_desc* claims, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  int rc = validate_folds("fp_fold_matrix", fold_dt, n_fold, folds);
  if (!rc) rc = validate_claims("fp_claim_eval_batched", claim_dt, n_claim, claims);
  if (rc) return rc;
  std::vector<Item> v;
  add_folds(v, fold_dt, n_fold, folds);
  add_claims(v, claim_dt, n_claim, claims);
  if (v.empty()) return fpi::ok();
  const size_t need = items_ws(v);
  if (need && (!ws || ws_bytes < need))
    return fpi::fail(FP_EWORKSPACE, "fold/claim: workspace %zu < %zu", ws_bytes, need);
  rc = run_items(v, (char*)ws, stream);
  return rc ? rc : fpi::ok();
}

// ---- MLE at a point ------------------------------------------------------
// Workspace: [claim workspace][E_rows: 2^n_rows][E_cols: 2^n_cols]
extern "C" size_t fp_mle_eval_workspace(fp_dtype dt, int32_t rows, int32_t cols, int32_t n_rows, int32_t n_cols) {
  if (n_rows < 0 || n_cols < 0 || n_rows > 24 || n_cols > 24) return 0;
  fp_claim_desc d{nullptr, cols, rows, cols, nullptr, nullptr, nullptr};
  return fpi::align_up(fp_claim_eval_batched_workspace(dt, 1, &d), 256) + fpi::align_up(((size_t)8) << n_rows, 256) +
         fpi::align_up(((size_t)8) << n_cols, 256);
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
  fp_claim_desc d0{nullptr, cols, rows, cols, nullptr, nullptr, nullptr};
  const size_t cw = fpi::align_up(fp_claim_eval_batched_workspace(dt, 1, &d0), 256);
  char* w = (char*)ws + cw;
  fp_elem* Er = (fp_elem*)w;
  w += fpi::align_up(((size_t)8) << n_rows, 256);
  fp_elem* Ec = (fp_elem*)w;
  int rc = fpi::launch_eq(r_rows, n_rows, Er, stream);
  if (rc) return rc;
  rc = fpi::launch_eq(r_cols, n_cols, Ec, stream);
  if (rc) return rc;
  fp_claim_desc d{M, ld, rows, cols, Er, Ec, out};
  return fp_claim_eval_batched(dt, 1, &d, ws, cw, stream);
}
