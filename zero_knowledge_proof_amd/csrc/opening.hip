// opening.hip - the committed tables of a layer proof whose rescale is
// committed, and the openings of claims about them.
//
// "How fast can FlashProve go", §2: the prover commits intermediate values, and
// sum-check leaves claims about the committed tables that openings settle; an
// opening sends a table's folded row (the eq-weighted sum of its rows) and
// opens a few columns of the encoded table. §3.1: the rescaled value g_w and
// the remainder r are committed (g^ never is), the matmul's claim about g^
// reads 2^k g_w + r, and the clamped value is committed beside them.
//
// fp_commit_tables writes each map's Q (the rounded value before the clamp),
// R and Y as field elements into runs of whole rows of the message matrix;
// fp_commit_fold_ext forms folded rows over F_p[u]/(u^2 - 7): the proximity row
// (every row i weighted by eq(r_prox, i)) and one row per claim (weights
// eq(z, i - row0) on the claim's rows); fp_merkle_open gathers the columns the
// transcript picked, their salts and their Merkle paths.
#include "common.hpp"
#include "ext.hpp"
#include "gl.hpp"
#include "sc_tail.hpp"

using namespace fpx;

namespace {

// ------------------------------------------------------------------ tables
struct TabArgs {
  fp_table_desc d[FP_MAX_MULTI];
  int64_t start[FP_MAX_MULTI + 1];  // first entry of each map in the launch's index space
  int32_t count, n_t, s, log_cols;
  uint64_t* msg;
  int64_t ld;
};

__device__ __forceinline__ uint64_t embed(int64_t v) {
  return v < 0 ? (uint64_t)v - 0xFFFFFFFFull : (uint64_t)v;  // p + v
}

__device__ __forceinline__ void rescale_embed(int64_t z, int s, uint64_t& q, uint64_t& r, uint64_t& y) {
  const int64_t qq = (z + ((int64_t)1 << (s - 1))) >> s;  // floor: arithmetic shift
  const int64_t rr = z - (qq << s);
  const int64_t yy = qq < -128 ? -128 : (qq > 127 ? 127 : qq);
  q = embed(qq);
  r = embed(rr);
  y = embed(yy);
}

// V consecutive entries of one map's padded [2^n_t, 2^n_o] tables per thread.
// With V = 2 every table has an even size, rows have an even number of
// columns and msg is 16-byte aligned, so a thread's two entries share a row
// and each table's pair is one 16-byte store.
template <int V>
__global__ __launch_bounds__(256) void tables_kernel(TabArgs a) {
  const int64_t e = V * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (e >= a.start[a.count]) return;
  int m = 0;
  while (e >= a.start[m + 1]) ++m;
  const fp_table_desc& d = a.d[m];
  const int64_t i = e - a.start[m];
  const int64_t row = i >> a.log_cols, col = i & (((int64_t)1 << a.log_cols) - 1);
  uint64_t q[V], r[V], y[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const int64_t ik = i + k;
    const int64_t t = ik >> d.n_o, o = ik & (((int64_t)1 << d.n_o) - 1);
    const int64_t z = (t < d.T && o < d.d_out) ? (int64_t)d.Z[t * d.ldz + o] : 0;
    rescale_embed(z, a.s, q[k], r[k], y[k]);
  }
  if constexpr (V == 2) {
    *(ulonglong2*)&a.msg[(d.row_q + row) * a.ld + col] = ulonglong2{q[0], q[1]};
    *(ulonglong2*)&a.msg[(d.row_r + row) * a.ld + col] = ulonglong2{r[0], r[1]};
    *(ulonglong2*)&a.msg[(d.row_y + row) * a.ld + col] = ulonglong2{y[0], y[1]};
  } else {
    a.msg[(d.row_q + row) * a.ld + col] = q[0];
    a.msg[(d.row_r + row) * a.ld + col] = r[0];
    a.msg[(d.row_y + row) * a.ld + col] = y[0];
  }
}

// ----------------------------------------------------------- folded rows
struct FoldArgs {
  fp_open_claim c[FP_MAX_OPEN_CLAIMS];
  int32_t n_claims, rows, n_prox, log_cols;
  const uint64_t* r_prox;
  const uint64_t* msg;
  int64_t ld;
  E2* wp;  // [rows] proximity weights
  E2* wc;  // [rows] claim weights (rows outside every claim: unused)
  uint64_t* U;
};

// Row weights, one row per thread.
__global__ __launch_bounds__(256) void row_weights_kernel(FoldArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.rows) return;
  a.wp[i] = eq_at([&](int j) { return E2{a.r_prox[2 * j], a.r_prox[2 * j + 1]}; }, a.n_prox, i);
  E2 w{0, 0};
  for (int k = 0; k < a.n_claims; ++k) {
    const fp_open_claim& c = a.c[k];
    if (i >= c.row0 && i < (int64_t)c.row0 + c.nrows) {
      w = eq_at(
          [&](int j) {
            const uint64_t* p = j < c.n1 ? c.z1 + 2 * j : c.z2 + 2 * (j - c.n1);
            return E2{p[0], p[1]};
          },
          c.n1 + c.n2, i - c.row0);
      break;
    }
  }
  a.wc[i] = w;
}

// One column per thread: the proximity row and every claim's row at that
// column, summed exactly (96-bit) over the rows and reduced once. Claims are
// sorted by row0 and disjoint, so one walk down the rows serves them all.
__global__ __launch_bounds__(256) void fold_rows_ext_kernel(FoldArgs a) {
  const int64_t cols = (int64_t)1 << a.log_cols;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  sct::S96 p0{0, 0, 0}, p1{0, 0, 0}, q0{0, 0, 0}, q1{0, 0, 0};
  int k = 0;
  int64_t end = a.n_claims > 0 ? (int64_t)a.c[0].row0 + a.c[0].nrows : -1;
  for (int64_t i = 0; i < a.rows; ++i) {
    const uint64_t v = a.msg[i * a.ld + c];
    const E2 wp = a.wp[i];
    p0 = sct::add96(p0, sct::to96(gl::mul(wp.a, v)));
    p1 = sct::add96(p1, sct::to96(gl::mul(wp.b, v)));
    if (k < a.n_claims && i >= a.c[k].row0) {
      const E2 wc = a.wc[i];
      q0 = sct::add96(q0, sct::to96(gl::mul(wc.a, v)));
      q1 = sct::add96(q1, sct::to96(gl::mul(wc.b, v)));
      if (i + 1 == end) {
        uint64_t* u = a.U + (int64_t)(1 + k) * 2 * cols;
        u[c] = sct::reduce96(q0);
        u[cols + c] = sct::reduce96(q1);
        q0 = q1 = sct::S96{0, 0, 0};
        ++k;
        end = k < a.n_claims ? (int64_t)a.c[k].row0 + a.c[k].nrows : -1;
      }
    }
  }
  a.U[c] = sct::reduce96(p0);
  a.U[cols + c] = sct::reduce96(p1);
}

// ------------------------------------------------------------ column opening
// One opened column per workgroup: j = (first word of challenge q) mod width.
__global__ __launch_bounds__(256) void open_kernel(const uint64_t* __restrict__ code, int64_t ld, int32_t rows,
                                                   int32_t log_width, const uint64_t* __restrict__ salts,
                                                   const uint64_t* __restrict__ tree, const uint64_t* __restrict__ chal,
                                                   uint64_t* __restrict__ cols, uint64_t* __restrict__ col_salts,
                                                   uint64_t* __restrict__ paths, int32_t* __restrict__ idx) {
  const int q = blockIdx.x, tid = threadIdx.x;
  const int64_t width = (int64_t)1 << log_width;
  const int64_t j = (int64_t)(chal[2 * q] & (uint64_t)(width - 1));
  for (int64_t i = tid; i < rows; i += 256) cols[(int64_t)q * rows + i] = code[i * ld + j];
  if (tid < 2) col_salts[2 * q + tid] = salts[2 * j + tid];
  if (tid == 0 && idx) idx[q] = (int32_t)j;
  if (tid < 4 * log_width) {
    const int d = tid / 4, w = tid % 4;
    const int64_t off = 2 * width - (2 * width >> d);  // first node of level d
    paths[((int64_t)q * log_width + d) * 4 + w] = tree[(off + ((j >> d) ^ 1)) * 4 + w];
  }
}

}  // namespace

extern "C" int fp_commit_tables(int32_t count, const fp_table_desc* d, int32_t n_t, int32_t s, int32_t log_cols,
                                fp_elem* msg, int64_t ld, int32_t rows, hipStream_t stream) {
  const char* fn = "fp_commit_tables";
  if (count < 1 || count > FP_MAX_MULTI) return fpi::fail(FP_EARG, "%s: count=%d outside [1, %d]", fn, count, FP_MAX_MULTI);
  if (!d || !msg) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  if (s < 1 || s > 8) return fpi::fail(FP_ERANGE, "%s: s=%d outside [1, 8]", fn, s);
  if (n_t < 0 || log_cols < 0 || log_cols > FP_MAX_RS_LOGN || ld < ((int64_t)1 << log_cols) || rows < 0)
    return fpi::fail(FP_ESHAPE, "%s: n_t=%d log_cols=%d ld=%lld rows=%d", fn, n_t, log_cols, (long long)ld, rows);
  TabArgs a{};
  a.count = count;
  a.n_t = n_t;
  a.s = s;
  a.log_cols = log_cols;
  a.msg = msg;
  a.ld = ld;
  for (int m = 0; m < count; ++m) {
    const fp_table_desc& x = d[m];
    const int lg = n_t + x.n_o;
    if (x.n_o < 0 || lg < log_cols || lg > FP_MAX_N || x.T < 0 || x.d_out < 0 || x.T > (1LL << n_t) ||
        x.d_out > (1LL << x.n_o) || x.ldz < x.d_out)
      return fpi::fail(FP_ESHAPE, "%s: map %d: T=%d d_out=%d ldz=%lld n_t=%d n_o=%d log_cols=%d", fn, m, x.T, x.d_out,
                       (long long)x.ldz, n_t, x.n_o, log_cols);
    if (!x.Z && (int64_t)x.T * x.d_out > 0) return fpi::fail(FP_EARG, "%s: map %d: null Z", fn, m);
    const int64_t tr = (int64_t)1 << (lg - log_cols);
    for (int32_t r0 : {x.row_q, x.row_r, x.row_y})
      if (r0 < 0 || r0 + tr > rows)
        return fpi::fail(FP_ESHAPE, "%s: map %d: rows [%d, %lld) outside the %d rows", fn, m, r0, (long long)(r0 + tr), rows);
    a.d[m] = x;
    a.start[m + 1] = a.start[m] + ((int64_t)1 << lg);
  }
  const int64_t total = a.start[count];
  if (total == 0) return fpi::ok();
  // two entries per thread (16-byte stores) when every table has an even size, the rows an even number of
  // columns and msg is 16-byte aligned; else one
  bool pairs = log_cols >= 1 && ld % 2 == 0 && ((uintptr_t)msg & 15) == 0;
  for (int m = 0; m < count; ++m) pairs = pairs && ((a.start[m + 1] - a.start[m]) % 2 == 0);
  if (pairs) hipLaunchKernelGGL(tables_kernel<2>, dim3((unsigned)((total / 2 + 255) / 256)), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(tables_kernel<1>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a);
  const int rc = fpi::check_launch("tables_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" size_t fp_commit_fold_ext_workspace(int32_t rows) {
  if (rows < 0) return 0;
  return fpi::align_up((size_t)rows * 2 * sizeof(E2), 256);
}

extern "C" int fp_commit_fold_ext(const fp_elem* msg, int64_t ld, int32_t rows, int32_t log_cols, const fp_elem* r_prox,
                                  int32_t n_prox, int32_t n_claims, const fp_open_claim* claims, fp_elem* U, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  const char* fn = "fp_commit_fold_ext";
  if (rows < 1 || log_cols < 0 || log_cols > FP_MAX_RS_LOGN || ld < ((int64_t)1 << log_cols))
    return fpi::fail(FP_ESHAPE, "%s: rows=%d log_cols=%d ld=%lld", fn, rows, log_cols, (long long)ld);
  if (n_prox < 0 || n_prox > FP_MAX_N || ((int64_t)1 << n_prox) < rows)
    return fpi::fail(FP_ESHAPE, "%s: 2^n_prox (n_prox=%d) must cover the %d rows", fn, n_prox, rows);
  if (n_claims < 0 || n_claims > FP_MAX_OPEN_CLAIMS)
    return fpi::fail(FP_EARG, "%s: n_claims=%d outside [0, %d]", fn, n_claims, FP_MAX_OPEN_CLAIMS);
  if (!msg || !U || (n_prox > 0 && !r_prox) || (n_claims > 0 && !claims)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  const size_t need = fp_commit_fold_ext_workspace(rows);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255))
    return fpi::fail(FP_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) needed, %zu given", fn, need, ws_bytes);
  FoldArgs a{};
  int64_t prev_end = 0;
  for (int k = 0; k < n_claims; ++k) {
    const fp_open_claim& c = claims[k];
    const int n = c.n1 + c.n2;
    if (c.n1 < 0 || c.n2 < 0 || n > FP_MAX_N || c.nrows != (1LL << n) || c.row0 < prev_end ||
        (int64_t)c.row0 + c.nrows > rows || (c.n1 > 0 && !c.z1) || (c.n2 > 0 && !c.z2))
      return fpi::fail(FP_ESHAPE, "%s: claim %d: rows [%d, +%d) with n1=%d n2=%d (claims sorted, disjoint, "
                       "2^(n1+n2) rows inside the matrix)", fn, k, c.row0, c.nrows, c.n1, c.n2);
    prev_end = (int64_t)c.row0 + c.nrows;
    a.c[k] = c;
  }
  a.n_claims = n_claims;
  a.rows = rows;
  a.n_prox = n_prox;
  a.log_cols = log_cols;
  a.r_prox = r_prox;
  a.msg = msg;
  a.ld = ld;
  a.wp = (E2*)ws;
  a.wc = a.wp + rows;
  a.U = U;
  hipLaunchKernelGGL(row_weights_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, a);
  int rc = fpi::check_launch("row_weights_kernel");
  if (rc) return rc;
  const int64_t cols = (int64_t)1 << log_cols;
  hipLaunchKernelGGL(fold_rows_ext_kernel, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, stream, a);
  rc = fpi::check_launch("fold_rows_ext_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" int fp_merkle_open(const fp_elem* code, int64_t ld_code, int32_t rows, int32_t log_width, const uint8_t* salts,
                              const uint8_t* tree, const fp_elem* chal, int32_t nq, fp_elem* cols, uint8_t* col_salts,
                              uint8_t* paths, int32_t* idx, hipStream_t stream) {
  const char* fn = "fp_merkle_open";
  if (rows < 0 || rows > FP_MAX_MERKLE_ROWS || log_width < 1 || log_width > FP_MAX_RS_LOGN + 1 ||
      ld_code < ((int64_t)1 << log_width) || nq < 0)
    return fpi::fail(FP_ESHAPE, "%s: rows=%d log_width=%d ld_code=%lld nq=%d", fn, rows, log_width, (long long)ld_code, nq);
  if (nq == 0) return fpi::ok();
  if (!code || !salts || !tree || !chal || !cols || !col_salts || !paths) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  if ((((uintptr_t)salts) | ((uintptr_t)tree) | ((uintptr_t)col_salts) | ((uintptr_t)paths)) & 7)
    return fpi::fail(FP_EARG, "%s: salts, tree, col_salts and paths must be 8-byte aligned", fn);
  hipLaunchKernelGGL(open_kernel, dim3(nq), dim3(256), 0, stream, code, ld_code, rows, log_width,
                     (const uint64_t*)salts, (const uint64_t*)tree, chal, cols, (uint64_t*)col_salts,
                     (uint64_t*)paths, idx);
  const int rc = fpi::check_launch("open_kernel");
  return rc ? rc : fpi::ok();
}
