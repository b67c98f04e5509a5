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
  uint64_t* corr;  // [n_claims + 1][2]: 2^31 times each weight vector's sum
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

// The offsets of the fast sums below: corr[k] = 2^31 sum_i w_k[i] over the
// rows of weight vector k (claims k < n_claims, the proximity weights at
// k = n_claims), one workgroup each.
__global__ __launch_bounds__(256) void weight_sums_kernel(FoldArgs a) {
  __shared__ sct::S96 red[4][2];
  const int k = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool prox = k == a.n_claims;
  const int64_t r0 = prox ? 0 : a.c[k].row0, r1 = prox ? a.rows : r0 + a.c[k].nrows;
  const E2* w = prox ? a.wp : a.wc;
  sct::S96 s0{0, 0, 0}, s1{0, 0, 0};
  for (int64_t i = r0 + tid; i < r1; i += 256) {
    s0 = sct::add96(s0, sct::to96(w[i].a));
    s1 = sct::add96(s1, sct::to96(w[i].b));
  }
  s0 = sct::wave_sum96(s0);
  s1 = sct::wave_sum96(s1);
  if (lane == 63) {
    red[wave][0] = s0;
    red[wave][1] = s1;
  }
  __syncthreads();
  if (tid < 2) {
    sct::S96 x = red[0][tid];
    for (int v = 1; v < 4; ++v) x = sct::add96(x, red[v][tid]);
    a.corr[2 * k + tid] = gl::mul(sct::reduce96(x), 0x80000000ull);
  }
}

// A fast sum: sum_i e_i m'_i for 64-bit e_i = e0 + 2^32 e1 and 32-bit m'_i,
// kept exactly as l + 2^64 lc + 2^32 (h + 2^64 hc).
struct Fast {
  uint64_t l, h;
  uint32_t lc, hc;
};

__device__ __forceinline__ void fast_add(Fast& f, uint64_t e, uint32_t m) {
  unsigned long long c0, c1;
  f.l = __builtin_addcll(f.l, (uint64_t)(uint32_t)e * m, 0ull, &c0);
  f.h = __builtin_addcll(f.h, (e >> 32) * m, 0ull, &c1);
  f.lc += (uint32_t)c0;
  f.hc += (uint32_t)c1;
}

// The fast sum mod p (2^64 = 2^32 - 1, 2^96 = -1), less its offset.
__device__ __forceinline__ uint64_t fast_value(const Fast& f, uint64_t corr) {
  uint64_t v = gl::canon(f.l);
  v = gl::add(v, ((uint64_t)f.lc << 32) - f.lc);
  v = gl::add(v, gl::reduce128(f.h << 32, f.h >> 32));
  v = gl::sub(v, f.hc);
  return gl::sub(v, corr);
}

// One column per thread: the proximity row and every claim's row at that
// column. The committed tables hold small signed integers m (|m| < 2^31), so
// an entry v = m mod p is taken as m' = m + 2^31 in [0, 2^32): each weight
// half times m' is one 32 x 32-bit product, summed exactly without reduction,
// and the offset 2^31 sum_i w_i (the same for every column) is taken off at the
// end. Any other entry is multiplied in full and summed exactly (96-bit) on
// the side, while its m' is 2^31, which the offset cancels. The rows stream
// through a ring of FR_D loads in flight per thread; the weights pass through
// LDS FR_CH rows at a time. Claims are sorted by row0 and disjoint, so one walk
// down the rows serves them all.
constexpr int FR_T = 256, FR_D = 8, FR_CH = 512;
static_assert(FR_CH % FR_D == 0, "weight chunks of whole groups of rows");

__global__ __launch_bounds__(FR_T) void fold_rows_ext_kernel(FoldArgs a) {
  __shared__ E2 swp[FR_CH], swc[FR_CH];
  const int64_t cols = (int64_t)1 << a.log_cols;
  const int64_t c = (int64_t)blockIdx.x * FR_T + threadIdx.x;
  const bool live = c < cols;
  const uint64_t* src = a.msg + (live ? c : 0);
  const int64_t ld = a.ld, rows = a.rows;
  Fast fp0{0, 0, 0, 0}, fp1{0, 0, 0, 0}, fq0{0, 0, 0, 0}, fq1{0, 0, 0, 0};
  sct::S96 gp0{0, 0, 0}, gp1{0, 0, 0}, gq0{0, 0, 0}, gq1{0, 0, 0};
  int k = 0;
  int64_t beg = a.n_claims > 0 ? a.c[0].row0 : rows, end = a.n_claims > 0 ? beg + a.c[0].nrows : rows;
  uint64_t nxt[FR_D];
#pragma unroll
  for (int d = 0; d < FR_D; ++d) nxt[d] = (live && d < rows) ? src[d * ld] : 0;
  for (int64_t i0 = 0; i0 < rows; i0 += FR_D) {
    if (i0 % FR_CH == 0) {
      __syncthreads();  // the previous chunk's weights read
      for (int t = threadIdx.x; t < FR_CH; t += FR_T) {
        const int64_t i = i0 + t;
        if (i < rows) {
          swp[t] = a.wp[i];
          swc[t] = a.wc[i];
        }
      }
      __syncthreads();
    }
    uint64_t cur[FR_D];
#pragma unroll
    for (int d = 0; d < FR_D; ++d) {
      cur[d] = nxt[d];
      const int64_t j = i0 + FR_D + d;
      nxt[d] = (live && j < rows) ? src[j * ld] : 0;
    }
#pragma unroll
    for (int d = 0; d < FR_D; ++d) {
      const int64_t i = i0 + d;
      if (i >= rows) continue;  // the last group's rows past the matrix
      const uint64_t v = cur[d];
      const uint64_t t = v + 0x80000000ull;
      const bool lo = t >= v && (t >> 32) == 0;  // v < 2^31
      const bool hi = t >= gl::P;                // v in [p - 2^31, p): v - p + 2^31 = t - p
      const uint32_t m = lo ? (uint32_t)t : (hi ? (uint32_t)(t - gl::P) : 0x80000000u);
      const E2 wp = swp[i % FR_CH];
      fast_add(fp0, wp.a, m);
      fast_add(fp1, wp.b, m);
      const bool claim = i >= beg;  // beg <= i < end
      E2 wc{0, 0};
      if (claim) {
        wc = swc[i % FR_CH];
        fast_add(fq0, wc.a, m);
        fast_add(fq1, wc.b, m);
      }
      if (!(lo || hi)) {
        gp0 = sct::add96(gp0, sct::to96(gl::mul(wp.a, v)));
        gp1 = sct::add96(gp1, sct::to96(gl::mul(wp.b, v)));
        if (claim) {
          gq0 = sct::add96(gq0, sct::to96(gl::mul(wc.a, v)));
          gq1 = sct::add96(gq1, sct::to96(gl::mul(wc.b, v)));
        }
      }
      if (i + 1 == end && claim) {
        if (live) {
          uint64_t* u = a.U + (int64_t)(1 + k) * 2 * cols;
          u[c] = gl::add(fast_value(fq0, a.corr[2 * k]), sct::reduce96(gq0));
          u[cols + c] = gl::add(fast_value(fq1, a.corr[2 * k + 1]), sct::reduce96(gq1));
        }
        fq0 = fq1 = Fast{0, 0, 0, 0};
        gq0 = gq1 = sct::S96{0, 0, 0};
        ++k;
        beg = k < a.n_claims ? a.c[k].row0 : rows;
        end = k < a.n_claims ? beg + a.c[k].nrows : rows;
      }
    }
  }
  if (!live) return;
  const uint64_t* cp = a.corr + 2 * a.n_claims;
  a.U[c] = gl::add(fast_value(fp0, cp[0]), sct::reduce96(gp0));
  a.U[cols + c] = gl::add(fast_value(fp1, cp[1]), sct::reduce96(gp1));
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
  return fpi::align_up((size_t)rows * 2 * sizeof(E2), 256) + fpi::align_up((FP_MAX_OPEN_CLAIMS + 1) * sizeof(E2), 256);
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
  a.corr = (uint64_t*)((char*)ws + fpi::align_up((size_t)rows * 2 * sizeof(E2), 256));
  a.U = U;
  hipLaunchKernelGGL(row_weights_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, a);
  int rc = fpi::check_launch("row_weights_kernel");
  if (rc) return rc;
  hipLaunchKernelGGL(weight_sums_kernel, dim3((unsigned)(n_claims + 1)), dim3(256), 0, stream, a);
  rc = fpi::check_launch("weight_sums_kernel");
  if (rc) return rc;
  const int64_t cols = (int64_t)1 << log_cols;
  hipLaunchKernelGGL(fold_rows_ext_kernel, dim3((unsigned)((cols + FR_T - 1) / FR_T)), dim3(FR_T), 0, stream, a);
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
