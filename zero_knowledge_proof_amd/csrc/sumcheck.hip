// sumcheck.hip - sum-check prover rounds over Goldilocks.
//
// "How fast can FlashProve go", §2: sum-check reduces each matmul to claims
// about committed tables. For the claim sum_j rho_j sum_k A_j[k] B_j[k] over
// 2^n-entry tables, round i sends the degree-2 polynomial
//     g_i(c) = sum_j rho_j sum_q A_j,c[q] B_j,c[q],  A_c[q] = A[2q] + c (A[2q+1] - A[2q])
// by its values at c = 0, 1, 2, and then binds the variable with the
// challenge r_i: A[q] <- A[2q] + r_i (A[2q+1] - A[2q]) (B likewise).
//
// Schedule. While the tables are large, each round is one launch over many
// workgroups: a workgroup folds its slice of the previous round's table with
// r_{i-1}, stores the new slice and emits its share of g_i. A launch boundary
// separates the last partial of g_{i-1} from any read of r_{i-1}, so no
// challenge is used before its round polynomial is complete. Once all of an
// instance's tables fit one workgroup (<= 8192 entries per side), one 512-thread
// workgroup per instance finishes the remaining rounds (sc_tail.hpp: register
// slices, then a single wave). Independent instances (one per MoE expert) run
// as one workgroup each in a single launch.
#include <vector>

#include "common.hpp"
#include "gl.hpp"
#include "sc_tail.hpp"

namespace {

using namespace sct;

constexpr int SC_SLICE = 2048;      // table entries per workgroup in a wide round
constexpr int SC_RT = 256;          // threads of a wide-round workgroup

// Reduce three field values over the workgroup; thread 0 returns the sums.
template <int NT>
__device__ __forceinline__ void block_sum3(uint64_t& a, uint64_t& b, uint64_t& c, uint64_t* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    a = gl::add(a, fpi::shfl_xor_u64(a, m));
    b = gl::add(b, fpi::shfl_xor_u64(b, m));
    c = gl::add(c, fpi::shfl_xor_u64(c, m));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[3 * w] = a;
    red[3 * w + 1] = b;
    red[3 * w + 2] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < NT / 64; ++k) {
      a = gl::add(a, red[3 * k]);
      b = gl::add(b, red[3 * k + 1]);
      c = gl::add(c, red[3 * k + 2]);
    }
  }
  __syncthreads();
}

// Terms of g(0), g(1), g(2) for one pair of entries.
__device__ __forceinline__ void round_terms(uint64_t a0, uint64_t a1, uint64_t b0, uint64_t b1, uint64_t& g0,
                                            uint64_t& g1, uint64_t& g2) {
  const uint64_t a2 = gl::sub(gl::add(a1, a1), a0);  // A at c = 2: 2 A1 - A0
  const uint64_t b2 = gl::sub(gl::add(b1, b1), b0);
  g0 = gl::add(g0, gl::mul(a0, b0));
  g1 = gl::add(g1, gl::mul(a1, b1));
  g2 = gl::add(g2, gl::mul(a2, b2));
}

// ---- wide round ------------------------------------------------------------
// Round i over n_pairs pairs, current table size m = 2^(n-i).
//   i == 0: read the caller's tables, emit partials of g_0.
//   i > 0 : read T_{i-1} (caller's tables when i == 1, else `src`), fold with
//           r_{i-1} into `dst`, emit partials of g_i; workgroup 0 also reduces
//           the partials of g_{i-1} into rounds[i-1].
struct RoundArgs {
  Tabs user;
  const fp_elem* src;   // ws buffer with T_{i-1} (i >= 2)
  fp_elem* dst;         // ws buffer for T_i (i >= 1)
  const fp_elem* rho;
  const fp_elem* r;
  const fp_elem* prev_part;
  fp_elem* part;
  fp_elem* rounds;
  fp_elem* claim0;
  int32_t i, n_pairs, m, nprev;
};

__global__ __launch_bounds__(SC_RT) void sc_round_kernel(RoundArgs a) {
  __shared__ uint64_t red[3 * (SC_RT / 64)];
  const int slices = (a.m + SC_SLICE - 1) / SC_SLICE;
  const int j = blockIdx.x / slices;
  const int s0 = (blockIdx.x - j * slices) * SC_SLICE;
  const int S = min(SC_SLICE, a.m);
  uint64_t g0 = 0, g1 = 0, g2 = 0;
  if (a.i == 0) {
    const fp_elem* A = a.user.A[j];
    const fp_elem* B = a.user.B[j];
    for (int p = threadIdx.x; p < S / 2; p += SC_RT) {
      const int q = s0 + 2 * p;
      round_terms(A[q], A[q + 1], B[q], B[q + 1], g0, g1, g2);
    }
  } else {
    if (blockIdx.x == 0 && threadIdx.x == 0) finish_prev(a.prev_part, a.nprev, a.rounds, a.i - 1, a.claim0);
    const uint64_t r = a.r[a.i - 1];
    const int mp = 2 * a.m;  // previous size
    const fp_elem* A = (a.i == 1) ? a.user.A[j] : a.src + (int64_t)j * mp;
    const fp_elem* B = (a.i == 1) ? a.user.B[j] : a.src + (int64_t)(a.n_pairs + j) * mp;
    fp_elem* dA = a.dst + (int64_t)j * a.m;
    fp_elem* dB = a.dst + (int64_t)(a.n_pairs + j) * a.m;
    for (int p = threadIdx.x; p < S / 2; p += SC_RT) {
      const int q = s0 + 2 * p;  // new pair (q, q+1) from old entries 2q .. 2q+3
      const uint64_t x0 = A[2 * q], x1 = A[2 * q + 1], x2 = A[2 * q + 2], x3 = A[2 * q + 3];
      const uint64_t y0 = B[2 * q], y1 = B[2 * q + 1], y2 = B[2 * q + 2], y3 = B[2 * q + 3];
      const uint64_t a0 = gl::add(x0, gl::mul(r, gl::sub(x1, x0)));
      const uint64_t a1 = gl::add(x2, gl::mul(r, gl::sub(x3, x2)));
      const uint64_t b0 = gl::add(y0, gl::mul(r, gl::sub(y1, y0)));
      const uint64_t b1 = gl::add(y2, gl::mul(r, gl::sub(y3, y2)));
      dA[q] = a0; dA[q + 1] = a1;
      dB[q] = b0; dB[q + 1] = b1;
      round_terms(a0, a1, b0, b1, g0, g1, g2);
    }
  }
  block_sum3<SC_RT>(g0, g1, g2, red);
  if (threadIdx.x == 0) {
    if (a.rho) {
      const uint64_t rj = a.rho[j];
      g0 = gl::mul(g0, rj); g1 = gl::mul(g1, rj); g2 = gl::mul(g2, rj);
    }
    a.part[3 * blockIdx.x] = g0;
    a.part[3 * blockIdx.x + 1] = g1;
    a.part[3 * blockIdx.x + 2] = g2;
  }
}

// The tail launch: one 512-thread workgroup per instance.
constexpr int ST = 512;
__global__ __launch_bounds__(ST) void sc_tail_kernel(TailArgs a) {
  __shared__ TailLds<ST> sh;
  tail_body<ST>(a, blockIdx.x, sh);
}

struct Sched {
  int i0;           // first round of the LDS tail
  int max_blocks;   // most workgroups in a wide round
};

Sched schedule(int n_pairs, int n) {
  Sched s{0, 0};
  int vp = 1;
  while (vp < n_pairs) vp <<= 1;
  // the tail holds at most ST * SLMAX virtual entries (VP * 2^(n - i0))
  while (((int64_t)vp << (n - s.i0)) > (int64_t)ST * SLMAX) ++s.i0;
  for (int i = 0; i < s.i0; ++i) {
    const int m = 1 << (n - i);
    const int blocks = n_pairs * ((m + SC_SLICE - 1) / SC_SLICE);
    if (blocks > s.max_blocks) s.max_blocks = blocks;
  }
  return s;
}

}  // namespace

// Workspace: [T buffers: 2 x (2 n_pairs 2^(n-1))][partials: 2 x max_blocks x 3]
extern "C" size_t fp_sumcheck_workspace(int32_t n_pairs, int32_t n) {
  if (n_pairs < 1 || n < 1 || n > FP_MAX_N) return 0;
  const Sched s = schedule(n_pairs, n);
  if (s.i0 == 0) return 0;
  const size_t tab = (size_t)2 * n_pairs * ((size_t)1 << (n - 1)) * 8;
  return 2 * fpi::align_up(tab, 256) + 2 * fpi::align_up((size_t)s.max_blocks * 3 * 8, 256);
}

extern "C" int fp_sumcheck_prove(int32_t n_pairs, const fp_elem* const* A, const fp_elem* const* B, const fp_elem* rho,
                                 int32_t n, const fp_elem* r, fp_elem* rounds, fp_elem* finals, fp_elem* claim0,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n_pairs < 1 || n_pairs > SC_MAX_PAIRS)
    return fpi::fail(FP_EARG, "fp_sumcheck_prove: n_pairs=%d outside [1, %d]", n_pairs, SC_MAX_PAIRS);
  if (n < 1 || n > FP_MAX_N) return fpi::fail(FP_ESHAPE, "fp_sumcheck_prove: n=%d outside [1, %d]", n, FP_MAX_N);
  if (!A || !B || !r || !rounds || !finals) return fpi::fail(FP_EARG, "fp_sumcheck_prove: null pointer");
  for (int j = 0; j < n_pairs; ++j)
    if (!A[j] || !B[j]) return fpi::fail(FP_EARG, "fp_sumcheck_prove: null table %d", j);
  if ((int64_t)n_pairs * ((int64_t)1 << n) > ((int64_t)1 << 31))
    return fpi::fail(FP_ESHAPE, "fp_sumcheck_prove: tables too large");
  const size_t need = fp_sumcheck_workspace(n_pairs, n);
  if (need && (!ws || ws_bytes < need)) return fpi::fail(FP_EWORKSPACE, "fp_sumcheck_prove: workspace %zu < %zu", ws_bytes, need);
  const Sched s = schedule(n_pairs, n);
  Tabs user{};
  for (int j = 0; j < n_pairs; ++j) {
    user.A[j] = A[j];
    user.B[j] = B[j];
  }
  fp_elem* buf[2] = {nullptr, nullptr};
  fp_elem* part[2] = {nullptr, nullptr};
  if (s.i0 > 0) {
    const size_t tab = fpi::align_up((size_t)2 * n_pairs * ((size_t)1 << (n - 1)) * 8, 256);
    char* w = (char*)ws;
    buf[0] = (fp_elem*)w;
    buf[1] = (fp_elem*)(w + tab);
    part[0] = (fp_elem*)(w + 2 * tab);
    part[1] = (fp_elem*)(w + 2 * tab + fpi::align_up((size_t)s.max_blocks * 3 * 8, 256));
  }
  int nprev = 0;
  for (int i = 0; i < s.i0; ++i) {
    const int m = 1 << (n - i);
    const int blocks = n_pairs * ((m + SC_SLICE - 1) / SC_SLICE);
    RoundArgs ra{};
    ra.user = user;
    ra.src = (i >= 2) ? buf[(i - 1) & 1] : nullptr;
    ra.dst = (i >= 1) ? buf[i & 1] : nullptr;
    ra.rho = rho; ra.r = r;
    ra.prev_part = (i >= 1) ? part[(i - 1) & 1] : nullptr;
    ra.part = part[i & 1];
    ra.rounds = rounds; ra.claim0 = claim0;
    ra.i = i; ra.n_pairs = n_pairs; ra.m = m; ra.nprev = nprev;
    hipLaunchKernelGGL(sc_round_kernel, dim3(blocks), dim3(SC_RT), 0, stream, ra);
    int rc = fpi::check_launch("sc_round_kernel");
    if (rc) return rc;
    nprev = blocks;
  }
  TailArgs ta{};
  ta.user = user;
  ta.src = (s.i0 >= 2) ? buf[(s.i0 - 1) & 1] : nullptr;
  ta.rho = rho; ta.r = r;
  ta.prev_part = (s.i0 >= 1) ? part[(s.i0 - 1) & 1] : nullptr;
  ta.rounds = rounds; ta.finals = finals; ta.claim0 = claim0;
  ta.i0 = s.i0; ta.n = n; ta.n_pairs = n_pairs; ta.nprev = nprev; ta.multi = 0;
  hipLaunchKernelGGL(sc_tail_kernel, dim3(1), dim3(ST), 0, stream, ta);
  int rc = fpi::check_launch("sc_tail_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" int fp_sumcheck_prove_multi(int32_t n_inst, int32_t n, const fp_elem* A, const fp_elem* B, const fp_elem* r,
                                       fp_elem* rounds, fp_elem* finals, fp_elem* claim0, hipStream_t stream) {
  if (n_inst < 0) return fpi::fail(FP_EARG, "fp_sumcheck_prove_multi: n_inst < 0");
  if (n < 1 || n > 13) return fpi::fail(FP_ESHAPE, "fp_sumcheck_prove_multi: n=%d outside [1, 13]", n);
  if (n_inst == 0) return fpi::ok();
  if (!A || !B || !r || !rounds || !finals) return fpi::fail(FP_EARG, "fp_sumcheck_prove_multi: null pointer");
  TailArgs ta{};
  ta.user.A[0] = A;
  ta.user.B[0] = B;
  ta.r = r; ta.rounds = rounds; ta.finals = finals; ta.claim0 = claim0;
  ta.i0 = 0; ta.n = n; ta.n_pairs = 1; ta.nprev = 0; ta.multi = 1;
  hipLaunchKernelGGL(sc_tail_kernel, dim3(n_inst), dim3(ST), 0, stream, ta);
  int rc = fpi::check_launch("sc_tail_kernel");
  return rc ? rc : fpi::ok();
}

// ---- random linear combination of finished claims --------------------------
namespace {
struct CombineArgs {
  const fp_elem* g[16];
  const fp_elem* x[16];
  const fp_elem* rho;
  fp_elem* out;
  int32_t count;
};

__global__ void combine_kernel(CombineArgs a) {
  if (threadIdx.x != 0) return;
  uint64_t s = 0;
  for (int j = 0; j < a.count; ++j) {
    const uint64_t v = gl::eval_deg2(a.g[j][0], a.g[j][1], a.g[j][2], a.x[j][0]);
    s = gl::add(s, gl::mul(a.rho[j], v));
  }
  a.out[0] = s;
}
}  // namespace

extern "C" int fp_combine_claims(int32_t count, const fp_elem* const* g_last, const fp_elem* const* x_last,
                                 const fp_elem* rho, fp_elem* out, hipStream_t stream) {
  if (count < 1 || count > 16) return fpi::fail(FP_EARG, "fp_combine_claims: count=%d outside [1, 16]", count);
  if (!g_last || !x_last || !rho || !out) return fpi::fail(FP_EARG, "fp_combine_claims: null pointer");
  CombineArgs a{};
  for (int j = 0; j < count; ++j) {
    if (!g_last[j] || !x_last[j]) return fpi::fail(FP_EARG, "fp_combine_claims: null entry %d", j);
    a.g[j] = g_last[j];
    a.x[j] = x_last[j];
  }
  a.rho = rho; a.out = out; a.count = count;
  hipLaunchKernelGGL(combine_kernel, dim3(1), dim3(64), 0, stream, a);
  int rc = fpi::check_launch("combine_kernel");
  return rc ? rc : fpi::ok();
}

// ---- plain random linear combination ----------------------------------------
namespace {
struct LinArgs {
  const fp_elem* v[16];
  const fp_elem* rho;
  fp_elem* out;
  int32_t count;
};

__global__ void linear_combine_kernel(LinArgs a) {
  if (threadIdx.x != 0) return;
  uint64_t s = 0;
  for (int j = 0; j < a.count; ++j) s = gl::add(s, gl::mul(a.rho[j], a.v[j][0]));
  a.out[0] = s;
}
}  // namespace

extern "C" int fp_linear_combine(int32_t count, const fp_elem* const* vals, const fp_elem* rho, fp_elem* out,
                                 hipStream_t stream) {
  if (count < 1 || count > 16) return fpi::fail(FP_EARG, "fp_linear_combine: count=%d outside [1, 16]", count);
  if (!vals || !rho || !out) return fpi::fail(FP_EARG, "fp_linear_combine: null pointer");
  LinArgs a{};
  for (int j = 0; j < count; ++j) {
    if (!vals[j]) return fpi::fail(FP_EARG, "fp_linear_combine: null entry %d", j);
    a.v[j] = vals[j];
  }
  a.rho = rho; a.out = out; a.count = count;
  hipLaunchKernelGGL(linear_combine_kernel, dim3(1), dim3(64), 0, stream, a);
  int rc = fpi::check_launch("linear_combine_kernel");
  return rc ? rc : fpi::ok();
}
