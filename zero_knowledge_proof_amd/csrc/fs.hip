// fs.hip - soundness-faithful challenges: a Fiat-Shamir transcript on the
// device and the matmul sum-check over an extension of Goldilocks.
//
// "How fast can FlashProve go", §2: every challenge is a BLAKE2b hash of all
// the prover has sent so far; §4 footnote 20: the protocol's challenge and
// lookup arithmetic runs in an extension of Goldilocks, a product costing
// several base products. Here the extension is F_p[u]/(u^2 - 7) (7 generates
// F_p*, so it is not a square); the transcript state is a 32-byte BLAKE2b-256
// digest s, absorbing a message sets s <- BLAKE2b-256(s || message), and
// challenges are read from s and, beyond the first two, from
// BLAKE2b-256(s || j) (j = 1, 2, ... as 32-bit little-endian), each digest's
// four little-endian words w0..w3 giving (w0 mod p) + u (w1 mod p) and
// (w2 mod p) + u (w3 mod p).
//
// The sum-check of sum_k A(k) B(k) over the extension runs in one workgroup:
// each round's values g(0), g(1), g(2) are absorbed and r_i is read from the
// new state before any table is bound by it, so the round chain includes one
// BLAKE2b compression per round, computed by wave 0.
#include <algorithm>

#include "blake2b.hpp"
#include "common.hpp"
#include "ext.hpp"
#include "gl.hpp"
#include "sc_tail.hpp"

namespace {

using namespace fpx;

// ----------------------------------------------------------- the transcript
constexpr int FS_MAX_INIT_WORDS = 16;
struct InitMsg {
  uint64_t w[FS_MAX_INIT_WORDS];
};

// d <- BLAKE2b-256 of nbytes bytes given as little-endian words (zero past the end)
template <typename F>
__device__ __forceinline__ void b2_digest(F word, int nbytes, uint64_t (&d)[4]) {
  uint64_t h[8];
  b2_init32(h);
  const int nw = (nbytes + 7) / 8;
  for (int w0 = 0; w0 < nw || w0 == 0; w0 += 16) {
    uint64_t m[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) m[i] = (w0 + i < nw) ? word(w0 + i) : 0;
    const bool last = w0 + 16 >= nw;
    b2_compress(h, m, last ? (uint64_t)nbytes : (uint64_t)(8 * (w0 + 16)), last);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = h[i];
}

// s <- BLAKE2b-256(s || g0 || g1 || g2): 10 words, one block
__device__ __forceinline__ void absorb_round(uint64_t (&s)[4], const E2 (&g)[3]) {
  uint64_t h[8], m[16];
  b2_init32(h);
#pragma unroll
  for (int i = 0; i < 4; ++i) m[i] = s[i];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    m[4 + 2 * c] = g[c].a;
    m[5 + 2 * c] = g[c].b;
  }
#pragma unroll
  for (int i = 10; i < 16; ++i) m[i] = 0;
  b2_compress(h, m, 80, true);
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = h[i];
}

__device__ __forceinline__ E2 first_challenge(const uint64_t (&s)[4]) { return E2{canon(s[0]), canon(s[1])}; }

__global__ void fs_init_kernel(InitMsg msg, int32_t nbytes, uint64_t* state) {
  if (threadIdx.x != 0) return;
  uint64_t d[4];
  b2_digest([&](int i) { return msg.w[i]; }, nbytes, d);
#pragma unroll
  for (int i = 0; i < 4; ++i) state[i] = d[i];
}

__global__ void fs_absorb_kernel(uint64_t* state, const uint64_t* __restrict__ data, int32_t nw) {
  if (threadIdx.x != 0) return;
  uint64_t d[4];
  b2_digest([&](int i) { return i < 4 ? state[i] : data[i - 4]; }, 8 * (4 + nw), d);
#pragma unroll
  for (int i = 0; i < 4; ++i) state[i] = d[i];
}

// challenge c (c < k) into out[2c], out[2c+1]; thread j reads digest j
__global__ __launch_bounds__(64) void fs_challenges_kernel(const uint64_t* __restrict__ state, int32_t k,
                                                           uint64_t* __restrict__ out) {
  const int j = blockIdx.x * 64 + threadIdx.x;
  if (2 * j >= k) return;
  uint64_t s[4], d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = state[i];
  if (j == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = s[i];
  } else {  // BLAKE2b-256(s || j): 36 bytes, one block
    uint64_t h[8], m[16];
    b2_init32(h);
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = s[i];
    m[4] = (uint32_t)j;
#pragma unroll
    for (int i = 5; i < 16; ++i) m[i] = 0;
    b2_compress(h, m, 36, true);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = h[i];
  }
  out[4 * j] = canon(d[0]);
  out[4 * j + 1] = canon(d[1]);
  if (2 * j + 1 < k) {
    out[4 * j + 2] = canon(d[2]);
    out[4 * j + 3] = canon(d[3]);
  }
}

// E[k] = prod_j (bit j of k ? r_j : 1 - r_j) over the extension, as E0 + u E1
__global__ __launch_bounds__(256) void eq_ext_kernel(const uint64_t* __restrict__ r, int32_t n,
                                                     uint64_t* __restrict__ E0, uint64_t* __restrict__ E1) {
  __shared__ E2 f[2][FP_MAX_N];
  if (threadIdx.x < n) {
    const E2 rj{r[2 * threadIdx.x], r[2 * threadIdx.x + 1]};
    f[1][threadIdx.x] = rj;
    f[0][threadIdx.x] = e2_sub(E2{1, 0}, rj);
  }
  __syncthreads();
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= ((int64_t)1 << n)) return;
  E2 e{1, 0};
  for (int j = 0; j < n; ++j) e = e2_mul(e, f[(k >> j) & 1][j]);
  E0[k] = e.a;
  E1[k] = e.b;
}

// c0 = (c00 + 7 c11) + u (c01 + c10) from the four base claims c4 = [c00, c11, c01, c10]
__global__ void ext_claim_kernel(const uint64_t* __restrict__ c4, uint64_t* __restrict__ c0) {
  if (threadIdx.x != 0) return;
  c0[0] = gl::add(c4[0], gl::mul_small(c4[1], 7u));
  c0[1] = gl::add(c4[2], c4[3]);
}

// ------------------------------------------------ the extension sum-check
constexpr int SE_T = 512;                  // threads
constexpr int SE_Q = 8;                    // entries per thread at the start (n <= 12)
constexpr int SE_MAXN = 12;

// terms of g(0), g(1), g(2) of one pair as exact 96-bit sums per component
__device__ __forceinline__ void pair_terms_e2(E2 a0, E2 a1, E2 b0, E2 b1, sct::S96 (&s)[6]) {
  const E2 da = e2_sub(a1, a0), db = e2_sub(b1, b0);
  E2 a = a0, b = b0;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const E2 p = e2_mul(a, b);
    s[2 * c] = sct::add96(s[2 * c], sct::to96(p.a));
    s[2 * c + 1] = sct::add96(s[2 * c + 1], sct::to96(p.b));
    if (c < 2) {
      a = e2_add(a, da);
      b = e2_add(b, db);
    }
  }
}

// wave totals of the 6 sums, canonical, in every lane
__device__ __forceinline__ void wave_g(sct::S96 (&s)[6], E2 (&g)[3]) {
  uint64_t v[6];
#pragma unroll
  for (int c = 0; c < 6; ++c) v[c] = sct::lane_value(sct::wave_sum96(s[c]), 63);
#pragma unroll
  for (int c = 0; c < 3; ++c) g[c] = E2{v[2 * c], v[2 * c + 1]};
}

// the round's message out, the transcript advanced, r_i returned (wave-uniform)
__device__ __forceinline__ E2 emit_round(uint64_t (&s)[4], const E2 (&g)[3], uint64_t* rounds, uint64_t* r_out,
                                         int i, bool writer) {
  absorb_round(s, g);
  const E2 r = first_challenge(s);
  if (writer) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      rounds[(int64_t)i * 6 + 2 * c] = g[c].a;
      rounds[(int64_t)i * 6 + 2 * c + 1] = g[c].b;
    }
    r_out[2 * i] = r.a;
    r_out[2 * i + 1] = r.b;
  }
  return r;
}

// Stage 1 of the extension sum-check: CNT entries per thread, pairs inside the
// thread; the round sums meet in LDS, wave 0 absorbs them and reads r_i, which
// every thread then applies.
template <int CNT>
__device__ __forceinline__ void s1_round(E2 (&a)[SE_Q], E2 (&b)[SE_Q], uint64_t (&s)[4], sct::S96 (*red)[6],
                                         uint64_t* rsh, uint64_t* rounds, uint64_t* r_out, int i) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  sct::S96 acc[6] = {};
#pragma unroll
  for (int p = 0; p < CNT / 2; ++p) pair_terms_e2(a[2 * p], a[2 * p + 1], b[2 * p], b[2 * p + 1], acc);
#pragma unroll
  for (int c = 0; c < 6; ++c) acc[c] = sct::wave_sum96(acc[c]);
  if (lane == 63)
#pragma unroll
    for (int c = 0; c < 6; ++c) red[wave][c] = acc[c];
  __syncthreads();
  if (wave == 0) {
    // every lane of wave 0 adds the wave totals and hashes the same message
    E2 g[3];
    uint64_t v[6];
#pragma unroll
    for (int c = 0; c < 6; ++c) {
      sct::S96 t = red[0][c];
#pragma unroll
      for (int w = 1; w < SE_T / 64; ++w) t = sct::add96(t, red[w][c]);
      v[c] = sct::reduce96(t);
    }
#pragma unroll
    for (int c = 0; c < 3; ++c) g[c] = E2{v[2 * c], v[2 * c + 1]};
    const E2 r = emit_round(s, g, rounds, r_out, i, lane == 0);
    if (lane == 0) {
      rsh[0] = r.a;
      rsh[1] = r.b;
    }
  }
  __syncthreads();
  // only wave 0 carries the transcript: the other waves stop after stage 1
  const E2 r{rsh[0], rsh[1]};
#pragma unroll
  for (int p = 0; p < CNT / 2; ++p) {
    a[p] = e2_lerp(a[2 * p], a[2 * p + 1], r);
    b[p] = e2_lerp(b[2 * p], b[2 * p + 1], r);
  }
}

// Stage 2: wave 0 alone, CNT entries per lane, pairs inside the lane.
template <int CNT>
__device__ __forceinline__ void s2_round(E2 (&a)[8], E2 (&b)[8], uint64_t (&s)[4], uint64_t* rounds, uint64_t* r_out,
                                         int i) {
  sct::S96 acc[6] = {};
#pragma unroll
  for (int p = 0; p < CNT / 2; ++p) pair_terms_e2(a[2 * p], a[2 * p + 1], b[2 * p], b[2 * p + 1], acc);
  E2 g[3];
  wave_g(acc, g);
  const E2 r = emit_round(s, g, rounds, r_out, i, (threadIdx.x & 63) == 0);
#pragma unroll
  for (int p = 0; p < CNT / 2; ++p) {
    a[p] = e2_lerp(a[2 * p], a[2 * p + 1], r);
    b[p] = e2_lerp(b[2 * p], b[2 * p + 1], r);
  }
}

__global__ __launch_bounds__(SE_T) void sc_ext_fs_kernel(const uint64_t* __restrict__ A0, const uint64_t* __restrict__ A1,
                                                         const uint64_t* __restrict__ B0, const uint64_t* __restrict__ B1,
                                                         int32_t n, uint64_t* __restrict__ state,
                                                         uint64_t* __restrict__ rounds, uint64_t* __restrict__ r_out,
                                                         uint64_t* __restrict__ finals) {
  __shared__ sct::S96 red[SE_T / 64][6];
  __shared__ uint64_t rsh[2];
  __shared__ E2 xa[SE_T], xb[SE_T];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t N = (int64_t)1 << n;
  uint64_t s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = state[i];
  // stage 1: thread t holds entries t q .. t q + q - 1
  int q = N >= SE_T ? (int)(N / SE_T) : 1;
  E2 a[SE_Q], b[SE_Q];
#pragma unroll
  for (int k = 0; k < SE_Q; ++k) {
    const int64_t x = (int64_t)tid * q + k;
    const bool ok = k < q && x < N;
    a[k] = ok ? E2{A0[x], A1[x]} : E2{0, 0};
    b[k] = ok ? E2{B0[x], B1[x]} : E2{0, 0};
  }
  int i = 0;
  if (q == 8) s1_round<8>(a, b, s, red, rsh, rounds, r_out, i++), q = 4;
  if (q == 4) s1_round<4>(a, b, s, red, rsh, rounds, r_out, i++), q = 2;
  if (q == 2) s1_round<2>(a, b, s, red, rsh, rounds, r_out, i++), q = 1;
  // stage 2: n2 = min(N, 512) entries, one per thread -> wave 0, q2 per lane
  const int n2 = N < SE_T ? (int)N : SE_T;
  xa[tid] = a[0];
  xb[tid] = b[0];
  __syncthreads();
  if (wave != 0) return;
  int q2 = n2 >= 64 ? n2 / 64 : 1;
  E2 a2[8], b2[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int x = lane * q2 + k;
    const bool ok = k < q2 && x < n2;
    a2[k] = ok ? xa[x] : E2{0, 0};
    b2[k] = ok ? xb[x] : E2{0, 0};
  }
  if (q2 == 8) s2_round<8>(a2, b2, s, rounds, r_out, i++), q2 = 4;
  if (q2 == 4) s2_round<4>(a2, b2, s, rounds, r_out, i++), q2 = 2;
  if (q2 == 2) s2_round<2>(a2, b2, s, rounds, r_out, i++), q2 = 1;
  // stage 3: entry x at lane x * dist, partners dist apart
  E2 av = a2[0], bv = b2[0];
  for (int dist = 1; i < n; dist <<= 1, ++i) {
    const E2 a1{fpi::shfl_down_u64(av.a, dist), fpi::shfl_down_u64(av.b, dist)};
    const E2 b1{fpi::shfl_down_u64(bv.a, dist), fpi::shfl_down_u64(bv.b, dist)};
    const bool lead = (lane & (2 * dist - 1)) == 0;
    sct::S96 acc[6] = {};
    if (lead) pair_terms_e2(av, a1, bv, b1, acc);
    E2 g[3];
    wave_g(acc, g);
    const E2 r = emit_round(s, g, rounds, r_out, i, lane == 0);
    if (lead) {
      av = e2_lerp(av, a1, r);
      bv = e2_lerp(bv, b1, r);
    }
  }
  // finals: A(r), B(r), absorbed like a round message (8 words, one block)
  const E2 fa{fpi::readlane_u64(av.a, 0), fpi::readlane_u64(av.b, 0)};
  const E2 fb{fpi::readlane_u64(bv.a, 0), fpi::readlane_u64(bv.b, 0)};
  uint64_t h[8], m[16];
  b2_init32(h);
#pragma unroll
  for (int k = 0; k < 4; ++k) m[k] = s[k];
  m[4] = fa.a;
  m[5] = fa.b;
  m[6] = fb.a;
  m[7] = fb.b;
#pragma unroll
  for (int k = 8; k < 16; ++k) m[k] = 0;
  b2_compress(h, m, 64, true);
  if (lane == 0) {
    finals[0] = fa.a;
    finals[1] = fa.b;
    finals[2] = fb.a;
    finals[3] = fb.b;
#pragma unroll
    for (int k = 0; k < 4; ++k) state[k] = h[k];
  }
}

// ------------------------------------- the multi-pair extension sum-check
// sum_j rho_j sum_k A_j[k] B_j[k] over 2^n with up to 8 pairs, for tables too
// large for registers, streamed through a workspace. T_i (the tables of round
// i) is the caller's base parts for i = 0, else it alternates between two
// workspace buffers (T_i in buffer (i-1) mod 2; pair j's A at 2j 2^(n-1), its
// B at (2j+1) 2^(n-1)). While the tables are large (rounds before i0), round i
// is two launches: workgroups own runs of one pair's entries, bind T_{i-1}
// with r_{i-1} into T_i and sum their terms of round i exactly (96-bit), each
// workgroup's sums weighted by its pair's rho_j into its partials; then one
// wave adds the partials, absorbs g_i and reads r_i. Rounds i0 onwards run in
// one workgroup with the tables in LDS (T_i0, bound from T_{i0-1} on the way
// in): round i lets every pair of entries of every table add its terms,
// completes g_i across the workgroup, lets wave 0 absorb it and read r_i, and
// only then binds the pairs in place.
constexpr int SM_T = 1024;
constexpr int SM_MAX_PAIRS = 8;
constexpr int SM_MAXN = 24;
constexpr int SM_LDS_ENTRIES = 1024;  // entries of all A tables (and of all B) at round i0

struct ExtScArgs {
  const uint64_t* A0[SM_MAX_PAIRS];
  const uint64_t* A1[SM_MAX_PAIRS];
  const uint64_t* B0[SM_MAX_PAIRS];
  const uint64_t* B1[SM_MAX_PAIRS];
  const uint64_t* rho;  // 2 n_pairs words, or NULL (all ones)
  int32_t np, n, i0;  // i0: the first round of the workgroup (n_pairs 2^(n - i0) <= SM_LDS_ENTRIES)
  uint64_t* state;
  uint64_t* rounds;  // [n][3][2]
  uint64_t* r_out;   // [n][2]
  uint64_t* finals;  // [np][4]: A_j(r), B_j(r)
  E2* ws;
};

__device__ __forceinline__ E2 rho_of(const ExtScArgs& a, int j) {
  return a.rho ? E2{a.rho[2 * j], a.rho[2 * j + 1]} : E2{1, 0};
}

// entry e of table (j, which) of T_i, i < i0, from the caller's parts (i = 0) or the workspace
__device__ __forceinline__ E2 ext_entry(const ExtScArgs& a, int i, int j, int which, int64_t e) {
  if (i == 0) return which ? E2{a.B0[j][e], a.B1[j][e]} : E2{a.A0[j][e], a.A1[j][e]};
  const int64_t H = (int64_t)1 << (a.n - 1);
  return a.ws[(int64_t)(2 * ((i - 1) & 1)) * a.np * H + (2 * j + which) * H + e];
}

__global__ __launch_bounds__(SM_T) void sc_ext_multi_kernel(ExtScArgs a) {
  __shared__ E2 TA[SM_LDS_ENTRIES], TB[SM_LDS_ENTRIES];
  __shared__ sct::S96 red[SM_T / 64][6];
  __shared__ uint64_t rsh[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int np = a.np, n = a.n, i0 = a.i0;
  const int lh0 = n - i0;  // log2 of the entries per table at round i0
  const int64_t H0 = (int64_t)1 << lh0;
  uint64_t s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = a.state[i];
  // T_i0 into LDS: pair j's entries at j H0
  if (i0 == 0) {
    for (int64_t p = tid; p < np * H0; p += SM_T) {
      const int j = (int)(p >> lh0);
      const int64_t e = p & (H0 - 1);
      TA[p] = ext_entry(a, 0, j, 0, e);
      TB[p] = ext_entry(a, 0, j, 1, e);
    }
  } else {
    const E2 r{a.r_out[2 * (i0 - 1)], a.r_out[2 * (i0 - 1) + 1]};
    for (int64_t p = tid; p < np * H0; p += SM_T) {
      const int j = (int)(p >> lh0);
      const int64_t e = p & (H0 - 1);
      TA[p] = e2_lerp(ext_entry(a, i0 - 1, j, 0, 2 * e), ext_entry(a, i0 - 1, j, 0, 2 * e + 1), r);
      TB[p] = e2_lerp(ext_entry(a, i0 - 1, j, 1, 2 * e), ext_entry(a, i0 - 1, j, 1, 2 * e + 1), r);
    }
  }
  __syncthreads();
  for (int i = i0; i < n; ++i) {
    const int lh = n - 1 - i;  // log2 of the pairs of entries per table in round i
    const bool act = tid < (np << lh);
    const int j = act ? tid >> lh : 0;
    const int64_t q = tid & (((int64_t)1 << lh) - 1);
    const int64_t base = j * H0;
    E2 a0{0, 0}, a1{0, 0}, b0{0, 0}, b1{0, 0};
    sct::S96 acc[6] = {};
    if (act) {
      a0 = TA[base + 2 * q];
      a1 = TA[base + 2 * q + 1];
      b0 = TB[base + 2 * q];
      b1 = TB[base + 2 * q + 1];
      pair_terms_e2(a0, a1, b0, b1, acc);
    }
    const E2 rj = rho_of(a, j);
    sct::S96 t[6];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const E2 g = act ? e2_mul(rj, E2{sct::reduce96(acc[2 * c]), sct::reduce96(acc[2 * c + 1])}) : E2{0, 0};
      t[2 * c] = sct::wave_sum96(sct::to96(g.a));
      t[2 * c + 1] = sct::wave_sum96(sct::to96(g.b));
    }
    if (lane == 63)
#pragma unroll
      for (int c = 0; c < 6; ++c) red[wave][c] = t[c];
    __syncthreads();
    if (wave == 0) {
      uint64_t v[6];
#pragma unroll
      for (int c = 0; c < 6; ++c) {
        sct::S96 x = red[0][c];
        for (int w = 1; w < SM_T / 64; ++w) x = sct::add96(x, red[w][c]);
        v[c] = sct::reduce96(x);
      }
      E2 G[3];
#pragma unroll
      for (int c = 0; c < 3; ++c) G[c] = E2{v[2 * c], v[2 * c + 1]};
      const E2 r = emit_round(s, G, a.rounds, a.r_out, i, lane == 0);
      if (lane == 0) {
        rsh[0] = r.a;
        rsh[1] = r.b;
      }
    }
    __syncthreads();  // r_i known to every wave, and every read of round i done
    if (act) {
      const E2 r{rsh[0], rsh[1]};
      TA[base + q] = e2_lerp(a0, a1, r);
      TB[base + q] = e2_lerp(b0, b1, r);
    }
    __syncthreads();  // T_{i+1} complete before round i+1 reads it
  }
  if (wave != 0) return;
  // finals A_j(r), B_j(r) of every pair, absorbed as one message
  auto fin = [&](int w) -> uint64_t {  // word w of the finals message
    const int j = w / 4, k = w % 4;
    const E2 x = k < 2 ? TA[j * H0] : TB[j * H0];
    return (k & 1) ? x.b : x.a;
  };
  uint64_t d[4];
  b2_digest([&](int w) { return w < 4 ? s[w] : fin(w - 4); }, 8 * (4 + 4 * np), d);
  if (lane < 4 * np) a.finals[lane] = fin(lane);
  if (lane < 4) a.state[lane] = d[lane];
}

// A wide round i < i0 of the streamed sum-check (see above): workgroup b owns
// pairs q of pair j = b / bpp's tables (runs of SW_T, every bpp-th); for i > 0
// it binds them from T_{i-1} with r_{i-1} into T_i, and it writes rho_j times
// its sums of their round-i terms into partials[b].
constexpr int SW_T = 256, SW_MAXB = 1024;
__global__ __launch_bounds__(SW_T) void sc_ext_wide_kernel(ExtScArgs a, int32_t i, int32_t bpp,
                                                          uint64_t* __restrict__ partials) {
  __shared__ sct::S96 red[SW_T / 64][6];
  const int n = a.n, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = blockIdx.x / bpp, chunk = blockIdx.x % bpp;
  const int64_t H = (int64_t)1 << (n - 1);
  const int64_t h = (int64_t)1 << (n - 1 - i);  // pairs per table in round i
  const E2 rp = i > 0 ? E2{a.r_out[2 * (i - 1)], a.r_out[2 * (i - 1) + 1]} : E2{0, 0};
  E2* DA = a.ws + (int64_t)(2 * ((i - 1) & 1)) * a.np * H + 2 * j * H;  // T_i's tables of pair j (i > 0)
  E2* DB = DA + H;
  sct::S96 acc[6] = {};
  for (int64_t q = (int64_t)chunk * SW_T + tid; q < h; q += (int64_t)bpp * SW_T) {
    E2 a0, a1, b0, b1;
    if (i == 0) {
      a0 = ext_entry(a, 0, j, 0, 2 * q);
      a1 = ext_entry(a, 0, j, 0, 2 * q + 1);
      b0 = ext_entry(a, 0, j, 1, 2 * q);
      b1 = ext_entry(a, 0, j, 1, 2 * q + 1);
    } else {
      a0 = e2_lerp(ext_entry(a, i - 1, j, 0, 4 * q), ext_entry(a, i - 1, j, 0, 4 * q + 1), rp);
      a1 = e2_lerp(ext_entry(a, i - 1, j, 0, 4 * q + 2), ext_entry(a, i - 1, j, 0, 4 * q + 3), rp);
      b0 = e2_lerp(ext_entry(a, i - 1, j, 1, 4 * q), ext_entry(a, i - 1, j, 1, 4 * q + 1), rp);
      b1 = e2_lerp(ext_entry(a, i - 1, j, 1, 4 * q + 2), ext_entry(a, i - 1, j, 1, 4 * q + 3), rp);
      DA[2 * q] = a0;
      DA[2 * q + 1] = a1;
      DB[2 * q] = b0;
      DB[2 * q + 1] = b1;
    }
    pair_terms_e2(a0, a1, b0, b1, acc);
  }
  sct::S96 t[6];
#pragma unroll
  for (int c = 0; c < 6; ++c) t[c] = sct::wave_sum96(sct::to96(sct::reduce96(acc[c])));
  if (lane == 63)
#pragma unroll
    for (int c = 0; c < 6; ++c) red[wave][c] = t[c];
  __syncthreads();
  if (tid < 3) {
    sct::S96 x0 = red[0][2 * tid], x1 = red[0][2 * tid + 1];
#pragma unroll
    for (int w = 1; w < SW_T / 64; ++w) {
      x0 = sct::add96(x0, red[w][2 * tid]);
      x1 = sct::add96(x1, red[w][2 * tid + 1]);
    }
    const E2 g = e2_mul(rho_of(a, j), E2{sct::reduce96(x0), sct::reduce96(x1)});
    partials[(int64_t)blockIdx.x * 6 + 2 * tid] = g.a;
    partials[(int64_t)blockIdx.x * 6 + 2 * tid + 1] = g.b;
  }
}

// The end of a wide round i: one wave adds the workgroups' partials, absorbs
// g_i, reads r_i and writes both out.
__global__ __launch_bounds__(64) void sc_ext_hash_kernel(ExtScArgs a, int32_t i, int32_t nb,
                                                         const uint64_t* __restrict__ partials) {
  const int lane = threadIdx.x;
  sct::S96 acc[6] = {};
  for (int b = lane; b < nb; b += 64)
#pragma unroll
    for (int c = 0; c < 6; ++c) acc[c] = sct::add96(acc[c], sct::to96(partials[(int64_t)b * 6 + c]));
  uint64_t s[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) s[k] = a.state[k];
  E2 g[3];
  wave_g(acc, g);
  emit_round(s, g, a.rounds, a.r_out, i, lane == 0);
  if (lane < 4) a.state[lane] = s[lane];
}

}  // namespace

extern "C" int fp_fs_init(uint8_t* state, const uint8_t* msg, int32_t nbytes, hipStream_t stream) {
  const char* fn = "fp_fs_init";
  if (nbytes < 0 || nbytes > 8 * FS_MAX_INIT_WORDS) return fpi::fail(FP_EARG, "%s: nbytes=%d outside [0, 128]", fn, nbytes);
  if (!state || (nbytes > 0 && !msg)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  if (((uintptr_t)state) & 7) return fpi::fail(FP_EARG, "%s: state must be 8-byte aligned", fn);
  InitMsg m{};
  for (int i = 0; i < nbytes; ++i) m.w[i / 8] |= (uint64_t)msg[i] << (8 * (i % 8));
  hipLaunchKernelGGL(fs_init_kernel, dim3(1), dim3(64), 0, stream, m, nbytes, (uint64_t*)state);
  const int rc = fpi::check_launch("fs_init_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" int fp_fs_absorb(uint8_t* state, const fp_elem* data, int32_t nwords, hipStream_t stream) {
  const char* fn = "fp_fs_absorb";
  if (nwords < 0 || nwords > (1 << 20)) return fpi::fail(FP_EARG, "%s: nwords=%d", fn, nwords);
  if (!state || (nwords > 0 && !data)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  if (((uintptr_t)state) & 7) return fpi::fail(FP_EARG, "%s: state must be 8-byte aligned", fn);
  hipLaunchKernelGGL(fs_absorb_kernel, dim3(1), dim3(64), 0, stream, (uint64_t*)state, data, nwords);
  const int rc = fpi::check_launch("fs_absorb_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" int fp_fs_challenges(const uint8_t* state, int32_t k, fp_elem* out, hipStream_t stream) {
  const char* fn = "fp_fs_challenges";
  if (k < 0 || k > (1 << 20)) return fpi::fail(FP_EARG, "%s: k=%d", fn, k);
  if (k == 0) return fpi::ok();
  if (!state || !out) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  if (((uintptr_t)state) & 7) return fpi::fail(FP_EARG, "%s: state must be 8-byte aligned", fn);
  const int digests = (k + 1) / 2;
  hipLaunchKernelGGL(fs_challenges_kernel, dim3((digests + 63) / 64), dim3(64), 0, stream, (const uint64_t*)state, k,
                     out);
  const int rc = fpi::check_launch("fs_challenges_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" int fp_eq_table_ext(const fp_elem* r, int32_t n, fp_elem* E0, fp_elem* E1, hipStream_t stream) {
  const char* fn = "fp_eq_table_ext";
  if (n < 0 || n > 24) return fpi::fail(FP_ESHAPE, "%s: n=%d outside [0, 24]", fn, n);
  if (!E0 || !E1 || (n > 0 && !r)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  const int64_t N = (int64_t)1 << n;
  hipLaunchKernelGGL(eq_ext_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, r, n, E0, E1);
  const int rc = fpi::check_launch("eq_ext_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" int fp_ext_claim_combine(const fp_elem* c4, fp_elem* c0, hipStream_t stream) {
  if (!c4 || !c0) return fpi::fail(FP_EARG, "fp_ext_claim_combine: null pointer");
  hipLaunchKernelGGL(ext_claim_kernel, dim3(1), dim3(64), 0, stream, c4, c0);
  const int rc = fpi::check_launch("ext_claim_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" int fp_sumcheck_ext_fs(const fp_elem* A0, const fp_elem* A1, const fp_elem* B0, const fp_elem* B1,
                                  int32_t n, uint8_t* state, fp_elem* rounds, fp_elem* r, fp_elem* finals,
                                  hipStream_t stream) {
  const char* fn = "fp_sumcheck_ext_fs";
  if (n < 0 || n > SE_MAXN) return fpi::fail(FP_ESHAPE, "%s: n=%d outside [0, %d]", fn, n, SE_MAXN);
  if (!A0 || !A1 || !B0 || !B1 || !state || !finals || (n > 0 && (!rounds || !r)))
    return fpi::fail(FP_EARG, "%s: null pointer", fn);
  if (((uintptr_t)state) & 7) return fpi::fail(FP_EARG, "%s: state must be 8-byte aligned", fn);
  hipLaunchKernelGGL(sc_ext_fs_kernel, dim3(1), dim3(SE_T), 0, stream, A0, A1, B0, B1, n, (uint64_t*)state, rounds,
                     r, finals);
  const int rc = fpi::check_launch("sc_ext_fs_kernel");
  return rc ? rc : fpi::ok();
}

// Rounds run wide before the single workgroup takes over: while the pairs' A tables hold more than
// SM_LDS_ENTRIES entries in all (the workgroup's LDS; one workgroup's round then costs little more than its
// hash).
static int ext_wide_rounds(int np, int n) {
  int i0 = 0;
  while (i0 < n && ((int64_t)np << (n - i0)) > SM_LDS_ENTRIES) ++i0;
  return i0;
}

extern "C" size_t fp_sumcheck_ext_fs_multi_workspace(int32_t n_pairs, int32_t n) {
  if (n_pairs < 1 || n_pairs > SM_MAX_PAIRS || n < 0 || n > SM_MAXN) return 0;
  if (n == 0) return 0;
  const size_t tables = fpi::align_up((size_t)n_pairs << (n + 5), 256);
  return tables + (ext_wide_rounds(n_pairs, n) > 0 ? (size_t)SW_MAXB * 6 * 8 : 0);
}

extern "C" int fp_sumcheck_ext_fs_multi(int32_t n_pairs, const fp_elem* const* A0, const fp_elem* const* A1,
                                        const fp_elem* const* B0, const fp_elem* const* B1, const fp_elem* rho,
                                        int32_t n, uint8_t* state, fp_elem* rounds, fp_elem* r, fp_elem* finals,
                                        void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "fp_sumcheck_ext_fs_multi";
  if (n_pairs < 1 || n_pairs > SM_MAX_PAIRS)
    return fpi::fail(FP_EARG, "%s: n_pairs=%d outside [1, %d]", fn, n_pairs, SM_MAX_PAIRS);
  if (n < 0 || n > SM_MAXN) return fpi::fail(FP_ESHAPE, "%s: n=%d outside [0, %d]", fn, n, SM_MAXN);
  if (!A0 || !A1 || !B0 || !B1 || !state || !finals || (n > 0 && (!rounds || !r)))
    return fpi::fail(FP_EARG, "%s: null pointer", fn);
  if (((uintptr_t)state) & 7) return fpi::fail(FP_EARG, "%s: state must be 8-byte aligned", fn);
  const size_t need = fp_sumcheck_ext_fs_multi_workspace(n_pairs, n);
  if (need > 0 && (!ws || ws_bytes < need || ((uintptr_t)ws & 255)))
    return fpi::fail(FP_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) needed, %zu given", fn, need,
                     ws_bytes);
  ExtScArgs a{};
  for (int j = 0; j < n_pairs; ++j) {
    if (!A0[j] || !A1[j] || !B0[j] || !B1[j]) return fpi::fail(FP_EARG, "%s: null table of pair %d", fn, j);
    a.A0[j] = A0[j];
    a.A1[j] = A1[j];
    a.B0[j] = B0[j];
    a.B1[j] = B1[j];
  }
  a.rho = rho;
  a.np = n_pairs;
  a.n = n;
  a.i0 = ext_wide_rounds(n_pairs, n);
  a.state = (uint64_t*)state;
  a.rounds = rounds;
  a.r_out = r;
  a.finals = finals;
  a.ws = (E2*)ws;
  if (a.i0 > 0) {
    uint64_t* partials = (uint64_t*)((char*)ws + fpi::align_up((size_t)n_pairs << (n + 5), 256));
    // rounds 0 .. i0-1 wide: each binds T_{i-1} into T_i for i > 0 and sums its terms, then the hash
    for (int i = 0; i < a.i0; ++i) {
      const int64_t h = (int64_t)1 << (n - 1 - i);
      const int bpp = (int)std::min<int64_t>(SW_MAXB / n_pairs, (h + SW_T - 1) / SW_T);
      const int nb = n_pairs * bpp;
      hipLaunchKernelGGL(sc_ext_wide_kernel, dim3(nb), dim3(SW_T), 0, stream, a, i, bpp, partials);
      int rc = fpi::check_launch("sc_ext_wide_kernel");
      if (rc) return rc;
      hipLaunchKernelGGL(sc_ext_hash_kernel, dim3(1), dim3(64), 0, stream, a, i, nb, (const uint64_t*)partials);
      rc = fpi::check_launch("sc_ext_hash_kernel");
      if (rc) return rc;
    }
  }
  hipLaunchKernelGGL(sc_ext_multi_kernel, dim3(1), dim3(SM_T), 0, stream, a);
  const int rc = fpi::check_launch("sc_ext_multi_kernel");
  return rc ? rc : fpi::ok();
}
