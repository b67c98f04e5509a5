// lookup.hip - the lookup that shows committed remainders are small.
//
// "How fast can FlashProve go", §3.1 (each rescale remainder is committed and
// range-checked by a lookup) and §4 (the lookup as a grand-product argument:
// the product of gamma - key over the keys is matched against the table's
// product, the key side computed as a binary product tree that is proved one
// level at a time by sum-check). Here the tree has 2^L leaves gamma - key
// (padded with gamma - 0), level d+1 entry i = level d entries 2i times 2i+1,
// and the claim on level d+1 at a point z is reduced to level d by the
// degree-3 sum-check of eq(z, x) V_d(2x) V_d(2x+1); the next point is
// (lambda, rho), rho the sum-check's challenges. The table side is the
// keys' multiplicities.
//
// Sum-check rounds: while the tables are large, one launch per round folds the
// three tables by the previous challenge and emits per-workgroup partial sums
// of the round polynomial's values at 0..3 (the next launch's first workgroup
// adds them); at most 2048 entries are finished by one workgroup, first 8 per
// thread in registers, then in one wave with no barriers. The levels'
// challenges are inputs, so the levels are independent instances: one launch
// runs round k of every level that still has wide rounds, and one launch runs
// every level's tail, a workgroup each.
#include <algorithm>

#include "common.hpp"
#include "gl.hpp"
#include "sc_tail.hpp"

namespace {

constexpr int LK_T = 256;        // threads of the tree and wide-round launches
constexpr int LK_K = 4;          // tree levels per launch (16 children per thread)
constexpr int SC3_TAIL = 2048;   // entries the single-workgroup tail takes
constexpr int SC3_TT = 256;      // tail threads
constexpr int SC3_MAXB = 1024;   // workgroups of a wide round
static_assert(SC3_TAIL == 8 * SC3_TT, "the tail starts with 8 entries per thread");

// --------------------------------------------------------------- the tree
// Thread t takes inputs [t 2^K, (t+1) 2^K) of level `in` (or, for the leaves,
// keys: gamma - key, 0 past n) and writes the K levels above them; with keys,
// the leaves themselves are written first. MODE 0: int8 keys; MODE 1: pair
// keys A[j] + scale B[j] + offset of two field tables; MODE 2: a level of the
// tree as input.
struct PairKeys {
  const uint64_t* A;
  const uint64_t* B;
  uint64_t scale, offset;
};

template <int K, int MODE>
__global__ __launch_bounds__(LK_T) void tree_kernel(const int8_t* __restrict__ keys, int64_t n, PairKeys pk,
                                                    const uint64_t* __restrict__ gamma, const uint64_t* __restrict__ in,
                                                    int64_t n_in, uint64_t* __restrict__ leaves_out,
                                                    uint64_t* __restrict__ out) {
  constexpr int W = 1 << K;
  // pair keys are 8-byte entries of two tables: the workgroup's LK_T W keys are formed from coalesced loads
  // into LDS (a pad word after every W, so that the threads' runs start on different banks)
  __shared__ uint64_t kl[MODE == 1 ? LK_T * (W + 1) : 1];
  const int64_t t = (int64_t)blockIdx.x * LK_T + threadIdx.x;
  if constexpr (MODE == 1) {
    const int64_t base = (int64_t)blockIdx.x * LK_T * W;
    for (int i = threadIdx.x; i < LK_T * W; i += LK_T) {
      const int64_t j = base + i;
      kl[i + i / W] = (j < n) ? gl::add(gl::add(pk.A[j], gl::mul(pk.scale, pk.B[j])), pk.offset) : 0;
    }
    __syncthreads();
  }
  if (t >= (n_in >> K)) return;
  uint64_t v[W];
  if constexpr (MODE != 2) {
    const uint64_t g = *gamma;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      uint64_t key;
      if constexpr (MODE == 0) {
        const int64_t j = t * W + i;
        key = gl::from_i64(j < n ? keys[j] : (int8_t)0);
      } else {
        key = kl[threadIdx.x * (W + 1) + i];
      }
      v[i] = gl::sub(g, key);
    }
#pragma unroll
    for (int i = 0; i < W; ++i) leaves_out[t * W + i] = v[i];
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) v[i] = in[t * W + i];
  }
  int64_t level_n = n_in >> 1;
  uint64_t* level = out;
#pragma unroll
  for (int lev = 0; lev < K; ++lev) {
    const int cnt = W >> (lev + 1);
#pragma unroll
    for (int i = 0; i < cnt; ++i) v[i] = gl::mul(v[2 * i], v[2 * i + 1]);
#pragma unroll
    for (int i = 0; i < cnt; ++i) level[t * cnt + i] = v[i];
    level += level_n;
    level_n >>= 1;
  }
}

// ------------------------------------------------------------ multiplicities
__global__ __launch_bounds__(256) void counts_zero_kernel(uint32_t* counts, int32_t nb) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < nb) counts[i] = 0;
}

// counts[i] += keys equal to -2^(s-1) + i; counts[2^s] += keys outside the table.
// One LDS histogram per workgroup, then one atomic add per bin.
__global__ __launch_bounds__(256) void counts_kernel(const int8_t* __restrict__ keys, int64_t n, int32_t s,
                                                     uint32_t* __restrict__ counts) {
  __shared__ uint32_t h[257];
  const int T = 1 << s;
  for (int i = threadIdx.x; i <= T; i += 256) h[i] = 0;
  __syncthreads();
  const int lo = -(1 << (s - 1));
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256) {
    const int k = keys[j] - lo;
    atomicAdd(&h[(k >= 0 && k < T) ? k : T], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i <= T; i += 256)
    if (h[i]) atomicAdd(&counts[i], h[i]);
}

// Multiplicities of field keys read as signed integers (a > p/2 as a - p):
// counts[v - lo] for lo <= v < lo + T, counts[T] for the rest. Table indices
// [c0, c0 + win) (the window around v = 0, where a rescaled output's values
// gather) are histogrammed in LDS per workgroup, the others go straight to the
// global bins.
constexpr int CF_WIN = 16384;
__global__ __launch_bounds__(256) void counts_field_kernel(const uint64_t* __restrict__ A, int64_t n, int64_t lo,
                                                           int64_t T, int64_t c0, int32_t win,
                                                           uint32_t* __restrict__ counts) {
  __shared__ uint32_t h[CF_WIN + 1];  // h[win]: keys outside the table
  for (int i = threadIdx.x; i <= win; i += 256) h[i] = 0;
  __syncthreads();
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256) {
    const uint64_t a = A[j];
    const int64_t v = a > (gl::P >> 1) ? -(int64_t)(gl::P - a) : (int64_t)a;
    const int64_t k = v - lo;
    if (k < 0 || k >= T) atomicAdd(&h[win], 1u);
    else if (k >= c0 && k < c0 + win) atomicAdd(&h[k - c0], 1u);
    else atomicAdd(&counts[k], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < win; i += 256)
    if (h[i]) atomicAdd(&counts[c0 + i], h[i]);
  if (threadIdx.x == 0 && h[win]) atomicAdd(&counts[T], h[win]);
}

__global__ void counts_pad_kernel(uint32_t* counts, int32_t s, uint32_t pad) {
  if (threadIdx.x == 0 && pad) counts[1 << (s - 1)] += pad;
}

// --------------------------------------------------------- degree-3 sum-check
// Sum over a workgroup of 4 field values per thread; every thread gets the totals.
template <int NT>
__device__ __forceinline__ void block_sum4(uint64_t (&g)[4], uint64_t* red) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int c = 0; c < 4; ++c) g[c] = fpi::wave_total(g[c]);
  if (lane == 0)
#pragma unroll
    for (int c = 0; c < 4; ++c) red[w * 4 + c] = g[c];
  __syncthreads();
  if (threadIdx.x < 4) {
    uint64_t s = 0;
    for (int i = 0; i < NW; ++i) s = gl::add(s, red[i * 4 + threadIdx.x]);
    red[NW * 4 + threadIdx.x] = s;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) g[c] = red[NW * 4 + c];
}

// adds E_c A_c B_c for c = 0..3 along the line between entries 0 and 1
__device__ __forceinline__ void pair_terms(uint64_t e0, uint64_t e1, uint64_t a0, uint64_t a1, uint64_t b0,
                                           uint64_t b1, uint64_t (&g)[4]) {
  const uint64_t de = gl::sub(e1, e0), da = gl::sub(a1, a0), db = gl::sub(b1, b0);
  uint64_t e = e0, a = a0, b = b0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    g[c] = gl::add(g[c], gl::mul(e, gl::mul(a, b)));
    if (c < 3) {
      e = gl::add(e, de);
      a = gl::add(a, da);
      b = gl::add(b, db);
    }
  }
}

// The same terms as exact 96-bit sums (each product < p), for wave reductions
// that carry no modular corrections.
__device__ __forceinline__ void pair_terms96(uint64_t e0, uint64_t e1, uint64_t a0, uint64_t a1, uint64_t b0,
                                             uint64_t b1, sct::S96 (&g)[4]) {
  const uint64_t de = gl::sub(e1, e0), da = gl::sub(a1, a0), db = gl::sub(b1, b0);
  uint64_t e = e0, a = a0, b = b0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    g[c] = sct::add96(g[c], sct::to96(gl::mul(e, gl::mul(a, b))));
    if (c < 3) {
      e = gl::add(e, de);
      a = gl::add(a, da);
      b = gl::add(b, db);
    }
  }
}

// Round sums of one wave: the 96-bit lane sums added across the wave (DPP),
// reduced once; lane 0 stores them.
__device__ __forceinline__ void wave_round(sct::S96 (&s)[4], uint64_t* rounds) {
  uint64_t g[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) g[c] = sct::lane_value(sct::wave_sum96(s[c]), 63);
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int c = 0; c < 4; ++c) rounds[c] = g[c];
}

__device__ __forceinline__ uint64_t lerp(uint64_t x0, uint64_t x1, uint64_t r) {
  return gl::add(x0, gl::mul(r, gl::sub(x1, x0)));
}

struct Sc3Tables {
  const uint64_t* E;  // E[x]
  const uint64_t* A;  // A[x] (interleaved: V, A[x] = V[2x], B[x] = V[2x+1])
  const uint64_t* B;
  int32_t interleaved;
};

__device__ __forceinline__ void load3(const Sc3Tables& t, int64_t x, uint64_t& e, uint64_t& a, uint64_t& b) {
  e = t.E[x];
  if (t.interleaved) {
    a = t.A[2 * x];
    b = t.A[2 * x + 1];
  } else {
    a = t.A[x];
    b = t.B[x];
  }
}

// Adds the previous launch's per-workgroup partial sums, kp rounds of 4
// values from each of nb workgroups (part[b][kp][4]), into out[kp][4]
// (workgroup-wide).
template <int NT>
__device__ __forceinline__ void add_partials(const uint64_t* __restrict__ part, int nb, int kp,
                                             uint64_t* __restrict__ out, uint64_t* red) {
  for (int rr = 0; rr < kp; ++rr) {
    uint64_t g[4] = {0, 0, 0, 0};
    for (int b = threadIdx.x; b < nb; b += NT)
#pragma unroll
      for (int c = 0; c < 4; ++c) g[c] = gl::add(g[c], part[((int64_t)b * kp + rr) * 4 + c]);
    block_sum4<NT>(g, red);
    if (threadIdx.x < 4) out[rr * 4 + threadIdx.x] = g[threadIdx.x];
  }
}

// Rounds i .. i+k-1 of one instance in one launch (1 <= k <= SC3_KMAX). The
// challenges are inputs, so a thread takes 2^k consecutive entries of E, A, B
// and runs the k rounds on them in registers: the pairs of round i + rr are
// adjacent entries after the folds by r_i .. r_{i+rr-1}, so they never leave
// the thread. It adds its pairs' terms to the k round sums and writes its
// entry of the tables folded by all k challenges (out, out + buf, out + 2 buf:
// chunks = size / 2^k entries). Per-workgroup partial sums go to
// part[block][k][4]; the instance's first workgroup first adds the previous
// launch's partials (prev, nb_prev workgroups of k_prev rounds) into
// prev_round.
constexpr int SC3_KMAX = 3;              // rounds per wide launch
constexpr int SC3_CW = 1 << SC3_KMAX;    // entries per thread

struct Sc3RoundJob {
  Sc3Tables in;
  uint64_t* out;
  int64_t buf;
  const uint64_t* r;  // r_i .. r_{i+k-1}
  int64_t chunks;
  uint64_t* part;
  const uint64_t* prev;
  uint64_t* prev_round;
  int32_t k, k_prev, nb_prev;
  int32_t block_start, nb;  // the instance's workgroups in the launch
};

constexpr int SC3_RJ = 12;  // instances per wide-round launch
struct Sc3RoundList {
  Sc3RoundJob j[SC3_RJ];
  int32_t count;
};

__global__ __launch_bounds__(LK_T) void sc3_round_kernel(Sc3RoundList jl) {
  __shared__ uint64_t red[(LK_T / 64) * 4 + 4];
  int q = 0;
#pragma unroll 1
  for (int x = 1; x < jl.count; ++x)
    if (jl.j[x].block_start <= (int)blockIdx.x) q = x;
  const Sc3RoundJob& j = jl.j[q];
  const int blk = (int)blockIdx.x - j.block_start;
  if (blk == 0 && j.nb_prev > 0) add_partials<LK_T>(j.prev, j.nb_prev, j.k_prev, j.prev_round, red);
  const int K = j.k, C = 1 << K;
  uint64_t rk[SC3_KMAX], g[SC3_KMAX][4];
#pragma unroll
  for (int rr = 0; rr < SC3_KMAX; ++rr) {
    rk[rr] = rr < K ? j.r[rr] : 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) g[rr][c] = 0;
  }
  const Sc3Tables in = j.in;
  uint64_t* __restrict__ Eo = j.out;
  uint64_t* __restrict__ Ao = j.out + j.buf;
  uint64_t* __restrict__ Bo = j.out + 2 * j.buf;
  const int64_t chunks = j.chunks, stride = (int64_t)j.nb * LK_T;
  for (int64_t t = (int64_t)blk * LK_T + threadIdx.x; t < chunks; t += stride) {
    // The chunk's C entries are taken a pair at a time and reduced like a
    // binary counter: a pair's round-0 terms are added and its fold is an
    // entry of level 1; two level-l entries make a pair of round l, whose
    // fold is an entry of level l+1. One pending entry per level stays live.
    // The whole chunk is loaded first, in one burst: a lane's entries are
    // consecutive, so each cache line is read by the loads of a few lanes
    // issued together, before L2 can evict it.
    uint64_t ve[SC3_CW], va[SC3_CW], vb[SC3_CW];
#pragma unroll
    for (int x = 0; x < SC3_CW; ++x) {
      ve[x] = va[x] = vb[x] = 0;
      if (x < C) load3(in, t * C + x, ve[x], va[x], vb[x]);
    }
    uint64_t se[SC3_KMAX + 1], sa[SC3_KMAX + 1], sb[SC3_KMAX + 1];
#pragma unroll
    for (int l = 0; l <= SC3_KMAX; ++l) se[l] = sa[l] = sb[l] = 0;
#pragma unroll
    for (int p = 0; p < SC3_CW / 2; ++p) {
      if (p < (C >> 1)) {
        const uint64_t e0 = ve[2 * p], a0 = va[2 * p], b0 = vb[2 * p];
        const uint64_t e1 = ve[2 * p + 1], a1 = va[2 * p + 1], b1 = vb[2 * p + 1];
        pair_terms(e0, e1, a0, a1, b0, b1, g[0]);
        uint64_t ce = lerp(e0, e1, rk[0]), ca = lerp(a0, a1, rk[0]), cb = lerp(b0, b1, rk[0]);
        int l = 1;
#pragma unroll
        for (; l < SC3_KMAX; ++l) {
          if (((p + 1) & ((1 << l) - 1)) != 0) break;  // the level-l entry waits for its partner
          pair_terms(se[l], ce, sa[l], ca, sb[l], cb, g[l]);
          ce = lerp(se[l], ce, rk[l]);
          ca = lerp(sa[l], ca, rk[l]);
          cb = lerp(sb[l], cb, rk[l]);
        }
        se[l] = ce;
        sa[l] = ca;
        sb[l] = cb;
      }
    }
    // p < C/2 = 2^(K-1) never completes a level past K-1, so the chunk's entry
    // folded by all K challenges is the pending entry of level K
    uint64_t oe = se[1], oa = sa[1], ob = sb[1];
#pragma unroll
    for (int l = 2; l <= SC3_KMAX; ++l)
      if (K == l) {
        oe = se[l];
        oa = sa[l];
        ob = sb[l];
      }
    Eo[t] = oe;
    Ao[t] = oa;
    Bo[t] = ob;
  }
#pragma unroll
  for (int rr = 0; rr < SC3_KMAX; ++rr) {
    if (rr < K) {
      block_sum4<LK_T>(g[rr], red);
      if (threadIdx.x < 4) j.part[((int64_t)blk * K + rr) * 4 + threadIdx.x] = g[rr][threadIdx.x];
    }
  }
}

// The last rounds of one instance in one workgroup of SC3_TT = 256 threads.
// The first adds the previous wide launch's partials (nb_prev > 0, k_prev
// rounds) into rounds[i0-k_prev .. i0-1]. Then `in` (size_in entries, folded by r[i0-1] first when fold;
// S <= 2048 entries after that) is held as 8 consecutive entries per thread,
// and rounds i0 .. m-1 run:
//  - while a thread holds 2 or more entries, pairs are inside the thread and
//    only the round sums cross threads (LDS, two barriers);
//  - the <= 256 left go to wave 0, up to 4 per lane, pairs inside the lane,
//    round sums by DPP within the wave, no barriers;
//  - with one entry per lane (<= 64), partners are lane distance 1, 2, 4 ...
//    apart (shuffles), round sums within the wave.
// r_i is applied only after g_i is complete. finals = E, A, B at the point.
struct Sc3TailJob {
  Sc3Tables in;
  int64_t size_in;
  const uint64_t* r;
  uint64_t* rounds;
  uint64_t* finals;
  const uint64_t* prev;
  int32_t fold, i0, m, nb_prev, k_prev;
};

constexpr int SC3_TJ = 24;  // instances per tail launch, one workgroup each
struct Sc3TailList {
  Sc3TailJob j[SC3_TJ];
  int32_t count;
};

constexpr int TQ = SC3_TAIL / SC3_TT;  // entries per thread in the first stage (8)

__global__ __launch_bounds__(SC3_TT) void sc3_tail_kernel(Sc3TailList jl) {
  __shared__ uint64_t red[(SC3_TT / 64) * 4 + 4];
  __shared__ uint64_t xE[SC3_TT], xA[SC3_TT], xB[SC3_TT];
  __shared__ uint64_t rs[FP_MAX_N];
  const Sc3TailJob& j = jl.j[blockIdx.x];
  const Sc3Tables in = j.in;
  const int32_t fold = j.fold, i0 = j.i0, m = j.m;
  const uint64_t* __restrict__ r = j.r;
  uint64_t* __restrict__ rounds = j.rounds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t g[4];
  if (j.nb_prev > 0) add_partials<SC3_TT>(j.prev, j.nb_prev, j.k_prev, rounds + (int64_t)(i0 - j.k_prev) * 4, red);
  if (tid < m - i0) rs[tid] = r[i0 + tid];
  const int64_t S = fold ? j.size_in / 2 : j.size_in;  // entries after the first fold
  const uint64_t r0 = fold ? r[i0 - 1] : 0;
  // stage 1: thread t holds entries t q .. t q + q - 1, q = max(1, S / 256)
  int q = S >= SC3_TT ? (int)(S / SC3_TT) : 1;
  uint64_t e[TQ], a[TQ], b[TQ];
#pragma unroll
  for (int k = 0; k < TQ; ++k) {
    e[k] = a[k] = b[k] = 0;
    const int64_t x = (int64_t)tid * q + k;
    if (k < q && x < S) {
      if (fold) {
        uint64_t e0, a0, b0, e1, a1, b1;
        load3(in, 2 * x, e0, a0, b0);
        load3(in, 2 * x + 1, e1, a1, b1);
        e[k] = lerp(e0, e1, r0);
        a[k] = lerp(a0, a1, r0);
        b[k] = lerp(b0, b1, r0);
      } else {
        load3(in, x, e[k], a[k], b[k]);
      }
    }
  }
  __syncthreads();  // rs visible
  int i = i0;
#pragma unroll
  for (int cnt = TQ; cnt >= 2; cnt >>= 1) {
    if (q == cnt) {
#pragma unroll
      for (int c = 0; c < 4; ++c) g[c] = 0;
#pragma unroll
      for (int p = 0; p < cnt / 2; ++p) pair_terms(e[2 * p], e[2 * p + 1], a[2 * p], a[2 * p + 1], b[2 * p], b[2 * p + 1], g);
      block_sum4<SC3_TT>(g, red);
      if (tid < 4) rounds[(int64_t)i * 4 + tid] = g[tid];
      const uint64_t ri = rs[i - i0];
#pragma unroll
      for (int p = 0; p < cnt / 2; ++p) {
        e[p] = lerp(e[2 * p], e[2 * p + 1], ri);
        a[p] = lerp(a[2 * p], a[2 * p + 1], ri);
        b[p] = lerp(b[2 * p], b[2 * p + 1], ri);
      }
      ++i;
      q = cnt / 2;
    }
  }
  // stage 2: n2 = min(S, 256) entries, one per thread -> wave 0, q2 per lane
  const int n2 = S < SC3_TT ? (int)S : SC3_TT;
  xE[tid] = e[0];
  xA[tid] = a[0];
  xB[tid] = b[0];
  __syncthreads();
  if (wave != 0) return;
  int q2 = n2 >= 64 ? n2 / 64 : 1;
  uint64_t e2[4], a2[4], b2[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int x = lane * q2 + k;
    const bool ok = k < q2 && x < n2;
    e2[k] = ok ? xE[x] : 0;
    a2[k] = ok ? xA[x] : 0;
    b2[k] = ok ? xB[x] : 0;
  }
#pragma unroll
  for (int cnt = 4; cnt >= 2; cnt >>= 1) {
    if (q2 == cnt) {
      sct::S96 s96[4] = {};
#pragma unroll
      for (int p = 0; p < cnt / 2; ++p)
        pair_terms96(e2[2 * p], e2[2 * p + 1], a2[2 * p], a2[2 * p + 1], b2[2 * p], b2[2 * p + 1], s96);
      wave_round(s96, rounds + (int64_t)i * 4);
      const uint64_t ri = rs[i - i0];
#pragma unroll
      for (int p = 0; p < cnt / 2; ++p) {
        e2[p] = lerp(e2[2 * p], e2[2 * p + 1], ri);
        a2[p] = lerp(a2[2 * p], a2[2 * p + 1], ri);
        b2[p] = lerp(b2[2 * p], b2[2 * p + 1], ri);
      }
      ++i;
      q2 = cnt / 2;
    }
  }
  // stage 3: entry x at lane x * dist, pairs dist apart
  uint64_t ev = e2[0], av = a2[0], bv = b2[0];
  for (int dist = 1; i < m; dist <<= 1, ++i) {
    const uint64_t e1 = fpi::shfl_down_u64(ev, dist), a1 = fpi::shfl_down_u64(av, dist), b1 = fpi::shfl_down_u64(bv, dist);
    const bool lead = (lane & (2 * dist - 1)) == 0;
    sct::S96 s96[4] = {};
    if (lead) pair_terms96(ev, e1, av, a1, bv, b1, s96);
    wave_round(s96, rounds + (int64_t)i * 4);
    const uint64_t ri = rs[i - i0];
    if (lead) {
      ev = lerp(ev, e1, ri);
      av = lerp(av, a1, ri);
      bv = lerp(bv, b1, ri);
    }
  }
  if (lane == 0) {
    j.finals[0] = ev;
    j.finals[1] = av;
    j.finals[2] = bv;
  }
}

struct Sc3Layout {
  size_t buf;  // entries of each folded table buffer
  int nb;      // workgroups of the wide rounds
  size_t bytes;
};

Sc3Layout sc3_layout(int32_t m) {
  Sc3Layout l{};
  const int64_t S = (int64_t)1 << m;
  l.buf = S > SC3_TAIL ? (size_t)(S / 2) : 0;
  const int64_t pairs = S / 2;  // bounds the threads of any wide launch
  l.nb = (int)std::min<int64_t>(SC3_MAXB, std::max<int64_t>(1, (pairs + LK_T - 1) / LK_T));
  l.bytes = 6 * l.buf * 8 + 2 * fpi::align_up((size_t)l.nb * SC3_KMAX * 4 * 8, 256);
  return l;
}

// One degree-3 sum-check: sum_x E[x] V[2x] V[2x+1] over x < 2^m, challenges
// r[0..m), ws of sc3_layout(m).bytes (its own; instances share nothing).
struct Sc3Inst {
  const uint64_t* E;
  const uint64_t* V;
  int32_t m;
  const uint64_t* r;
  uint64_t* rounds;
  uint64_t* finals;
  void* ws;
};

// Where an instance stands between launches.
struct Sc3State {
  Sc3Tables in;
  int64_t size;  // entries of `in` (folded by every challenge so far)
  int i;         // next round
  int cur, lc;   // table buffer and partials buffer to write next
  int nb_prev, k_prev, nb;
  const uint64_t* last;  // the last launch's partials
  uint64_t* bufs;
  size_t buf;
  uint64_t* parts[2];
};

// Enqueues `count` independent instances (m <= FP_MAX_N - 1 each). Since
// their challenges are inputs, each wide launch runs up to SC3_KMAX rounds of
// every instance whose tables still exceed the tail's 2048 entries, and one
// launch runs all the tails, one workgroup per instance.
int sc3_enqueue_many(int count, const Sc3Inst* inst, hipStream_t st) {
  Sc3State s[FP_MAX_N];
  if (count < 0 || count > FP_MAX_N) return fpi::fail(FP_EARG, "sc3: %d instances", count);
  for (int k = 0; k < count; ++k) {
    const Sc3Layout l = sc3_layout(inst[k].m);
    Sc3State& t = s[k];
    t.in = Sc3Tables{inst[k].E, inst[k].V, nullptr, 1};
    t.size = (int64_t)1 << inst[k].m;
    t.i = t.cur = t.lc = t.nb_prev = t.k_prev = 0;
    t.nb = l.nb;
    t.last = nullptr;
    t.bufs = (uint64_t*)inst[k].ws;
    t.buf = l.buf;
    t.parts[0] = t.bufs + 6 * l.buf;
    t.parts[1] = t.parts[0] + fpi::align_up((size_t)l.nb * SC3_KMAX * 4 * 8, 256) / 8;
  }
  for (;;) {
    Sc3RoundList jl{};
    int64_t blocks = 0;
    bool any = false;
    for (int k = 0; k <= count; ++k) {
      const bool wide = k < count && s[k].size > SC3_TAIL;
      if ((k == count || (wide && jl.count == SC3_RJ)) && jl.count > 0) {
        hipLaunchKernelGGL(sc3_round_kernel, dim3((unsigned)blocks), dim3(LK_T), 0, st, jl);
        const int rc = fpi::check_launch("sc3_round_kernel");
        if (rc) return rc;
        jl = Sc3RoundList{};
        blocks = 0;
      }
      if (!wide) continue;
      any = true;
      Sc3State& t = s[k];
      int left = 0;  // rounds until the tables fit the tail
      while ((t.size >> left) > SC3_TAIL) ++left;
      const int kk = std::min(left, SC3_KMAX);
      const int64_t chunks = t.size >> kk;
      const int nb = (int)std::min<int64_t>(t.nb, (chunks + LK_T - 1) / LK_T);
      uint64_t* out = t.bufs + (size_t)(3 * t.cur) * t.buf;
      uint64_t* part = t.parts[t.lc & 1];
      jl.j[jl.count++] = Sc3RoundJob{t.in, out, (int64_t)t.buf, inst[k].r + t.i, chunks, part, t.last,
                                     inst[k].rounds + (size_t)(t.i - t.k_prev) * 4, kk, t.k_prev, t.nb_prev,
                                     (int32_t)blocks, nb};
      blocks += nb;
      t.in = Sc3Tables{out, out + t.buf, out + 2 * t.buf, 0};
      t.size = chunks;
      t.i += kk;
      t.cur ^= 1;
      t.lc ^= 1;
      t.last = part;
      t.nb_prev = nb;
      t.k_prev = kk;
    }
    if (!any) break;
  }
  Sc3TailList tl{};
  for (int k = 0; k <= count; ++k) {
    if ((k == count || tl.count == SC3_TJ) && tl.count > 0) {
      hipLaunchKernelGGL(sc3_tail_kernel, dim3((unsigned)tl.count), dim3(SC3_TT), 0, st, tl);
      const int rc = fpi::check_launch("sc3_tail_kernel");
      if (rc) return rc;
      tl = Sc3TailList{};
    }
    if (k == count) break;
    const Sc3State& t = s[k];
    tl.j[tl.count++] = Sc3TailJob{t.in, t.size, inst[k].r, inst[k].rounds, inst[k].finals, t.last, 0, t.i,
                                  inst[k].m, t.nb_prev, t.k_prev};
  }
  return FP_OK;
}

int64_t level_offset(int32_t L, int32_t d) { return ((int64_t)2 << L) - ((int64_t)2 << (L - d)); }

}  // namespace

static int tree_launch(int mode, const int8_t* keys, int64_t n, PairKeys pk, int32_t L, const fp_elem* gamma,
                       fp_elem* tree, hipStream_t stream) {
  // leaves, with up to LK_K levels above them
  int64_t n_in = (int64_t)1 << L;
  int k = L < LK_K ? L : LK_K;
  {
    const int64_t threads = n_in >> k;
    const dim3 grid((unsigned)((threads + LK_T - 1) / LK_T));
    uint64_t* out = tree + n_in;
#define LEAF_LAUNCH(KK)                                                                                        \
  if (mode == 0)                                                                                               \
    hipLaunchKernelGGL((tree_kernel<KK, 0>), grid, dim3(LK_T), 0, stream, keys, n, pk, gamma, nullptr, n_in, tree, out); \
  else                                                                                                         \
    hipLaunchKernelGGL((tree_kernel<KK, 1>), grid, dim3(LK_T), 0, stream, keys, n, pk, gamma, nullptr, n_in, tree, out)
    switch (k) {
      case 0: LEAF_LAUNCH(0); break;
      case 1: LEAF_LAUNCH(1); break;
      case 2: LEAF_LAUNCH(2); break;
      case 3: LEAF_LAUNCH(3); break;
      default: LEAF_LAUNCH(4); break;
    }
#undef LEAF_LAUNCH
    const int rc = fpi::check_launch("tree_kernel");
    if (rc) return rc;
  }
  int32_t d = k;  // levels written so far above the leaves
  while (d < L) {
    k = (L - d) < LK_K ? (L - d) : LK_K;
    const int64_t w = (int64_t)1 << (L - d);  // entries of level d
    const uint64_t* in = tree + level_offset(L, d);
    uint64_t* out = tree + level_offset(L, d + 1);
    const dim3 grid((unsigned)(((w >> k) + LK_T - 1) / LK_T));
    const PairKeys none{};
    switch (k) {
      case 1: hipLaunchKernelGGL((tree_kernel<1, 2>), grid, dim3(LK_T), 0, stream, nullptr, 0, none, nullptr, in, w, nullptr, out); break;
      case 2: hipLaunchKernelGGL((tree_kernel<2, 2>), grid, dim3(LK_T), 0, stream, nullptr, 0, none, nullptr, in, w, nullptr, out); break;
      case 3: hipLaunchKernelGGL((tree_kernel<3, 2>), grid, dim3(LK_T), 0, stream, nullptr, 0, none, nullptr, in, w, nullptr, out); break;
      default: hipLaunchKernelGGL((tree_kernel<4, 2>), grid, dim3(LK_T), 0, stream, nullptr, 0, none, nullptr, in, w, nullptr, out); break;
    }
    const int rc = fpi::check_launch("tree_kernel");
    if (rc) return rc;
    d += k;
  }
  return fpi::ok();
}

extern "C" int fp_lookup_tree(const int8_t* keys, int64_t n, int32_t L, const fp_elem* gamma, fp_elem* tree,
                              hipStream_t stream) {
  const char* fn = "fp_lookup_tree";
  if (L < 0 || L > FP_MAX_N) return fpi::fail(FP_ESHAPE, "%s: L=%d outside [0, %d]", fn, L, FP_MAX_N);
  if (n < 0 || n > ((int64_t)1 << L)) return fpi::fail(FP_ESHAPE, "%s: n=%lld outside [0, 2^L]", fn, (long long)n);
  if (!gamma || !tree || (n > 0 && !keys)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  return tree_launch(0, keys, n, PairKeys{}, L, gamma, tree, stream);
}

extern "C" int fp_lookup_tree_pairs(const fp_elem* A, const fp_elem* B, int64_t n, uint64_t scale, uint64_t offset,
                                    int32_t L, const fp_elem* gamma, fp_elem* tree, hipStream_t stream) {
  const char* fn = "fp_lookup_tree_pairs";
  if (L < 0 || L > FP_MAX_N) return fpi::fail(FP_ESHAPE, "%s: L=%d outside [0, %d]", fn, L, FP_MAX_N);
  if (n < 0 || n > ((int64_t)1 << L)) return fpi::fail(FP_ESHAPE, "%s: n=%lld outside [0, 2^L]", fn, (long long)n);
  if (!gamma || !tree || (n > 0 && (!A || !B))) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  const PairKeys pk{A, B, scale % gl::P, offset % gl::P};
  return tree_launch(1, nullptr, n, pk, L, gamma, tree, stream);
}

extern "C" int fp_lookup_counts_field(const fp_elem* A, int64_t n, int64_t lo, int32_t bits, uint32_t* counts,
                                      hipStream_t stream) {
  const char* fn = "fp_lookup_counts_field";
  if (bits < 1 || bits > 24) return fpi::fail(FP_ERANGE, "%s: bits=%d outside [1, 24]", fn, bits);
  if (n < 0 || n > ((int64_t)1 << FP_MAX_N) || lo < -(1LL << 40) || lo > (1LL << 40))
    return fpi::fail(FP_ESHAPE, "%s: n=%lld, lo=%lld", fn, (long long)n, (long long)lo);
  if (!counts || (n > 0 && !A)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  const int64_t T = (int64_t)1 << bits;
  const int nbins = (int)(T + 1);
  hipLaunchKernelGGL(counts_zero_kernel, dim3((nbins + 255) / 256), dim3(256), 0, stream, counts, nbins);
  int rc = fpi::check_launch("counts_zero_kernel");
  if (rc) return rc;
  if (n == 0) return fpi::ok();
  const int32_t win = (int32_t)std::min<int64_t>(T, CF_WIN);
  const int64_t c0 = std::min<int64_t>(std::max<int64_t>(-lo - win / 2, 0), T - win);
  const int64_t blocks = std::min<int64_t>(1024, (n + 255) / 256);
  hipLaunchKernelGGL(counts_field_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, A, n, lo, T, c0, win, counts);
  rc = fpi::check_launch("counts_field_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" int fp_lookup_counts(const int8_t* keys, int64_t n, int32_t L, int32_t s, uint32_t* counts,
                                hipStream_t stream) {
  const char* fn = "fp_lookup_counts";
  if (s < 1 || s > 8) return fpi::fail(FP_ERANGE, "%s: s=%d outside [1, 8]", fn, s);
  if (L < 0 || L > FP_MAX_N || n < 0 || n > ((int64_t)1 << L))
    return fpi::fail(FP_ESHAPE, "%s: n=%lld, L=%d", fn, (long long)n, L);
  if (!counts || (n > 0 && !keys)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  const int nbins = (1 << s) + 1;
  hipLaunchKernelGGL(counts_zero_kernel, dim3((nbins + 255) / 256), dim3(256), 0, stream, counts, nbins);
  int rc = fpi::check_launch("counts_zero_kernel");
  if (rc) return rc;
  if (n > 0) {
    const int64_t blocks = std::min<int64_t>(1024, (n + 255) / 256);
    hipLaunchKernelGGL(counts_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, keys, n, s, counts);
    rc = fpi::check_launch("counts_kernel");
    if (rc) return rc;
  }
  const int64_t pad = ((int64_t)1 << L) - n;
  if (pad > 0xFFFFFFFFll) return fpi::fail(FP_ESHAPE, "%s: padding count exceeds 32 bits", fn);
  hipLaunchKernelGGL(counts_pad_kernel, dim3(1), dim3(64), 0, stream, counts, s, (uint32_t)pad);
  rc = fpi::check_launch("counts_pad_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" size_t fp_sumcheck3_workspace(int32_t m) {
  if (m < 0 || m >= FP_MAX_N) return 0;
  return sc3_layout(m).bytes;
}

extern "C" int fp_sumcheck3_prove(const fp_elem* E, const fp_elem* V, int32_t m, const fp_elem* r, fp_elem* rounds,
                                  fp_elem* finals, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "fp_sumcheck3_prove";
  if (m < 0 || m >= FP_MAX_N) return fpi::fail(FP_ESHAPE, "%s: m=%d outside [0, %d)", fn, m, FP_MAX_N);
  if (!E || !V || !finals || (m > 0 && (!r || !rounds))) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  const Sc3Layout l = sc3_layout(m);
  if (!ws || ws_bytes < l.bytes) return fpi::fail(FP_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, l.bytes);
  const Sc3Inst one{E, V, m, r, rounds, finals, ws};
  const int rc = sc3_enqueue_many(1, &one, stream);
  return rc ? rc : fpi::ok();
}

// Workspace: every level's eq table (the level with m variables at entry
// 2^m - 1, 2^L - 1 entries in all), then each level's sum-check tables (its
// own, so that the levels run side by side).
size_t lookup_sc_bytes(int32_t L) {
  size_t b = 0;
  for (int32_t m = 0; m < L; ++m) b += fpi::align_up(sc3_layout(m).bytes, 256);
  return b;
}

extern "C" size_t fp_lookup_prove_workspace(int32_t L) {
  if (L < 1 || L > FP_MAX_N) return 0;
  return fpi::align_up(((size_t)1 << L) * 8, 256) + lookup_sc_bytes(L);
}

extern "C" int fp_lookup_prove(const fp_elem* tree, int32_t L, const fp_elem* chal, fp_elem* rounds, fp_elem* finals,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "fp_lookup_prove";
  if (L < 1 || L > FP_MAX_N) return fpi::fail(FP_ESHAPE, "%s: L=%d outside [1, %d]", fn, L, FP_MAX_N);
  if (!tree || !chal || !finals || (L > 1 && !rounds)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  const size_t need = fp_lookup_prove_workspace(L);
  if (!ws || ws_bytes < need) return fpi::fail(FP_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  if (((uintptr_t)ws) & 255) return fpi::fail(FP_EARG, "%s: workspace must be 256-byte aligned", fn);
  uint64_t* E = (uint64_t*)ws;
  char* sc_ws = (char*)ws + fpi::align_up(((size_t)1 << L) * 8, 256);
  // The claim on level d+1 sits at z = level d+1's challenges (empty at the
  // root). The challenges are inputs, so no level waits for another: every
  // level's eq table is built up front in one batched launch (level d's
  // table: m = L-1-d variables, at E + 2^m - 1), and the levels' sum-checks
  // run side by side.
  fp_eq_desc eq[FP_MAX_N];
  Sc3Inst inst[FP_MAX_N];
  int64_t round_off = 0;
  for (int32_t d = L - 1; d >= 0; --d) {
    const int32_t m = L - 1 - d;
    const int64_t off_next = (int64_t)(L - 2 - d) * (L - 1 - d) / 2;  // start of level d+1's challenges
    const int64_t off = (int64_t)(L - 1 - d) * (L - d) / 2;           // [lambda_d, rho_1 .. rho_m]
    eq[m] = fp_eq_desc{m ? chal + off_next : nullptr, m, E + ((int64_t)1 << m) - 1};
    inst[m] = Sc3Inst{E + ((int64_t)1 << m) - 1, tree + level_offset(L, d), m, chal + off + 1,
                      rounds + round_off * 4, finals + (int64_t)m * 3, sc_ws};
    sc_ws += fpi::align_up(sc3_layout(m).bytes, 256);
    round_off += m;
  }
  int rc = fpi::launch_eq_list(L, eq, stream);
  if (rc) return rc;
  rc = sc3_enqueue_many(L, inst, stream);
  return rc ? rc : fpi::ok();
}
