// sc_tail.hpp - the single-workgroup sum-check tail, shared by the sum-check
// launches and by the witness launch that overlaps a finished layer's
// sum-check with the next layer's GEMM.
//
// "How fast can FlashProve go", §2: sum-check reduces each matmul to claims
// about committed tables. Round i sends g_i at 0, 1, 2 with
//     g_i(c) = sum_j rho_j sum_q A_j,c[q] B_j,c[q],  A_c[q] = A[2q] + c (A[2q+1] - A[2q]),
// then binds A[q] <- A[2q] + r_i (A[2q+1] - A[2q]) (B likewise).
#pragma once
#include "common.hpp"
#include "gl.hpp"

namespace sct {

constexpr int SC_MAX_PAIRS = 16;

struct Tabs {
  const fp_elem* A[SC_MAX_PAIRS];
  const fp_elem* B[SC_MAX_PAIRS];
};


// An exact sum of field values, w0 + 2^32 w1 + 2^64 w2 (below 2^96).
struct S96 {
  uint32_t w0, w1, w2;
};

__device__ __forceinline__ S96 to96(uint64_t v) { return S96{(uint32_t)v, (uint32_t)(v >> 32), 0u}; }

__device__ __forceinline__ S96 add96(S96 a, S96 b) {
  unsigned int c0, c1, c2;
  S96 r;
  r.w0 = __builtin_addc(a.w0, b.w0, 0u, &c0);
  r.w1 = __builtin_addc(a.w1, b.w1, c0, &c1);
  r.w2 = __builtin_addc(a.w2, b.w2, c1, &c2);
  return r;
}

// DPP move of all three words; lanes of rows outside RM (and lanes without a
// source) read 0.
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ S96 dpp96(S96 a) {
  return S96{(uint32_t)__builtin_amdgcn_update_dpp(0, (int)a.w0, CTRL, RM, 0xF, false),
             (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a.w1, CTRL, RM, 0xF, false),
             (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a.w2, CTRL, RM, 0xF, false)};
}

__device__ __forceinline__ uint64_t reduce96(S96 v) {
  return gl::reduce128(((uint64_t)v.w1 << 32) | v.w0, v.w2);
}

// Terms of g(0), g(1), g(2) for one pair of entries, added exactly into 96-bit
// sums. Returns the differences A1 - A0 and B1 - B0, which binding reuses:
// A(r) = A0 + r (A1 - A0), and A at 2 is A1 + (A1 - A0).
__device__ __forceinline__ void round_terms96(uint64_t a0, uint64_t a1, uint64_t b0, uint64_t b1, S96& g0, S96& g1,
                                              S96& g2, uint64_t& da, uint64_t& db) {
  da = gl::sub(a1, a0);
  db = gl::sub(b1, b0);
  g0 = add96(g0, to96(gl::mul(a0, b0)));
  g1 = add96(g1, to96(gl::mul(a1, b1)));
  g2 = add96(g2, to96(gl::mul(gl::add(a1, da), gl::add(b1, db))));
}


// Reduce the previous round's partials: g_{i-1} -> rounds, and the claim.
__device__ __forceinline__ void finish_prev(const fp_elem* __restrict__ part, int nparts, fp_elem* rounds, int iprev,
                                            fp_elem* claim0) {
  uint64_t s0 = 0, s1 = 0, s2 = 0;
  for (int k = 0; k < nparts; ++k) {
    s0 = gl::add(s0, part[3 * k]);
    s1 = gl::add(s1, part[3 * k + 1]);
    s2 = gl::add(s2, part[3 * k + 2]);
  }
  rounds[3 * iprev] = s0;
  rounds[3 * iprev + 1] = s1;
  rounds[3 * iprev + 2] = s2;
  if (iprev == 0 && claim0) claim0[0] = gl::add(s0, s1);
}


// ---- tail ------------------------------------------------------------------
// One workgroup of ST threads (256 or 512) finishes rounds i0..n-1 of one
// instance.
//   i0 == 0: start from the caller's tables (2^n entries per pair).
//   i0 > 0 : reduce the partials of g_{i0-1}, then fold T_{i0-1} with r_{i0-1}
//            while loading.
// Pairs are padded to a power of two VP of "virtual" pairs (zero tables,
// weight 0) so that every slice lies inside one pair. With mt virtual entries:
//   Stage A (mt >= 2 ST, all waves): thread t holds entries [t L, (t+1) L) of
//     A and B in registers (L = mt / ST); while L >= 2 the pairs (2q, 2q+1)
//     of a round lie in the slice, binding a variable moves no data, and only
//     the three round sums cross threads (one barrier per round).
//   Stage B (wave 0 alone, no barriers): the <= ST remaining entries are
//     re-sliced through LDS to L = mt / 64 entries per lane; rounds as in A.
//   Stage C (wave 0, one entry per lane): partners at lane distance 1, 2, 4, ...
// Round sums are carried as exact 96-bit integers while they cross lanes (DPP
// row butterflies, then row broadcasts into lane 63) and reduced mod p once;
// across waves they meet in LDS, and every wave completes g_i before it
// applies r_i. The challenges are inputs and are staged in LDS at the start.
// Multi-instance mode: instance b uses A + b 2^n, B + b 2^n, r + b n,
// rounds + 3 b n, finals + 2 b, claim0 + b.
constexpr int SLMAX = 16;   // register entries per thread and table
struct TailArgs {
  Tabs user;
  const fp_elem* src;  // ws buffer with T_{i0-1} when i0 >= 2
  const fp_elem* rho;
  const fp_elem* r;
  const fp_elem* prev_part;
  fp_elem* rounds;
  fp_elem* finals;
  fp_elem* claim0;
  int32_t i0, n, n_pairs, nprev;
  int32_t multi;
};

constexpr int DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

// Sum over the 64 lanes (all active); the total lands in lane 63.
__device__ __forceinline__ S96 wave_sum96(S96 v) {
  v = add96(v, dpp96<fpi::DPP_XOR1>(v));
  v = add96(v, dpp96<fpi::DPP_XOR2>(v));
  v = add96(v, dpp96<fpi::DPP_HALF_MIRROR>(v));
  v = add96(v, dpp96<fpi::DPP_MIRROR>(v));            // row sums in every lane
  v = add96(v, dpp96<DPP_ROW_BCAST15, 0xA>(v));       // rows 1, 3 += rows 0, 2
  v = add96(v, dpp96<DPP_ROW_BCAST31, 0xC>(v));       // rows 2, 3 += rows 0 + 1
  return v;
}

__device__ __forceinline__ uint64_t lane_value(S96 v, int lane) {
  const uint32_t w0 = (uint32_t)__builtin_amdgcn_readlane((int)v.w0, lane);
  const uint32_t w1 = (uint32_t)__builtin_amdgcn_readlane((int)v.w1, lane);
  const uint32_t w2 = (uint32_t)__builtin_amdgcn_readlane((int)v.w2, lane);
  return gl::reduce128(((uint64_t)w1 << 32) | w0, w2);
}

// Round sums of one wave (stages B and C): canonical g values in every lane.
__device__ __forceinline__ void wave_round(S96 s0, S96 s1, S96 s2, uint64_t& g0, uint64_t& g1, uint64_t& g2) {
  const S96 a = wave_sum96(s0), b = wave_sum96(s1), c = wave_sum96(s2);
  g0 = lane_value(a, 63);
  g1 = lane_value(b, 63);
  g2 = lane_value(c, 63);
}

// Round sums of the workgroup (stage A): each wave's total goes to LDS
// (double-buffered by round parity), one barrier, and every wave adds the SW
// (<= 8) wave totals itself. Canonical g values in every lane.
template <int SW>
__device__ __forceinline__ void block_round(S96 s0, S96 s1, S96 s2, uint64_t& g0, uint64_t& g1, uint64_t& g2, S96* red,
                                            int par) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const S96 a = wave_sum96(s0), b = wave_sum96(s1), c = wave_sum96(s2);
  S96* slot = red + (par * SW) * 3;
  if (lane == 63) {
    slot[3 * wave] = a;
    slot[3 * wave + 1] = b;
    slot[3 * wave + 2] = c;
  }
  __syncthreads();
  S96 x{0, 0, 0}, y{0, 0, 0}, z{0, 0, 0};
  if (lane < SW) {
    x = slot[3 * lane];
    y = slot[3 * lane + 1];
    z = slot[3 * lane + 2];
  }
  // up to 8 values in lanes 0..7: two quad butterflies and a half-row mirror
  x = add96(x, dpp96<fpi::DPP_XOR1>(x));
  y = add96(y, dpp96<fpi::DPP_XOR1>(y));
  z = add96(z, dpp96<fpi::DPP_XOR1>(z));
  x = add96(x, dpp96<fpi::DPP_XOR2>(x));
  y = add96(y, dpp96<fpi::DPP_XOR2>(y));
  z = add96(z, dpp96<fpi::DPP_XOR2>(z));
  x = add96(x, dpp96<fpi::DPP_HALF_MIRROR>(x));
  y = add96(y, dpp96<fpi::DPP_HALF_MIRROR>(y));
  z = add96(z, dpp96<fpi::DPP_HALF_MIRROR>(z));
  g0 = lane_value(x, 0);
  g1 = lane_value(y, 0);
  g2 = lane_value(z, 0);
}

__device__ __forceinline__ void emit_round(fp_elem* rounds, fp_elem* claim0, int i, uint64_t g0, uint64_t g1,
                                           uint64_t g2) {
  rounds[3 * i] = g0;
  rounds[3 * i + 1] = g1;
  rounds[3 * i + 2] = g2;
  if (i == 0 && claim0) claim0[0] = gl::add(g0, g1);
}

__device__ __forceinline__ uint64_t bind(uint64_t x0, uint64_t x1, uint64_t r) {
  return gl::add(x0, gl::mul(r, gl::sub(x1, x0)));
}

// Weight three exact sums by a field element.
__device__ __forceinline__ void weigh(S96& a, S96& b, S96& c, uint64_t w) {
  a = to96(gl::mul(reduce96(a), w));
  b = to96(gl::mul(reduce96(b), w));
  c = to96(gl::mul(reduce96(c), w));
}

// Shared memory of one tail workgroup.
template <int ST>
struct TailLds {
  uint64_t lA[ST], lB[ST];
  S96 red[2 * (ST / 64) * 3];
  uint64_t rl[FP_MAX_N];
};

// Instance `inst` of the tail, run by one workgroup of ST threads.
template <int ST>
__device__ __forceinline__ void tail_body(const TailArgs& a, int inst, TailLds<ST>& sh) {
  constexpr int SW = ST / 64;
  uint64_t* lA = sh.lA;
  uint64_t* lB = sh.lB;
  S96* red = sh.red;
  uint64_t* rl = sh.rl;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int np = a.n_pairs;
  const fp_elem* r = a.r;
  fp_elem* rounds = a.rounds;
  fp_elem* finals = a.finals;
  fp_elem* claim0 = a.claim0;
  const fp_elem* uA[SC_MAX_PAIRS];
  const fp_elem* uB[SC_MAX_PAIRS];
  if (a.multi) {
    const int64_t b = inst;
    uA[0] = a.user.A[0] + (b << a.n);
    uB[0] = a.user.B[0] + (b << a.n);
    r += b * a.n;
    rounds += b * 3 * a.n;
    finals += 2 * b;
    if (claim0) claim0 += b;
  } else {
    for (int j = 0; j < np; ++j) {
      uA[j] = a.user.A[j];
      uB[j] = a.user.B[j];
    }
  }
  if (tid >= a.i0 && tid < a.n) rl[tid] = r[tid];
  int vp = 1;
  while (vp < np) vp <<= 1;
  int m = 1 << (a.n - a.i0);  // per-pair entries after the entry fold
  int i = a.i0;
  if (i > 0 && tid == 0) finish_prev(a.prev_part, a.nprev, rounds, i - 1, claim0);
  const uint64_t r_entry = (i > 0) ? r[i - 1] : 0;
  const int mp = 2 * m;
  // entry q of pair j at the start of the tail
  auto load_entry = [&](int j, int q, uint64_t& x, uint64_t& y) {
    if (j >= np) { x = 0; y = 0; return; }
    if (a.i0 == 0) { x = uA[j][q]; y = uB[j][q]; return; }
    const fp_elem* A = (a.i0 == 1) ? uA[j] : a.src + (int64_t)j * mp;
    const fp_elem* B = (a.i0 == 1) ? uB[j] : a.src + (int64_t)(np + j) * mp;
    x = bind(A[2 * q], A[2 * q + 1], r_entry);
    y = bind(B[2 * q], B[2 * q + 1], r_entry);
  };
  auto weight = [&](int j) -> uint64_t { return j < np ? (a.rho ? a.rho[j] : 1ull) : 0ull; };
  const bool weighted = (a.rho != nullptr) || (vp != np);

  int mt = vp * m;
  int par = 0;
  if (mt >= 2 * ST) {
    // ---- stage A: register slices over all waves --------------------------
    int L = mt / ST;
    const int e0 = tid * L;
    const int j = e0 / m;
    const int q0 = e0 - j * m;
    uint64_t xa[SLMAX], xb[SLMAX];
#pragma unroll
    for (int k = 0; k < SLMAX; ++k)
      if (k < L) load_entry(j, q0 + k, xa[k], xb[k]);
    const uint64_t wj = weight(j);
    while (L >= 2) {
      S96 s0{0, 0, 0}, s1{0, 0, 0}, s2{0, 0, 0};
#pragma unroll
      for (int q = 0; q < SLMAX / 2; ++q)
        if (2 * q < L)  // the odd entry becomes the pair's difference
          round_terms96(xa[2 * q], xa[2 * q + 1], xb[2 * q], xb[2 * q + 1], s0, s1, s2, xa[2 * q + 1], xb[2 * q + 1]);
      if (weighted) weigh(s0, s1, s2, wj);
      uint64_t g0, g1, g2;
      block_round<SW>(s0, s1, s2, g0, g1, g2, red, par);
      if (tid == 0) emit_round(rounds, claim0, i, g0, g1, g2);
      const uint64_t ri = rl[i];
#pragma unroll
      for (int q = 0; q < SLMAX / 2; ++q)
        if (2 * q < L) {
          xa[q] = gl::add(xa[2 * q], gl::mul(ri, xa[2 * q + 1]));
          xb[q] = gl::add(xb[2 * q], gl::mul(ri, xb[2 * q + 1]));
        }
      L >>= 1;
      m >>= 1;
      ++i;
      par ^= 1;
    }
    lA[tid] = xa[0];
    lB[tid] = xb[0];
    mt = ST;
  } else {
    for (int e = tid; e < mt; e += ST) {
      const int j = e / m;
      load_entry(j, e - j * m, lA[e], lB[e]);
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // ---- stage B: wave 0, L = mt / 64 entries per lane ----------------------
  constexpr int BL = ST / 64;
  int L = mt >= 64 ? mt / 64 : 1;
  const bool live = lane * L < mt;
  const int jb = live ? (lane * L) / m : 0;
  uint64_t xa[BL], xb[BL];
#pragma unroll
  for (int k = 0; k < BL; ++k) {
    xa[k] = (k < L && live) ? lA[lane * L + k] : 0;
    xb[k] = (k < L && live) ? lB[lane * L + k] : 0;
  }
  const uint64_t wb = live ? weight(jb) : 0;
  while (L >= 2) {
    S96 s0{0, 0, 0}, s1{0, 0, 0}, s2{0, 0, 0};
#pragma unroll
    for (int q = 0; q < BL / 2; ++q)
      if (2 * q < L)
        round_terms96(xa[2 * q], xa[2 * q + 1], xb[2 * q], xb[2 * q + 1], s0, s1, s2, xa[2 * q + 1], xb[2 * q + 1]);
    if (weighted) weigh(s0, s1, s2, wb);
    uint64_t g0, g1, g2;
    wave_round(s0, s1, s2, g0, g1, g2);
    if (lane == 0) emit_round(rounds, claim0, i, g0, g1, g2);
    const uint64_t ri = rl[i];
#pragma unroll
    for (int q = 0; q < BL / 2; ++q)
      if (2 * q < L) {
        xa[q] = gl::add(xa[2 * q], gl::mul(ri, xa[2 * q + 1]));
        xb[q] = gl::add(xb[2 * q], gl::mul(ri, xb[2 * q + 1]));
      }
    L >>= 1;
    m >>= 1;
    mt >>= 1;
    ++i;
  }

  // ---- stage C: wave 0, one entry per lane --------------------------------
  const bool on = lane < mt;
  uint64_t x = on ? xa[0] : 0, y = on ? xb[0] : 0;
  const int m0 = m;
  const int jl = lane / m0;
  const uint64_t wl = on ? weight(jl) : 0;
  for (int d = 1; d < m0; d <<= 1) {
    const uint64_t x1 = fpi::shfl_xor_u64(x, d);
    const uint64_t y1 = fpi::shfl_xor_u64(y, d);
    const bool even = on && ((lane & (2 * d - 1)) == 0);
    S96 s0{0, 0, 0}, s1{0, 0, 0}, s2{0, 0, 0};
    uint64_t dx = 0, dy = 0;
    if (even) round_terms96(x, x1, y, y1, s0, s1, s2, dx, dy);
    if (weighted) weigh(s0, s1, s2, even ? wl : 0);
    uint64_t g0, g1, g2;
    wave_round(s0, s1, s2, g0, g1, g2);
    if (lane == 0) emit_round(rounds, claim0, i, g0, g1, g2);
    const uint64_t ri = rl[i];
    if (even) {
      x = gl::add(x, gl::mul(ri, dx));
      y = gl::add(y, gl::mul(ri, dy));
    }
    ++i;
  }
  if (on && (lane % m0) == 0 && jl < np) {
    finals[2 * jl] = x;
    finals[2 * jl + 1] = y;
  }
}


}  // namespace sct
