// sc_stream.hpp - a whole sum-check instance in ONE workgroup, for tables too
// large for the register tail: the first rounds stream the tables through a
// workspace, the rest is the tail of sc_tail.hpp.
//
// "How fast can FlashProve go", §2: sum-check reduces each matmul to claims
// about its folded tables; round i sends g_i(0), g_i(1), g_i(2),
//     g_i(c) = sum_j rho_j sum_q A_j,c[q] B_j,c[q],  A_c[q] = A[2q] + c (A[2q+1] - A[2q]),
// then binds A[q] <- A[2q] + r_i (A[2q+1] - A[2q]) (B likewise).
//
// Such a workgroup runs beside the GEMM tiles of a later proof (a chain of
// dependent rounds occupies one compute unit, not the GPU). The round
// challenges are known in advance here, so streamed round i (i < i0) forms
// T_i and sums its terms in one pass: round 0 reads the caller's tables, round
// i > 0 binds T_{i-1} with r_{i-1} into T_i on the way (T_i ping-pongs between
// two workspace buffers, T_i in buffer i mod 2: pair j's A at j 2^(n-i), its B
// at (n_pairs + j) 2^(n-i)). The terms of every pair are summed exactly
// (96-bit) and weighted by rho_j, and g_i is completed across the workgroup.
// Round i0-1 leaves g as the tail's partial sum and T_{i0-1} unbound: the
// tail binds it with r_{i0-1} while loading (sc_tail.hpp, entry at i0). i0 is
// the first round after which the virtual pairs fit the tail's registers.
#pragma once
#include "common.hpp"
#include "gl.hpp"
#include "sc_tail.hpp"

namespace scs {

constexpr int ST = 256;         // threads of the workgroup
constexpr int MAX_PAIRS = 8;    // pairs of one instance
constexpr int TAIL_ENTRIES = ST * sct::SLMAX;

struct Inst {
  const fp_elem* A[MAX_PAIRS];
  const fp_elem* B[MAX_PAIRS];
  const fp_elem* rho;  // n_pairs weights, or NULL (all ones)
  const fp_elem* r;    // n round challenges
  fp_elem* rounds;     // [n][3]
  fp_elem* finals;     // [n_pairs][2]
  fp_elem* claim0;     // 1, or NULL
  fp_elem* scratch;    // workspace_entries(n_pairs, n) entries
  int32_t n, n_pairs, i0;
};

__host__ __device__ inline int virtual_pairs(int np) {
  int vp = 1;
  while (vp < np) vp <<= 1;
  return vp;
}

// Rounds streamed before the tail: the first i with vp 2^(n - i) <= TAIL_ENTRIES.
__host__ __device__ inline int stream_rounds(int np, int n) {
  int i0 = 0;
  while (((int64_t)virtual_pairs(np) << (n - i0)) > TAIL_ENTRIES) ++i0;
  return i0;
}

// Workspace entries of an instance: two table buffers and the partial sums.
inline int64_t workspace_entries(int np, int n) { return (int64_t)2 * np * ((int64_t)1 << n) + 4; }

__device__ __forceinline__ void load2(const fp_elem* p, int64_t q, uint64_t& x0, uint64_t& x1) {
  const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(p + 2 * q);
  x0 = v.x;
  x1 = v.y;
}

__device__ __forceinline__ void store2(fp_elem* p, int64_t q, uint64_t x0, uint64_t x1) {
  *reinterpret_cast<ulonglong2*>(p + 2 * q) = ulonglong2{x0, x1};
}

constexpr int SU = 4;  // pairs of entries per thread whose loads are in flight together

// One pair's run of a streamed round i (see the file comment): FIRST (i = 0)
// reads T_0's pairs of entries from the caller's tables; otherwise pair q of
// T_i is bound from entries 4q .. 4q+3 of T_{i-1} with r_{i-1} and written to
// the workspace in the same pass. The terms of round i are added into s.
template <bool FIRST>
__device__ __forceinline__ void stream_pair(const fp_elem* A, const fp_elem* B, fp_elem* DA, fp_elem* DB,
                                            int64_t half, uint64_t rp, sct::S96& s0, sct::S96& s1, sct::S96& s2) {
  constexpr int E = FIRST ? 2 : 4;  // entries of the source tables per pair of T_i
  for (int64_t q0 = threadIdx.x; q0 < half; q0 += SU * ST) {
    uint64_t a[SU][E], b[SU][E];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int64_t q = q0 + (int64_t)u * ST;
      if (q < half) {
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          load2(A, (E / 2) * q + e / 2, a[u][e], a[u][e + 1]);
          load2(B, (E / 2) * q + e / 2, b[u][e], b[u][e + 1]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int64_t q = q0 + (int64_t)u * ST;
      if (q < half) {
        uint64_t a0, a1, b0, b1, da, db;
        if constexpr (FIRST) {
          a0 = a[u][0];
          a1 = a[u][1];
          b0 = b[u][0];
          b1 = b[u][1];
        } else {
          a0 = sct::bind(a[u][0], a[u][1], rp);
          a1 = sct::bind(a[u][2], a[u][3], rp);
          b0 = sct::bind(b[u][0], b[u][1], rp);
          b1 = sct::bind(b[u][2], b[u][3], rp);
          store2(DA, q, a0, a1);
          store2(DB, q, b0, b1);
        }
        sct::round_terms96(a0, a1, b0, b1, s0, s1, s2, da, db);
      }
    }
  }
}

// The instance, run by one workgroup of ST threads (sh: the tail's LDS).
__device__ __forceinline__ void stream_body(const Inst& in, sct::TailLds<ST>& sh) {
  constexpr int SW = ST / 64;
  const int tid = threadIdx.x;
  const int np = in.n_pairs, n = in.n, i0 = in.i0;
  fp_elem* buf[2] = {in.scratch, in.scratch + ((int64_t)np << n)};
  fp_elem* part = in.scratch + ((int64_t)2 * np << n);
  int par = 0;
  for (int i = 0; i < i0; ++i) {
    const int64_t m = (int64_t)1 << (n - i), half = m >> 1;  // entries of each table of T_i, its pairs
    const uint64_t rp = i > 0 ? in.r[i - 1] : 0;
    fp_elem* D = buf[i & 1];
    const fp_elem* S = buf[(i - 1) & 1];  // T_{i-1} (i >= 2): 2m entries per table
    sct::S96 t0{0, 0, 0}, t1{0, 0, 0}, t2{0, 0, 0};
    for (int j = 0; j < np; ++j) {
      sct::S96 s0{0, 0, 0}, s1{0, 0, 0}, s2{0, 0, 0};
      if (i == 0) {
        stream_pair<true>(in.A[j], in.B[j], nullptr, nullptr, half, 0, s0, s1, s2);
      } else {
        const fp_elem* A = i == 1 ? in.A[j] : S + j * 2 * m;
        const fp_elem* B = i == 1 ? in.B[j] : S + (np + j) * 2 * m;
        stream_pair<false>(A, B, D + j * m, D + (np + j) * m, half, rp, s0, s1, s2);
      }
      if (in.rho) sct::weigh(s0, s1, s2, in.rho[j]);
      t0 = sct::add96(t0, s0);
      t1 = sct::add96(t1, s1);
      t2 = sct::add96(t2, s2);
    }
    uint64_t g0, g1, g2;
    // g_i complete in every wave; its barrier also orders this round's writes of T_i before the next round
    sct::block_round<SW>(t0, t1, t2, g0, g1, g2, sh.red, par);
    par ^= 1;
    if (tid == 0) {
      if (i + 1 < i0) {
        sct::emit_round(in.rounds, in.claim0, i, g0, g1, g2);
      } else {
        part[0] = g0;
        part[1] = g1;
        part[2] = g2;
      }
    }
  }
  __syncthreads();
  sct::TailArgs ta{};
  for (int j = 0; j < np; ++j) {
    ta.user.A[j] = in.A[j];
    ta.user.B[j] = in.B[j];
  }
  ta.src = i0 >= 2 ? buf[(i0 - 1) & 1] : nullptr;
  ta.rho = in.rho;
  ta.r = in.r;
  ta.prev_part = part;
  ta.nprev = i0 > 0 ? 1 : 0;
  ta.rounds = in.rounds;
  ta.finals = in.finals;
  ta.claim0 = in.claim0;
  ta.i0 = i0;
  ta.n = n;
  ta.n_pairs = np;
  ta.multi = 0;
  sct::tail_body<ST>(ta, 0, sh);
}

}  // namespace scs
