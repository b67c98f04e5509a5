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
// dependent rounds occupies one compute unit, not the GPU). Rounds 0..i0-2
// read T_i (the caller's tables for i = 0, else the workspace), sum the terms
// of every pair weighted by rho_j exactly (96-bit), complete g_i across the
// workgroup, and only then bind with r_i into T_{i+1}, which ping-pongs
// between two workspace buffers: pair j's A at j 2^(n-i-1), its B at
// (n_pairs + j) 2^(n-i-1). Round i0-1 leaves g as the tail's partial sum and
// T_{i0-1} unbound: the tail binds it with r_{i0-1} while loading (sc_tail.hpp,
// entry at i0). i0 is the first round after which the virtual pairs fit the
// tail's registers.
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

// The instance, run by one workgroup of ST threads (sh: the tail's LDS).
__device__ __forceinline__ void stream_body(const Inst& in, sct::TailLds<ST>& sh) {
  constexpr int SW = ST / 64;
  const int tid = threadIdx.x;
  const int np = in.n_pairs, n = in.n, i0 = in.i0;
  fp_elem* buf[2] = {in.scratch, in.scratch + ((int64_t)np << n)};
  fp_elem* part = in.scratch + ((int64_t)2 * np << n);
  int par = 0;
  for (int i = 0; i < i0; ++i) {
    const int64_t m = (int64_t)1 << (n - i), half = m >> 1;
    auto tabA = [&](int j) -> const fp_elem* { return i == 0 ? in.A[j] : buf[i & 1] + j * m; };
    auto tabB = [&](int j) -> const fp_elem* { return i == 0 ? in.B[j] : buf[i & 1] + (np + j) * m; };
    sct::S96 t0{0, 0, 0}, t1{0, 0, 0}, t2{0, 0, 0};
    for (int j = 0; j < np; ++j) {
      const fp_elem* A = tabA(j);
      const fp_elem* B = tabB(j);
      sct::S96 s0{0, 0, 0}, s1{0, 0, 0}, s2{0, 0, 0};
      for (int64_t q = tid; q < half; q += ST) {
        uint64_t a0, a1, b0, b1, da, db;
        load2(A, q, a0, a1);
        load2(B, q, b0, b1);
        sct::round_terms96(a0, a1, b0, b1, s0, s1, s2, da, db);
      }
      if (in.rho) sct::weigh(s0, s1, s2, in.rho[j]);
      t0 = sct::add96(t0, s0);
      t1 = sct::add96(t1, s1);
      t2 = sct::add96(t2, s2);
    }
    uint64_t g0, g1, g2;
    sct::block_round<SW>(t0, t1, t2, g0, g1, g2, sh.red, par);  // g_i complete in every wave
    par ^= 1;
    if (i + 1 < i0) {
      if (tid == 0) sct::emit_round(in.rounds, in.claim0, i, g0, g1, g2);
      const uint64_t ri = in.r[i];
      fp_elem* D = buf[(i + 1) & 1];
      for (int j = 0; j < np; ++j) {
        const fp_elem* A = tabA(j);
        const fp_elem* B = tabB(j);
        fp_elem* DA = D + j * half;
        fp_elem* DB = D + (np + j) * half;
        for (int64_t q = tid; q < half; q += ST) {
          uint64_t a0, a1, b0, b1;
          load2(A, q, a0, a1);
          load2(B, q, b0, b1);
          DA[q] = sct::bind(a0, a1, ri);
          DB[q] = sct::bind(b0, b1, ri);
        }
      }
      __syncthreads();  // T_{i+1} complete before the next round reads it
    } else if (tid == 0) {
      part[0] = g0;
      part[1] = g1;
      part[2] = g2;
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
