// fold.hpp - the row-fold and claim workgroups ("How fast can FlashProve go",
// §2: a folded row is the eq-weighted sum of a table's rows; §3.1: the claim
// about the rescaled product), shared by the fold launch and by the fused
// layer-step launch. fold.hip describes the arithmetic.
#pragma once
#include "common.hpp"
#include "gl.hpp"

namespace foldk {

constexpr int FT = 256;         // threads per workgroup
constexpr int FCT = 64;         // column threads (one wave wide)
constexpr int FRG = FT / FCT;   // row groups (waves)
constexpr int FCOLS = FCT * 4;  // columns per workgroup
constexpr int FMAX_CHUNK = 1024;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct FoldJob {
  const void* M;
  int64_t ld;
  const fp_elem* E;     // row weights
  const fp_elem* Ecol;  // claim: column weights; nullptr for a folded row
  fp_elem* out;         // folded row (cols_pad) or the claim (1)
  fp_elem* part;        // per-chunk column values [n_chunks][cols] or per-workgroup values
  const fp_elem* E2;    // a second row-weight vector folded from the same read of M (int8 rows), or nullptr
  fp_elem* out2;        // its folded row (cols_pad)
  fp_elem* part2;       // its per-chunk column values [n_chunks][cols]
  int32_t rows, cols, cols_pad;
  int32_t chunk_rows, n_chunks, n_strips;  // strips holding data columns
  int32_t n_pad_strips;                    // strips wholly inside [cols, cols_pad)
  int32_t block_start;
  int32_t vec;  // whole aligned 4-column groups (see fold_body)
  int32_t eb;   // bytes per element: 1 (int8) or 4 (int32)
  int32_t ctr;  // (arrival mode) first counter: one per strip of several chunks, or one per claim
};


// The last job whose first workgroup is <= b (block_start ascends; job 0 starts at 0).
template <typename Job>
__device__ __forceinline__ int find_job(const Job* j, int count, int b) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (j[mid].block_start <= b) lo = mid;
    else hi = mid - 1;
  }
  return lo;
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

// 4-row groups per wave and batch: int8 rows are 4 bytes a lane, int32 rows 16.
// kU: the fold launch's batches; kUMax: the step launches' int8 batches, whose
// fold workgroups run at the GEMM's occupancy (two per CU) and so keep twice
// the loads in flight each, in registers the GEMM has reserved anyway.
template <int EB> constexpr int kU = (EB == 1) ? 2 : 1;
template <int EB> constexpr int kUMax = (EB == 1) ? 4 : 1;
template <int EB> constexpr int kStep = FRG * kUMax<EB>;                 // groups per batch (workgroup), at most
template <int EB> constexpr int kMaxG = FMAX_CHUNK / 4 + 2 * kStep<EB>;  // digit groups incl. padding
// rows of a chunk are a multiple of this (whole pairs of batches)
template <int EB> constexpr int kRowQuantum = 8 * kStep<EB>;

template <int EB> constexpr int kNL = (EB == 1) ? 8 : 11;  // limb accumulators per column
template <int EB> constexpr int kLdsWords =
    (kMaxG<EB> * 8 > 3 * FRG * FCT * kNL<EB>) ? kMaxG<EB> * 8 : 3 * FRG * FCT * kNL<EB>;

// One workgroup's (chunk, strip). VEC: every lane's 4 columns are whole and
// aligned (cols % 4 == 0, aligned rows), so a row is one dword (int8) or one
// dwordx4 (int32) load per lane; otherwise each column is loaded alone.
// Per-chunk values that another workgroup of the same launch adds (arrival
// mode) cross XCDs: agent-scope atomic stores and loads, written through to
// and read from the point where the XCDs' memory traffic is coherent.
__device__ __forceinline__ void store_part(uint64_t* p, uint64_t v, bool coherent) {
  if (coherent) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
__device__ __forceinline__ uint64_t load_part(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// NE = 2: the rows are folded by E and E2 from one read of them (int8 rows;
// the second vector's digits follow the first's in LDS, and its weight sum
// travels through four words after the exchange area).
template <int EB> constexpr int kDig2 = kMaxG<EB> * 8;       // LDS word of the second vector's digits
template <int EB> constexpr int kEs2 = 3 * FRG * FCT * kNL<EB>;  // LDS word of its per-wave weight sums

template <int EB, bool VEC, bool COH, int NE = 1, int U = kU<EB>>
__device__ __forceinline__ void fold_body(const FoldJob& job, int lb, uint32_t* lds, uint64_t* gsum) {
  static_assert(NE == 1 || (NE == 2 && EB == 1), "two row-weight vectors for int8 rows only");
  static_assert(U >= 1 && U <= kUMax<EB>, "batch within the digit table's padding");
  constexpr int NL = kNL<EB>;
  constexpr int STEP = FRG * U;
  constexpr int W = (EB == 1) ? 1 : 4;    // dwords per lane and row
  const int tid = threadIdx.x;
  const int ct = tid % FCT;
  const int rg = __builtin_amdgcn_readfirstlane(tid / FCT);  // wave index (uniform)
  const int chunk = lb / job.n_strips;
  const int strip = lb - chunk * job.n_strips;
  const int row0 = chunk * job.chunk_rows;
  const int nrows = min(job.chunk_rows, job.rows - row0);
  const int ngroups = (nrows + 3) >> 2;
  const int nb = (ngroups + STEP - 1) / STEP;  // batches
  const int nbp = (nb + 1) & ~1;               // whole pairs for the two-stage loop
  const int gpad = nbp * STEP;                 // groups with digits (zero past the rows)
  const int c0 = strip * FCOLS + 4 * ct;
  const int col = c0 + rg;                     // the column this wave finishes

  // Rows go through a buffer descriptor: the chunk's base in SGPRs, the lane's
  // column byte offset as the VGPR offset and the row's byte offset (wave-
  // uniform) as the scalar offset. Rows past the chunk are clamped to its last
  // row (their digits are zero); columns past cols are read from inside the
  // row and never stored.
  const uint32_t ldb = (uint32_t)job.ld * EB;
  const char* cbase = (const char*)job.M + (int64_t)row0 * job.ld * EB;
  const uint32_t extent = (uint32_t)(nrows - 1) * ldb + (uint32_t)job.cols * EB;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)cbase, (short)0, (int)extent, 0x00020000);
  const int cl = VEC ? min(c0, job.cols - 4) : 0;  // idle lanes read inside the row
  uint32_t A[U][4][W], B[U][4][W];
  auto load = [&](uint32_t (&v)[U][4][W], int bi) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = min(4 * (bi * STEP + rg + FRG * u) + i, nrows - 1);
        const int soff = (int)((uint32_t)t * ldb);
        if constexpr (VEC && EB == 1) {
          v[u][i][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, cl, soff, 0);
        } else if constexpr (VEC) {
          const u32x4 q = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, cl * 4, soff, 0));
          v[u][i][0] = q[0]; v[u][i][1] = q[1]; v[u][i][2] = q[2]; v[u][i][3] = q[3];
        } else if constexpr (EB == 1) {
          uint32_t w = 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int cc = min(c0 + c, job.cols - 1);
            w |= (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(rsrc, cc, soff, 0) << (8 * c);
          }
          v[u][i][0] = w;
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int cc = min(c0 + c, job.cols - 1);
            v[u][i][c] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, cc * 4, soff, 0);
          }
        }
      }
  };

  uint32_t acc[NE][4][NL];
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int l = 0; l < NL; ++l) acc[e][c][l] = 0;
  auto compute = [&](const uint32_t (&v)[U][4][W], int bi) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = bi * STEP + rg + FRG * u;
      const u32x4 d0 = *(const u32x4*)&lds[g * 8];
      const u32x4 d1 = *(const u32x4*)&lds[g * 8 + 4];
      const uint32_t dg[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
      if constexpr (EB == 1) {
        uint32_t dh[8];
        if constexpr (NE == 2) {
          const u32x4 h0 = *(const u32x4*)&lds[kDig2<EB> + g * 8];
          const u32x4 h1 = *(const u32x4*)&lds[kDig2<EB> + g * 8 + 4];
          dh[0] = h0[0]; dh[1] = h0[1]; dh[2] = h0[2]; dh[3] = h0[3];
          dh[4] = h1[0]; dh[5] = h1[1]; dh[6] = h1[2]; dh[7] = h1[3];
        }
        uint32_t w[4];
        transpose4(v[u][0][0], v[u][1][0], v[u][2][0], v[u][3][0], w[0], w[1], w[2], w[3]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t uu = w[c] ^ 0x80808080u;  // m + 128 per byte
#pragma unroll
          for (int l = 0; l < 8; ++l) acc[0][c][l] = udot4(uu, dg[l], acc[0][c][l]);
          if constexpr (NE == 2) {
#pragma unroll
            for (int l = 0; l < 8; ++l) acc[1][c][l] = udot4(uu, dh[l], acc[1][c][l]);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t pl[4];  // byte planes of this column's 4 rows
          transpose4(v[u][0][c], v[u][1][c], v[u][2][c], v[u][3][c], pl[0], pl[1], pl[2], pl[3]);
          pl[3] ^= 0x80808080u;  // m + 2^31 as an unsigned 32-bit value
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int l = 0; l < 8; ++l) acc[0][c][b + l] = udot4(pl[b], dg[l], acc[0][c][b + l]);
        }
      }
    }
  };

  // the first batch is in flight while the digits are built
  const uint64_t ecol = (job.Ecol && col < job.cols) ? job.Ecol[col] : 0;
  load(A, 0);

  // ---- digits of E for this chunk (zero past its rows), and group sums of E ----
  uint64_t es2 = 0;  // NE = 2: this thread's share of the chunk's sum of E2
  for (int g = tid; g < gpad; g += FT) {
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const fp_elem* Ev = e == 0 ? job.E : job.E2;
      uint32_t dg[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      uint64_t es = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * g + i;
        const uint64_t x = (t < nrows) ? Ev[row0 + t] : 0;
        es = gl::add(es, x);
#pragma unroll
        for (int l = 0; l < 8; ++l) dg[l] |= (uint32_t)((x >> (8 * l)) & 0xFF) << (8 * i);
      }
      const int base = e == 0 ? 0 : kDig2<EB>;
      *(u32x4*)&lds[base + g * 8] = u32x4{dg[0], dg[1], dg[2], dg[3]};
      *(u32x4*)&lds[base + g * 8 + 4] = u32x4{dg[4], dg[5], dg[6], dg[7]};
      if (e == 0) gsum[g] = es;
      else es2 = gl::add(es2, es);
    }
  }
  __syncthreads();

  // ---- main loop: batch bi covers groups bi*STEP .. bi*STEP+STEP-1; two
  // register sets so one batch's loads are in flight while the other is used ----
  int bi = 0;
  for (; bi + 2 < nbp; bi += 2) {
    load(B, bi + 1);
    compute(A, bi);
    load(A, bi + 2);
    compute(B, bi + 1);
  }
  load(B, bi + 1);
  compute(A, bi);
  compute(B, bi + 1);

  // ---- exchange: wave v stores its other three columns (lane-contiguous), and
  // each wave finishes column c0 + v of its lanes (for each weight vector in turn) ----
  uint64_t* es2w = reinterpret_cast<uint64_t*>(lds + kEs2<EB>);
  if constexpr (NE == 2) es2 = fpi::wave_total(es2);
  uint64_t val[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    __syncthreads();  // digits (or the previous vector's exchange) no longer needed
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c == rg) continue;
      const int slot = rg * 3 + (c < rg ? c : c - 1);
#pragma unroll
      for (int l = 0; l < NL; ++l) lds[(slot * NL + l) * FCT + ct] = acc[e][c][l];
    }
    if (NE == 2 && e == 0 && ct == 0) es2w[rg] = es2;
    __syncthreads();
    uint32_t sl[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l)
      sl[l] = rg == 0 ? acc[e][0][l] : rg == 1 ? acc[e][1][l] : rg == 2 ? acc[e][2][l] : acc[e][3][l];
#pragma unroll
    for (int v = 0; v < FRG; ++v) {
      if (v == rg) continue;
      const int slot = v * 3 + (rg < v ? rg : rg - 1);
#pragma unroll
      for (int l = 0; l < NL; ++l) sl[l] += lds[(slot * NL + l) * FCT + ct];  // exact: < 2^32
    }
    uint64_t es = 0;
    if (e == 0) {
      for (int g = ct; g < gpad; g += FCT) es = gl::add(es, gsum[g]);
      es = fpi::wave_total(es);
    } else {
#pragma unroll
      for (int v = 0; v < FRG; ++v) es = gl::add(es, es2w[v]);
    }
    // offset correction: off * sum E, off = 128 (int8) or 2^31 (int32)
    const uint64_t corr = gl::mul_small(es, EB == 1 ? 128u : 0x80000000u);
    uint64_t lo = 0, hi = 0;
#pragma unroll
    for (int l = 0; l < NL; ++l) acc128(lo, hi, sl[l], 8 * l);
    val[e] = gl::sub(gl::reduce128(lo, hi), corr);
  }

  if (job.Ecol) {
    // claim: weight the column by its eq value; one value per wave
    const uint64_t s = fpi::wave_total(gl::mul(val[0], ecol));
    if (ct == 0) store_part(job.part + lb * FRG + rg, s, COH);
    return;
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    fp_elem* out = e == 0 ? job.out : job.out2;
    fp_elem* part = e == 0 ? job.part : job.part2;
    if (job.n_chunks == 1) {
      if (col < job.cols) out[col] = val[e];
      else if (col < job.cols_pad) out[col] = 0;
    } else if (col < job.cols) {
      store_part(part + (int64_t)chunk * job.cols + col, val[e], COH);
    }
  }
}

constexpr int LDS_WORDS = kLdsWords<1> > kLdsWords<4> ? kLdsWords<1> : kLdsWords<4>;
static_assert(2 * kDig2<1> <= LDS_WORDS && kEs2<1> + 2 * FRG <= LDS_WORDS,
              "the second vector's digits and weight sums fit the fold's LDS");
constexpr int MAXG_ALL = kMaxG<1> > kMaxG<4> ? kMaxG<1> : kMaxG<4>;


// Workgroup lb of a job: strips wholly in the padding write zeros; the others
// fold their chunk of rows over their 256 columns.
// DUAL (the step launches' folds): jobs with a second row-weight vector may
// occur, and int8 rows go in the larger batches.
template <bool COH, bool DUAL = false>
__device__ __forceinline__ void fold_block(const FoldJob& job, int lb, uint32_t* lds, uint64_t* gsum) {
  if (lb >= job.n_chunks * job.n_strips) {
    const int strip = job.n_strips + (lb - job.n_chunks * job.n_strips);
    for (int c = strip * FCOLS + (int)threadIdx.x; c < min((strip + 1) * FCOLS, job.cols_pad); c += FT) {
      job.out[c] = 0;
      if (job.E2) job.out2[c] = 0;
    }
    return;
  }
  if (DUAL && job.eb == 1) {
    constexpr int U = kUMax<1>;
    if (job.E2) {
      if (job.vec) fold_body<1, true, COH, 2, U>(job, lb, lds, gsum);
      else fold_body<1, false, COH, 2, U>(job, lb, lds, gsum);
    } else {
      if (job.vec) fold_body<1, true, COH, 1, U>(job, lb, lds, gsum);
      else fold_body<1, false, COH, 1, U>(job, lb, lds, gsum);
    }
  } else if (job.eb == 1) {
    if (job.vec) fold_body<1, true, COH>(job, lb, lds, gsum);
    else fold_body<1, false, COH>(job, lb, lds, gsum);
  } else {
    if (job.vec) fold_body<4, true, COH>(job, lb, lds, gsum);
    else fold_body<4, false, COH>(job, lb, lds, gsum);
  }
}

// ---- arrival mode: the cross-chunk sums inside the same launch -----------
// The last workgroup of a strip to finish (one arrival counter per strip, at
// the start of the workspace: zero on entry, left zero) adds the chunks of its
// columns; the last of a claim adds the claim's per-wave values.

// True in the workgroup whose arrival is the n-th at *ctr, which also resets
// the counter. Each thread first waits until its agent-scope stores have
// completed, so by the time the n-th arrival is counted every workgroup's
// values are visible to agent-scope loads.
__device__ __forceinline__ bool arrive_last(uint32_t* ctr, uint32_t n, uint32_t* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old + 1 == n;
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last ? 1u : 0u;
  }
  __syncthreads();
  return *flag != 0;
}

// out[c] = sum over chunks of part[chunk][c]; zeros for the strip's padding.
__device__ __forceinline__ void strip_total(const FoldJob& job, int strip) {
  const int c = strip * FCOLS + (int)threadIdx.x;
  for (int e = 0; e < (job.E2 ? 2 : 1); ++e) {
    const fp_elem* part = e == 0 ? job.part : job.part2;
    fp_elem* out = e == 0 ? job.out : job.out2;
    if (c < job.cols) {
      uint64_t v = 0;
      for (int ch = 0; ch < job.n_chunks; ++ch) v = gl::add(v, load_part(part + (int64_t)ch * job.cols + c));
      out[c] = v;
    } else if (c < job.cols_pad) {
      out[c] = 0;
    }
  }
}

// out[0] = sum of the claim's per-wave values.
__device__ __forceinline__ void claim_total(const FoldJob& job, uint64_t* red) {
  const int nv = job.n_chunks * job.n_strips * FRG;
  uint64_t v = 0;
  for (int i = (int)threadIdx.x; i < nv; i += FT) v = gl::add(v, load_part(job.part + i));
  v = fpi::wave_total(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
    for (int w = 0; w < FRG; ++w) t = gl::add(t, red[w]);
    job.out[0] = t;
  }
}

// Workgroup lb of a job in arrival mode: fold, then the sums by the last.
__device__ __forceinline__ void fold_block_arrive(const FoldJob& job, int lb, uint32_t* ctrs, uint32_t* lds,
                                                  uint64_t* gsum, uint32_t* flag) {
  fold_block<true, true>(job, lb, lds, gsum);
  if (lb >= job.n_chunks * job.n_strips) return;
  if (job.Ecol) {
    if (arrive_last(ctrs + job.ctr, (uint32_t)(job.n_chunks * job.n_strips), flag)) claim_total(job, gsum);
  } else if (job.n_chunks > 1) {
    const int strip = lb % job.n_strips;
    if (arrive_last(ctrs + job.ctr + strip, (uint32_t)job.n_chunks, flag)) strip_total(job, strip);
  }
}

// ---- planning (host) ------------------------------------------------------
struct Plan {
  int32_t chunk_rows, n_chunks, n_strips, n_pad_strips;
  size_t part_bytes;
  int64_t blocks, sum_blocks;  // fold workgroups; cross-chunk sum workgroups of the separate sum launch
  int32_t ctrs;                // arrival counters (arrival mode)
};

// arrive: the sums are done by the last workgroups of the same launch (the
// padding strips are then always workgroups of their own).
inline Plan plan_job(int32_t rows, int32_t cols, int32_t cols_pad, int eb, bool claim, bool arrive,
                     int target_blocks = 256) {
  Plan p{};
  p.n_strips = (cols + FCOLS - 1) / FCOLS;
  const int pad_total = (cols_pad + FCOLS - 1) / FCOLS;
  p.n_pad_strips = claim ? 0 : (pad_total - p.n_strips);
  // a launch of its own: about target_blocks workgroups per job (fold.hip
  // asks for two per compute unit when a launch holds int8 folds only, one
  // otherwise), chunks in whole pairs of batches. Inside a step launch
  // the folds of several tables share the GPU with the GEMM's last tiles:
  // the longest chunks (measured against 256-row and 512-row minimums on the
  // seven-map layer: 6 us per step less than one workgroup per CU per job).
  const int q = eb == 1 ? kRowQuantum<1> : kRowQuantum<4>;
  const int want_chunks = (target_blocks + p.n_strips - 1) / p.n_strips;
  int64_t cr = (rows + want_chunks - 1) / want_chunks;
  cr = (cr + q - 1) / q * q;
  if (arrive) cr = FMAX_CHUNK;
  if (cr > FMAX_CHUNK) cr = FMAX_CHUNK;
  if (cr >= rows) cr = rows;
  p.chunk_rows = (int32_t)cr;
  p.n_chunks = (int32_t)((rows + cr - 1) / cr);
  if (claim) {
    p.part_bytes = fpi::align_up((size_t)p.n_chunks * p.n_strips * FRG * 8, 256);
    p.sum_blocks = 1;
    p.ctrs = 1;
  } else if (p.n_chunks > 1) {
    p.part_bytes = fpi::align_up((size_t)p.n_chunks * (size_t)cols * 8, 256);
    p.sum_blocks = (cols_pad + 15) / 16;
    p.ctrs = p.n_strips;
  }
  if (arrive) {
    p.blocks = (int64_t)p.n_chunks * p.n_strips + p.n_pad_strips;
    p.sum_blocks = 0;
    return p;
  }
  // a single chunk writes the folded row (and its zero tail) directly
  p.blocks = (int64_t)p.n_chunks * p.n_strips + (p.n_chunks == 1 ? p.n_pad_strips : 0);
  if (p.n_chunks > 1) p.n_pad_strips = 0;  // the sum kernel writes the tail
  p.ctrs = 0;
  return p;
}

}  // namespace foldk
