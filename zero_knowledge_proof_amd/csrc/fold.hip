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
// Rows are split into chunks, one workgroup per (chunk, 256-column strip).
// Each workgroup stores its per-column field values, and a second small kernel
// adds the chunks per column (16 chunk lanes per column, so the adds are not
// one long dependent chain). For a claim, each workgroup weights its columns
// with the column eq table and stores one value; one workgroup per claim then
// adds them. The two kernels need no atomics and no cross-XCD fences.
#include <vector>

#include "common.hpp"
#include "gl.hpp"

namespace {

constexpr int FT = 256;         // threads per workgroup
constexpr int FCT = 64;         // column threads (one wave wide)
constexpr int FRG = FT / FCT;   // row groups (waves)
constexpr int FCOLS = FCT * 4;  // columns per workgroup
constexpr int FMAX_CHUNK = 1024;
constexpr int INLINE = 32;      // jobs carried in one launch's arguments (kernel arguments <= 4 KB)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct FoldJob {
  const void* M;
  int64_t ld;
  const fp_elem* E;     // row weights
  const fp_elem* Ecol;  // claim: column weights; nullptr for a folded row
  fp_elem* out;         // folded row (cols_pad) or the claim (1)
  fp_elem* part;        // per-chunk column values [n_chunks][cols] or per-workgroup values
  int32_t rows, cols, cols_pad;
  int32_t chunk_rows, n_chunks, n_strips;  // strips holding data columns
  int32_t n_pad_strips;                    // strips wholly inside [cols, cols_pad)
  int32_t block_start;
  int32_t vec;  // whole aligned 4-column groups (see fold_body)
  int32_t eb;   // bytes per element: 1 (int8) or 4 (int32)
};

struct JobList {
  FoldJob j[INLINE];
  int32_t count;
};
static_assert(sizeof(JobList) <= 4096, "a job list travels in the kernel arguments");

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
template <int EB> constexpr int kU = (EB == 1) ? 2 : 1;
template <int EB> constexpr int kStep = FRG * kU<EB>;                  // groups per batch (workgroup)
template <int EB> constexpr int kMaxG = FMAX_CHUNK / 4 + 2 * kStep<EB>;  // digit groups incl. padding
// rows of a chunk are a multiple of this (whole pairs of batches)
template <int EB> constexpr int kRowQuantum = 8 * kStep<EB>;

template <int EB> constexpr int kNL = (EB == 1) ? 8 : 11;  // limb accumulators per column
template <int EB> constexpr int kLdsWords =
    (kMaxG<EB> * 8 > 3 * FRG * FCT * kNL<EB>) ? kMaxG<EB> * 8 : 3 * FRG * FCT * kNL<EB>;

// One workgroup's (chunk, strip). VEC: every lane's 4 columns are whole and
// aligned (cols % 4 == 0, aligned rows), so a row is one dword (int8) or one
// dwordx4 (int32) load per lane; otherwise each column is loaded alone.
template <int EB, bool VEC>
__device__ __forceinline__ void fold_body(const FoldJob& job, int lb, uint32_t* lds, uint64_t* gsum) {
  constexpr int NL = kNL<EB>;
  constexpr int U = kU<EB>;
  constexpr int STEP = kStep<EB>;
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

  uint32_t acc[4][NL];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int l = 0; l < NL; ++l) acc[c][l] = 0;
  auto compute = [&](const uint32_t (&v)[U][4][W], int bi) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = bi * STEP + rg + FRG * u;
      const u32x4 d0 = *(const u32x4*)&lds[g * 8];
      const u32x4 d1 = *(const u32x4*)&lds[g * 8 + 4];
      const uint32_t dg[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
      if constexpr (EB == 1) {
        uint32_t w[4];
        transpose4(v[u][0][0], v[u][1][0], v[u][2][0], v[u][3][0], w[0], w[1], w[2], w[3]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t uu = w[c] ^ 0x80808080u;  // m + 128 per byte
#pragma unroll
          for (int l = 0; l < 8; ++l) acc[c][l] = udot4(uu, dg[l], acc[c][l]);
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
            for (int l = 0; l < 8; ++l) acc[c][b + l] = udot4(pl[b], dg[l], acc[c][b + l]);
        }
      }
    }
  };

  // the first batch is in flight while the digits are built
  const uint64_t ecol = (job.Ecol && col < job.cols) ? job.Ecol[col] : 0;
  load(A, 0);

  // ---- digits of E for this chunk (zero past its rows), and group sums of E ----
  for (int g = tid; g < gpad; g += FT) {
    uint32_t dg[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint64_t es = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g + i;
      const uint64_t e = (t < nrows) ? job.E[row0 + t] : 0;
      es = gl::add(es, e);
#pragma unroll
      for (int l = 0; l < 8; ++l) dg[l] |= (uint32_t)((e >> (8 * l)) & 0xFF) << (8 * i);
    }
    *(u32x4*)&lds[g * 8] = u32x4{dg[0], dg[1], dg[2], dg[3]};
    *(u32x4*)&lds[g * 8 + 4] = u32x4{dg[4], dg[5], dg[6], dg[7]};
    gsum[g] = es;
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
  // each wave finishes column c0 + v of its lanes ----
  __syncthreads();  // digits no longer needed
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c == rg) continue;
    const int slot = rg * 3 + (c < rg ? c : c - 1);
#pragma unroll
    for (int l = 0; l < NL; ++l) lds[(slot * NL + l) * FCT + ct] = acc[c][l];
  }
  __syncthreads();
  uint32_t sl[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) sl[l] = rg == 0 ? acc[0][l] : rg == 1 ? acc[1][l] : rg == 2 ? acc[2][l] : acc[3][l];
#pragma unroll
  for (int v = 0; v < FRG; ++v) {
    if (v == rg) continue;
    const int slot = v * 3 + (rg < v ? rg : rg - 1);
#pragma unroll
    for (int l = 0; l < NL; ++l) sl[l] += lds[(slot * NL + l) * FCT + ct];  // exact: < 2^32
  }
  uint64_t es = 0;
  for (int g = ct; g < gpad; g += FCT) es = gl::add(es, gsum[g]);
  es = fpi::wave_total(es);
  // offset correction: off * sum E, off = 128 (int8) or 2^31 (int32)
  const uint64_t corr = gl::mul_small(es, EB == 1 ? 128u : 0x80000000u);
  uint64_t lo = 0, hi = 0;
#pragma unroll
  for (int l = 0; l < NL; ++l) acc128(lo, hi, sl[l], 8 * l);
  const uint64_t val = gl::sub(gl::reduce128(lo, hi), corr);

  if (job.Ecol) {
    // claim: weight the column by its eq value; one value per wave
    const uint64_t s = fpi::wave_total(gl::mul(val, ecol));
    if (ct == 0) job.part[lb * FRG + rg] = s;
    return;
  }
  if (job.n_chunks == 1) {
    if (col < job.cols) job.out[col] = val;
    else if (col < job.cols_pad) job.out[col] = 0;
    return;
  }
  if (col < job.cols) job.part[(int64_t)chunk * job.cols + col] = val;
}

constexpr int LDS_WORDS = kLdsWords<1> > kLdsWords<4> ? kLdsWords<1> : kLdsWords<4>;
constexpr int MAXG_ALL = kMaxG<1> > kMaxG<4> ? kMaxG<1> : kMaxG<4>;

// Every job of the list, int8 or int32, folds or claims, in one launch.
__global__ __launch_bounds__(FT) void fold_rows_kernel(JobList jl) {
  __shared__ __align__(16) uint32_t lds[LDS_WORDS];
  __shared__ uint64_t gsum[MAXG_ALL];
  const FoldJob& job = jl.j[find_job(jl.j, jl.count, blockIdx.x)];
  const int lb = blockIdx.x - job.block_start;
  // strips wholly in the padding: write zeros and leave
  if (lb >= job.n_chunks * job.n_strips) {
    const int strip = job.n_strips + (lb - job.n_chunks * job.n_strips);
    for (int c = strip * FCOLS + (int)threadIdx.x; c < min((strip + 1) * FCOLS, job.cols_pad); c += FT) job.out[c] = 0;
    return;
  }
  if (job.eb == 1) {
    if (job.vec) fold_body<1, true>(job, lb, lds, gsum);
    else fold_body<1, false>(job, lb, lds, gsum);
  } else {
    if (job.vec) fold_body<4, true>(job, lb, lds, gsum);
    else fold_body<4, false>(job, lb, lds, gsum);
  }
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
struct Plan {
  int32_t chunk_rows, n_chunks, n_strips, n_pad_strips;
  size_t part_bytes;
  int64_t blocks, sum_blocks;  // fold workgroups; cross-chunk sum workgroups (0: none)
};

Plan plan_job(int32_t rows, int32_t cols, int32_t cols_pad, int eb, bool claim) {
  Plan p{};
  p.n_strips = (cols + FCOLS - 1) / FCOLS;
  const int pad_total = (cols_pad + FCOLS - 1) / FCOLS;
  p.n_pad_strips = claim ? 0 : (pad_total - p.n_strips);
  // about one workgroup per compute unit (measured against 128-1536 on the
  // up-projection: fewer chunks also shorten the cross-chunk sums), chunks in
  // whole pairs of batches
  const int target_blocks = 256;
  const int q = eb == 1 ? kRowQuantum<1> : kRowQuantum<4>;
  const int want_chunks = (target_blocks + p.n_strips - 1) / p.n_strips;
  int64_t cr = (rows + want_chunks - 1) / want_chunks;
  cr = (cr + q - 1) / q * q;
  if (cr > FMAX_CHUNK) cr = FMAX_CHUNK;
  if (cr >= rows) cr = rows;
  p.chunk_rows = (int32_t)cr;
  p.n_chunks = (int32_t)((rows + cr - 1) / cr);
  if (claim) {
    p.part_bytes = fpi::align_up((size_t)p.n_chunks * p.n_strips * FRG * 8, 256);
    p.sum_blocks = 1;
  } else if (p.n_chunks > 1) {
    p.part_bytes = fpi::align_up((size_t)p.n_chunks * (size_t)cols * 8, 256);
    p.sum_blocks = (cols_pad + 15) / 16;
  }
  // a single chunk writes the folded row (and its zero tail) directly
  p.blocks = (int64_t)p.n_chunks * p.n_strips + (p.n_chunks == 1 ? p.n_pad_strips : 0);
  if (p.n_chunks > 1) p.n_pad_strips = 0;  // the sum kernel writes the tail
  return p;
}

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

// Workspace: the partials of every job, back to back.
size_t items_ws(const std::vector<Item>& v) {
  size_t parts = 0;
  for (const Item& it : v) {
    if (it.j.rows <= 0 || it.j.cols <= 0) continue;
    parts += plan_job(it.j.rows, it.j.cols, it.j.cols_pad, it.j.eb, it.claim).part_bytes;
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
    const Plan p = plan_job(j.rows, j.cols, j.cols_pad, eb, claim);
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
    int rc = validate_fold(fn, dt, d[i].M, d[i].ld, d[i].rows, d[i].cols, d[i].E, d[i].out, d[i].cols_pad);
    if (rc) return rc;
  }
  return FP_OK;
}

}  // namespace

extern "C" size_t fp_fold_matrix_workspace(fp_dtype dt, int32_t rows, int32_t cols) {
  fp_fold_desc d{nullptr, cols, rows, cols, cols, nullptr, nullptr};
  return fp_fold_matrix_batched_workspace(dt, 1, &d);
}

extern "C" int fp_fold_matrix(fp_dtype dt, const void* M, int64_t ld, int32_t rows, int32_t cols, const fp_elem* E,
                              fp_elem* out, int32_t cols_pad, void* ws, size_t ws_bytes, hipStream_t stream) {
  fp_fold_desc d{M, ld, rows, cols, cols_pad, E, out};
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
