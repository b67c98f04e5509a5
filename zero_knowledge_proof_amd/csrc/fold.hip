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
#include "common.hpp"
#include "gl.hpp"

namespace {

constexpr int FT = 256;         // threads per workgroup
constexpr int FCT = 64;         // column threads (one wave wide)
constexpr int FRG = FT / FCT;   // row groups (waves)
constexpr int FCOLS = FCT * 4;  // columns per workgroup
constexpr int FMAX_CHUNK = 1024;
constexpr int INLINE = 12;      // jobs carried in one launch's arguments
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
};

struct JobList {
  FoldJob j[INLINE];
  int32_t count;
};

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

__device__ __forceinline__ uint64_t wave_sum(uint64_t s) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s = gl::add(s, fpi::shfl_xor_u64(s, m));
  return s;
}

template <int EB>
__global__ __launch_bounds__(FT) void fold_rows_kernel(JobList jl) {
  constexpr int NL = (EB == 1) ? 8 : 11;  // limb accumulators per column
  constexpr int U = (EB == 1) ? 4 : 2;    // row groups of 4 rows in flight per thread
  constexpr int DIG_WORDS = FMAX_CHUNK / 4 * 8;
  constexpr int RED_WORDS = (FRG - 1) * FCT * 4 * NL;
  constexpr int LDS_WORDS = DIG_WORDS > RED_WORDS ? DIG_WORDS : RED_WORDS;
  __shared__ __align__(16) uint32_t lds[LDS_WORDS];
  __shared__ uint64_t wpart[FT / 64];

  int ji = 0;
#pragma unroll 1
  for (int k = 1; k < jl.count; ++k)
    if (jl.j[k].block_start <= (int)blockIdx.x) ji = k;
  const FoldJob& job = jl.j[ji];
  const int lb = blockIdx.x - job.block_start;
  const int tid = threadIdx.x;
  const int ct = tid % FCT, rg = tid / FCT;

  // strips wholly in the padding: write zeros and leave
  if (lb >= job.n_chunks * job.n_strips) {
    const int strip = job.n_strips + (lb - job.n_chunks * job.n_strips);
    for (int c = strip * FCOLS + tid; c < min((strip + 1) * FCOLS, job.cols_pad); c += FT) job.out[c] = 0;
    return;
  }
  const int chunk = lb / job.n_strips;
  const int strip = lb - chunk * job.n_strips;
  const int row0 = chunk * job.chunk_rows;
  const int nrows = min(job.chunk_rows, job.rows - row0);
  const int ngroups = (nrows + 3) >> 2;

  // ---- digits of E for this chunk, and the chunk's sum of E ----
  uint64_t esum = 0;
  for (int g = tid; g < ngroups; g += FT) {
    uint32_t dg[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g + i;
      const uint64_t e = (t < nrows) ? job.E[row0 + t] : 0;
      esum = gl::add(esum, e);
#pragma unroll
      for (int l = 0; l < 8; ++l) dg[l] |= (uint32_t)((e >> (8 * l)) & 0xFF) << (8 * i);
    }
    *(u32x4*)&lds[g * 8] = u32x4{dg[0], dg[1], dg[2], dg[3]};
    *(u32x4*)&lds[g * 8 + 4] = u32x4{dg[4], dg[5], dg[6], dg[7]};
  }
  esum = wave_sum(esum);
  if ((tid & 63) == 0) wpart[tid >> 6] = esum;
  __syncthreads();

  // ---- main loop: 4-row groups g = rg, rg + FRG, ... ----
  const int c0 = strip * FCOLS + 4 * ct;
  uint32_t acc[4][NL];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int l = 0; l < NL; ++l) acc[c][l] = 0;

  if (c0 < job.cols) {
    const bool full_cols = (c0 + 4 <= job.cols);
    if constexpr (EB == 1) {
      const int8_t* base = (const int8_t*)job.M + (int64_t)row0 * job.ld + c0;
      const bool vec = full_cols && ((job.ld & 3) == 0) && ((((uintptr_t)job.M) & 3) == 0);
      for (int g0 = rg; g0 < ngroups; g0 += FRG * U) {
        uint32_t v[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 4 * (g0 + FRG * u) + i;
            const int8_t* p = base + (int64_t)t * job.ld;
            uint32_t w = 0;
            if (t < nrows) {
              if (vec) {
                w = __builtin_nontemporal_load((const uint32_t*)p);
              } else {
                for (int c = 0; c < 4; ++c)
                  if (c0 + c < job.cols) w |= (uint32_t)(uint8_t)p[c] << (8 * c);
              }
            }
            v[u][i] = w;
          }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int g = g0 + FRG * u;
          if (g >= ngroups) break;
          uint32_t w[4];
          transpose4(v[u][0], v[u][1], v[u][2], v[u][3], w[0], w[1], w[2], w[3]);
          const u32x4 d0 = *(const u32x4*)&lds[g * 8];
          const u32x4 d1 = *(const u32x4*)&lds[g * 8 + 4];
          const uint32_t dg[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t uu = w[c] ^ 0x80808080u;  // m + 128 per byte
#pragma unroll
            for (int l = 0; l < 8; ++l) acc[c][l] = udot4(uu, dg[l], acc[c][l]);
          }
        }
      }
    } else {
      const int32_t* base = (const int32_t*)job.M + (int64_t)row0 * job.ld + c0;
      const bool vec = full_cols && ((job.ld & 3) == 0) && ((((uintptr_t)job.M) & 15) == 0);
      for (int g0 = rg; g0 < ngroups; g0 += FRG * U) {
        uint32_t v[U][4][4];  // [group][row][col]
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 4 * (g0 + FRG * u) + i;
            const int32_t* p = base + (int64_t)t * job.ld;
            if (t < nrows && vec) {
              const u32x4 q = __builtin_nontemporal_load((const u32x4*)p);
              v[u][i][0] = q[0]; v[u][i][1] = q[1]; v[u][i][2] = q[2]; v[u][i][3] = q[3];
            } else {
#pragma unroll
              for (int c = 0; c < 4; ++c) v[u][i][c] = (t < nrows && c0 + c < job.cols) ? (uint32_t)p[c] : 0u;
            }
          }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int g = g0 + FRG * u;
          if (g >= ngroups) break;
          const u32x4 d0 = *(const u32x4*)&lds[g * 8];
          const u32x4 d1 = *(const u32x4*)&lds[g * 8 + 4];
          const uint32_t dg[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
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
    }
  }

  // ---- cross-wave reduction of the limb sums (exact in u32) ----
  __syncthreads();  // digits no longer needed
  if (rg > 0) {
    uint32_t* dst = &lds[((rg - 1) * FCT + ct) * 4 * NL];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int l = 0; l < NL; ++l) dst[c * NL + l] = acc[c][l];
  }
  __syncthreads();
  uint64_t vals[4] = {0, 0, 0, 0};
  if (rg == 0) {
#pragma unroll
    for (int w = 0; w < FRG - 1; ++w) {
      const uint32_t* src = &lds[(w * FCT + ct) * 4 * NL];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int l = 0; l < NL; ++l) acc[c][l] += src[c * NL + l];
    }
    uint64_t es = 0;
#pragma unroll
    for (int w = 0; w < FT / 64; ++w) es = gl::add(es, wpart[w]);
    // offset correction: off * sum E, off = 128 (int8) or 2^31 (int32)
    const uint64_t corr = gl::mul_small(es, EB == 1 ? 128u : 0x80000000u);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint64_t lo = 0, hi = 0;
#pragma unroll
      for (int l = 0; l < NL; ++l) acc128(lo, hi, acc[c][l], 8 * l);
      vals[c] = gl::sub(gl::reduce128(lo, hi), corr);
    }
  }

  if (job.Ecol) {
    // claim: weight each column by its eq value; one value per workgroup
    if (rg == 0) {
      uint64_t s = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c0 + c < job.cols) s = gl::add(s, gl::mul(vals[c], job.Ecol[c0 + c]));
      s = wave_sum(s);
      if (ct == 0) job.part[lb] = s;
    }
    return;
  }

  if (job.n_chunks == 1) {
    if (rg == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = c0 + c;
        if (col < job.cols) job.out[col] = vals[c];
        else if (col < job.cols_pad) job.out[col] = 0;
      }
    }
    return;
  }
  if (rg == 0) {
    fp_elem* dst = job.part + (int64_t)chunk * job.cols;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c0 + c < job.cols) dst[c0 + c] = vals[c];
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
  int ji = 0;
#pragma unroll 1
  for (int k = 1; k < sl.count; ++k)
    if (sl.j[k].block_start <= (int)blockIdx.x) ji = k;
  const SumJob& j = sl.j[ji];
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

Plan plan_job(int32_t rows, int32_t cols, int32_t cols_pad, bool claim) {
  Plan p{};
  p.n_strips = (cols + FCOLS - 1) / FCOLS;
  const int pad_total = (cols_pad + FCOLS - 1) / FCOLS;
  p.n_pad_strips = claim ? 0 : (pad_total - p.n_strips);
  const int target_blocks = 2048;
  const int want_chunks = (target_blocks + p.n_strips - 1) / p.n_strips;
  int cr = (rows + want_chunks - 1) / want_chunks;
  cr = (cr + 15) / 16 * 16;
  const int min_cr = claim ? 32 : 256;
  if (cr < min_cr) cr = min_cr;
  if (cr > FMAX_CHUNK) cr = FMAX_CHUNK;
  if (cr >= rows) cr = (rows + 3) / 4 * 4;
  if (cr < 4) cr = 4;
  p.chunk_rows = cr;
  p.n_chunks = (rows + cr - 1) / cr;
  if (claim) {
    p.part_bytes = fpi::align_up((size_t)p.n_chunks * p.n_strips * 8, 256);
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

// Workspace: the partials of every job, back to back.
template <typename Desc>
size_t layout(int32_t count, const Desc* d, bool claim, int32_t (*rows)(const Desc&), int32_t (*cols)(const Desc&),
              int32_t (*pad)(const Desc&)) {
  size_t parts = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (rows(d[i]) <= 0 || cols(d[i]) <= 0) continue;
    parts += plan_job(rows(d[i]), cols(d[i]), pad(d[i]), claim).part_bytes;
  }
  return parts;
}

int32_t f_rows(const fp_fold_desc& d) { return d.rows; }
int32_t f_cols(const fp_fold_desc& d) { return d.cols; }
int32_t f_pad(const fp_fold_desc& d) { return d.cols_pad; }
int32_t c_rows(const fp_claim_desc& d) { return d.rows; }
int32_t c_cols(const fp_claim_desc& d) { return d.cols; }
int32_t c_pad(const fp_claim_desc& d) { return d.cols; }

int launch_list(int eb, const JobList& jl, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return FP_OK;
  if (blocks > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "fold: too many workgroups");
  if (eb == 1) hipLaunchKernelGGL(fold_rows_kernel<1>, dim3((unsigned)blocks), dim3(FT), 0, st, jl);
  else hipLaunchKernelGGL(fold_rows_kernel<4>, dim3((unsigned)blocks), dim3(FT), 0, st, jl);
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
  jl.count = 1;
  return launch_list(1, jl, j.n_pad_strips, st);
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

// Enqueue a list of fold or claim jobs, INLINE at a time: one fold launch and
// (when needed) one cross-chunk sum launch per INLINE jobs.
template <typename Desc, typename Fill>
int run_jobs(int eb, int32_t count, const Desc* d, bool claim, char* ws, Fill fill, hipStream_t st) {
  char* parts = ws;
  JobList jl{};
  SumList sl{};
  int64_t blocks = 0, sblocks = 0;
  auto flush = [&]() -> int {
    int rc = launch_list(eb, jl, blocks, st);
    if (!rc && sblocks > 0) {
      hipLaunchKernelGGL(fold_sum_kernel, dim3((unsigned)sblocks), dim3(256), 0, st, sl);
      rc = fpi::check_launch("fold_sum_kernel");
    }
    jl = JobList{};
    sl = SumList{};
    blocks = sblocks = 0;
    return rc;
  };
  for (int32_t i = 0; i < count; ++i) {
    FoldJob j{};
    fill(d[i], j);
    if (j.rows <= 0 || j.cols <= 0) {
      // empty matrix: zero output
      int rc = claim ? zero_only(j.out, 1, st) : zero_only(j.out, j.cols_pad, st);
      if (rc) return rc;
      continue;
    }
    const Plan p = plan_job(j.rows, j.cols, j.cols_pad, claim);
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
      sj.n_chunks = claim ? (int32_t)(p.n_chunks * p.n_strips) : p.n_chunks;
      sj.block_start = (int32_t)sblocks;
      sl.j[sl.count++] = sj;
      sblocks += p.sum_blocks;
    }
  }
  return jl.count ? flush() : FP_OK;
}

size_t fold_ws(int32_t count, const fp_fold_desc* d) { return layout(count, d, false, f_rows, f_cols, f_pad); }
size_t claim_ws(int32_t count, const fp_claim_desc* d) { return layout(count, d, true, c_rows, c_cols, c_pad); }

}  // namespace

extern "C" size_t fp_fold_matrix_workspace(fp_dtype dt, int32_t rows, int32_t cols) {
  (void)dt;
  fp_fold_desc d{nullptr, cols, rows, cols, cols, nullptr, nullptr};
  return fold_ws(1, &d);
}

extern "C" int fp_fold_matrix(fp_dtype dt, const void* M, int64_t ld, int32_t rows, int32_t cols, const fp_elem* E,
                              fp_elem* out, int32_t cols_pad, void* ws, size_t ws_bytes, hipStream_t stream) {
  fp_fold_desc d{M, ld, rows, cols, cols_pad, E, out};
  return fp_fold_matrix_batched(dt, 1, &d, ws, ws_bytes, stream);
}

extern "C" size_t fp_fold_matrix_batched_workspace(fp_dtype dt, int32_t count, const fp_fold_desc* d) {
  (void)dt;
  if (count <= 0 || !d) return 0;
  return fold_ws(count, d);
}

extern "C" int fp_fold_matrix_batched(fp_dtype dt, int32_t count, const fp_fold_desc* d, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  if (count < 0) return fpi::fail(FP_EARG, "fp_fold_matrix_batched: count < 0");
  if (count == 0) return fpi::ok();
  if (!d) return fpi::fail(FP_EARG, "fp_fold_matrix_batched: null descs");
  for (int32_t i = 0; i < count; ++i) {
    int rc = validate_fold("fp_fold_matrix", dt, d[i].M, d[i].ld, d[i].rows, d[i].cols, d[i].E, d[i].out,
                           d[i].cols_pad);
    if (rc) return rc;
  }
  const size_t need = layout(count, d, false, f_rows, f_cols, f_pad);
  if (need && (!ws || ws_bytes < need))
    return fpi::fail(FP_EWORKSPACE, "fp_fold_matrix: workspace %zu < %zu", ws_bytes, need);
  auto fill = [](const fp_fold_desc& s, FoldJob& j) {
    j.M = s.M; j.ld = s.ld; j.E = s.E; j.Ecol = nullptr; j.out = s.out;
    j.rows = s.rows; j.cols = s.cols; j.cols_pad = s.cols_pad;
  };
  int rc = run_jobs(dt == FP_I8 ? 1 : 4, count, d, false, (char*)ws, fill, stream);
  return rc ? rc : fpi::ok();
}

extern "C" size_t fp_claim_eval_batched_workspace(fp_dtype dt, int32_t count, const fp_claim_desc* d) {
  (void)dt;
  if (count <= 0 || !d) return 0;
  return claim_ws(count, d);
}

extern "C" int fp_claim_eval_batched(fp_dtype dt, int32_t count, const fp_claim_desc* d, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  if (dt != FP_I8 && dt != FP_I32) return fpi::fail(FP_EARG, "fp_claim_eval_batched: unknown dtype %d", (int)dt);
  if (count < 0) return fpi::fail(FP_EARG, "fp_claim_eval_batched: count < 0");
  if (count == 0) return fpi::ok();
  if (!d) return fpi::fail(FP_EARG, "fp_claim_eval_batched: null descs");
  for (int32_t i = 0; i < count; ++i) {
    if (d[i].rows < 0 || d[i].cols < 0 || d[i].ld < d[i].cols)
      return fpi::fail(FP_ESHAPE, "fp_claim_eval_batched: desc %d has bad sizes", i);
    if (!d[i].out || (d[i].rows > 0 && d[i].cols > 0 && (!d[i].M || !d[i].E_rows || !d[i].E_cols)))
      return fpi::fail(FP_EARG, "fp_claim_eval_batched: desc %d has a null pointer", i);
  }
  const size_t need = layout(count, d, true, c_rows, c_cols, c_pad);
  if (need && (!ws || ws_bytes < need))
    return fpi::fail(FP_EWORKSPACE, "fp_claim_eval_batched: workspace %zu < %zu", ws_bytes, need);
  auto fill = [](const fp_claim_desc& s, FoldJob& j) {
    j.M = s.M; j.ld = s.ld; j.E = s.E_rows; j.Ecol = s.E_cols; j.out = s.out;
    j.rows = s.rows; j.cols = s.cols; j.cols_pad = s.cols;
  };
  int rc = run_jobs(dt == FP_I8 ? 1 : 4, count, d, true, (char*)ws, fill, stream);
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
