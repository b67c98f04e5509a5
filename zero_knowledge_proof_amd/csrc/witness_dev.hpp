// witness_dev.hpp - device helpers shared by the witness kernels: the launch
// arguments, the rescale epilogue ("How fast can FlashProve go", §3.1: the
// rescaled value and its committed remainder; §2: the clamp that follows),
// the claim of a launch's own product taken from the GEMM's accumulators, and
// the eq tables that spare workgroups of a witness launch build.
#pragma once

#include "common.hpp"
#include "eq.hpp"
#include "fold.hpp"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int MAXG = 128;  // groups per grouped launch

struct WitArgs {
  const int8_t* X;
  int64_t ldx;
  const int8_t* W;
  int64_t ldw;
  int32_t T, N, K, s;  // tokens, outputs (d_out), reduction (d_in), shift
  int32_t* Z;
  int8_t* Y;
  int8_t* R;
  int32_t tiles_t, tiles_o;
  int32_t vecX, vecW, vecZ, vecYR;
  // split K: each tile is computed by ksplit workgroups, workgroup j reducing
  // over [j kchunk, (j+1) kchunk) (0 or 1: no split)
  int32_t ksplit, kchunk;
  // limb-fold epilogue: field value of each group of 8 output rows at token t
  // into part[j psplit + (o / 8) ldp + t], plus the column-sum term in split 0
  const int32_t* colsum;
  uint64_t* part;
  int64_t ldp, psplit;
  // packed weights (W then points at them): 32-row blocks and WP_BK-byte K blocks
  int32_t wp_rb, wp_kb;
  // packed kernel: the claim sum_{t,o} cEt[t] cEo[o] Z[t, o] of the launch's own
  // product, taken from the accumulators (none when cEt is NULL): one value per
  // wave into cpart, and the last tile to arrive at *cctr writes the sum to *cout
  const uint64_t* cEt = nullptr;
  const uint64_t* cEo = nullptr;
  uint64_t* cpart = nullptr;
  uint64_t* cout = nullptr;
  uint32_t* cctr = nullptr;
  // weight fold beside the GEMM (the first token tile of each weight panel):
  // sum_o E_o[o] W[o, k] over the panel's rows into fpart[panel fpitch + k]
  // (cEo: the E_o table), none when fpart is NULL
  uint64_t* fpart = nullptr;
  int64_t fpitch = 0;
};

struct GroupTab {
  const int8_t* W[MAXG];
  int32_t row_off[MAXG + 1];   // token rows of each group
  int32_t tile_off[MAXG + 1];  // first token tile of each group
  int32_t G;
};

__device__ __forceinline__ v4i load16(const int8_t* rowp, int k, int K, bool vec) {
  if (vec && k + 16 <= K) return *(const v4i*)(rowp + k);
  int w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int b = 0; b < 16; ++b)
    if (k + b < K) w[b >> 2] |= (int)((uint32_t)(uint8_t)rowp[k + b] << (8 * (b & 3)));
  v4i r = {w[0], w[1], w[2], w[3]};
  return r;
}

// Map a linear workgroup id to a tile id so that each XCD gets a contiguous
// range of tiles (ids are dealt to XCDs round-robin).
__device__ __forceinline__ int xcd_tile(int bid, int nb) {
  constexpr int NX = 8;
  const int x = bid % NX, li = bid / NX;
  const int q = nb / NX, rm = nb % NX;
  const int start = (x < rm) ? x * (q + 1) : rm * (q + 1) + (x - rm) * q;
  return start + li;
}

// Q = floor((z + 2^(s-1)) / 2^s) by an arithmetic shift, R = z - 2^s Q, Y = Q
// clamped to int8. The sum cannot overflow: |z| <= 2^14 d_in <= 2^31 - 2^14
// (d_in <= FP_MAX_DIN) and 2^(s-1) <= 128 (s in [1, 8]). Results in the low
// byte (the packing keeps only that byte).
__device__ __forceinline__ void rescale(int32_t z, int s, int32_t& y, int32_t& r) {
  const int32_t q = (z + (1 << (s - 1))) >> s;
  r = z - (q << s);
  y = q < -128 ? -128 : (q > 127 ? 127 : q);
}

// Low bytes of a, b, c, d as one dword (byte 0 = a).
__device__ __forceinline__ uint32_t pack_low_bytes(int32_t a, int32_t b, int32_t c, int32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0c0c0400u);  // a0 b0 0 0
  const uint32_t cd = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x0c0c0400u);  // c0 d0 0 0
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// One 32x32 accumulator fragment as 16 consecutive outputs per lane: lanes
// 0-31 keep o = 0..15 of the 32-block, lanes 32-63 take o = 16..31 (two
// v_permlane32_swap per 4 accumulators), then the o offsets are in register
// order 0-3, 8-11, 4-7, 12-15.
__device__ __forceinline__ void fragment_outputs(const v16i& accv, int32_t (&z)[16]) {
  int32_t v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = accv[k];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)v[k], (unsigned)v[k + 8], false, false);
    v[k] = (int32_t)sw[0];
    v[k + 8] = (int32_t)sw[1];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    z[q] = v[q];
    z[4 + q] = v[8 + q];
    z[8 + q] = v[4 + q];
    z[12 + q] = v[12 + q];
  }
}

// The Y and R bytes of 16 outputs, four to a word.
__device__ __forceinline__ void yr_bytes(const int32_t (&z)[16], int s, uint32_t (&yw)[4], uint32_t (&rw)[4]) {
  int32_t y[16], r[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) rescale(z[q], s, y[q], r[q]);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    yw[g] = pack_low_bytes(y[4 * g], y[4 * g + 1], y[4 * g + 2], y[4 * g + 3]);
    rw[g] = pack_low_bytes(r[4 * g], r[4 * g + 1], r[4 * g + 2], r[4 * g + 3]);
  }
}

// Y, R (and Z unless NULL) of 16 consecutive outputs o0.. of token t, held by one
// lane after the swap; the caller has checked t < T and o0 < N.
__device__ __forceinline__ void store_fragment(const WitArgs& a, const int32_t (&z)[16], int t, int o0, int s) {
  const int64_t idx = (int64_t)t * a.N + o0;
  uint32_t yw[4], rw[4];
  yr_bytes(z, s, yw, rw);
  if (o0 + 16 <= a.N) {
    if (a.Z) {
      if (a.vecZ) {
#pragma unroll
        for (int q = 0; q < 4; ++q) *(v4i*)(a.Z + idx + 4 * q) = v4i{z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]};
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) a.Z[idx + q] = z[q];
      }
    }
    if (a.vecYR) {
      *(v4i*)(a.Y + idx) = v4i{(int)yw[0], (int)yw[1], (int)yw[2], (int)yw[3]};
      *(v4i*)(a.R + idx) = v4i{(int)rw[0], (int)rw[1], (int)rw[2], (int)rw[3]};
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        a.Y[idx + q] = (int8_t)(yw[q >> 2] >> (8 * (q & 3)));
        a.R[idx + q] = (int8_t)(rw[q >> 2] >> (8 * (q & 3)));
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (o0 + q < a.N) {
        if (a.Z) a.Z[idx + q] = z[q];
        a.Y[idx + q] = (int8_t)(yw[q >> 2] >> (8 * (q & 3)));
        a.R[idx + q] = (int8_t)(rw[q >> 2] >> (8 * (q & 3)));
      }
    }
  }
}

// Limb-fold epilogue: a lane's 16 outputs o0.. of token t are the byte limbs
// l = 0..7 of digit-row group o0 / 8 (z[0..7]) and of the next group
// (z[8..15]); the group's value sum_l 2^(8l) z[l] is exact as L + 2^32 H with
// |L|, |H| < 2^55, then reduced, plus the digits' offset term in chunk 0.
__device__ __forceinline__ void limb_fold_store(const WitArgs& a, const int32_t (&z)[16], int t, int o0, int ks) {
  uint64_t cterm = 0;
  if (ks == 0) cterm = gl::mul(gl::from_i64(128 * (int64_t)a.colsum[t]), 0x0101010101010101ull);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int o = o0 + 8 * g;
    if (o >= a.N) break;
    const int32_t* zz = z + 8 * g;
    const int64_t L = (int64_t)zz[0] + (int64_t)zz[1] * 256 + (int64_t)zz[2] * 65536 + (int64_t)zz[3] * 16777216;
    const int64_t H = (int64_t)zz[4] + (int64_t)zz[5] * 256 + (int64_t)zz[6] * 65536 + (int64_t)zz[7] * 16777216;
    const uint64_t v = gl::add(gl::from_i64(L), gl::mul(gl::from_i64(H), 1ull << 32));
    a.part[(int64_t)ks * a.psplit + (int64_t)(o >> 3) * a.ldp + t] = gl::add(v, cterm);
  }
}

// Bytes of K per packed weight block (the K step of the packed-weight kernels).
constexpr int WP_BK = fpi::PACK_BK;

// ---- the claim of a launch's own product, from the accumulators ---------
// Each wave contracts its fragments over the outputs on the matrix cores:
// the 7-bit limbs of E_o (CL_LIMBS per element, rows 0..9 of the A operand)
// against the four byte planes of Z (the B operand: after the swap a lane
// holds 16 consecutive outputs of one token, which is the operand's layout
// with the outputs as k). Planes 0-2 are unsigned bytes, fed as b - 128;
// plane 3 is Z's signed top byte. Row m of the products, weighted
// 2^(7m + 8p), plus the offsets' share, then gives sum_o E_o[o] Z[t, o] for
// the lane's token t, which E_t[t] weights.
constexpr int CL_LIMBS = 10;

// Lane (t, h) of the plane products D[p]: register v holds row m = 8 (v / 4)
// + 4 h + v % 4; rows below CL_LIMBS carry limbs (v < 4 for both halves,
// v = 4, 5 for h = 0). Returns sum_m 2^(7m) sum_p 2^(8p) D_p[m] mod p (the
// offsets of planes 0-2 are added back per wave: sum_m 2^(7m) 128 (1 + 2^8 +
// 2^16) sum_o limb_m(E_o[o]) is 128 * 65793 * sum_o E_o[o]).
__device__ __forceinline__ uint64_t claim_row_value(const v16i (&D)[4], int h) {
  // sum_p 2^(8p) D_p for register v, |.| < 2^46
  auto rowsum = [&](int v) -> __int128 {
    const int32_t s01 = D[0][v] + (D[1][v] << 8);  // |D| < 2^21: exact in 32 bits
    const int32_t s23 = D[2][v] + (D[3][v] << 8);
    return (__int128)((int64_t)s01 + ((int64_t)s23 << 16));
  };
  // registers 0-3 hold rows v + 4h: scale by 2^(7v), then by 2^28 in the upper half
  __int128 x = rowsum(0) + (rowsum(1) << 7) + (rowsum(2) << 14) + (rowsum(3) << 21);
  x = h ? (x << 28) : x;
  // registers 4, 5 hold rows 8, 9 (h = 0; rows 12, 13 of the upper half are zero)
  x += (rowsum(4) << 56) + (rowsum(5) << 63);
  // p 2^48 keeps the sum positive (|x| < 2^110)
  const unsigned __int128 y = (unsigned __int128)x + ((unsigned __int128)0xFFFFFFFF00000001ull << 48);
  return gl::reduce128((uint64_t)y, (uint64_t)(y >> 64));
}

// The wave's claim value to its slot; the last tile to arrive adds them all.
__device__ __forceinline__ void claim_arrive(const WitArgs& a, uint64_t wsum, int bid, int nblocks, int nwaves,
                                             uint64_t* red, uint32_t* flag) {
  const int tid = threadIdx.x;
  wsum = fpi::wave_total(wsum);
  if ((tid & 63) == 0) foldk::store_part(a.cpart + (int64_t)bid * nwaves + (tid >> 6), wsum, true);
  if (!foldk::arrive_last(a.cctr, (uint32_t)nblocks, flag)) return;
  const int nv = nblocks * nwaves;
  uint64_t v = 0;
  for (int i = tid; i < nv; i += (int)blockDim.x) v = gl::add(v, foldk::load_part(a.cpart + i));
  v = fpi::wave_total(v);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  if (tid == 0) {
    uint64_t t = 0;
    for (int w = 0; w < nwaves; ++w) t = gl::add(t, red[w]);
    *a.cout = t;
  }
}

// eq tables built by spare workgroups of a witness launch (a proof's eq
// tables depend on its challenges only, so they can be made while its GEMM
// runs): table i takes aux workgroups [block_start[i], block_start[i+1]),
// each writing 2^(8 + eq_aux_mid(n)) entries.
constexpr int WIT_MAX_EQ = 8;
struct EqAux {
  const fp_elem* r[WIT_MAX_EQ];
  fp_elem* E[WIT_MAX_EQ];
  int32_t n[WIT_MAX_EQ];
  int32_t block_start[WIT_MAX_EQ + 1];
  int32_t count;
};
__host__ __device__ inline int eq_aux_mid(int n) {
  return n <= 8 ? 0 : (n - 8 < eqk::EQ_MAX_MID ? n - 8 : eqk::EQ_MAX_MID);
}
inline int64_t eq_aux_blocks(int n) { return n <= 8 ? 1 : (int64_t)1 << (n - 8 - eq_aux_mid(n)); }

// Aux workgroup b of the launch's eq tables.
__device__ __forceinline__ void eq_aux_block(const EqAux& eq, int b) {
  int k = 0;
#pragma unroll 1
  for (int q = 1; q < eq.count; ++q)
    if (eq.block_start[q] <= b) k = q;
  eqk::eq_block(eq.r[k], eq.n[k], eq.E[k], b - eq.block_start[k], eq_aux_mid(eq.n[k]));
}

// The eq tables a packed witness launch builds beside its GEMM.
inline int eq_aux(const char* fn, int32_t n_eq, const fp_eq_desc* eq, EqAux& aux) {
  aux = EqAux{};
  if (n_eq < 0 || n_eq > WIT_MAX_EQ) return fpi::fail(FP_EARG, "%s: n_eq=%d outside [0, %d]", fn, n_eq, WIT_MAX_EQ);
  if (n_eq > 0 && !eq) return fpi::fail(FP_EARG, "%s: null eq descs", fn);
  int64_t blocks = 0;
  for (int32_t i = 0; i < n_eq; ++i) {
    if (eq[i].n < 0 || eq[i].n > FP_MAX_N)
      return fpi::fail(FP_ESHAPE, "%s: eq table %d has n=%d outside [0, %d]", fn, i, eq[i].n, FP_MAX_N);
    if (!eq[i].E || (eq[i].n > 0 && !eq[i].r)) return fpi::fail(FP_EARG, "%s: eq table %d has a null pointer", fn, i);
    aux.r[i] = eq[i].r;
    aux.E[i] = eq[i].E;
    aux.n[i] = eq[i].n;
    aux.block_start[i] = (int32_t)blocks;
    blocks += eq_aux_blocks(eq[i].n);
    if (blocks > (1 << 24)) return fpi::fail(FP_ESHAPE, "%s: eq tables too large for one launch", fn);
  }
  aux.block_start[n_eq] = (int32_t)blocks;
  aux.count = n_eq;
  return FP_OK;
}

// Fold and claim jobs run by workgroups of a witness launch in arrival mode
// (the last workgroup of each column strip, or of a claim, adds the chunks):
// their descriptors, the arrival counters at the start of the workspace
// (FP_FOLD_COUNTER_BYTES, zero on entry and left zero) and the workgroups.
template <int MAXJ>
struct FoldAuxT {
  foldk::FoldJob j[MAXJ];
  uint32_t* ctrs;
  int32_t count;
  int32_t blocks;
};

// Plans the folds (int8) and claims (int32) of a launch's fold workgroups:
// workspace = arrival counters, then every job's partial values, then (with
// own_parts > 0) own_parts slots for the claim taken from the accumulators,
// whose counter follows the jobs'.
template <int MAXJ>
int plan_folds(const char* fn, int32_t n_fold, const fp_fold_desc* folds, int32_t n_claim,
               const fp_claim_desc* claims, int64_t own_parts, void* ws, size_t ws_bytes, bool plan_only,
               size_t* need, FoldAuxT<MAXJ>& fa, uint64_t** own_part, uint32_t** own_ctr) {
  fa = FoldAuxT<MAXJ>{};
  if (n_fold < 0 || n_claim < 0 || n_fold + n_claim > MAXJ)
    return fpi::fail(FP_EARG, "%s: %d folds and %d claims (at most %d in all)", fn, n_fold, n_claim, MAXJ);
  if ((n_fold > 0 && !folds) || (n_claim > 0 && !claims)) return fpi::fail(FP_EARG, "%s: null descs", fn);
  size_t off = FP_FOLD_COUNTER_BYTES;
  int64_t blocks = 0;
  int32_t nctr = 0;
  for (int32_t i = 0; i < n_fold + n_claim; ++i) {
    const bool claim = i >= n_fold;
    foldk::FoldJob j{};
    if (!claim) {
      const fp_fold_desc& d = folds[i];
      if (d.rows < 0 || d.cols < 0 || d.cols_pad < d.cols || d.ld < d.cols)
        return fpi::fail(FP_ESHAPE, "%s: fold %d has bad sizes", fn, i);
      if ((d.cols_pad > 0 && !d.out) || (d.rows > 0 && d.cols > 0 && (!d.M || !d.E)))
        return fpi::fail(FP_EARG, "%s: fold %d has a null pointer", fn, i);
      if ((d.E2 != nullptr) != (d.out2 != nullptr))
        return fpi::fail(FP_EARG, "%s: fold %d has a second weight vector without its output, or the reverse", fn, i);
      j.M = d.M; j.ld = d.ld; j.E = d.E; j.Ecol = nullptr; j.out = d.out;
      j.E2 = d.E2; j.out2 = d.out2;
      j.rows = d.rows; j.cols = d.cols; j.cols_pad = d.cols_pad; j.eb = 1;
    } else {
      const fp_claim_desc& d = claims[i - n_fold];
      if (d.rows < 0 || d.cols < 0 || d.ld < d.cols) return fpi::fail(FP_ESHAPE, "%s: claim %d has bad sizes", fn, i);
      if (!d.out || (d.rows > 0 && d.cols > 0 && (!d.M || !d.E_rows || !d.E_cols)))
        return fpi::fail(FP_EARG, "%s: claim %d has a null pointer", fn, i);
      j.M = d.M; j.ld = d.ld; j.E = d.E_rows; j.Ecol = d.E_cols; j.out = d.out;
      j.rows = d.rows; j.cols = d.cols; j.cols_pad = d.cols; j.eb = 4;
    }
    if (j.rows == 0 || j.cols == 0)
      return fpi::fail(FP_ESHAPE, "%s: job %d is empty (the step's folds and claims need rows and columns)", fn, i);
    const int64_t span = (int64_t)j.ld * j.eb * (j.rows < foldk::FMAX_CHUNK ? j.rows : foldk::FMAX_CHUNK);
    if (span > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "%s: job %d spans more than 2^31 bytes per chunk", fn, i);
    const foldk::Plan p = foldk::plan_job(j.rows, j.cols, j.cols_pad, j.eb, claim, true);
    const uintptr_t align = j.eb == 1 ? 3 : 15;
    j.vec = (j.cols % 4 == 0) && (j.ld % 4 == 0) && (((uintptr_t)j.M & align) == 0);
    j.chunk_rows = p.chunk_rows;
    j.n_chunks = p.n_chunks;
    j.n_strips = p.n_strips;
    j.n_pad_strips = p.n_pad_strips;
    j.part = p.part_bytes ? (fp_elem*)((char*)ws + off) : nullptr;
    off += p.part_bytes;
    j.part2 = nullptr;
    if (j.E2 && p.part_bytes) {  // the second vector's chunk values after the first's
      j.part2 = (fp_elem*)((char*)ws + off);
      off += p.part_bytes;
    }
    j.block_start = (int32_t)blocks;
    j.ctr = nctr;
    blocks += p.blocks;
    nctr += p.ctrs;
    fa.j[fa.count++] = j;
  }
  *own_part = nullptr;
  *own_ctr = nullptr;
  if (own_parts > 0) {
    *own_part = (uint64_t*)((char*)ws + off);
    off += fpi::align_up((size_t)own_parts * 8, 256);
    *own_ctr = (uint32_t*)ws + nctr;
    nctr += 1;
  }
  if (nctr > (int32_t)(FP_FOLD_COUNTER_BYTES / 4) || blocks > (1 << 24))
    return fpi::fail(FP_ESHAPE, "%s: folds too large for one step", fn);
  fa.blocks = (int32_t)blocks;
  fa.ctrs = (uint32_t*)ws;
  *need = (n_fold + n_claim || own_parts > 0) ? off : 0;
  if (plan_only) return FP_OK;
  if (*need && (!ws || ws_bytes < *need)) return fpi::fail(FP_EWORKSPACE, "%s: workspace %zu < %zu", fn, ws_bytes, *need);
  if (*need && (((uintptr_t)ws) & 255)) return fpi::fail(FP_EARG, "%s: workspace not 256-byte aligned", fn);
  return FP_OK;
}

}  // namespace
