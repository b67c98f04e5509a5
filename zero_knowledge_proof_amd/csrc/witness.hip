// witness.hip - the witness of a fixed-point linear layer on int8 matrix cores.
//
// "How fast can FlashProve go", §2: the model is integer-quantized, so every
// product is rescaled and many results are clamped; §3.1: the rescale
// g_w = round(g^ / 2^k) commits its remainder r = g^ - 2^k g_w, which the
// matmul's sum-check uses in place of g^ (so Z itself is kept for the claim).
// Per output entry:
//   Z = sum_k X[t,k] W[o,k]          (int8 x int8 -> int32, exact)
//   Q = floor((Z + 2^(s-1)) / 2^s)   (ties up), computed as (Z + 2^(s-1)) >> s
//   R = Z - 2^s Q
//   Y = clamp(Q, -128, 127)
// Z + 2^(s-1) cannot overflow int32: |Z| <= 2^14 d_in <= 2^31 - 2^14 for
// d_in <= FP_MAX_DIN, and 2^(s-1) <= 128.
//
// Kernel. X [T, K] and W [d_out, K] are both K-contiguous, the operand order
// of v_mfma_i32_32x32x32_i8: lane l feeds row l%32 with the 16 bytes at
// k = 16*(l/32) of a 32-wide K slice, for both operands, so the products pair
// equal k. W rows are the MFMA rows and X rows its columns: a lane's 16
// accumulators then hold one token t and output columns o = 8g + 4h + (0..3)
// (g = 0..3, h = l/32). Two v_permlane32_swap per 4 accumulators exchange the
// g = 1,3 halves between lanes l and l+32, after which each lane holds 16
// consecutive o of one t: Z leaves as four 16-byte stores and Y, R as one
// 16-byte store each. Workgroup tiles are BO x BT (outputs x tokens), wave
// tiles WO x WT; K steps of BK bytes are double-buffered through LDS with the
// next steps' tiles staged in registers, rows padded by 16 bytes so the
// 16-byte reads of 16 consecutive rows hit distinct bank groups (an unpadded
// 64- or 128-byte pitch measures 3-6x slower). Workgroup ids are remapped so that each XCD (ids are dealt to
// the 8 XCDs round-robin) works on a contiguous run of tiles; tokens vary
// fastest, so one W panel is shared by the XCD's tiles in its L2.
#include <utility>

#include "common.hpp"
#include "eq.hpp"
#include "fold.hpp"
#include "sc_tail.hpp"
#include "witness_dev.hpp"

namespace {

// LDS of one GEMM workgroup: double-buffered W and X tiles.
template <int BO, int BT, int BK>
struct WitLds {
  __align__(16) int8_t sA[2][BO * (BK + 16)];  // W rows
  __align__(16) int8_t sB[2][BT * (BK + 16)];  // X rows
};

// Tile `bid` of `nblocks` GEMM workgroups.
template <int BO, int BT, int WO, int WT, bool GROUPED, int PF, int BK, int EPI>
__device__ __forceinline__ void witness_body(const WitArgs& a, const GroupTab& gt, int bid, int nblocks,
                                             WitLds<BO, BT, BK>& sh) {
  constexpr int PITCH = BK + 16;  // LDS row pitch: 16 consecutive rows start in distinct bank groups
  constexpr int CPR = BK / 16;    // 16-byte chunks per row
  constexpr int WAVES_T = BT / WT;
  constexpr int NT = (BO / WO) * WAVES_T * 64;
  constexpr int TM = WO / 32, TN = WT / 32;
  constexpr int NCA = BO * CPR, NCB = BT * CPR;  // 16-byte chunks per K step
  constexpr int CA = (NCA + NT - 1) / NT;
  constexpr int CB = (NCB + NT - 1) / NT;
  auto& sA = sh.sA;
  auto& sB = sh.sB;

  int tile = xcd_tile(bid, nblocks);
  int ks = 0;
  if (a.ksplit > 1) {
    const int per = a.tiles_t * a.tiles_o;
    ks = tile / per;
    tile -= ks * per;
  }
  const int tt = tile % a.tiles_t;
  const int to = tile / a.tiles_t;
  const int kb = ks * a.kchunk;                                   // this workgroup's K range
  const int klen = (a.ksplit > 1) ? min(a.kchunk, a.K - kb) : a.K;

  const int8_t* Wb = a.W;
  int t_base, t_lim;  // token rows [t_base, t_lim) valid for this tile's group
  if constexpr (GROUPED) {
    int lo = 0, hi = gt.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gt.tile_off[mid] <= tt) lo = mid; else hi = mid - 1;
    }
    Wb = gt.W[lo];
    t_base = gt.row_off[lo] + (tt - gt.tile_off[lo]) * BT;
    t_lim = gt.row_off[lo + 1];
  } else {
    t_base = tt * BT;
    t_lim = a.T;
  }
  const int o_base = to * BO;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wo0 = (wave / WAVES_T) * WO;
  const int wt0 = (wave % WAVES_T) * WT;

  // Rows past the matrix are clamped to its last row: their products land in
  // outputs that are never stored, and every load stays in bounds.
  const int8_t* pa[CA];
  const int8_t* pb[CB];
  int sa_off[CA], sb_off[CB], ka[CA], kb_[CB];
#pragma unroll
  for (int c = 0; c < CA; ++c) {
    const int ch = tid + c * NT;
    const int row = ch / CPR, kc = (ch % CPR) * 16;
    const int g = min(o_base + row, a.N - 1);
    pa[c] = Wb + (int64_t)g * a.ldw + kb;
    ka[c] = kc;
    sa_off[c] = (ch < NCA) ? row * PITCH + kc : -1;
  }
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int ch = tid + c * NT;
    const int row = ch / CPR, kc = (ch % CPR) * 16;
    const int g = min(t_base + row, t_lim - 1);
    pb[c] = a.X + (int64_t)g * a.ldx + kb;
    kb_[c] = kc;
    sb_off[c] = (ch < NCB) ? row * PITCH + kc : -1;
  }
  // register staging for PF K steps ahead; whole 16-byte chunks when the K step
  // lies inside the matrix and the rows are 16-byte aligned (a uniform branch)
  const bool vec_all = a.vecX && a.vecW;
  v4i ra[PF][CA], rb[PF][CB];
  auto gload = [&](int slot, int k0) {
    if (vec_all && k0 + BK <= klen) {
#pragma unroll
      for (int c = 0; c < CA; ++c) ra[slot][c] = *(const v4i*)(pa[c] + k0 + ka[c]);
#pragma unroll
      for (int c = 0; c < CB; ++c) rb[slot][c] = *(const v4i*)(pb[c] + k0 + kb_[c]);
    } else {
#pragma unroll
      for (int c = 0; c < CA; ++c) ra[slot][c] = load16(pa[c], k0 + ka[c], klen, a.vecW);
#pragma unroll
      for (int c = 0; c < CB; ++c) rb[slot][c] = load16(pb[c], k0 + kb_[c], klen, a.vecX);
    }
  };
  auto sstore = [&](int slot, int buf) {
#pragma unroll
    for (int c = 0; c < CA; ++c)
      if (NCA % NT == 0 || sa_off[c] >= 0) *(v4i*)&sA[buf][sa_off[c]] = ra[slot][c];
#pragma unroll
    for (int c = 0; c < CB; ++c)
      if (NCB % NT == 0 || sb_off[c] >= 0) *(v4i*)&sB[buf][sb_off[c]] = rb[slot][c];
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  const int KT = (klen + BK - 1) / BK;
  const int lrow = lane & 31, lk = (lane >> 5) * 16;
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      v4i fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = *(const v4i*)&sA[buf][(wo0 + 32 * i + lrow) * PITCH + kk * 32 + lk];
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = *(const v4i*)&sB[buf][(wt0 + 32 * j + lrow) * PITCH + kk * 32 + lk];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  // Pipeline: while step s is multiplied out of LDS buffer s%2, the loads of
  // step s+PF are in flight into register slot s%PF; step s+1's registers go
  // to the other LDS buffer after the MFMAs, then one barrier. U = lcm(PF, 2)
  // steps are unrolled so that slots and buffers are compile-time indices.
  constexpr int U = (PF % 2 == 0) ? PF : 2 * PF;
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < KT) gload(p, p * BK);
  sstore(0, 0);
  __syncthreads();
  for (int kt = 0; kt < KT; kt += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = kt + u;
      if (st < KT) {
        if (st + PF < KT) gload(u % PF, (st + PF) * BK);
        compute(u % 2);
        if (st + 1 < KT) sstore((u + 1) % PF, (u + 1) % 2);
        __syncthreads();
      }
    }
  }

  // ---- epilogue: 16 consecutive outputs per lane, rescale, clamp, remainder
  const int s = a.s;
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int32_t z[16];
      fragment_outputs(acc[i][j], z);
      const int t = t_base + wt0 + 32 * j + (lane & 31);
      const int o0 = o_base + wo0 + 32 * i + 16 * h;
      if (t >= t_lim || o0 >= a.N) continue;
      if constexpr (EPI == 1) {
        limb_fold_store(a, z, t, o0, ks);
        continue;
      }
      store_fragment(a, z, t, o0, s);
    }
  }
}

template <int BO, int BT, int WO, int WT, bool GROUPED, int PF = 1, int BK = 64, int EPI = 0>
__global__ __launch_bounds__((BO / WO) * (BT / WT) * 64) void witness_kernel(WitArgs a, GroupTab gt) {
  __shared__ WitLds<BO, BT, BK> sh;
  witness_body<BO, BT, WO, WT, GROUPED, PF, BK, EPI>(a, gt, blockIdx.x, gridDim.x, sh);
}

// The GEMM together with sum-check tails: workgroups [0, n_tail) each run one
// tail instance (they are dispatched first, so the latency-bound tail overlaps
// the GEMM), the rest are GEMM tiles. The tail's LDS is carved from the GEMM's.
template <int BO, int BT, int WO, int WT, bool GROUPED, int PF = 1, int BK = 64>
__global__ __launch_bounds__((BO / WO) * (BT / WT) * 64) void witness_sc_kernel(WitArgs a, GroupTab gt,
                                                                               sct::TailArgs ta, int n_tail) {
  constexpr int NT = (BO / WO) * (BT / WT) * 64;
  __shared__ WitLds<BO, BT, BK> sh;
  static_assert(sizeof(sct::TailLds<NT>) <= sizeof(WitLds<BO, BT, BK>), "tail LDS must fit the GEMM's");
  if ((int)blockIdx.x < n_tail) {
    sct::tail_body<NT>(ta, blockIdx.x, *reinterpret_cast<sct::TailLds<NT>*>(&sh));
    return;
  }
  witness_body<BO, BT, WO, WT, GROUPED, PF, BK, 0>(a, gt, blockIdx.x - n_tail, gridDim.x - n_tail, sh);
}


// ---- packed weights: W streamed straight into the MFMA registers ----------
// The weights of a layer are fixed, so they can be laid out once in the order
// the matrix cores read them: fragment (row block b, K block c, step q) is
// 1 KiB, lane l holding W[32 b + l%32][WP_BK c + (l/32) WP_BK/2 + 16 q + 0..15]
// (zero past d_out and d_in). Within a K block the two lane halves take
// different byte ranges of the same rows; X is staged in LDS in the same
// order, so both operands pair equal k and the sum over k is unchanged. A
// wave's weight fragments are then single coalesced 1 KiB loads that no other
// wave needs, and only X (shared by the workgroup's waves) passes through LDS:
// half the LDS traffic per MFMA of the tile above, and the register copy of
// each W byte is used against all of the workgroup's tokens.

__global__ __launch_bounds__(256) void pack_weights_kernel(const int8_t* __restrict__ W, int64_t ldw, int32_t N,
                                                           int32_t K, int32_t nrb, int32_t nkb, int vec,
                                                           int8_t* __restrict__ Wp) {
  constexpr int KS = WP_BK / 32;
  const int64_t units = (int64_t)nrb * nkb * KS * 64;  // 16-byte units
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    const int l = (int)(u & 63);
    int64_t f = u >> 6;  // (b nkb + c) KS + q
    const int q = (int)(f % KS);
    f /= KS;
    const int c = (int)(f % nkb);
    const int b = (int)(f / nkb);
    const int row = 32 * b + (l & 31);
    const int k = WP_BK * c + (l >> 5) * (WP_BK / 2) + 16 * q;
    v4i val = {0, 0, 0, 0};
    if (row < N) val = load16(W + (int64_t)row * ldw, k, K, vec != 0);
    *(v4i*)(Wp + u * 16) = val;
  }
}

// Tile `bid` of `nblocks`: NW waves, wave w owning weight rows
// [o_base + 32 TM w, +32 TM) (fragments from the packed weights, PFW K blocks
// ahead) and all BT = 32 TN tokens of the tile (X through double-buffered
// LDS, PFX K blocks ahead in registers). Every K block issues its loads
// unconditionally (past the end they re-read the last block), so the code
// between barriers is straight-line and the compiler's wait counts let the
// prefetches stay in flight. X chunks past d_in are read from column 0: they
// meet zero weights. Requires d_in % 16 == 0 and 16-byte aligned X rows.
template <int NW, int TM, int TN, int PFW, int PFX, int UNR>
struct WsCfg {
  static constexpr int NT = NW * 64, BO = NW * 32 * TM, BT = 32 * TN, BK = WP_BK;
  static constexpr int PITCH = BK + 16, CPR = BK / 16, CB = BT * CPR / NT, KS = BK / 32, HB = BK / 2;
  // the epilogue stages each wave's 32x32 int32 fragments in rows of EP words;
  // the claim's limb table [CL_LIMBS][BO], the tile's E_t, reduction words and
  // the waves' offset terms sit past both that and the X tiles
  static constexpr int EP = 36, STAGE_BYTES = NW * 32 * EP * 4;
  static constexpr int LOOP_BYTES = 2 * BT * PITCH;
  // the claim's tables sit past the X tiles and the Z staging: they are
  // filled while the K loop runs
  static constexpr int CLAIM_OFF = LOOP_BYTES > STAGE_BYTES ? LOOP_BYTES : STAGE_BYTES;
  static constexpr int CLAIM_BYTES = CL_LIMBS * BO + 8 * BT + 16 * 8 + 8 * NW;
  static constexpr int LDS_BYTES = CLAIM_OFF + CLAIM_BYTES;
  static_assert((BT * CPR) % NT == 0, "X chunks per thread");
};

template <int NW, int TM, int TN, int PFW, int PFX, int UNR, int EPI = 0>
__device__ __forceinline__ void witness_body_ws(const WitArgs& a, int bid, int nblocks, int8_t* lds) {
  using C = WsCfg<NW, TM, TN, PFW, PFX, UNR>;
  constexpr int NT = C::NT, BO = C::BO, BT = C::BT, BK = C::BK, PITCH = C::PITCH, CPR = C::CPR, CB = C::CB;
  constexpr int KS = C::KS, HB = C::HB;
  int8_t (*sB)[BT * PITCH] = reinterpret_cast<int8_t (*)[BT * PITCH]>(lds);
  int tile = xcd_tile(bid, nblocks);
  int ks = 0;  // split K: workgroup (tile, ks) reduces over K blocks [kb0, kb0 + KT)
  if (a.ksplit > 1) {
    const int per = a.tiles_t * a.tiles_o;
    ks = tile / per;
    tile -= ks * per;
  }
  const int kb0 = a.ksplit > 1 ? ks * (a.kchunk / BK) : 0;
  const int KT = a.ksplit > 1 ? min(a.kchunk / BK, a.wp_kb - kb0) : a.wp_kb;
  const int klim = a.K - kb0 * BK;  // X columns left from the range's start
  const int tt = tile % a.tiles_t, to = tile / a.tiles_t;
  const int t_base = tt * BT, o_base = to * BO;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int wo0 = wave * 32 * TM;
  const int64_t rb_bytes = (int64_t)a.wp_kb * BK * 32;  // one 32-row block of the packed weights
  const int8_t* pw[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
    pw[i] = a.W + (int64_t)min((o_base + wo0) / 32 + i, a.wp_rb - 1) * rb_bytes + (int64_t)kb0 * (BK * 32) + lane * 16;
  const int8_t* px[CB];
  int kc[CB], so[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int ch = tid + c * NT, row = ch / CPR;
    kc[c] = (ch % CPR) * 16;
    px[c] = a.X + (int64_t)min(t_base + row, a.T - 1) * a.ldx + (int64_t)kb0 * BK;
    so[c] = row * PITCH + kc[c];
  }
  // the claim's tables: E_t and E_o are read before the K loop's first loads
  // and put in LDS once those are issued (the loop's barriers order the
  // writes before the epilogue's reads). The layer step runs one wave of
  // tiles, so the tables' latency was on its critical path: 1% of a T=512
  // step. (Y and R staged through LDS as whole row pieces measured 2% slower.)
  uint8_t* limbs = reinterpret_cast<uint8_t*>(lds) + C::CLAIM_OFF;
  uint64_t* etl = reinterpret_cast<uint64_t*>(lds + C::CLAIM_OFF + CL_LIMBS * BO);  // E_t of the tile's tokens
  uint64_t* red = etl + BT;
  uint64_t* wcorr = red + 16;
  const bool claim = EPI == 0 && a.cEt != nullptr;
  static_assert(BT <= NT && BO <= NT, "one E_t and one E_o entry per thread");
  uint64_t et_v = 0, eo_v = 0;
  auto load_tables = [&]() {
    if (!claim) return;
    if (tid < BT && t_base + tid < a.T) et_v = a.cEt[t_base + tid];
    // zero past d_out, so rows of Z there, computed from clamped weight blocks, do not count
    if (tid < BO && o_base + tid < a.N) eo_v = a.cEo[o_base + tid];
  };
  auto write_tables = [&]() {
    if (!claim) return;
    if (tid < BT) etl[tid] = et_v;
    uint64_t se = 0;
    if (tid < BO) {
#pragma unroll
      for (int m = 0; m < CL_LIMBS; ++m) limbs[m * BO + tid] = (uint8_t)((eo_v >> (7 * m)) & 127u);
      if constexpr (BO == NT) se = eo_v;  // output tid is lane tid % 64 of its wave's range
    }
    if constexpr (BO != NT) {
#pragma unroll
      for (int x = lane; x < 32 * TM; x += 64) {
        const int o = o_base + wo0 + x;
        if (o < a.N) se = gl::add(se, a.cEo[o]);
      }
    }
    se = fpi::wave_total(se);  // every lane takes part
    if (lane == 0) wcorr[wave] = gl::mul_small(se, 128u * 65793u);
  };
  load_tables();
  v4i wf[PFW][TM][KS];
  v4i xr[PFX][CB];
  auto wload = [&](int slot, int kblk) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < KS; ++q) wf[slot][i][q] = *(const v4i*)(pw[i] + (int64_t)kblk * (BK * 32) + 1024 * q);
  };
  auto xload = [&](int slot, int kblk) {
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int k = kblk * BK + kc[c];
      xr[slot][c] = *(const v4i*)(px[c] + (k < klim ? k : 0));
    }
  };
  auto sstore = [&](int slot, int buf) {
#pragma unroll
    for (int c = 0; c < CB; ++c) *(v4i*)&sB[buf][so[c]] = xr[slot][c];
  };
  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;
  auto compute = [&](int buf, int ws) {
    const int8_t* B = &sB[buf][r * PITCH + HB * h];
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      v4i fb[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = *(const v4i*)(B + 32 * j * PITCH + 16 * q);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[ws][i][q], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  // K block s: multiply out of LDS buffer s%2 with weight slot s%PFW, refill
  // that slot with block s+PFW, store block s+1 (register slot (s+1)%PFX) into
  // the other buffer and refill its slot with block s+1+PFX; one barrier.
  constexpr int L1 = (PFW % 2 == 0) ? PFW : 2 * PFW;
  constexpr int U = ((L1 % PFX == 0) ? L1 : L1 * PFX) * UNR;
  if (KT > 0) {  // d_in = 0: every output is 0
#pragma unroll
    for (int p = 0; p < PFW; ++p) wload(p, min(p, KT - 1));
#pragma unroll
    for (int p = 0; p < PFX; ++p) xload(p, min(p, KT - 1));
    sstore(0, 0);
    xload(0, min(PFX, KT - 1));
    write_tables();
    __syncthreads();
    auto step = [&](auto uc, int st) {
      constexpr int u = decltype(uc)::value;
      compute(u % 2, u % PFW);
      wload(u % PFW, min(st + PFW, KT - 1));
      sstore((u + 1) % PFX, (u + 1) % 2);
      xload((u + 1) % PFX, min(st + 1 + PFX, KT - 1));
      __syncthreads();
    };
    int kt = 0;
    for (; kt + U <= KT; kt += U) {
      [&]<int... I>(std::integer_sequence<int, I...>) { (step(std::integral_constant<int, I>{}, kt + I), ...); }(
          std::make_integer_sequence<int, U>{});
    }
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((kt + I < KT ? step(std::integral_constant<int, I>{}, kt + I) : void()), ...);
    }(std::make_integer_sequence<int, U>{});
  } else {
    write_tables();
  }

  if constexpr (EPI == 1) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int32_t z[16];
        fragment_outputs(acc[i][j], z);
        const int t = t_base + 32 * j + r;
        const int o0 = o_base + wo0 + 32 * i + 16 * h;
        if (t < a.T && o0 < a.N) limb_fold_store(a, z, t, o0, ks);
      }
    return;
  }
  const int s = a.s;
  // Z leaves through LDS: a lane's fragment holds 16 outputs of one token,
  // so direct stores write 32-byte pieces of 32 rows; staged, eight lanes
  // write a row's whole 128 bytes.
  const bool stage = a.Z != nullptr && a.vecZ;
  if (stage || claim) __syncthreads();  // every wave is done with the X tiles
  int32_t* E = reinterpret_cast<int32_t*>(lds) + wave * 32 * C::EP;
  v4i Aop[TM];
  uint64_t corr = 0;  // the planes' offsets, added once per token (by the h = 0 lanes)
  if (claim) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      Aop[i] = r < CL_LIMBS ? *(const v4i*)&limbs[r * BO + wo0 + 32 * i + 16 * h] : v4i{0, 0, 0, 0};
    corr = h == 0 ? wcorr[wave] : 0;
  }
  WitArgs yr = a;
  if (stage) yr.Z = nullptr;
  uint64_t wsum = 0;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    v16i D[4];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      int32_t z[16];
      fragment_outputs(acc[i][j], z);
      const int t = t_base + 32 * j + r;
      const int o0 = o_base + wo0 + 32 * i + 16 * h;
      if (t < a.T && o0 < a.N) store_fragment(yr, z, t, o0, s);
      if (stage) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(v4i*)&E[r * C::EP + 16 * h + 4 * q] = v4i{z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]};
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int row = 8 * p + (lane >> 3), c4 = (lane & 7) * 4;
          const v4i v = *(const v4i*)&E[row * C::EP + c4];
          const int tz = t_base + 32 * j + row, oz = o_base + wo0 + 32 * i + c4;
          if (tz < a.T && oz < a.N) *(v4i*)(a.Z + (int64_t)tz * a.N + oz) = v;  // N % 4 == 0
        }
        __builtin_amdgcn_wave_barrier();
      }
      if (claim) {
        v4i P[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint32_t w0, w1, w2, w3;
          foldk::transpose4((uint32_t)z[4 * g], (uint32_t)z[4 * g + 1], (uint32_t)z[4 * g + 2], (uint32_t)z[4 * g + 3],
                            w0, w1, w2, w3);
          P[0][g] = (int)(w0 ^ 0x80808080u);
          P[1][g] = (int)(w1 ^ 0x80808080u);
          P[2][g] = (int)(w2 ^ 0x80808080u);
          P[3][g] = (int)w3;
        }
        const v16i zero = {};
#pragma unroll
        for (int p = 0; p < 4; ++p)
          D[p] = __builtin_amdgcn_mfma_i32_32x32x32_i8(Aop[i], P[p], i == 0 ? zero : D[p], 0, 0, 0);
      }
    }
    if (claim) wsum = gl::add(wsum, gl::mul(gl::add(claim_row_value(D, h), corr), etl[32 * j + r]));
  }
  if (claim) claim_arrive(a, wsum, bid, nblocks, NW, red, reinterpret_cast<uint32_t*>(red + 8));
}

// 256x64 workgroup tiles (outputs x tokens): 4 waves of 64x64, weight
// fragments two K blocks ahead, X two blocks ahead; two workgroups per CU.
#define WIT_WS 4, 2, 2, 2, 2, 4
// 256x128 tiles (4 waves of 64x128): each weight fragment in registers meets
// twice the tokens, for shapes with enough tiles to fill the GPU.
#define WIT_WS_L 4, 2, 4, 2, 2, 2

// Workgroups [0, n_tail): sum-check tails (as witness_sc_kernel); the next
// eq.block_start[eq.count]: eq tables; the rest: GEMM tiles (times the K
// split). EPI 1: the limb-fold epilogue instead of the rescale.
template <int NW, int TM, int TN, int PFW, int PFX, int UNR, int EPI = 0>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void witness_ws_kernel(
    WitArgs a, sct::TailArgs ta, int n_tail, EqAux eq) {
  constexpr int NT = NW * 64;
  static_assert(NT == 256, "the eq blocks and the tail are written for 256 threads");
  constexpr int GEMM_LDS = WsCfg<NW, TM, TN, PFW, PFX, UNR>::LDS_BYTES;
  constexpr int BYTES = GEMM_LDS > (int)sizeof(sct::TailLds<NT>) ? GEMM_LDS : (int)sizeof(sct::TailLds<NT>);
  __shared__ __align__(16) int8_t lds[BYTES];
  int b = blockIdx.x;
  if (b < n_tail) {
    sct::tail_body<NT>(ta, b, *reinterpret_cast<sct::TailLds<NT>*>(lds));
    return;
  }
  b -= n_tail;
  const int n_eq = eq.block_start[eq.count];
  if (b < n_eq) {
    eq_aux_block(eq, b);
    return;
  }
  witness_body_ws<NW, TM, TN, PFW, PFX, UNR, EPI>(a, b - n_eq, gridDim.x - n_tail - n_eq, lds);
}

template <int NW, int TM, int TN, int PFW, int PFX, int UNR, int EPI = 0>
int launch_ws(WitArgs a, const sct::TailArgs* ta, int n_tail, const EqAux& eq, hipStream_t st) {
  using C = WsCfg<NW, TM, TN, PFW, PFX, UNR>;
  a.tiles_t = (a.T + C::BT - 1) / C::BT;
  a.tiles_o = (a.N + C::BO - 1) / C::BO;
  const int64_t tiles =
      (a.T > 0 && a.N > 0) ? (int64_t)a.tiles_t * a.tiles_o * (a.ksplit > 1 ? a.ksplit : 1) : 0;
  const int64_t total = tiles + n_tail + eq.block_start[eq.count];
  if (total > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "witness: too many tiles");
  if (total == 0) return FP_OK;
  sct::TailArgs none{};
  hipLaunchKernelGGL((witness_ws_kernel<NW, TM, TN, PFW, PFX, UNR, EPI>), dim3((unsigned)total), dim3(C::NT), 0, st,
                     a, ta ? *ta : none, n_tail, eq);
  return fpi::check_launch("witness_ws_kernel");
}

// ---- one step of a stream of layer proofs in one launch ------------------
// Proof k's witness GEMM and eq tables, proof k-1's folds and claim and proof
// k-2's sum-check: the three touch different data, so one launch runs them
// side by side. Workgroups: [0, n_tail) sum-check tail, then the eq tables,
// then the GEMM tiles, then the fold and claim workgroups in arrival mode (the
// last workgroup of each strip or claim adds the chunks), whose work hides
// under the GEMM's on the compute units it leaves free.
constexpr int STEP_MAX_FOLD = 4;
using FoldAux = FoldAuxT<STEP_MAX_FOLD>;

template <int NW, int TM, int TN, int PFW, int PFX, int UNR>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void layer_step_kernel(
    WitArgs a, sct::TailArgs ta, int n_tail, EqAux eq, FoldAux fa) {
  constexpr int NT = NW * 64;
  static_assert(NT == foldk::FT, "the fold, eq and tail workgroups are written for 256 threads");
  constexpr int GEMM_LDS = WsCfg<NW, TM, TN, PFW, PFX, UNR>::LDS_BYTES;
  constexpr int FOLD_LDS = foldk::LDS_WORDS * 4 + foldk::MAXG_ALL * 8 + 16;
  constexpr int TAIL_LDS = (int)sizeof(sct::TailLds<NT>);
  constexpr int B1 = GEMM_LDS > TAIL_LDS ? GEMM_LDS : TAIL_LDS;
  constexpr int BYTES = B1 > FOLD_LDS ? B1 : FOLD_LDS;
  __shared__ __align__(16) int8_t lds[BYTES];
  int b = blockIdx.x;
  if (b < n_tail) {
    sct::tail_body<NT>(ta, b, *reinterpret_cast<sct::TailLds<NT>*>(lds));
    return;
  }
  b -= n_tail;
  const int n_eq = eq.block_start[eq.count];
  if (b < n_eq) {
    eq_aux_block(eq, b);
    return;
  }
  b -= n_eq;
  const int tiles = (int)gridDim.x - n_tail - n_eq - fa.blocks;
  if (b < tiles) {
    witness_body_ws<NW, TM, TN, PFW, PFX, UNR>(a, b, tiles, lds);
    return;
  }
  b -= tiles;
  const foldk::FoldJob& job = fa.j[foldk::find_job(fa.j, fa.count, b)];
  uint32_t* fl = reinterpret_cast<uint32_t*>(lds);
  uint64_t* gsum = reinterpret_cast<uint64_t*>(lds + foldk::LDS_WORDS * 4);
  uint32_t* flag = reinterpret_cast<uint32_t*>(gsum + foldk::MAXG_ALL);
  foldk::fold_block_arrive(job, b - job.block_start, fa.ctrs, fl, gsum, flag);
}

template <int NW, int TM, int TN, int PFW, int PFX, int UNR>
int launch_step(WitArgs a, const sct::TailArgs* ta, int n_tail, const EqAux& eq, const FoldAux& fa,
                hipStream_t st) {
  using C = WsCfg<NW, TM, TN, PFW, PFX, UNR>;
  a.tiles_t = (a.T + C::BT - 1) / C::BT;
  a.tiles_o = (a.N + C::BO - 1) / C::BO;
  const int64_t tiles = (a.T > 0 && a.N > 0) ? (int64_t)a.tiles_t * a.tiles_o : 0;
  const int64_t total = tiles + n_tail + eq.block_start[eq.count] + fa.blocks;
  if (total > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "layer step: too many workgroups");
  if (total == 0) return FP_OK;
  sct::TailArgs none{};
  hipLaunchKernelGGL((layer_step_kernel<NW, TM, TN, PFW, PFX, UNR>), dim3((unsigned)total), dim3(C::NT), 0, st, a,
                     ta ? *ta : none, n_tail, eq, fa);
  return fpi::check_launch("layer_step_kernel");
}

// Tile configurations (BO, BT, WO, WT, grouped, prefetch distance, K step),
// chosen from measurements on the up-projection and layer shapes:
//   XL: 256x256 outputs x tokens, 8 waves of 64x128, K step 64
//   M : 128x128, 4 waves of 64x64, K step 128
//   S : 256x32 for few tokens (and MoE groups), 4 waves of 64x32
#define WIT_XL 256, 256, 64, 128, false, 1, 64
#define WIT_M 128, 128, 64, 64, false, 1, 128
#define WIT_S 256, 32, 64, 32, false, 1, 64
#define WIT_SG 256, 32, 64, 32, true, 1, 64

template <int BO, int BT, int WO, int WT, bool GROUPED, int PF = 1, int BK = 64, int EPI = 0>
int launch(WitArgs a, const GroupTab& gt, hipStream_t st) {
  if (!GROUPED) a.tiles_t = (a.T + BT - 1) / BT;
  a.tiles_o = (a.N + BO - 1) / BO;
  const int64_t blocks = (int64_t)a.tiles_t * a.tiles_o * (a.ksplit > 1 ? a.ksplit : 1);
  if (blocks <= 0) return FP_OK;
  if (blocks > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "witness: too many tiles");
  hipLaunchKernelGGL((witness_kernel<BO, BT, WO, WT, GROUPED, PF, BK, EPI>), dim3((unsigned)blocks),
                     dim3((BO / WO) * (BT / WT) * 64), 0, st, a, gt);
  return fpi::check_launch("witness_kernel");
}

template <int BO, int BT, int WO, int WT, bool GROUPED, int PF = 1, int BK = 64>
int launch_with_tail(WitArgs a, const GroupTab& gt, const sct::TailArgs& ta, int n_tail, hipStream_t st) {
  constexpr int NT = (BO / WO) * (BT / WT) * 64;
  if (!GROUPED) a.tiles_t = (a.T + BT - 1) / BT;
  a.tiles_o = (a.N + BO - 1) / BO;
  const int64_t tiles = (a.T > 0 && a.N > 0) ? (int64_t)a.tiles_t * a.tiles_o : 0;
  if (tiles + n_tail > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "witness: too many tiles");
  hipLaunchKernelGGL((witness_sc_kernel<BO, BT, WO, WT, GROUPED, PF, BK>), dim3((unsigned)(tiles + n_tail)), dim3(NT),
                     0, st, a, gt, ta, n_tail);
  return fpi::check_launch("witness_sc_kernel");
}

// Threads of the workgroups the witness launch uses for a shape.
int witness_threads(int32_t T, int32_t d_out) {
  const int64_t xl_tiles = (int64_t)((d_out + 255) / 256) * ((T + 255) / 256);
  if (T <= 32) return 256;
  return xl_tiles >= 256 ? 512 : 256;
}

int validate(const char* fn, int64_t ldx, int64_t ldw, int32_t T, int32_t d_in, int32_t d_out, int32_t s,
             const int8_t* Y, const int8_t* R) {
  if (T < 0 || d_in < 0 || d_out < 0) return fpi::fail(FP_EARG, "%s: negative size", fn);
  if (d_in > FP_MAX_DIN) return fpi::fail(FP_ESHAPE, "%s: d_in=%d > %d (int32 Z would not be exact)", fn, d_in, FP_MAX_DIN);
  if (s < 1 || s > 8) return fpi::fail(FP_ERANGE, "%s: s=%d outside [1, 8]", fn, s);
  if (ldx < d_in || ldw < d_in) return fpi::fail(FP_ESHAPE, "%s: leading dimension < d_in", fn);
  if ((int64_t)T * d_out > 0 && (!Y || !R)) return fpi::fail(FP_EARG, "%s: null Y or R", fn);
  return FP_OK;
}

void vec_flags(WitArgs& a) {
  a.vecX = ((a.ldx & 15) == 0) && ((((uintptr_t)a.X) & 15) == 0);
  a.vecZ = ((a.N & 3) == 0) && ((((uintptr_t)a.Z) & 15) == 0);
  a.vecYR = ((a.N & 15) == 0) && ((((uintptr_t)a.Y) & 15) == 0) && ((((uintptr_t)a.R) & 15) == 0);
}

// Checks and packs the arguments of a sum-check that runs as the tail of a
// witness launch of nt-thread workgroups.
int tail_args(const char* fn, int32_t n_pairs, const fp_elem* const* A, const fp_elem* const* B, const fp_elem* rho,
              int32_t n, const fp_elem* r, fp_elem* rounds, fp_elem* finals, fp_elem* claim0, int nt,
              sct::TailArgs& ta) {
  if (n_pairs < 1 || n_pairs > sct::SC_MAX_PAIRS)
    return fpi::fail(FP_EARG, "%s: n_pairs=%d outside [1, %d]", fn, n_pairs, sct::SC_MAX_PAIRS);
  if (n < 1 || n > FP_MAX_N) return fpi::fail(FP_ESHAPE, "%s: n=%d outside [1, %d]", fn, n, FP_MAX_N);
  if (!A || !B || !r || !rounds || !finals) return fpi::fail(FP_EARG, "%s: null sum-check pointer", fn);
  for (int j = 0; j < n_pairs; ++j)
    if (!A[j] || !B[j]) return fpi::fail(FP_EARG, "%s: null table %d", fn, j);
  int vp = 1;
  while (vp < n_pairs) vp <<= 1;
  if (((int64_t)vp << n) > (int64_t)nt * sct::SLMAX)
    return fpi::fail(FP_ESHAPE, "%s: %d x 2^%d table entries exceed one %d-thread workgroup (%d)", fn, vp, n, nt,
                     nt * sct::SLMAX);
  ta = sct::TailArgs{};
  for (int j = 0; j < n_pairs; ++j) {
    ta.user.A[j] = A[j];
    ta.user.B[j] = B[j];
  }
  ta.rho = rho; ta.r = r; ta.rounds = rounds; ta.finals = finals; ta.claim0 = claim0;
  ta.i0 = 0; ta.n = n; ta.n_pairs = n_pairs; ta.nprev = 0; ta.multi = 0;
  return FP_OK;
}

}  // namespace

extern "C" int fp_witness_linear(const int8_t* X, int64_t ldx, const int8_t* W, int64_t ldw, int32_t T, int32_t d_in,
                                 int32_t d_out, int32_t s, int32_t* Z, int8_t* Y, int8_t* R, hipStream_t stream) {
  int rc = validate("fp_witness_linear", ldx, ldw, T, d_in, d_out, s, Y, R);
  if (rc) return rc;
  if (T == 0 || d_out == 0) return fpi::ok();
  if (d_in > 0 && (!X || !W)) return fpi::fail(FP_EARG, "fp_witness_linear: null X or W");
  WitArgs a{};
  a.X = X; a.ldx = ldx; a.W = W; a.ldw = ldw;
  a.T = T; a.N = d_out; a.K = d_in; a.s = s;
  a.Z = Z; a.Y = Y; a.R = R;
  vec_flags(a);
  a.vecW = ((ldw & 15) == 0) && ((((uintptr_t)W) & 15) == 0);
  GroupTab gt{};
  const int64_t xl_tiles = (int64_t)((d_out + 255) / 256) * ((T + 255) / 256);
  if (T <= 32) rc = launch<WIT_S>(a, gt, stream);
  else if (xl_tiles >= 256) rc = launch<WIT_XL>(a, gt, stream);
  else rc = launch<WIT_M>(a, gt, stream);
  return rc ? rc : fpi::ok();
}

extern "C" int fp_witness_linear_grouped(const int8_t* X, int64_t ldx, const int8_t* const* W_ptrs, int64_t ldw,
                                         const int32_t* row_off, int32_t G, int32_t d_in, int32_t d_out, int32_t s,
                                         int32_t* Z, int8_t* Y, int8_t* R, hipStream_t stream) {
  if (G < 0 || G > FP_MAX_GROUPS) return fpi::fail(FP_EARG, "fp_witness_linear_grouped: G=%d outside [0, %d]", G, FP_MAX_GROUPS);
  if (G == 0) return fpi::ok();
  if (!row_off || !W_ptrs) return fpi::fail(FP_EARG, "fp_witness_linear_grouped: null host array");
  if (row_off[0] != 0) return fpi::fail(FP_EARG, "fp_witness_linear_grouped: row_off[0] != 0");
  for (int g = 0; g < G; ++g)
    if (row_off[g + 1] < row_off[g]) return fpi::fail(FP_EARG, "fp_witness_linear_grouped: row_off decreases at %d", g);
  const int32_t total = row_off[G];
  int rc = validate("fp_witness_linear_grouped", ldx, ldw, total, d_in, d_out, s, Y, R);
  if (rc) return rc;
  if (total == 0 || d_out == 0) return fpi::ok();
  if (d_in > 0 && !X) return fpi::fail(FP_EARG, "fp_witness_linear_grouped: null X");
  for (int g = 0; g < G; ++g)
    if (row_off[g + 1] > row_off[g] && d_in > 0 && !W_ptrs[g])
      return fpi::fail(FP_EARG, "fp_witness_linear_grouped: null W for non-empty group %d", g);
  WitArgs a{};
  a.X = X; a.ldx = ldx; a.W = nullptr; a.ldw = ldw;
  a.T = total; a.N = d_out; a.K = d_in; a.s = s;
  a.Z = Z; a.Y = Y; a.R = R;
  vec_flags(a);
  bool vw = (ldw & 15) == 0;
  for (int g = 0; g < G; ++g) vw = vw && ((((uintptr_t)W_ptrs[g]) & 15) == 0);
  a.vecW = vw;
  constexpr int GBT = 32;  // token tile of the grouped launch
  for (int g0 = 0; g0 < G; g0 += MAXG) {
    const int gc = (G - g0) < MAXG ? (G - g0) : MAXG;
    GroupTab gt{};
    int tiles = 0, ng = 0;
    for (int g = g0; g < g0 + gc; ++g) {
      const int rows = row_off[g + 1] - row_off[g];
      if (rows == 0) continue;  // empty groups own no tiles
      gt.W[ng] = W_ptrs[g];
      gt.row_off[ng] = row_off[g];
      gt.row_off[ng + 1] = row_off[g + 1];
      gt.tile_off[ng] = tiles;
      tiles += (rows + GBT - 1) / GBT;
      ++ng;
    }
    if (ng == 0) continue;
    gt.tile_off[ng] = tiles;
    gt.G = ng;
    a.tiles_t = tiles;
    rc = launch<WIT_SG>(a, gt, stream);
    if (rc) return rc;
  }
  return fpi::ok();
}

extern "C" int fp_witness_linear_with_sumcheck(const int8_t* X, int64_t ldx, const int8_t* W, int64_t ldw, int32_t T,
                                               int32_t d_in, int32_t d_out, int32_t s, int32_t* Z, int8_t* Y,
                                               int8_t* R, int32_t n_pairs, const fp_elem* const* A,
                                               const fp_elem* const* B, const fp_elem* rho, int32_t n,
                                               const fp_elem* r, fp_elem* rounds, fp_elem* finals, fp_elem* claim0,
                                               hipStream_t stream) {
  const char* fn = "fp_witness_linear_with_sumcheck";
  int rc = validate(fn, ldx, ldw, T, d_in, d_out, s, Y, R);
  if (rc) return rc;
  if (T > 0 && d_out > 0 && d_in > 0 && (!X || !W)) return fpi::fail(FP_EARG, "%s: null X or W", fn);
  const int nt = witness_threads(T, d_out);
  sct::TailArgs ta;
  rc = tail_args(fn, n_pairs, A, B, rho, n, r, rounds, finals, claim0, nt, ta);
  if (rc) return rc;
  WitArgs a{};
  a.X = X; a.ldx = ldx; a.W = W; a.ldw = ldw;
  a.T = T; a.N = d_out; a.K = d_in; a.s = s;
  a.Z = Z; a.Y = Y; a.R = R;
  vec_flags(a);
  a.vecW = ((ldw & 15) == 0) && ((((uintptr_t)W) & 15) == 0);
  GroupTab gt{};
  const int64_t xl_tiles = (int64_t)((d_out + 255) / 256) * ((T + 255) / 256);
  if (T <= 32) rc = launch_with_tail<WIT_S>(a, gt, ta, 1, stream);
  else if (xl_tiles >= 256) rc = launch_with_tail<WIT_XL>(a, gt, ta, 1, stream);
  else rc = launch_with_tail<WIT_M>(a, gt, ta, 1, stream);
  return rc ? rc : fpi::ok();
}

// ---- limb folds: the int8 product of a weight matrix's transpose (as the
// token operand) with byte-digit rows (as the weight operand), reduced per
// group of 8 digit rows to a field value in the epilogue. One tile shape, the
// 128 x 128 one, measured best or within 2% of best from 1 to 128 requests on
// the up-projection's weights, with the split picked for about two workgroups
// per CU.
namespace fpi {

SplitK splitk_plan(int32_t T, int32_t K, int32_t N) {
  constexpr int BO = 128, BT = 128, BK = 128;  // WIT_M
  SplitK p{};
  const int64_t tiles = (int64_t)((T + BT - 1) / BT) * ((N + BO - 1) / BO);
  int64_t want = tiles > 0 ? (512 + tiles - 1) / tiles : 1;
  const int64_t kb = ((int64_t)K + BK - 1) / BK;  // K steps
  if (want > kb) want = kb > 0 ? kb : 1;
  int64_t chunk = (kb + want - 1) / want * BK;
  if (chunk > SPLITK_MAX_CHUNK) chunk = SPLITK_MAX_CHUNK;
  p.kchunk = (int32_t)chunk;
  p.ksplit = (int32_t)(K > 0 ? ((int64_t)K + chunk - 1) / chunk : 1);
  return p;
}

int witness_fold_splitk(const int8_t* Xt, int64_t ldx, const int8_t* D, int64_t ldd, int32_t T, int32_t K, int32_t N,
                        const int32_t* colsum, const SplitK& p, uint64_t* part, int64_t ldp, int64_t psplit,
                        hipStream_t st) {
  WitArgs a{};
  a.X = Xt; a.ldx = ldx; a.W = D; a.ldw = ldd;
  a.T = T; a.N = N; a.K = K; a.s = 1;
  a.ksplit = p.ksplit; a.kchunk = p.kchunk;
  a.colsum = colsum; a.part = part; a.ldp = ldp; a.psplit = psplit;
  vec_flags(a);
  a.vecW = ((ldd & 15) == 0) && ((((uintptr_t)D) & 15) == 0);
  GroupTab gt{};
  return launch<WIT_M, 1>(a, gt, st);
}

// The packed-weight kernel's 256x128 tiles (digit rows x columns of Xt), the
// reduction split so that there is about one workgroup per compute unit.
SplitK splitk_plan_packed(int32_t T, int32_t K, int32_t N) {
  SplitK p{};
  const int64_t tiles = (int64_t)((T + 127) / 128) * ((N + 255) / 256);
  int64_t want = tiles > 0 ? (256 + tiles - 1) / tiles : 1;
  const int64_t kb = ((int64_t)K + WP_BK - 1) / WP_BK;  // K blocks
  if (want > kb) want = kb > 0 ? kb : 1;
  int64_t chunk = (kb + want - 1) / want * WP_BK;
  if (chunk > SPLITK_MAX_CHUNK) chunk = SPLITK_MAX_CHUNK;
  p.kchunk = (int32_t)chunk;
  p.ksplit = (int32_t)(K > 0 ? ((int64_t)K + chunk - 1) / chunk : 1);
  return p;
}

size_t packed_rows_bytes(int32_t N, int32_t K) {
  return (size_t)((N + 31) / 32) * 32 * (size_t)((K + WP_BK - 1) / WP_BK) * WP_BK;
}

int witness_fold_splitk_packed(const int8_t* Xt, int64_t ldx, const int8_t* Dp, int32_t T, int32_t K, int32_t N,
                               const int32_t* colsum, const SplitK& p, uint64_t* part, int64_t ldp, int64_t psplit,
                               hipStream_t st) {
  WitArgs a{};
  a.X = Xt; a.ldx = ldx; a.W = Dp; a.ldw = 0;
  a.T = T; a.N = N; a.K = K; a.s = 1;
  a.wp_rb = (N + 31) / 32;
  a.wp_kb = (K + WP_BK - 1) / WP_BK;
  a.ksplit = p.ksplit; a.kchunk = p.kchunk;
  a.colsum = colsum; a.part = part; a.ldp = ldp; a.psplit = psplit;
  vec_flags(a);
  return launch_ws<WIT_WS_L, 1>(a, nullptr, 0, EqAux{}, st);
}

}  // namespace fpi

// ---- packed weights ------------------------------------------------------
namespace {

bool packed_dims(int32_t d_out, int32_t d_in, int32_t& nrb, int32_t& nkb) {
  if (d_out < 0 || d_in < 0) return false;
  nrb = (d_out + 31) / 32;
  nkb = (d_in + WP_BK - 1) / WP_BK;
  return true;
}

// The packed-weight tile for a shape: 256x128 once it gives at least 3/4 of a
// workgroup per CU (measured 1-17% faster than 256x64 from T = 512 up on the
// workloads' projections), 256x64 for fewer, smaller outputs (4096 -> 1024 at
// T = 4096 has 128 large tiles and runs 23% faster with 256 small ones).
int launch_ws_auto(WitArgs a, const sct::TailArgs* ta, int n_tail, const EqAux& eq, hipStream_t st) {
  const int64_t large_tiles = (int64_t)((a.N + 255) / 256) * ((a.T + 127) / 128);
  if (large_tiles >= 192) return launch_ws<WIT_WS_L>(a, ta, n_tail, eq, st);
  return launch_ws<WIT_WS>(a, ta, n_tail, eq, st);
}

// Shared checks of the packed-weight witness entry points.
int packed_args(const char* fn, const int8_t* X, int64_t ldx, const int8_t* Wp, int32_t T, int32_t d_in,
                int32_t d_out, int32_t s, const int8_t* Y, const int8_t* R, WitArgs& a) {
  int rc = validate(fn, ldx, d_in, T, d_in, d_out, s, Y, R);
  if (rc) return rc;
  if (T > 0 && d_out > 0 && d_in > 0) {
    if (!X || !Wp) return fpi::fail(FP_EARG, "%s: null X or packed W", fn);
    if (d_in % 16 != 0 || ldx % 16 != 0 || (((uintptr_t)X) & 15) != 0)
      return fpi::fail(FP_ESHAPE, "%s: needs d_in %% 16 == 0 and 16-byte aligned X rows (d_in=%d, ldx=%lld)", fn, d_in,
                       (long long)ldx);
    if ((((uintptr_t)Wp) & 15) != 0) return fpi::fail(FP_EARG, "%s: packed W not 16-byte aligned", fn);
  }
  a = WitArgs{};
  a.X = X; a.ldx = ldx; a.W = Wp; a.ldw = 0;
  a.T = T; a.N = d_out; a.K = d_in; a.s = s;
  packed_dims(d_out, d_in, a.wp_rb, a.wp_kb);
  vec_flags(a);
  a.vecW = 1;
  return FP_OK;
}

}  // namespace

extern "C" size_t fp_witness_packed_weights_bytes(int32_t d_out, int32_t d_in) {
  int32_t nrb, nkb;
  if (!packed_dims(d_out, d_in, nrb, nkb)) return 0;
  return (size_t)nrb * 32 * (size_t)nkb * WP_BK;
}

extern "C" int fp_witness_pack_weights(const int8_t* W, int64_t ldw, int32_t d_out, int32_t d_in, int8_t* Wp,
                                       hipStream_t stream) {
  const char* fn = "fp_witness_pack_weights";
  int32_t nrb, nkb;
  if (!packed_dims(d_out, d_in, nrb, nkb)) return fpi::fail(FP_EARG, "%s: negative size", fn);
  if (d_in > FP_MAX_DIN) return fpi::fail(FP_ESHAPE, "%s: d_in=%d > %d", fn, d_in, FP_MAX_DIN);
  if (ldw < d_in) return fpi::fail(FP_ESHAPE, "%s: ldw < d_in", fn);
  const int64_t units = (int64_t)nrb * nkb * (WP_BK / 32) * 64;
  if (units == 0) return fpi::ok();
  if (!Wp || (d_out > 0 && d_in > 0 && !W)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  if ((((uintptr_t)Wp) & 15) != 0) return fpi::fail(FP_EARG, "%s: Wp not 16-byte aligned", fn);
  const int vec = ((ldw & 15) == 0) && ((((uintptr_t)W) & 15) == 0);
  const int64_t want = (units + 255) / 256;
  const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(blocks), dim3(256), 0, stream, W, ldw, d_out, d_in, nrb, nkb, vec, Wp);
  int rc = fpi::check_launch("pack_weights_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" int fp_witness_linear_packed(const int8_t* X, int64_t ldx, const int8_t* Wp, int32_t T, int32_t d_in,
                                        int32_t d_out, int32_t s, int32_t* Z, int8_t* Y, int8_t* R, int32_t n_eq,
                                        const fp_eq_desc* eq, hipStream_t stream) {
  const char* fn = "fp_witness_linear_packed";
  WitArgs a;
  int rc = packed_args(fn, X, ldx, Wp, T, d_in, d_out, s, Y, R, a);
  if (rc) return rc;
  EqAux aux;
  rc = eq_aux(fn, n_eq, eq, aux);
  if (rc) return rc;
  a.Z = Z; a.Y = Y; a.R = R;
  vec_flags(a);
  rc = launch_ws_auto(a, nullptr, 0, aux, stream);
  return rc ? rc : fpi::ok();
}

extern "C" int fp_witness_linear_packed_with_sumcheck(const int8_t* X, int64_t ldx, const int8_t* Wp, int32_t T,
                                                      int32_t d_in, int32_t d_out, int32_t s, int32_t* Z, int8_t* Y,
                                                      int8_t* R, int32_t n_pairs, const fp_elem* const* A,
                                                      const fp_elem* const* B, const fp_elem* rho, int32_t n,
                                                      const fp_elem* r, fp_elem* rounds, fp_elem* finals,
                                                      fp_elem* claim0, int32_t n_eq, const fp_eq_desc* eq,
                                                      hipStream_t stream) {
  const char* fn = "fp_witness_linear_packed_with_sumcheck";
  WitArgs a;
  int rc = packed_args(fn, X, ldx, Wp, T, d_in, d_out, s, Y, R, a);
  if (rc) return rc;
  sct::TailArgs ta;
  rc = tail_args(fn, n_pairs, A, B, rho, n, r, rounds, finals, claim0, WsCfg<WIT_WS>::NT, ta);
  if (rc) return rc;
  EqAux aux;
  rc = eq_aux(fn, n_eq, eq, aux);
  if (rc) return rc;
  a.Z = Z; a.Y = Y; a.R = R;
  vec_flags(a);
  rc = launch_ws_auto(a, &ta, 1, aux, stream);
  return rc ? rc : fpi::ok();
}

// ---- one step of a stream of layer proofs ----------------------------------
namespace {

// Plans the folds (int8) and claims (int32) of the step's fold workgroups:
// workspace = arrival counters, then every job's partial values.
// GEMM tiles of the layer step for a shape (256x128 once there are >= 192 of them, else 256x64).
int64_t step_tiles(int32_t T, int32_t d_out, bool* large) {
  const int64_t large_tiles = (int64_t)((d_out + 255) / 256) * ((T + 127) / 128);
  *large = large_tiles >= 192;
  return *large ? large_tiles : (int64_t)((d_out + 255) / 256) * ((T + 63) / 64);
}
constexpr int STEP_WAVES = 4;  // waves of both layer-step tile configurations

// Workspace of a layer step: arrival counters, the folds' partial values and
// (own_parts > 0) one slot per GEMM wave for the claim taken from the
// accumulators, whose counter follows the folds'.
int step_folds(const char* fn, int32_t n_fold, const fp_fold_desc* folds, int32_t n_claim,
               const fp_claim_desc* claims, int64_t own_parts, void* ws, size_t ws_bytes, bool plan_only,
               size_t* need, FoldAux& fa, uint64_t** own_part, uint32_t** own_ctr) {
  return plan_folds<STEP_MAX_FOLD>(fn, n_fold, folds, n_claim, claims, own_parts, ws, ws_bytes, plan_only, need, fa,
                                   own_part, own_ctr);
}

}  // namespace

extern "C" size_t fp_layer_step_workspace(int32_t T, int32_t d_out, int32_t own_claim, int32_t n_fold,
                                          const fp_fold_desc* folds, int32_t n_claim, const fp_claim_desc* claims) {
  if (T < 0 || d_out < 0) return 0;
  FoldAux fa;
  size_t need = 0;
  bool large;
  const int64_t own = own_claim ? step_tiles(T, d_out, &large) * STEP_WAVES : 0;
  uint64_t* op;
  uint32_t* oc;
  if (step_folds("fp_layer_step_workspace", n_fold, folds, n_claim, claims, own, nullptr, 0, true, &need, fa, &op,
                 &oc))
    return 0;
  return need;
}

extern "C" int fp_layer_step(const int8_t* X, int64_t ldx, const int8_t* Wp, int32_t T, int32_t d_in, int32_t d_out,
                             int32_t s, int32_t* Z, int8_t* Y, int8_t* R, const fp_elem* claim_E_t,
                             const fp_elem* claim_E_o, fp_elem* claim, int32_t n_eq, const fp_eq_desc* eq,
                             int32_t n_fold, const fp_fold_desc* folds, int32_t n_claim, const fp_claim_desc* claims,
                             void* ws, size_t ws_bytes, int32_t n_pairs, const fp_elem* const* A,
                             const fp_elem* const* B, const fp_elem* rho, int32_t n, const fp_elem* r,
                             fp_elem* rounds, fp_elem* finals, fp_elem* claim0, hipStream_t stream) {
  const char* fn = "fp_layer_step";
  WitArgs a;
  int rc = packed_args(fn, X, ldx, Wp, T, d_in, d_out, s, Y, R, a);
  if (rc) return rc;
  EqAux aux;
  rc = eq_aux(fn, n_eq, eq, aux);
  if (rc) return rc;
  const bool own = claim_E_t != nullptr;
  if (own && (!claim_E_o || !claim)) return fpi::fail(FP_EARG, "%s: the claim needs E_t, E_o and its output", fn);
  if (own && (T == 0 || d_out == 0)) return fpi::fail(FP_ESHAPE, "%s: the claim needs tokens and outputs", fn);
  bool large;
  const int64_t own_parts = own ? step_tiles(T, d_out, &large) * STEP_WAVES : 0;
  FoldAux fa;
  size_t need = 0;
  uint64_t* own_part;
  uint32_t* own_ctr;
  rc = step_folds(fn, n_fold, folds, n_claim, claims, own_parts, ws, ws_bytes, false, &need, fa, &own_part, &own_ctr);
  if (rc) return rc;
  sct::TailArgs ta;
  const bool tail = n_pairs > 0;
  if (tail) {
    rc = tail_args(fn, n_pairs, A, B, rho, n, r, rounds, finals, claim0, 256, ta);
    if (rc) return rc;
  }
  a.Z = Z; a.Y = Y; a.R = R;
  if (own) {
    a.cEt = claim_E_t;
    a.cEo = claim_E_o;
    a.cout = claim;
    a.cpart = own_part;
    a.cctr = own_ctr;
  }
  vec_flags(a);
  step_tiles(T, d_out, &large);
  if (large) rc = launch_step<WIT_WS_L>(a, tail ? &ta : nullptr, tail ? 1 : 0, aux, fa, stream);
  else rc = launch_step<WIT_WS>(a, tail ? &ta : nullptr, tail ? 1 : 0, aux, fa, stream);
  return rc ? rc : fpi::ok();
}
