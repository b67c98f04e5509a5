// witness_multi.hip - the witness GEMMs of all the linear maps of one layer in
// one launch, each map's claim taken from its GEMM's accumulators.
//
// "How fast can FlashProve go", §2: every linear map of the integer model is a
// matmul whose rescaled output and remainder are committed and whose claim is
// reduced by sum-check; §3.1: the claim is about the product g^ = 2^k g_w + r,
// i.e. about Z, which therefore never has to be stored: each map's claim
//   c0_m = sum_t sum_o E_t[t] E_o[o] Z_m[t, o]
// is contracted out of the int32 accumulators where Z is produced (the
// claim epilogue in witness_dev.hpp), and only Y and R leave the chip.
//
// One grid covers every map's tiles (the seven maps of a transformer layer:
// Q, K, V and O over d, gate and up over d_ff, down; or the dense MLP's three),
// so that no map's tail wave idles the GPU and maps sharing an input (Q/K/V,
// gate/up) keep it in the L2s together. Tiles are dealt to the 8 XCDs
// (workgroup b runs on XCD b % 8) map by map: each map's tiles are cut into 8
// contiguous chunks, chunk x to XCD x, so every XCD gets an equal share of
// every map (the long-K down projection included) and a run of neighbouring
// weight panels that its L2 shares; maps run in the caller's order (longest
// reduction first balances the end of the launch). Within a chunk, tiles walk
// `group_o` weight panels at a time with the token tiles outermost.
//
// The K loop: weights come packed (fp_witness_pack_weights: a wave's operand
// for one v_mfma_i32_32x32x32_i8 is one coalesced 1 KiB load), PFW K blocks
// ahead into registers; X passes through NBUF LDS stages, loaded PFX blocks
// ahead; with three stages the next block's first X fragments are read before
// the block's barrier, so the matrix cores restart at once after it.
#include <mutex>
#include <utility>

#include "common.hpp"
#include "eq.hpp"
#include "sc_stream.hpp"
#include "witness_dev.hpp"

namespace {

constexpr int MM_MAX = FP_MAX_MULTI;
constexpr int NXCD = 8;

struct MmDev {
  const int8_t* X;
  int64_t ldx;
  const int8_t* Wp;
  int32_t* Z;
  int8_t* Y;
  int8_t* R;
  const uint64_t* Et;
  const uint64_t* Eo;
  uint64_t* cout;
  uint64_t* cpart;
  uint32_t* cctr;
  int32_t T, K, N, wp_rb, wp_kb, tiles_t, tiles_o, vecZ, vecYR;
};

struct MultiArgs {
  MmDev m[MM_MAX];
  int32_t split[MM_MAX][NXCD + 1];  // map m's tiles [split[m][x], split[m][x+1]) run on XCD x
  int32_t count, s, group_o, gemm_blocks;
  // the last `pool` tiles of each XCD's list are taken by `ndyn` workgroups at
  // run time (qctr: the pool's counters in the workspace's first lines)
  int32_t pool, ndyn;
  uint32_t* qctr;
};

// The tiles of one launch are dealt to the XCDs in equal shares, but the XCDs
// do not run at one speed (on the seven-map layer one finishes its share up to
// 100 us, ~12%, after another, and which one varies from launch to launch). So
// each XCD's last tiles form a pool: after the statically placed tiles come
// 2 x 8 x pool workgroups that each reserve one pool tile (a reservation
// counter bounds the takers), take it from their own XCD's pool or else from
// another's, and exit at once when every tile is taken; those on the XCDs that
// are ahead arrive first. The counters sit in the workspace's claim-counter
// lines (word 16x + 8: XCD x's pool; word 9: reservations; word 25: exits),
// zero on entry; the last workgroup to exit sets them to zero again.
constexpr int POOL_PERCENT = 12;  // of an XCD's tiles, from 2 full waves of tiles on
constexpr int GPU_SLOTS = 512;    // GEMM workgroups resident at once (2 per CU)
__device__ __forceinline__ uint32_t* q_pool(uint32_t* q, int x) { return q + 16 * x + 8; }
__device__ __forceinline__ uint32_t q_add(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The pool tile of a dynamic workgroup on XCD y (x * pool + j), or -1.
__device__ __forceinline__ int pool_pick(const MultiArgs& ma, int y) {
  uint32_t* q = ma.qctr;
  int pick = -1;
  if (q_add(q + 9) < (uint32_t)(NXCD * ma.pool)) {
    // a reservation guarantees a tile: every pool full would mean as many other takers as tiles
    for (int j = 0; j < NXCD; ++j) {
      const int x = (y + j) % NXCD;
      const uint32_t g = q_add(q_pool(q, x));
      if (g < (uint32_t)ma.pool) {
        pick = x * ma.pool + (int)g;
        break;
      }
    }
  }
  if (q_add(q + 25) == (uint32_t)(ma.ndyn - 1)) {  // every taker is done taking
    for (int x = 0; x < NXCD; ++x) __hip_atomic_store(q_pool(q, x), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 9, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 25, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return pick;
}

// Fold jobs of another proof (arrival mode) and whole sum-check instances of a
// third, run by workgroups of the same launch.
constexpr int MULTI_MAX_FOLD = FP_STEP_MULTI_MAX_FOLD;
constexpr int MULTI_MAX_SC = FP_STEP_MULTI_MAX_SUMCHECK;
using MultiFolds = FoldAuxT<MULTI_MAX_FOLD>;
struct SumAux {
  scs::Inst inst[MULTI_MAX_SC];
  int32_t count;
  int32_t blocks;  // count rounded up to a multiple of 8, so the GEMM tiles keep blockIdx % 8 as their XCD
};
// the claim counters come first in the workspace, the folds' counters and parts after them
constexpr size_t CLAIM_CTR_BYTES = (size_t)MM_MAX * 64;

// Tile config: NW waves of 32 TM weight rows x 32 TN tokens; SB packed K blocks per LDS stage.
template <int NW, int TM, int TN, int PFW, int PFX, int NBUF, int SB = 1>
struct MCfg {
  static constexpr int NWAVES = NW, NT = NW * 64, BO = NW * 32 * TM, BT = 32 * TN, BK = WP_BK * SB;
  static constexpr int PITCH = BK + 16, CPR = BK / 16, NCB = BT * CPR, CB = (NCB + NT - 1) / NT, KS = BK / 32;
  static constexpr int EP = 36, STAGE_BYTES = NW * 32 * EP * 4;
  static constexpr int CLAIM_BYTES = CL_LIMBS * BO + 8 * BT + 16 * 8;
  static constexpr int LOOP_BYTES = NBUF * BT * PITCH;
  static constexpr int EPI_BYTES = STAGE_BYTES + CLAIM_BYTES;
  static constexpr int LDS_BYTES = LOOP_BYTES > EPI_BYTES ? LOOP_BYTES : EPI_BYTES;
  // Y and R of one 32-token block of the tile staged below the claim's tables
  // ([2][32][YP] bytes, double-buffered when it fits)
  static constexpr int YP = BO + 16, YS_BYTES = 2 * 32 * YP;
  static constexpr int NYB = 2 * YS_BYTES <= STAGE_BYTES ? 2 : (YS_BYTES <= STAGE_BYTES ? 1 : 0);
  // the weight fold's region after it: the panel's limb table, then 2 NW K
  // blocks of int32 limb sums [2 k-steps][32 columns][FL words] (two groups
  // of NW blocks: one filling while the other is turned into field values)
  static constexpr int FL = 11;  // an odd row pitch: the 32 columns of one limb fall in distinct banks
  static constexpr int FOLD_ACC_WORDS = 2 * 32 * FL;
  static constexpr int FOLD_SLOTS = 2 * NW;
  static constexpr int FOLD_BYTES = CL_LIMBS * BO + FOLD_SLOTS * FOLD_ACC_WORDS * 4;
  static constexpr int LDS_FOLD_BYTES = LDS_BYTES + FOLD_BYTES;
  static_assert(NCB % NT == 0 || NCB < NT, "X chunks: whole rounds, or fewer chunks than threads");
  static_assert(KS == 2 * SB, "two k-steps per packed K block");
};

// Tile `lt` of `nt` tiles of one map (a already holds the map's arguments).
// FOLDW: the first token tile of each weight panel also folds the panel's
// rows by E_o (a.fpart), from the weight fragments the GEMM streams: an MFMA
// against the identity puts a fragment's 32 rows x 32 columns into the
// accumulator layout, where after the v_permlane32_swap a lane holds 16
// consecutive rows of one column, which is an MFMA B operand with the rows as
// the reduction index; an MFMA with the 7-bit limbs of E_o as the A operand
// then gives sum_o limb_m(E_o[o]) W[o, k] for the fragment's columns. The
// waves' int32 limb sums meet in LDS (exact: |sum| < 2^7 2^7 BO), and once a
// group of NW K blocks is complete (after a barrier) each wave turns one block's
// limbs into field values sum_m 2^(7m) sum_o ... = sum_o E_o[o] W[o, k] mod p
// for the panel, at the end of the step that completes the next group, after
// its products are issued (wave 0 turning every block at the start of the next
// step held the matrix cores: the MoE block's step 2.70 ms, 2.32 without it).
template <int NW, int TM, int TN, int PFW, int PFX, int NBUF, int SCHED, int FOLDW = 0, int SB = 1>
__device__ __forceinline__ void multi_body(const WitArgs& a, int lt, int nt, int group_o, int8_t* lds) {
  static_assert(SB == 1 || SB == 2, "one or two packed K blocks per stage");
  static_assert(!FOLDW || SB == 1, "the weight folds work per packed K block");
  using C = MCfg<NW, TM, TN, PFW, PFX, NBUF, SB>;
  constexpr int NT = C::NT, BO = C::BO, BT = C::BT, BK = C::BK, PITCH = C::PITCH, CPR = C::CPR, CB = C::CB;
  constexpr int KS = C::KS;
  int8_t (*sB)[BT * PITCH] = reinterpret_cast<int8_t (*)[BT * PITCH]>(lds);
  // tile -> (token tile, output tile): groups of group_o output tiles, token tiles outermost
  const int gsz = group_o * a.tiles_t;
  const int g = lt / gsz, in = lt - g * gsz;
  const int go = min(group_o, a.tiles_o - g * group_o);
  const int to = g * group_o + in % go, tt = in / go;
  const int t_base = tt * BT, o_base = to * BO;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int wo0 = wave * 32 * TM;
  const int NB = a.wp_kb;               // packed K blocks
  const int NS = (NB + SB - 1) / SB;    // LDS stages
  const int64_t rb_bytes = (int64_t)NB * WP_BK * 32;
  const int8_t* pw[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) pw[i] = a.W + (int64_t)min((o_base + wo0) / 32 + i, a.wp_rb - 1) * rb_bytes + lane * 16;
  const int8_t* px[CB];
  int kc[CB], so[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    // with fewer chunks than threads the upper threads load a duplicate and do not store it
    const int ch = (tid + c * NT) % C::NCB, row = ch / CPR;
    kc[c] = (ch % CPR) * 16;
    px[c] = a.X + (int64_t)min(t_base + row, a.T - 1) * a.ldx;  // rows past T: the last row (never stored)
    so[c] = row * PITCH + kc[c];
  }
  const bool xstore = C::NCB >= NT || tid < C::NCB;  // wave-uniform
  const int klim = a.K;
  v4i wf[PFW][TM][KS];
  v4i xr[PFX][CB];
  v4i fb[2][TN];
  // stage st's weight fragments: k-step q of packed block st SB + q / 2 (the last block past the end)
  auto wload = [&](int slot, int st) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < KS; ++q)
        wf[slot][i][q] = *(const v4i*)(pw[i] + (int64_t)min(st * SB + q / 2, NB - 1) * (WP_BK * 32) + 1024 * (q % 2));
  };
  // X chunks past d_in are read from column 0: they meet zero weights
  auto xload = [&](int slot, int st) {
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int k = st * BK + kc[c];
      xr[slot][c] = *(const v4i*)(px[c] + (k < klim ? k : 0));
    }
  };
  auto sstore = [&](int slot, int buf) {
    if (xstore) {
#pragma unroll
      for (int c = 0; c < CB; ++c) *(v4i*)&sB[buf][so[c]] = xr[slot][c];
    }
  };
  // X fragments of k-step q of LDS stage buf (lane: token r of each 32-row block,
  // the 16 bytes of k the weight fragment's lane half holds)
  auto fread = [&](int fs, int buf, int q) {
    const int8_t* B = &sB[buf][r * PITCH + WP_BK * (q / 2) + 32 * h + 16 * (q % 2)];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[fs][j] = *(const v4i*)(B + 32 * j * PITCH);
  };
  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;
  auto mma = [&](int fs, int ws, int q) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[ws][i][q], fb[fs][j], acc[i][j], 0, 0, 0);
  };
  // ---- the weight fold's set-up (FOLDW, first token tile of the panel)
  const bool fold_on = FOLDW && a.fpart != nullptr && tt == 0;  // uniform over the workgroup
  uint8_t* flimbs = reinterpret_cast<uint8_t*>(lds + C::LDS_BYTES);
  int32_t* facc = reinterpret_cast<int32_t*>(lds + C::LDS_BYTES + CL_LIMBS * BO);  // [FOLD_SLOTS][FOLD_ACC_WORDS]
  v4i FA[TM];   // limbs of E_o for the wave's row blocks (A operand, reduction over the rows)
  v4i FI = {};  // the identity as a B operand: lane (n, h) holds rows 16 h .. 16 h + 15 of column n
  if constexpr (FOLDW) {
    if (fold_on) {
      for (int x = tid; x < BO; x += NT) {
        const int o = o_base + x;
        const uint64_t e = o < a.N ? a.cEo[o] : 0;
#pragma unroll
        for (int m = 0; m < CL_LIMBS; ++m) flimbs[m * BO + x] = (uint8_t)((e >> (7 * m)) & 127u);
      }
      for (int x = tid; x < C::FOLD_SLOTS * C::FOLD_ACC_WORDS; x += NT) facc[x] = 0;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) w |= (16 * h + 4 * d + b == r ? 1u : 0u) << (8 * b);
        FI[d] = (int)w;
      }
      __syncthreads();
      // byte j = 4 d + b of lane (r, h): limb r of row 8 d + 4 h + b of the row block
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          FA[i][d] = r < CL_LIMBS ? *(const int*)&flimbs[r * BO + wo0 + 32 * i + 8 * d + 4 * h] : 0;
    }
  }
  // K block st's fragments folded into LDS slot st % FOLD_SLOTS. The transpose's
  // accumulators hold, in lane (r, h) register v, row 8 (v / 4) + 4 h + v % 4
  // of column r: packed in register order they are the B operand, the limb
  // operand FA pairing the same rows with the same reduction index.
  auto fold_block = [&](int ws, int st) {
    int32_t* F = facc + (st % C::FOLD_SLOTS) * C::FOLD_ACC_WORDS;
    const v16i zero = {};
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      v16i Ff = zero;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const v16i T = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[ws][i][q], FI, zero, 0, 0, 0);
        const v4i Bf = {(int)pack_low_bytes(T[0], T[1], T[2], T[3]), (int)pack_low_bytes(T[4], T[5], T[6], T[7]),
                        (int)pack_low_bytes(T[8], T[9], T[10], T[11]),
                        (int)pack_low_bytes(T[12], T[13], T[14], T[15])};
        Ff = __builtin_amdgcn_mfma_i32_32x32x32_i8(FA[i], Bf, Ff, 0, 0, 0);
      }
      // lane (r, h), register v: limb row 8 (v / 4) + 4 h + v % 4 of column r
#pragma unroll
      for (int v = 0; v < 6; ++v) {
        const int m = v < 4 ? 4 * h + v : 8 + (v - 4);
        if (v < 4 || h == 0) atomicAdd(&F[(q * 32 + r) * C::FL + m], Ff[v]);
      }
    }
  };
  // the calling wave: K block st's limb sums -> one field value per column,
  // then its slot cleared for block st + FOLD_SLOTS. The limbs of each half are
  // exact in int64 (|sum| < 2^22, 5 limbs of 7 bits): lo + 2^35 hi.
  auto fold_flush = [&](int st) {
    int32_t* F = facc + (st % C::FOLD_SLOTS) * C::FOLD_ACC_WORDS + lane * C::FL;  // lane = column q * 32 + n
    int64_t lo = 0, hi = 0;
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      lo += (int64_t)F[m] << (7 * m);
      hi += (int64_t)F[m + 5] << (7 * m);
    }
    const int q = lane >> 5, n = lane & 31;
    const int k = st * BK + 32 * (n >> 4) + 16 * q + (n & 15);
    a.fpart[(int64_t)to * a.fpitch + k] = gl::add(gl::from_i64(lo), gl::mul(gl::from_i64(hi), 1ull << 35));
#pragma unroll
    for (int m = 0; m < CL_LIMBS; ++m) F[m] = 0;
  };
  // Block st: multiply stage st % NBUF with weight slot st % PFW; store block
  // st + NBUF - 1 (loaded PFX blocks ago) into its stage and load block
  // st + NBUF - 1 + PFX; refill the weight slot with block st + PFW; one
  // barrier. Every load is issued unconditionally (past the end the last block
  // is re-read), so the code between barriers is straight-line.
  constexpr int L2 = (PFW % 2 == 0) ? PFW : 2 * PFW;
  constexpr int L3 = (L2 % PFX == 0) ? L2 : L2 * PFX;
  constexpr int U = (L3 % NBUF == 0) ? L3 : L3 * NBUF;
  if (NS > 0) {  // d_in = 0: every output is 0
    // The steps before block 0, without their products: step v stores X block v + NBUF - 1, loads X block
    // v + NBUF - 1 + PFX, then weight block v + PFW, as every step of the loop does. Entering the loop with
    // the loads in the loop's own order lets every X store wait for its own loads only (the waits at the loop
    // head hold for both ways in); block b uses X slot b % PFX and weight slot b % PFW.
    constexpr int V0 = (PFW > NBUF - 1 + PFX) ? PFW : NBUF - 1 + PFX;
#pragma unroll
    for (int v = -V0; v < 0; ++v) {
      if (v + NBUF - 1 >= 0) sstore((v + NBUF - 1) % PFX, (v + NBUF - 1) % NBUF);
      if (v + NBUF - 1 + PFX >= 0) xload((v + NBUF - 1 + PFX) % PFX, min(v + NBUF - 1 + PFX, NS - 1));
      if (v + PFW >= 0) wload((v + PFW) % PFW, min(v + PFW, NS - 1));
    }
    __syncthreads();
    if constexpr (NBUF >= 3) fread(0, 0, 0);
    auto step = [&](auto uc, int st) {
      constexpr int u = decltype(uc)::value;
      constexpr int buf = u % NBUF, ws = u % PFW;

      if constexpr (NBUF < 3) fread(0, buf, 0);
      fread(1, buf, 1);
      mma(0, ws, 0);
      constexpr int ss = (u + NBUF - 1) % PFX;
      sstore(ss, (u + NBUF - 1) % NBUF);
      xload(ss, min(st + NBUF - 1 + PFX, NS - 1));
      if constexpr (SB == 2) {
        fread(0, buf, 2);
        mma(1, ws, 1);
        fread(1, buf, 3);
        if (st * SB + 1 < NB) {  // the stage's second packed block exists (wave-uniform)
          mma(0, ws, 2);
          mma(1, ws, 3);
        }
      } else {
        mma(1, ws, 1);
      }
      if constexpr (FOLDW) {
        if (fold_on) fold_block(ws, st);
        // a group of NW blocks ends with this one: the group before it (complete
        // since an earlier barrier) is turned into field values, one block per
        // wave, while this step's products are still in the matrix cores
        if (fold_on && (st + 1) % NW == 0 && st + 1 >= 2 * NW) fold_flush(st + 1 - 2 * NW + wave);
      }
      wload(ws, min(st + PFW, NS - 1));
      if constexpr (NBUF >= 3) fread(0, (u + 1) % NBUF, 0);
      if constexpr (SCHED == 1) {
#pragma unroll
        for (int m = 0; m < TM * TN * KS; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
        }
      }
      __syncthreads();
    };
    int kt = 0;
    for (; kt + U <= NS; kt += U) {
      [&]<int... I>(std::integer_sequence<int, I...>) { (step(std::integral_constant<int, I>{}, kt + I), ...); }(
          std::make_integer_sequence<int, U>{});
    }
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((kt + I < NS ? step(std::integral_constant<int, I>{}, kt + I) : void()), ...);
    }(std::make_integer_sequence<int, U>{});
    if constexpr (FOLDW) {  // the groups not yet turned (complete after the last barrier)
      if (fold_on) {
        for (int g = (NS / NW >= 1 ? NS / NW - 1 : 0) * NW; g < NS; g += NW)
          if (g + wave < NS) fold_flush(g + wave);
      }
    }
  }

  // ---- epilogue: Y and R (and Z through LDS if asked), the claim from the accumulators
  const int s = a.s;
  const bool stage = a.Z != nullptr && a.vecZ;
  const bool claim = a.cEt != nullptr;
  // Y and R through LDS (the grouped launch, whose tiles are 32 tokens): each
  // token block of the tile leaves as whole BO-byte row pieces (lanes of a
  // fragment hold 16 bytes of 32 rows each). 0.8% faster on the MoE block;
  // the layer's 128-token tiles measured no faster, so they store directly.
  const bool yrs = FOLDW && C::NYB > 0 && a.Z == nullptr && a.vecYR;
  if (stage || claim || yrs) __syncthreads();  // every wave is done with the X stages
  int32_t* E = reinterpret_cast<int32_t*>(lds) + wave * 32 * C::EP;
  uint8_t* limbs = reinterpret_cast<uint8_t*>(lds) + C::STAGE_BYTES;
  uint64_t* etl = reinterpret_cast<uint64_t*>(lds + C::STAGE_BYTES + CL_LIMBS * BO);  // E_t of the tile's tokens
  uint64_t* red = etl + BT;
  v4i Aop[TM];
  uint64_t corr = 0;  // the planes' offsets, added once per token (by the h = 0 lanes)
  if (claim) {
    for (int x = tid; x < BT; x += NT) {
      const int t = t_base + x;
      etl[x] = t < a.T ? a.cEt[t] : 0;
    }
    // limb table of the tile's outputs (zero past d_out: rows of Z there come
    // from clamped weight blocks and must not count)
    uint64_t se = 0;
    for (int x = tid; x < BO; x += NT) {
      const int o = o_base + x;
      const uint64_t e = o < a.N ? a.cEo[o] : 0;
#pragma unroll
      for (int m = 0; m < CL_LIMBS; ++m) limbs[m * BO + x] = (uint8_t)((e >> (7 * m)) & 127u);
      if constexpr (BO == NT) se = e;  // output tid is lane tid % 64 of its wave's range
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i)
      Aop[i] = r < CL_LIMBS ? *(const v4i*)&limbs[r * BO + wo0 + 32 * i + 16 * h] : v4i{0, 0, 0, 0};
    if constexpr (BO != NT) {
#pragma unroll
      for (int x = lane; x < 32 * TM; x += 64) {
        const int o = o_base + wo0 + x;
        if (o < a.N) se = gl::add(se, a.cEo[o]);
      }
    }
    se = fpi::wave_total(se);  // every lane takes part
    corr = h == 0 ? gl::mul_small(se, 128u * 65793u) : 0;
  }
  WitArgs yr = a;
  if (stage) yr.Z = nullptr;
  uint64_t wsum = 0;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    uint8_t* yb = reinterpret_cast<uint8_t*>(lds) + (C::NYB > 1 ? j % C::NYB : 0) * C::YS_BYTES;
    v16i D[4];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      int32_t z[16];
      fragment_outputs(acc[i][j], z);
      const int t = t_base + 32 * j + r;
      const int o0 = o_base + wo0 + 32 * i + 16 * h;
      if (yrs) {
        uint32_t yw[4], rw[4];
        yr_bytes(z, s, yw, rw);
        const int c = wo0 + 32 * i + 16 * h;
        *(v4i*)&yb[r * C::YP + c] = v4i{(int)yw[0], (int)yw[1], (int)yw[2], (int)yw[3]};
        *(v4i*)&yb[(32 + r) * C::YP + c] = v4i{(int)rw[0], (int)rw[1], (int)rw[2], (int)rw[3]};
      } else if (t < a.T && o0 < a.N) {
        store_fragment(yr, z, t, o0, s);
      }
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
        for (int gg = 0; gg < 4; ++gg) {
          uint32_t w0, w1, w2, w3;
          foldk::transpose4((uint32_t)z[4 * gg], (uint32_t)z[4 * gg + 1], (uint32_t)z[4 * gg + 2],
                            (uint32_t)z[4 * gg + 3], w0, w1, w2, w3);
          P[0][gg] = (int)(w0 ^ 0x80808080u);
          P[1][gg] = (int)(w1 ^ 0x80808080u);
          P[2][gg] = (int)(w2 ^ 0x80808080u);
          P[3][gg] = (int)w3;
        }
        const v16i zero = {};
#pragma unroll
        for (int p = 0; p < 4; ++p)
          D[p] = __builtin_amdgcn_mfma_i32_32x32x32_i8(Aop[i], P[p], i == 0 ? zero : D[p], 0, 0, 0);
      }
    }
    if (claim) wsum = gl::add(wsum, gl::mul(gl::add(claim_row_value(D, h), corr), etl[32 * j + r]));
    if (yrs) {
      __syncthreads();  // the block's rows are in LDS
      constexpr int PR = BO / 16;  // 16-byte pieces per row
      for (int q = tid; q < 2 * 32 * PR; q += NT) {
        const int row = q / PR, c16 = q % PR;  // rows 0-31: Y, 32-63: R
        const int t = t_base + 32 * j + (row & 31), o = o_base + 16 * c16;
        if (t < a.T && o < a.N)  // N % 16 == 0: a piece is inside or past the row
          *(v4i*)((row < 32 ? a.Y : a.R) + (int64_t)t * a.N + o) = *(const v4i*)&yb[row * C::YP + 16 * c16];
      }
      if constexpr (C::NYB == 1) __syncthreads();  // before the next block overwrites them
    }
  }
  if (claim) claim_arrive(a, wsum, lt, nt, NW, red, reinterpret_cast<uint32_t*>(red + 8));
}

// Workgroups, in order: [0, sa.blocks) whole sum-check instances (first, so
// their chains of rounds start at once; the count is padded to a multiple of
// 8); then the GEMM tiles of every map placed by the XCD split, all but each
// XCD's last ma.pool; then the pool's takers; then fold jobs in arrival mode;
// then eq tables. The sum-checks, folds and eq
// tables belong to other proofs than the GEMMs (this launch's claims read eq
// tables that are complete before it starts), so nothing in one launch waits
// for another part of it.
template <int NW, int TM, int TN, int PFW, int PFX, int NBUF, int SCHED, int SB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void witness_multi_kernel(
    MultiArgs ma, EqAux eq, MultiFolds mf, SumAux sa) {
  using C = MCfg<NW, TM, TN, PFW, PFX, NBUF, SB>;
  static_assert(C::NT == 256 && scs::ST == 256 && foldk::FT == 256,
                "the eq, fold and sum-check workgroups are written for 256 threads");
  constexpr int FOLD_LDS = foldk::LDS_WORDS * 4 + foldk::MAXG_ALL * 8 + 16;
  constexpr int TAIL_LDS = (int)sizeof(sct::TailLds<256>);
  constexpr int B1 = C::LDS_BYTES > TAIL_LDS ? C::LDS_BYTES : TAIL_LDS;
  constexpr int BYTES = B1 > FOLD_LDS ? B1 : FOLD_LDS;
  __shared__ __align__(16) int8_t lds[BYTES];
  __shared__ int pick;
  int b = blockIdx.x;
  if (b < sa.blocks) {
    if (b < sa.count) scs::stream_body(sa.inst[b], *reinterpret_cast<sct::TailLds<256>*>(lds));
    return;
  }
  b -= sa.blocks;
  const int nstat = ma.gemm_blocks - NXCD * ma.pool;  // statically placed tiles
  int x = b % NXCD, li = b / NXCD, m = 0;
  if (b >= nstat) {
    // after the placed tiles: the pool's takers, then fold jobs, then eq tables
    // (folds ahead of the takers measured slower: their stream then meets
    // the last tiles' reuse in L2)
    int c = b - nstat;
    if (c >= ma.ndyn) {
      c -= ma.ndyn;
      if (c < mf.blocks) {
        const foldk::FoldJob& job = mf.j[foldk::find_job(mf.j, mf.count, c)];
        uint32_t* fl = reinterpret_cast<uint32_t*>(lds);
        uint64_t* gsum = reinterpret_cast<uint64_t*>(lds + foldk::LDS_WORDS * 4);
        uint32_t* flag = reinterpret_cast<uint32_t*>(gsum + foldk::MAXG_ALL);
        foldk::fold_block_arrive(job, c - job.block_start, mf.ctrs, fl, gsum, flag);
        return;
      }
      eq_aux_block(eq, c - mf.blocks);
      return;
    }
    // a pool tile, if one is left
    if (threadIdx.x == 0) pick = pool_pick(ma, (int)(blockIdx.x % NXCD));
    __syncthreads();
    const int t = pick;
    if (t < 0) return;
    x = t / ma.pool;
    li = (ma.gemm_blocks - x + NXCD - 1) / NXCD - ma.pool + t % ma.pool;  // XCD x holds tiles [0, L_x)
  }
  for (; m < ma.count - 1; ++m) {
    const int c = ma.split[m][x + 1] - ma.split[m][x];
    if (li < c) break;
    li -= c;
  }
  const MmDev& d = ma.m[m];
  WitArgs a{};
  a.X = d.X; a.ldx = d.ldx; a.W = d.Wp;
  a.T = d.T; a.N = d.N; a.K = d.K; a.s = ma.s;
  a.Z = d.Z; a.Y = d.Y; a.R = d.R;
  a.tiles_t = d.tiles_t; a.tiles_o = d.tiles_o;
  a.vecZ = d.vecZ; a.vecYR = d.vecYR;
  a.wp_rb = d.wp_rb; a.wp_kb = d.wp_kb;
  a.cEt = d.Et; a.cEo = d.Eo; a.cpart = d.cpart; a.cout = d.cout; a.cctr = d.cctr;
  multi_body<NW, TM, TN, PFW, PFX, NBUF, SCHED, 0, SB>(a, ma.split[m][x] + li, d.tiles_t * d.tiles_o, ma.group_o, lds);
}

// 256 x 128 tiles (4 waves of 64 x 128); each LDS stage holds two packed K
// blocks (128 bytes of k: half the barriers per product, and a row pitch of
// 144 bytes keeps the X stores off each other's banks); weights 2 stages
// ahead, X 1 stage ahead through 2 LDS stages.
#define WIT_MULTI 4, 2, 4, 2, 1, 2, 0, 2

// ---- groups of rows, one weight matrix each (the experts of an MoE block) --
// Group g owns rows [row_off[g], row_off[g+1]) of X and of the outputs and its
// own packed weights; its tiles are [tile_off[g], tile_off[g+1]) of the
// launch (256 outputs x 32 tokens: an expert holds few tokens), dealt to the
// XCDs in contiguous runs, so a weight panel's token tiles share one L2.
constexpr int GRP_MAX = 128;
struct GroupArgs {
  const int8_t* X;
  int64_t ldx;
  int32_t* Z;
  int8_t* Y;
  int8_t* R;
  const int8_t* Wp[GRP_MAX];
  const uint64_t* Et[GRP_MAX];  // group g's E_t (claims), or all NULL
  const uint64_t* Eo;           // group g's E_o at Eo + g ldeo
  int64_t ldeo;
  uint64_t* cout;               // group g's claim at cout[g]
  uint64_t* cpart;              // one slot per GEMM wave of the launch
  uint32_t* cctr;               // one 64-byte counter line per group
  int32_t row_off[GRP_MAX + 1];
  int32_t tile_off[GRP_MAX + 1];
  int32_t gid[GRP_MAX];         // the caller's index of each (non-empty) group of the launch
  uint64_t* fpart;              // the weight folds' panel values: group g's at fpart + g tiles_o fpitch (or NULL)
  int64_t fpitch;
  int32_t G, N, K, s, wp_rb, wp_kb, vecZ, vecYR, tiles_o;
};
#define WIT_GROUPED 4, 2, 1, 3, 3, 3, 0

template <int NW, int TM, int TN, int PFW, int PFX, int NBUF, int SCHED>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3, 3))) void witness_grouped_kernel(
    GroupArgs ga) {
  using C = MCfg<NW, TM, TN, PFW, PFX, NBUF>;
  __shared__ __align__(16) int8_t lds[C::LDS_FOLD_BYTES];
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  int lo = 0, hi = ga.G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ga.tile_off[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int r0 = ga.row_off[g];
  WitArgs a{};
  a.X = ga.X + (int64_t)r0 * ga.ldx; a.ldx = ga.ldx; a.W = ga.Wp[g];
  a.T = ga.row_off[g + 1] - r0; a.N = ga.N; a.K = ga.K; a.s = ga.s;
  a.Z = ga.Z ? ga.Z + (int64_t)r0 * ga.N : nullptr;
  a.Y = ga.Y + (int64_t)r0 * ga.N;
  a.R = ga.R + (int64_t)r0 * ga.N;
  a.tiles_t = (a.T + C::BT - 1) / C::BT; a.tiles_o = ga.tiles_o;
  a.vecZ = ga.vecZ; a.vecYR = ga.vecYR;
  a.wp_rb = ga.wp_rb; a.wp_kb = ga.wp_kb;
  const int id = ga.gid[g];
  if (ga.Eo) a.cEo = ga.Eo + (int64_t)id * ga.ldeo;
  if (ga.Et[g]) {
    a.cEt = ga.Et[g];
    a.cout = ga.cout + id;
    a.cpart = ga.cpart + (int64_t)ga.tile_off[g] * NW;
    a.cctr = ga.cctr + 16 * id;
  }
  if (ga.fpart) {
    a.fpart = ga.fpart + (int64_t)id * ga.tiles_o * ga.fpitch;
    a.fpitch = ga.fpitch;
  }
  multi_body<NW, TM, TN, PFW, PFX, NBUF, SCHED, 1>(a, tile - ga.tile_off[g], ga.tile_off[g + 1] - ga.tile_off[g], 1,
                                                   lds);
}

// The weight folds from their panels' values: out[g ldout + k] = sum over the
// panels p of part[(g tiles_o + p) fpitch + k] for k < K, zero up to cols_pad;
// groups whose flag is 0 (no rows, so no tiles and no panel values) are left alone.
struct PanelSumArgs {
  const uint64_t* part;
  uint64_t* out;
  int64_t fpitch, ldout;
  int32_t tiles_o, K, cols_pad;
  uint8_t live[FP_MAX_GROUPS];
};
__global__ __launch_bounds__(256) void panel_sum_kernel(PanelSumArgs pa) {
  const int g = blockIdx.y;
  if (!pa.live[g]) return;
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= pa.cols_pad) return;
  uint64_t v = 0;
  if (k < pa.K) {
    const uint64_t* p = pa.part + (int64_t)g * pa.tiles_o * pa.fpitch + k;
    for (int t = 0; t < pa.tiles_o; ++t) v = gl::add(v, p[(int64_t)t * pa.fpitch]);
  }
  pa.out[(int64_t)g * pa.ldout + k] = v;
}

using GC = MCfg<4, 2, 1, 3, 3, 3>;

// Workspace of a grouped call: a 64-byte counter line per group, one claim slot
// per GEMM wave of every tile, then (with weight folds) each group's panel values.
struct GroupedWs {
  size_t ctr_bytes, part_bytes, fold_bytes;
  int64_t fpitch;
};
GroupedWs grouped_ws(const int32_t* row_off, int32_t G, int32_t d_in, int32_t d_out, bool fold) {
  int64_t tiles = 0;
  for (int g = 0; g < G; ++g) tiles += (int64_t)((row_off[g + 1] - row_off[g] + GC::BT - 1) / GC::BT);
  const int64_t tiles_o = (d_out + GC::BO - 1) / GC::BO;
  tiles *= tiles_o;
  GroupedWs w{};
  w.ctr_bytes = fpi::align_up((size_t)G * 64, 256);
  w.part_bytes = fpi::align_up((size_t)tiles * GC::NWAVES * 8, 256);
  w.fpitch = (int64_t)((d_in + WP_BK - 1) / WP_BK) * WP_BK;
  w.fold_bytes = fold ? fpi::align_up((size_t)G * tiles_o * w.fpitch * 8, 256) : 0;
  return w;
}

struct MultiPlan {
  int64_t tiles[MM_MAX];
  size_t part_off[MM_MAX];
  size_t sc_off[MULTI_MAX_SC];
  size_t bytes;
};

// Workspace: the claims' arrival counters (one 64-byte line per map); the
// folds' counters and partial values (fold_bytes of them, from plan_folds;
// the counters' FP_FOLD_COUNTER_BYTES even without folds);
// one slot per GEMM wave of every map that forms a claim; each sum-check's
// table buffers.
template <int NW, int TM, int TN, int PFW, int PFX, int NBUF, int SCHED, int SB>
int multi_plan(const char* fn, int32_t count, const fp_matmul_desc* mm, size_t fold_bytes, int32_t n_sc,
               const fp_sumcheck_desc* sc, MultiPlan& p) {
  using MC = MCfg<NW, TM, TN, PFW, PFX, NBUF, SB>;
  if (count < 1 || count > MM_MAX) return fpi::fail(FP_EARG, "%s: count=%d outside [1, %d]", fn, count, MM_MAX);
  if (!mm) return fpi::fail(FP_EARG, "%s: null descs", fn);
  size_t off = CLAIM_CTR_BYTES + fpi::align_up(fold_bytes, 256);
  for (int i = 0; i < count; ++i) {
    const fp_matmul_desc& d = mm[i];
    if (d.T < 0 || d.d_in < 0 || d.d_out < 0) return fpi::fail(FP_EARG, "%s: map %d has a negative size", fn, i);
    const int64_t tiles = (int64_t)((d.T + MC::BT - 1) / MC::BT) * ((d.d_out + MC::BO - 1) / MC::BO);
    p.tiles[i] = tiles;
    p.part_off[i] = off;
    if (d.E_t) off += fpi::align_up((size_t)tiles * NW * 8, 256);
  }
  if (n_sc < 0 || n_sc > MULTI_MAX_SC)
    return fpi::fail(FP_EARG, "%s: %d sum-checks (at most %d)", fn, n_sc, MULTI_MAX_SC);
  if (n_sc > 0 && !sc) return fpi::fail(FP_EARG, "%s: null sum-check descs", fn);
  for (int k = 0; k < n_sc; ++k) {
    if (sc[k].n_pairs < 1 || sc[k].n_pairs > scs::MAX_PAIRS)
      return fpi::fail(FP_EARG, "%s: sum-check %d has n_pairs=%d outside [1, %d]", fn, k, sc[k].n_pairs, scs::MAX_PAIRS);
    if (sc[k].n < 1 || sc[k].n > FP_STEP_MULTI_MAX_SC_N)
      return fpi::fail(FP_ESHAPE, "%s: sum-check %d has n=%d outside [1, %d]", fn, k, sc[k].n, FP_STEP_MULTI_MAX_SC_N);
    p.sc_off[k] = off;
    off += fpi::align_up((size_t)scs::workspace_entries(sc[k].n_pairs, sc[k].n) * 8, 256);
  }
  p.bytes = off;
  return FP_OK;
}

// Scratch of the allocation-free variant: arrival counters and claim slots in
// a file-scope device array (each GPU holds its own copy until the process
// ends). Host code reaches it only through the per-device address that
// hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[FP_WITNESS_MULTI_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The scratch array's device address on the current device (looked up once per device).
int scratch_address(const char* fn, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
    return fpi::fail(FP_EHIP, "%s: no current device (or device index >= %d)", fn, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fpi::fail(FP_EHIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", fn, dev,
                       hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FP_OK;
}

// Zeroes n 32-bit words (the arrival counters before an allocation-free call).
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += 256) p[i] = 0;
}

}  // namespace

extern "C" size_t fp_witness_grouped_packed_workspace(const int32_t* row_off, int32_t G, int32_t d_in, int32_t d_out,
                                                      int32_t with_fold) {
  if (G < 0 || G > FP_MAX_GROUPS || !row_off || d_out < 0 || d_in < 0) return 0;
  for (int g = 0; g < G; ++g)
    if (row_off[g + 1] < row_off[g]) return 0;
  const GroupedWs w = grouped_ws(row_off, G, d_in, d_out, with_fold != 0);
  return w.ctr_bytes + w.part_bytes + w.fold_bytes;
}

extern "C" int fp_witness_grouped_packed(const int8_t* X, int64_t ldx, const int8_t* const* Wp, const int32_t* row_off,
                                         int32_t G, int32_t d_in, int32_t d_out, int32_t s, int32_t* Z, int8_t* Y,
                                         int8_t* R, const fp_elem* const* E_t, const fp_elem* E_o, int64_t ldeo,
                                         fp_elem* claims, fp_elem* w_fold, int64_t ld_fold, int32_t fold_cols_pad,
                                         void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "fp_witness_grouped_packed";
  if (G < 0 || G > FP_MAX_GROUPS) return fpi::fail(FP_EARG, "%s: G=%d outside [0, %d]", fn, G, FP_MAX_GROUPS);
  if (G == 0) return fpi::ok();
  if (!row_off || !Wp) return fpi::fail(FP_EARG, "%s: null host array", fn);
  if (row_off[0] != 0) return fpi::fail(FP_EARG, "%s: row_off[0] != 0", fn);
  for (int g = 0; g < G; ++g)
    if (row_off[g + 1] < row_off[g]) return fpi::fail(FP_EARG, "%s: row_off decreases at %d", fn, g);
  const int32_t total = row_off[G];
  if (d_in < 0 || d_out < 0) return fpi::fail(FP_EARG, "%s: negative size", fn);
  if (d_in > FP_MAX_DIN) return fpi::fail(FP_ESHAPE, "%s: d_in=%d > %d", fn, d_in, FP_MAX_DIN);
  if (s < 1 || s > 8) return fpi::fail(FP_ERANGE, "%s: s=%d outside [1, 8]", fn, s);
  if (ldx < d_in) return fpi::fail(FP_ESHAPE, "%s: ldx < d_in", fn);
  if (total == 0 || d_out == 0) return fpi::ok();
  if (!Y || !R) return fpi::fail(FP_EARG, "%s: null Y or R", fn);
  if (d_in > 0) {
    if (!X) return fpi::fail(FP_EARG, "%s: null X", fn);
    if (d_in % 16 != 0 || ldx % 16 != 0 || (((uintptr_t)X) & 15) != 0)
      return fpi::fail(FP_ESHAPE, "%s: needs d_in %% 16 == 0 and 16-byte aligned X rows", fn);
  }
  const bool claim = E_t != nullptr;
  const bool fold = w_fold != nullptr;
  if (claim && !claims) return fpi::fail(FP_EARG, "%s: claims need an output", fn);
  if ((claim || fold) && (!E_o || ldeo < d_out)) return fpi::fail(FP_EARG, "%s: claims and folds need E_o, ldeo >= d_out", fn);
  if (fold && (fold_cols_pad < d_in || ld_fold < fold_cols_pad))
    return fpi::fail(FP_ESHAPE, "%s: weight folds need d_in <= fold_cols_pad <= ld_fold", fn);
  const GroupedWs gw = grouped_ws(row_off, G, d_in, d_out, fold);
  if (claim || fold) {
    const size_t need = gw.ctr_bytes + gw.part_bytes + gw.fold_bytes;
    if (!ws || ws_bytes < need) return fpi::fail(FP_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
    if ((((uintptr_t)ws) & 255) != 0) return fpi::fail(FP_EARG, "%s: workspace not 256-byte aligned", fn);
  }
  for (int g = 0; g < G; ++g) {
    if (row_off[g + 1] == row_off[g]) continue;
    if (d_in > 0 && (!Wp[g] || (((uintptr_t)Wp[g]) & 15)))
      return fpi::fail(FP_EARG, "%s: packed W of group %d is null or not 16-byte aligned", fn, g);
    if (claim && !E_t[g]) return fpi::fail(FP_EARG, "%s: null E_t for group %d", fn, g);
  }
  GroupArgs ga{};
  ga.X = X; ga.ldx = ldx; ga.Z = Z; ga.Y = Y; ga.R = R;
  ga.N = d_out; ga.K = d_in; ga.s = s;
  ga.wp_rb = (d_out + 31) / 32;
  ga.wp_kb = (d_in + WP_BK - 1) / WP_BK;
  ga.tiles_o = (d_out + GC::BO - 1) / GC::BO;
  ga.vecZ = ((d_out & 3) == 0) && ((((uintptr_t)Z) & 15) == 0);
  ga.vecYR = ((d_out & 15) == 0) && ((((uintptr_t)Y) & 15) == 0) && ((((uintptr_t)R) & 15) == 0);
  ga.Eo = E_o;
  ga.ldeo = ldeo;
  static_assert(sizeof(GroupArgs) <= 4096, "kernel arguments must fit 4 KiB");
  const size_t ctr_bytes = gw.ctr_bytes;
  ga.cout = claims;
  ga.fpart = fold ? (uint64_t*)((char*)ws + gw.ctr_bytes + gw.part_bytes) : nullptr;
  ga.fpitch = gw.fpitch;
  ga.cctr = claim ? (uint32_t*)ws : nullptr;
  int64_t tile_base = 0;  // tiles of the launches before (their claim slots)
  for (int g0 = 0; g0 < G; g0 += GRP_MAX) {
    const int gc = (G - g0) < GRP_MAX ? (G - g0) : GRP_MAX;
    int ng = 0;
    int64_t tiles = 0;
    for (int g = g0; g < g0 + gc; ++g) {
      const int rows = row_off[g + 1] - row_off[g];
      if (rows == 0) continue;  // empty groups own no tiles
      ga.Wp[ng] = Wp[g];
      ga.Et[ng] = claim ? E_t[g] : nullptr;
      ga.gid[ng] = g;
      ga.row_off[ng] = row_off[g];
      ga.row_off[ng + 1] = row_off[g + 1];
      ga.tile_off[ng] = (int32_t)tiles;
      tiles += (int64_t)((rows + GC::BT - 1) / GC::BT) * ga.tiles_o;
      ++ng;
    }
    if (ng == 0) continue;
    if (tiles > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "%s: too many tiles", fn);
    ga.tile_off[ng] = (int32_t)tiles;
    ga.G = ng;
    ga.cpart = claim ? (uint64_t*)((char*)ws + ctr_bytes) + tile_base * GC::NWAVES : nullptr;
    hipLaunchKernelGGL((witness_grouped_kernel<WIT_GROUPED>), dim3((unsigned)tiles), dim3(GC::NT), 0, stream, ga);
    const int rc = fpi::check_launch("witness_grouped_kernel");
    if (rc) return rc;
    tile_base += tiles;
  }
  if (fold && fold_cols_pad > 0) {
    PanelSumArgs pa{};
    pa.part = ga.fpart;
    pa.out = w_fold;
    pa.fpitch = gw.fpitch;
    pa.ldout = ld_fold;
    pa.tiles_o = ga.tiles_o;
    pa.K = d_in;
    pa.cols_pad = fold_cols_pad;
    for (int g = 0; g < G; ++g) pa.live[g] = row_off[g + 1] > row_off[g] ? 1 : 0;
    hipLaunchKernelGGL(panel_sum_kernel, dim3((unsigned)((fold_cols_pad + 255) / 256), (unsigned)G), dim3(256), 0,
                       stream, pa);
    const int rc = fpi::check_launch("panel_sum_kernel");
    if (rc) return rc;
  }
  return fpi::ok();
}

extern "C" size_t fp_witness_multi_workspace(int32_t count, const fp_matmul_desc* mm) {
  MultiPlan p;
  if (multi_plan<WIT_MULTI>("fp_witness_multi_workspace", count, mm, 0, 0, nullptr, p)) return 0;
  return p.bytes;
}

namespace {

// fp_witness_multi's checks and launch for one tile configuration; noalloc:
// ws is the scratch array (its counters cleared first on the stream).
template <int NW, int TM, int TN, int PFW, int PFX, int NBUF, int SCHED, int SB>
int multi_launch(const char* fn, int32_t count, const fp_matmul_desc* mm, int32_t s, int32_t group_o, int32_t n_eq,
                 const fp_eq_desc* eq, int32_t n_fold, const fp_fold_desc* folds, int32_t n_sc,
                 const fp_sumcheck_desc* sc, void* ws, size_t ws_bytes, bool noalloc, bool plan_only, size_t* need,
                 hipStream_t stream) {
  using MC = MCfg<NW, TM, TN, PFW, PFX, NBUF, SB>;
  // the folds' counters and parts follow the claims' counters
  MultiFolds mf;
  size_t fold_bytes = 0;
  uint64_t* unused_part;
  uint32_t* unused_ctr;
  int rc = plan_folds<MULTI_MAX_FOLD>(fn, n_fold, folds, 0, nullptr, 0, ws ? (char*)ws + CLAIM_CTR_BYTES : nullptr, 0,
                                      true, &fold_bytes, mf, &unused_part, &unused_ctr);
  if (rc) return rc;
  // the folds' counter region is always there, so that one workspace serves
  // calls with and without folds (its counters stay zero between calls)
  if (fold_bytes < (size_t)FP_FOLD_COUNTER_BYTES) fold_bytes = FP_FOLD_COUNTER_BYTES;
  MultiPlan p;
  rc = multi_plan<NW, TM, TN, PFW, PFX, NBUF, SCHED, SB>(fn, count, mm, fold_bytes, n_sc, sc, p);
  if (rc) return rc;
  if (plan_only) {
    *need = p.bytes;
    return FP_OK;
  }
  if (s < 1 || s > 8) return fpi::fail(FP_ERANGE, "%s: s=%d outside [1, 8]", fn, s);
  if (group_o < 1) return fpi::fail(FP_EARG, "%s: group_o=%d < 1", fn, group_o);
  bool any_claim = false;
  MultiArgs ma{};
  ma.count = count;
  ma.s = s;
  ma.group_o = group_o;
  int64_t total = 0, rem_before = 0;
  for (int i = 0; i < count; ++i) {
    const fp_matmul_desc& d = mm[i];
    if (d.d_in > FP_MAX_DIN) return fpi::fail(FP_ESHAPE, "%s: map %d has d_in=%d > %d", fn, i, d.d_in, FP_MAX_DIN);
    const bool work = d.T > 0 && d.d_out > 0;
    if (work && (!d.Y || !d.R)) return fpi::fail(FP_EARG, "%s: map %d has a null Y or R", fn, i);
    if (work && d.d_in > 0) {
      if (!d.X || !d.Wp) return fpi::fail(FP_EARG, "%s: map %d has a null X or packed W", fn, i);
      if (d.d_in % 16 != 0 || d.ldx % 16 != 0 || (((uintptr_t)d.X) & 15) != 0 || (((uintptr_t)d.Wp) & 15) != 0)
        return fpi::fail(FP_ESHAPE, "%s: map %d needs d_in %% 16 == 0 and 16-byte aligned X rows and packed W", fn,
                         i);
    }
    if (d.ldx < d.d_in) return fpi::fail(FP_ESHAPE, "%s: map %d has ldx < d_in", fn, i);
    if (d.E_t) {
      if (!work) return fpi::fail(FP_ESHAPE, "%s: map %d forms a claim but has no outputs", fn, i);
      if (!d.E_o || !d.claim) return fpi::fail(FP_EARG, "%s: map %d has E_t but a null E_o or claim", fn, i);
      any_claim = true;
    }
    MmDev& m = ma.m[i];
    m.X = d.X; m.ldx = d.ldx; m.Wp = d.Wp;
    m.Z = d.Z; m.Y = d.Y; m.R = d.R;
    m.T = d.T; m.K = d.d_in; m.N = d.d_out;
    m.wp_rb = (d.d_out + 31) / 32;
    m.wp_kb = (d.d_in + WP_BK - 1) / WP_BK;
    m.tiles_t = (d.T + MC::BT - 1) / MC::BT;
    m.tiles_o = (d.d_out + MC::BO - 1) / MC::BO;
    m.vecZ = ((d.d_out & 3) == 0) && ((((uintptr_t)d.Z) & 15) == 0);
    m.vecYR = ((d.d_out & 15) == 0) && ((((uintptr_t)d.Y) & 15) == 0) && ((((uintptr_t)d.R) & 15) == 0);
    if (d.E_t) {
      m.Et = d.E_t; m.Eo = d.E_o; m.cout = d.claim;
      m.cctr = (uint32_t*)((char*)ws + 64 * i);
      m.cpart = (uint64_t*)((char*)ws + p.part_off[i]);
    }
    // deal the map's tiles to the XCDs: equal contiguous chunks, the remainders
    // rotating across maps so that XCD x gets exactly the workgroups b % 8 == x
    const int64_t n = work ? p.tiles[i] : 0;
    const int64_t base = n / NXCD, rem = n % NXCD;
    int64_t off = 0;
    for (int x = 0; x < NXCD; ++x) {
      ma.split[i][x] = (int32_t)off;
      const int64_t extra = ((x - rem_before) % NXCD + NXCD) % NXCD < rem ? 1 : 0;
      off += base + extra;
    }
    ma.split[i][NXCD] = (int32_t)off;
    rem_before += rem;
    total += n;
  }
  if (any_claim || n_fold > 0 || n_sc > 0) {
    if (noalloc && p.bytes > FP_WITNESS_MULTI_SCRATCH_BYTES)
      return fpi::fail(FP_EWORKSPACE, "%s: these maps need %zu bytes of scratch, more than the %d the library holds", fn,
                       p.bytes, FP_WITNESS_MULTI_SCRATCH_BYTES);
    if (!ws || ws_bytes < p.bytes)
      return fpi::fail(FP_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, p.bytes);
    if ((((uintptr_t)ws) & 255) != 0) return fpi::fail(FP_EARG, "%s: workspace not 256-byte aligned", fn);
  }
  EqAux aux;
  rc = eq_aux(fn, n_eq, eq, aux);
  if (rc) return rc;
  SumAux sa{};
  sa.count = n_sc;
  sa.blocks = (n_sc + NXCD - 1) / NXCD * NXCD;
  for (int k = 0; k < n_sc; ++k) {
    const fp_sumcheck_desc& d = sc[k];
    if (!d.r || !d.rounds || !d.finals) return fpi::fail(FP_EARG, "%s: sum-check %d has a null pointer", fn, k);
    scs::Inst& in = sa.inst[k];
    for (int j = 0; j < d.n_pairs; ++j) {
      if (!d.A[j] || !d.B[j] || (((uintptr_t)d.A[j]) & 15) || (((uintptr_t)d.B[j]) & 15))
        return fpi::fail(FP_EARG, "%s: sum-check %d table %d is null or not 16-byte aligned", fn, k, j);
      in.A[j] = d.A[j];
      in.B[j] = d.B[j];
    }
    in.rho = d.rho; in.r = d.r; in.rounds = d.rounds; in.finals = d.finals; in.claim0 = d.claim0;
    in.scratch = (fp_elem*)((char*)ws + p.sc_off[k]);
    in.n = d.n;
    in.n_pairs = d.n_pairs;
    in.i0 = scs::stream_rounds(d.n_pairs, d.n);
  }
  // the fold jobs again, now against the real workspace
  if (n_fold > 0) {
    rc = plan_folds<MULTI_MAX_FOLD>(fn, n_fold, folds, 0, nullptr, 0, (char*)ws + CLAIM_CTR_BYTES,
                                    ws_bytes - CLAIM_CTR_BYTES, false, &fold_bytes, mf, &unused_part, &unused_ctr);
    if (rc) return rc;
  }
  // the tile pool needs the workspace's counter lines (zero on entry)
  ma.pool = 0;
  ma.ndyn = 0;
  ma.qctr = nullptr;
  if (!noalloc && (any_claim || n_fold > 0 || n_sc > 0) && total >= 2 * GPU_SLOTS) {
    ma.pool = (int32_t)(total / NXCD * POOL_PERCENT / 100);
    ma.ndyn = 2 * NXCD * ma.pool;
    ma.qctr = (uint32_t*)ws;
  }
  const int64_t grid = (int64_t)sa.blocks + total + (ma.ndyn - NXCD * ma.pool) + mf.blocks + aux.block_start[aux.count];
  if (grid > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "%s: too many workgroups", fn);
  ma.gemm_blocks = (int32_t)total;
  if (grid == 0) return fpi::ok();
  if (noalloc && any_claim) {
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, stream, (uint32_t*)ws, (int)(CLAIM_CTR_BYTES / 4));
    rc = fpi::check_launch("clear_words_kernel");
    if (rc) return rc;
  }
  static_assert(sizeof(MultiArgs) + sizeof(EqAux) + sizeof(MultiFolds) + sizeof(SumAux) <= 4096,
                "kernel arguments must fit 4 KiB");
  hipLaunchKernelGGL((witness_multi_kernel<NW, TM, TN, PFW, PFX, NBUF, SCHED, SB>), dim3((unsigned)grid), dim3(MC::NT), 0,
                     stream, ma, aux, mf, sa);
  rc = fpi::check_launch("witness_multi_kernel");
  return rc ? rc : fpi::ok();
}

}  // namespace

extern "C" int fp_witness_multi(int32_t count, const fp_matmul_desc* mm, int32_t s, int32_t group_o, int32_t n_eq,
                                const fp_eq_desc* eq, void* ws, size_t ws_bytes, hipStream_t stream) {
  return multi_launch<WIT_MULTI>("fp_witness_multi", count, mm, s, group_o, n_eq, eq, 0, nullptr, 0, nullptr, ws,
                                 ws_bytes, false, false, nullptr, stream);
}

extern "C" int fp_layer_step_multi(int32_t count, const fp_matmul_desc* mm, int32_t s, int32_t group_o, int32_t n_eq,
                                   const fp_eq_desc* eq, int32_t n_fold, const fp_fold_desc* folds, int32_t n_sc,
                                   const fp_sumcheck_desc* sc, void* ws, size_t ws_bytes, hipStream_t stream) {
  return multi_launch<WIT_MULTI>("fp_layer_step_multi", count, mm, s, group_o, n_eq, eq, n_fold, folds, n_sc, sc, ws,
                                 ws_bytes, false, false, nullptr, stream);
}

extern "C" size_t fp_layer_step_multi_workspace(int32_t count, const fp_matmul_desc* mm, int32_t n_fold,
                                                const fp_fold_desc* folds, int32_t n_sc, const fp_sumcheck_desc* sc) {
  size_t need = 0;
  if (multi_launch<WIT_MULTI>("fp_layer_step_multi_workspace", count, mm, 8, 1, 0, nullptr, n_fold, folds, n_sc, sc,
                              nullptr, 0, false, true, &need, nullptr))
    return 0;
  return need;
}

extern "C" int fp_witness_multi_noalloc(int32_t count, const fp_matmul_desc* mm, int32_t s, int32_t group_o,
                                        int32_t n_eq, const fp_eq_desc* eq, hipStream_t stream) {
  const char* fn = "fp_witness_multi_noalloc";
  void* ws = nullptr;
  const int rc = scratch_address(fn, &ws);
  if (rc) return rc;
  return multi_launch<WIT_MULTI>(fn, count, mm, s, group_o, n_eq, eq, 0, nullptr, 0, nullptr, ws,
                                 FP_WITNESS_MULTI_SCRATCH_BYTES, true, false, nullptr, stream);
}
