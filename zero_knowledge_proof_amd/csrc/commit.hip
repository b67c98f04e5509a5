// commit.hip - commitment of committed tables: limb packing, Reed-Solomon
// encoding by NTT, and a salted BLAKE2b Merkle tree over the columns.
//
// "How fast can FlashProve go", §3.1: to commit a table, each row is
// Reed-Solomon encoded (an NTT; a row of 2^22 elements becomes 2^23) and each
// column is Merkle hashed with BLAKE2b; values are cut into 8-bit limbs and
// three limbs share a field element in 20-bit slots. Here a row c_0..c_{n-1} is
// the coefficient vector of a polynomial evaluated at w^j, j < 2n, with w =
// 7^((p-1)/2n); column j's leaf is BLAKE2b-256(salt_j || code[0][j] || ... ||
// code[rows-1][j]) and a parent is BLAKE2b-256(left || right). BLAKE2b follows
// RFC 7693 (Saarinen and Aumasson, 2015).
//
// NTT of N = 2^L points (L <= 24) in P = ceil(L/8) passes over HBM. With
// N = N_1 ... N_P, n = sum_p n_p S_p (S_p = N_{p+1} ... N_P) and
// k = sum_p k_p T_p (T_p = N_1 ... N_{p-1}), n k = sum_p n_p S_p (k_p T_p + K_{p-1})
// (mod N) with K_{p-1} = sum_{q<p} k_q T_q, so pass p multiplies each element by
// w^(n_p S_p K_{p-1}) and transforms along n_p (N_p <= 256 points, inside LDS);
// k_p takes n_p's place in memory, and the last pass writes X[K_P] in natural
// order. A pass works on a [N_p x 16] tile: 16 neighbouring columns (or, in the
// last pass, 16 neighbouring K), so that global accesses are 128-byte runs. An
// N_p-point transform is two register transforms of at most 16 points: the
// first reads its elements straight from HBM, the second reads the first's
// results through LDS. Their internal twiddles are powers of w_16 = 2^156
// (w_64 = 2^39 for this generator, and 2^96 = -1), i.e. shifts.
#include "blake2b.hpp"
#include "common.hpp"
#include "gl.hpp"

namespace {

// ----------------------------------------------------------------- packing
// msg[e] = l_{3e} + 2^20 l_{3e+1} + 2^40 l_{3e+2}: limb l is byte l of the
// stream A (na bytes) followed by B (nb bytes), 0 past both.
__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ A, int64_t na,
                                                   const int8_t* __restrict__ B, int64_t nb, int64_t total,
                                                   uint64_t* __restrict__ msg) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  uint64_t v = 0;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int64_t l = 3 * e + q;
    uint32_t limb = 0;
    if (l < na) limb = (uint8_t)A[l];
    else if (l - na < nb) limb = (uint8_t)B[l - na];
    v |= (uint64_t)limb << (20 * q);
  }
  msg[e] = v;
}

// --------------------------------------------------------------------- NTT
constexpr int NTT_MAXP = 3;   // passes (N <= 2^24)
// Columns (or transforms) per workgroup of a pass of 2^lp points: NTT_T / R_b, so that stage A's R_b TC
// tasks fill the workgroup (and stage B's NTT_T / TC groups cover the R_a outputs); at least 16 (the
// 256-point pass). The LDS tile [N_p][TC + 1] fits 256 x 17 words for every lp <= 8.
constexpr int tile_cols(int lp) { return (256 >> (lp / 2)) < 16 ? 16 : (256 >> (lp / 2)); }
constexpr int TILE_WORDS = 256 * 17;
constexpr int NTT_T = 256;    // threads
constexpr int TW_BITS = 12;   // w^e = hi[e >> 12] * lo[e & 4095]

// x * 2^e mod p for 0 <= e < 192 (e is a compile-time constant after unrolling):
// 2^96 = -1 and 2^64 = 2^32 - 1.
__device__ __forceinline__ uint64_t mul_pow2(uint64_t x, int e) {
  const bool neg = e >= 96;
  if (neg) e -= 96;
  if (e >= 64) {
    x = gl::sub(gl::reduce128(x << 32, x >> 32), x);  // x (2^32 - 1)
    e -= 64;
  }
  if (e > 0) x = gl::reduce128(x << e, x >> (64 - e));
  return neg ? gl::sub(0, x) : x;
}

// exponent of w_m as a power of 2, for m | 64: w_64 = 2^39
constexpr int root_exp(int m) { return (39 * (64 / m)) % 192; }

// In-register DFT of R <= 16 points, natural order in and out:
// v[k] <- sum_n v[n] w_R^(nk). Radix-2 decimation in frequency, then the
// bit-reversal permutation as a register renaming.
template <int R>
__device__ __forceinline__ void dft_small(uint64_t (&v)[16]) {
  if constexpr (R == 1) return;
#pragma unroll
  for (int half = R / 2; half >= 1; half >>= 1) {
#pragma unroll
    for (int g = 0; g < R; g += 2 * half) {
#pragma unroll
      for (int j = 0; j < half; ++j) {
        const uint64_t a = v[g + j], b = v[g + j + half];
        v[g + j] = gl::add(a, b);
        v[g + j + half] = mul_pow2(gl::sub(a, b), (root_exp(2 * half) * j) % 192);
      }
    }
  }
  uint64_t t[16];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    int r = 0;
#pragma unroll
    for (int b = 1, kk = k; b < R; b <<= 1, kk >>= 1) r = (r << 1) | (kk & 1);
    t[k] = v[r];
  }
#pragma unroll
  for (int k = 0; k < R; ++k) v[k] = t[k];
}


struct NttArgs {
  const uint64_t* src;
  uint64_t* dst;
  int64_t src_rs, dst_rs;    // row strides (elements)
  const uint64_t* tw_lo;     // w_N^i, i < 4096
  const uint64_t* tw_hi;     // w_N^(4096 i)
  int32_t L;                 // log2 N
  int32_t P, p;              // passes, this pass (0-based)
  int32_t lN[NTT_MAXP];      // log2 N_q
  int32_t first, last;
  int32_t blocks_per_row;
  int32_t lS, lT;            // log2 S_p, log2 T_p of this pass
  // base(K) = sum_{q<p} k_q S_q with k_q = (K >> dT[q]) & dM[q], S_q = 2^dS[q]
  int32_t dT[NTT_MAXP - 1], dM[NTT_MAXP - 1], dS[NTT_MAXP - 1];
};

__device__ __forceinline__ uint64_t w_pow(const NttArgs& a, int64_t e) {
  const uint64_t lo = a.tw_lo[e & ((1 << TW_BITS) - 1)];
  if (a.L <= TW_BITS) return lo;
  return gl::mul(a.tw_hi[e >> TW_BITS], lo);
}

// One pass of N_p = 2^LP points: see the file comment. LDS tile [N_p][TILE_C]
// (between the two register transforms) plus the pass's in-tile twiddles w_{N_p}^i.
template <int LP>
__global__ __launch_bounds__(NTT_T) void ntt_pass_kernel(NttArgs a) {
  constexpr int TILE_C = tile_cols(LP), TILE_P = TILE_C + 1;  // an odd pitch: column walks spread over banks
  static_assert((1 << LP) * TILE_P <= TILE_WORDS, "LDS tile");
  __shared__ uint64_t tile[TILE_WORDS];
  __shared__ uint64_t twp[256];
  __shared__ uint64_t twk[256];  // a middle pass's twiddles w^(n S_p K) for the tile's one K
  const int tid = threadIdx.x;
  const int row = blockIdx.x / a.blocks_per_row;
  const int blk = blockIdx.x % a.blocks_per_row;
  const int p = a.p;
  constexpr int lp = LP;
  constexpr int Np = 1 << LP;
  const int lS = a.lS, lT = a.lT;
  const uint64_t* src = a.src + (int64_t)row * a.src_rs;
  uint64_t* dst = a.dst + (int64_t)row * a.dst_rs;

  // which transforms: not last -> K = kidx, columns c0 + c; last -> K = kidx0 + c
  int64_t kidx = 0, c0 = 0;
  int ncols;  // valid columns of the tile
  if (!a.last) {
    const int64_t S = (int64_t)1 << lS;
    const int64_t cblocks = (S + TILE_C - 1) / TILE_C;
    kidx = blk / cblocks;
    c0 = (blk % cblocks) * TILE_C;
    ncols = (int)min<int64_t>(TILE_C, S - c0);
  } else {
    c0 = (int64_t)blk * TILE_C;  // first K of the tile
    ncols = (int)min<int64_t>(TILE_C, ((int64_t)1 << lT) - c0);
  }
  // base(K) = sum_{q<p} k_q S_q for K = sum_{q<p} k_q T_q
  auto base_of = [&](int64_t K) {
    int64_t b = 0;
#pragma unroll
    for (int q = 0; q < NTT_MAXP - 1; ++q)
      if (q < p) b += ((K >> a.dT[q]) & a.dM[q]) << a.dS[q];
    return b;
  };

  // in-tile twiddles w_{N_p}^i = w_N^(i N / N_p); in a middle pass (neither the first nor the last) every
  // column of the tile has the same K, so its pass twiddles are one table of N_p values
  const bool mid = p > 0 && !a.last;
  for (int i = tid; i < Np; i += NTT_T) {
    twp[i] = w_pow(a, (int64_t)i << (a.L - lp));
    if (mid) twk[i] = w_pow(a, ((int64_t)i << lS) * kidx);
  }
  __syncthreads();

  // ---- N_p = R_a R_b. Stage A: each task (n_b, column) loads its R_a elements
  // n = i R_b + n_b straight from HBM, applies the pass twiddle w^(n S_p K)
  // as x y^i (x = w^(n_b S_p K), y = w^(R_b S_p K)), transforms over i, applies
  // w_{N_p}^(n_b k_a) and leaves the result in LDS at (k_a R_b + n_b).
  constexpr int la = (LP + 1) / 2, lb = LP / 2;
  constexpr int Ra = 1 << la, Rb = 1 << lb;
  constexpr int TASKS = Rb * TILE_C;
  uint64_t v[16];
  const int64_t b0 = a.last ? 0 : base_of(kidx);
  for (int q = tid; q < TASKS; q += NTT_T) {
    int nb, cc;
    int64_t rowbase, K;
    int sh;
    if (!a.last) {  // lanes along columns: 256-byte runs
      cc = q % TILE_C;
      nb = q / TILE_C;
      K = kidx;
      rowbase = b0 + c0 + cc;
      sh = lS;
    } else {  // lanes along n_b, then transforms: R_b-element runs
      cc = q / Rb;
      nb = q % Rb;
      K = c0 + cc;
      rowbase = cc < ncols ? base_of(K) : 0;
      sh = 0;
    }
    const bool ok = cc < ncols;
#pragma unroll
    for (int i = 0; i < Ra; ++i) {
      const int n = i * Rb + nb;
      v[i] = (ok && !(a.first && n >= Np / 2)) ? src[rowbase + ((int64_t)n << sh)] : 0;
    }
    if (mid && K != 0) {
#pragma unroll
      for (int i = 0; i < Ra; ++i) v[i] = gl::mul(v[i], twk[i * Rb + nb]);
    } else if (p > 0 && K != 0) {  // the last pass: K differs between the tile's columns
      uint64_t cur = w_pow(a, ((int64_t)nb << sh) * K);
      const uint64_t y = w_pow(a, ((int64_t)Rb << sh) * K);
#pragma unroll
      for (int i = 0; i < Ra; ++i) {
        v[i] = gl::mul(v[i], cur);
        if (i + 1 < Ra) cur = gl::mul(cur, y);
      }
    }
    dft_small<Ra>(v);
#pragma unroll
    for (int ka = 0; ka < Ra; ++ka) {
      const uint64_t x = (nb * ka) ? gl::mul(v[ka], twp[nb * ka]) : v[ka];
      tile[(ka * Rb + nb) * TILE_P + cc] = x;
    }
  }
  __syncthreads();
  // stage B over n_b (contiguous), k_p = k_a + R_a k_b
  const int c = tid % TILE_C, g = tid / TILE_C, G = NTT_T / TILE_C;
  for (int ka = g; ka < Ra; ka += G) {
#pragma unroll
    for (int i = 0; i < Rb; ++i) v[i] = tile[(ka * Rb + i) * TILE_P + c];
    dft_small<Rb>(v);
    if (c < ncols) {
      if (!a.last) {
#pragma unroll
        for (int kb = 0; kb < Rb; ++kb) dst[b0 + ((int64_t)(ka + Ra * kb) << lS) + c0 + c] = v[kb];
      } else {
#pragma unroll
        for (int kb = 0; kb < Rb; ++kb) dst[c0 + c + ((int64_t)(ka + Ra * kb) << lT)] = v[kb];
      }
    }
  }
}

// tw_lo[i] = w^i (i < 4096), tw_hi[i] = w^(4096 i) (i < N / 4096)
__global__ __launch_bounds__(256) void twiddle_kernel(uint64_t w, int32_t L, uint64_t* tw_lo, uint64_t* tw_hi) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int nlo = 1 << min(L, TW_BITS);
  const int nhi = L > TW_BITS ? 1 << (L - TW_BITS) : 0;
  if (i >= nlo + nhi) return;
  uint64_t base = w;
  int64_t e = i;
  uint64_t* out = tw_lo + i;
  if (i >= nlo) {
    e = i - nlo;
    for (int s = 0; s < TW_BITS; ++s) base = gl::mul(base, base);
    out = tw_hi + e;
  }
  uint64_t r = 1;
  while (e) {
    if (e & 1) r = gl::mul(r, base);
    base = gl::mul(base, base);
    e >>= 1;
  }
  *out = r;
}

constexpr int SALT_WORDS = 2;  // 16-byte salts

// leaf j = BLAKE2b-256(salt_j || code[0][j] || ... || code[rows-1][j]); the
// message is SALT_WORDS + rows 8-byte words, in 16-word blocks.
__global__ __launch_bounds__(256) void leaf_kernel(const uint64_t* __restrict__ code, int64_t ld, int32_t rows,
                                                   int64_t width, const uint64_t* __restrict__ salts,
                                                   uint64_t* __restrict__ leaves) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= width) return;
  uint64_t h[8];
  b2_init32(h);
  const int words = SALT_WORDS + rows;
  const int64_t bytes = 8 * (int64_t)words;
  for (int w0 = 0; w0 < words; w0 += 16) {
    uint64_t m[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int w = w0 + i;
      uint64_t x = 0;
      if (w < SALT_WORDS) x = salts[j * SALT_WORDS + w];
      else if (w < words) x = code[(int64_t)(w - SALT_WORDS) * ld + j];
      m[i] = x;
    }
    const bool last = w0 + 16 >= words;
    b2_compress(h, m, last ? (uint64_t)bytes : (uint64_t)(8 * (w0 + 16)), last);
  }
  uint64_t* out = leaves + 4 * j;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = h[i];
}

// K levels above level `in` (n_in digests): thread t hashes its 2^K children
// [t 2^K, (t+1) 2^K) up to one node, writing every node of its subtree to its
// level (out: the level above `in`, then the next, ...). Whole lanes stay busy
// at every level, and each thread reads and writes contiguous runs.
template <int K>
__global__ __launch_bounds__(256) void subtree_kernel(const uint64_t* __restrict__ in, int64_t n_in,
                                                      uint64_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (n_in >> K)) return;
  constexpr int H = 1 << (K - 1);  // nodes of the first level above the children
  uint64_t d[H][4];
  int64_t n_level = n_in >> 1;     // nodes in the level being written
  uint64_t* level = out;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    uint64_t m[16];
    const uint64_t* c = in + (t * (2 * H) + 2 * i) * 4;
#pragma unroll
    for (int w = 0; w < 8; ++w) m[w] = c[w];
#pragma unroll
    for (int w = 8; w < 16; ++w) m[w] = 0;
    uint64_t h[8];
    b2_init32(h);
    b2_compress(h, m, 64, true);
#pragma unroll
    for (int w = 0; w < 4; ++w) d[i][w] = h[w];
  }
#pragma unroll
  for (int lev = 0; lev < K; ++lev) {
    const int cnt = H >> lev;  // nodes of this level in the subtree
    if (lev > 0) {
#pragma unroll
      for (int i = 0; i < cnt; ++i) {
        uint64_t m[16];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          m[w] = d[2 * i][w];
          m[w + 4] = d[2 * i + 1][w];
        }
#pragma unroll
        for (int w = 8; w < 16; ++w) m[w] = 0;
        uint64_t h[8];
        b2_init32(h);
        b2_compress(h, m, 64, true);
#pragma unroll
        for (int w = 0; w < 4; ++w) d[i][w] = h[w];
      }
    }
    uint64_t* o = level + t * cnt * 4;
#pragma unroll
    for (int i = 0; i < cnt; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) o[i * 4 + w] = d[i][w];
    level += n_level * 4;
    n_level >>= 1;
  }
}

// The levels near the root, where a level holds too few nodes to fill the chip
// and each level waits for one compression: workgroup b takes children
// [b 2^L, (b+1) 2^L) of level `in` (n_in digests) and climbs L <= TOP_LEVELS
// levels, each node hashed by the four lanes of a quad (b2q_compress: a
// shorter chain per level than one lane's compression). Lane k of node q's
// quad brings message words 2k, 2k+1 (child 2q + k/2, words 2(k%2), 2(k%2)+1:
// from memory at level 1, later from LDS), and after the compression holds
// digest word k, which it writes to the node's level (out: the level above
// `in`, then the next, ...) and to LDS for the level above.
constexpr int TOP_T = 1024, TOP_LEVELS = 9;
__global__ __launch_bounds__(TOP_T) void tree_top_kernel(const uint64_t* __restrict__ in, int64_t n_in, int32_t L,
                                                        uint64_t* __restrict__ out) {
  __shared__ uint64_t nd[TOP_T / 4][4];   // the last level's digests of the workgroup's subtree
  __shared__ uint64_t mq[TOP_T / 4][16];  // each quad's message block
  const int t = threadIdx.x, q = t >> 2, k = t & 3;
  const int64_t b = blockIdx.x;
  int64_t n_level = n_in >> 1;  // nodes in the level being written
  uint64_t* level = out;
  for (int lev = 1; lev <= L; ++lev) {
    const int cnt = 1 << (L - lev);  // nodes of this level in the workgroup's subtree (whole quads: uniform)
    const int ch = 2 * q + (k >> 1), w = 2 * (k & 1);
    if (q < cnt) {
      uint64_t x0, x1;
      if (lev == 1) {
        const uint64_t* c = in + ((b << L) + ch) * 4 + w;
        x0 = c[0];
        x1 = c[1];
      } else {
        x0 = nd[ch][w];
        x1 = nd[ch][w + 1];
      }
      mq[q][2 * k] = x0;
      mq[q][2 * k + 1] = x1;
      mq[q][8 + 2 * k] = 0;
      mq[q][9 + 2 * k] = 0;
    }
    __syncthreads();  // this level's blocks complete, and every read of nd done
    if (q < cnt) {
      uint64_t h0, h1;
      b2q_init32(k, h0, h1);
      b2q_compress(h0, h1, mq[q], 64, true, k);
      nd[q][k] = h0;
      level[(b * cnt + q) * 4 + k] = h0;
    }
    __syncthreads();  // nd holds this level before the next reads it
    level += n_level * 4;
    n_level >>= 1;
  }
}

int plan_passes(int L, int (&lN)[NTT_MAXP]) {
  const int P = (L + 7) / 8;
  for (int q = 0; q < P; ++q) lN[q] = L / P + (q < L % P ? 1 : 0);
  for (int q = P; q < NTT_MAXP; ++q) lN[q] = 0;
  return P;
}

uint64_t host_mul(uint64_t a, uint64_t b) { return (uint64_t)(((unsigned __int128)a * b) % gl::P); }
uint64_t host_pow(uint64_t a, uint64_t e) {
  uint64_t r = 1;
  while (e) {
    if (e & 1) r = host_mul(r, a);
    a = host_mul(a, a);
    e >>= 1;
  }
  return r;
}

struct EncLayout {
  int P;
  size_t tw_bytes, tmp_bytes;
};

EncLayout enc_layout(int32_t rows, int32_t logn) {
  EncLayout e{};
  const int L = logn + 1;
  int lN[NTT_MAXP];
  e.P = plan_passes(L, lN);
  const size_t nlo = (size_t)1 << (L < TW_BITS ? L : TW_BITS);
  const size_t nhi = L > TW_BITS ? (size_t)1 << (L - TW_BITS) : 1;
  e.tw_bytes = fpi::align_up((nlo + nhi) * 8, 256);
  e.tmp_bytes = e.P > 1 ? fpi::align_up((size_t)rows << L, 32) * 8 : 0;
  return e;
}

}  // namespace

extern "C" int fp_commit_pack(const int8_t* A, int64_t na, const int8_t* B, int64_t nb, int32_t logn, int32_t rows,
                              fp_elem* msg, hipStream_t stream) {
  const char* fn = "fp_commit_pack";
  if (na < 0 || nb < 0 || rows < 0) return fpi::fail(FP_EARG, "%s: negative size", fn);
  if (logn < 0 || logn > FP_MAX_RS_LOGN) return fpi::fail(FP_ESHAPE, "%s: logn=%d outside [0, %d]", fn, logn, FP_MAX_RS_LOGN);
  const int64_t total = (int64_t)rows << logn;
  if ((na + nb + 2) / 3 > total) return fpi::fail(FP_ESHAPE, "%s: %lld limbs do not fit %d rows of 2^%d", fn,
                                                 (long long)(na + nb), rows, logn);
  if (total == 0) return fpi::ok();
  if (!msg || (na > 0 && !A) || (nb > 0 && !B)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, A, na, B, nb, total,
                     msg);
  const int rc = fpi::check_launch("pack_kernel");
  return rc ? rc : fpi::ok();
}

extern "C" size_t fp_rs_encode_workspace(int32_t rows, int32_t logn) {
  if (rows <= 0 || logn < 0 || logn > FP_MAX_RS_LOGN) return 0;
  const EncLayout e = enc_layout(rows, logn);
  return e.tw_bytes + e.tmp_bytes;
}

extern "C" int fp_rs_encode(const fp_elem* msg, int64_t ld_msg, int32_t rows, int32_t logn, fp_elem* code,
                            int64_t ld_code, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "fp_rs_encode";
  if (rows < 0) return fpi::fail(FP_EARG, "%s: negative rows", fn);
  if (logn < 0 || logn > FP_MAX_RS_LOGN) return fpi::fail(FP_ESHAPE, "%s: logn=%d outside [0, %d]", fn, logn, FP_MAX_RS_LOGN);
  const int L = logn + 1;
  if (ld_msg < ((int64_t)1 << logn) || ld_code < ((int64_t)1 << L))
    return fpi::fail(FP_ESHAPE, "%s: leading dimensions below 2^logn / 2^(logn+1)", fn);
  if (rows == 0) return fpi::ok();
  if (!msg || !code) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  const EncLayout e = enc_layout(rows, logn);
  if (!ws || ws_bytes < e.tw_bytes + e.tmp_bytes)
    return fpi::fail(FP_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, e.tw_bytes + e.tmp_bytes);
  if (((uintptr_t)ws) & 255) return fpi::fail(FP_EARG, "%s: workspace must be 256-byte aligned", fn);
  uint64_t* tw_lo = (uint64_t*)ws;
  uint64_t* tw_hi = tw_lo + ((size_t)1 << (L < TW_BITS ? L : TW_BITS));
  uint64_t* tmp = (uint64_t*)((char*)ws + e.tw_bytes);
  const uint64_t w = host_pow(7, (gl::P - 1) >> L);
  {
    const int n = (1 << (L < TW_BITS ? L : TW_BITS)) + (L > TW_BITS ? 1 << (L - TW_BITS) : 0);
    hipLaunchKernelGGL(twiddle_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, w, L, tw_lo, tw_hi);
    const int rc = fpi::check_launch("twiddle_kernel");
    if (rc) return rc;
  }
  NttArgs a{};
  a.tw_lo = tw_lo;
  a.tw_hi = tw_hi;
  a.L = L;
  a.P = plan_passes(L, a.lN);
  const int64_t N = (int64_t)1 << L;
  for (int p = 0; p < a.P; ++p) {
    a.p = p;
    a.first = p == 0;
    a.last = p == a.P - 1;
    a.src = p == 0 ? msg : tmp;
    a.src_rs = p == 0 ? ld_msg : N;
    a.dst = a.last ? code : tmp;
    a.dst_rs = a.last ? ld_code : N;
    int lS = 0, lT = 0;
    for (int q = p + 1; q < a.P; ++q) lS += a.lN[q];
    for (int q = 0; q < p; ++q) lT += a.lN[q];
    a.lS = lS;
    a.lT = lT;
    for (int q = 0, t = 0; q < NTT_MAXP - 1; ++q) {
      int sq = 0;
      for (int r = q + 1; r < a.P; ++r) sq += a.lN[r];
      a.dT[q] = t;
      a.dM[q] = (1 << a.lN[q]) - 1;
      a.dS[q] = sq;
      t += a.lN[q];
    }
    const int tc = tile_cols(a.lN[p]);
    int64_t bpr;
    if (!a.last) bpr = ((int64_t)1 << lT) * ((((int64_t)1 << lS) + tc - 1) / tc);
    else bpr = (((int64_t)1 << lT) + tc - 1) / tc;
    if (bpr * rows > 0x7FFFFFFF) return fpi::fail(FP_ESHAPE, "%s: too many rows", fn);
    a.blocks_per_row = (int32_t)bpr;
    const dim3 grid((unsigned)(bpr * rows));
    switch (a.lN[p]) {
      case 1: hipLaunchKernelGGL(ntt_pass_kernel<1>, grid, dim3(NTT_T), 0, stream, a); break;
      case 2: hipLaunchKernelGGL(ntt_pass_kernel<2>, grid, dim3(NTT_T), 0, stream, a); break;
      case 3: hipLaunchKernelGGL(ntt_pass_kernel<3>, grid, dim3(NTT_T), 0, stream, a); break;
      case 4: hipLaunchKernelGGL(ntt_pass_kernel<4>, grid, dim3(NTT_T), 0, stream, a); break;
      case 5: hipLaunchKernelGGL(ntt_pass_kernel<5>, grid, dim3(NTT_T), 0, stream, a); break;
      case 6: hipLaunchKernelGGL(ntt_pass_kernel<6>, grid, dim3(NTT_T), 0, stream, a); break;
      case 7: hipLaunchKernelGGL(ntt_pass_kernel<7>, grid, dim3(NTT_T), 0, stream, a); break;
      default: hipLaunchKernelGGL(ntt_pass_kernel<8>, grid, dim3(NTT_T), 0, stream, a); break;
    }
    const int rc = fpi::check_launch("ntt_pass_kernel");
    if (rc) return rc;
  }
  return fpi::ok();
}

extern "C" int fp_merkle_commit(const fp_elem* code, int64_t ld_code, int32_t rows, int32_t log_width,
                                const uint8_t* salts, uint8_t* tree, hipStream_t stream) {
  const char* fn = "fp_merkle_commit";
  if (rows < 0 || rows > FP_MAX_MERKLE_ROWS) return fpi::fail(FP_EARG, "%s: rows=%d outside [0, %d]", fn, rows,
                                                             FP_MAX_MERKLE_ROWS);
  if (log_width < 0 || log_width > FP_MAX_RS_LOGN + 1)
    return fpi::fail(FP_ESHAPE, "%s: log_width=%d outside [0, %d]", fn, log_width, FP_MAX_RS_LOGN + 1);
  const int64_t width = (int64_t)1 << log_width;
  if (rows > 0 && ld_code < width) return fpi::fail(FP_ESHAPE, "%s: ld_code < width", fn);
  if (!salts || !tree || (rows > 0 && !code)) return fpi::fail(FP_EARG, "%s: null pointer", fn);
  if ((((uintptr_t)salts) & 7) || (((uintptr_t)tree) & 7))
    return fpi::fail(FP_EARG, "%s: salts and tree must be 8-byte aligned", fn);
  uint64_t* nodes = (uint64_t*)tree;
  hipLaunchKernelGGL(leaf_kernel, dim3((unsigned)((width + 255) / 256)), dim3(256), 0, stream, code, ld_code, rows,
                     width, (const uint64_t*)salts, nodes);
  int rc = fpi::check_launch("leaf_kernel");
  if (rc) return rc;
  // levels above the leaves: 3 per launch (a subtree of 8 children per thread) while a level holds at least
  // 2^17 nodes, then up to TOP_LEVELS per launch (one node per quad of lanes and level)
  int64_t n_in = width;
  uint64_t* in = nodes;
  while (n_in > 1) {
    int levels;
    uint64_t* out = in + n_in * 4;
    if (n_in >= ((int64_t)1 << 17)) {
      levels = 3;
      hipLaunchKernelGGL(subtree_kernel<3>, dim3((unsigned)(((n_in >> 3) + 255) / 256)), dim3(256), 0, stream, in,
                         n_in, out);
      rc = fpi::check_launch("subtree_kernel");
    } else {
      levels = 0;
      while (levels < TOP_LEVELS && (n_in >> levels) > 1) ++levels;
      hipLaunchKernelGGL(tree_top_kernel, dim3((unsigned)(n_in >> levels)), dim3(TOP_T), 0, stream, in, n_in, levels,
                         out);
      rc = fpi::check_launch("tree_top_kernel");
    }
    if (rc) return rc;
    // the last level this launch wrote starts after the levels before it
    uint64_t* last = out;
    for (int d = 1; d < levels; ++d) last += (n_in >> d) * 4;
    in = last;
    n_in >>= levels;
  }
  return fpi::ok();
}
