/*
 * oracle.c - plain, slow CPU oracle for the matmul sum-check prover.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may call this code; the product path never does.
 * It shares no source, header or table with the GPU library.
 *
 * Every function computes the exact defined result with the most direct
 * arithmetic available: field values are reduced with unsigned __int128 and
 * '%', integer results are computed in int64. Sources:
 *   [HF]  "How fast can FlashProve go", §2 Background (sum-check reduces each
 *         matmul to claims about committed tables and the weights; a table's
 *         folded row is the eq-weighted sum of its rows), §3.1 (the rescale
 *         g_w = round(g^ / 2^k) and its committed remainder r = g^ - 2^k g_w,
 *         which the matmul's sum-check uses in place of g^; the field is
 *         Goldilocks, 2^64 - 2^32 + 1), §4 footnote 20 (a Goldilocks product
 *         takes several 32-bit multiplies, which is why the GPU side differs).
 * Conventions where the pages are silent (each is a stated reading):
 *   - table bits are LSB-first; eq(r,k) = prod_j (k_j ? r_j : 1 - r_j);
 *   - a row-major [rows, cols] matrix flattens with the column in the low bits;
 *   - round i of the sum-check binds bit i-1 (pairs 2j, 2j+1) and sends the
 *     degree-2 round polynomial as its values at 0, 1 and 2;
 *   - rounding ties go up: Q = floor((Z + 2^(s-1)) / 2^s), R = Z - 2^s Q,
 *     Y = clamp(Q, -128, 127); R is taken against the unclamped Q.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef unsigned __int128 u128;
typedef __int128 i128;

#define OR_P 0xFFFFFFFF00000001ULL

/* ---------------------------------------------------------------- field -- */
/* [HF §3.1] Goldilocks arithmetic, each op by its definition. */
uint64_t or_add(uint64_t a, uint64_t b) { return (uint64_t)(((u128)a + (u128)b) % OR_P); }
uint64_t or_sub(uint64_t a, uint64_t b) { return (uint64_t)(((u128)a + (u128)OR_P - (u128)(b % OR_P)) % OR_P); }
uint64_t or_mul(uint64_t a, uint64_t b) { return (uint64_t)(((u128)a * (u128)b) % OR_P); }

/* An integer as a field element: v mod p, negative v mapped to v + p. */
uint64_t or_from_int(int64_t v) {
  i128 r = (i128)v % (i128)OR_P;
  if (r < 0) r += (i128)OR_P;
  return (uint64_t)r;
}

uint64_t or_pow(uint64_t a, uint64_t e) {
  uint64_t r = 1, b = a % OR_P;
  while (e) {
    if (e & 1) r = or_mul(r, b);
    b = or_mul(b, b);
    e >>= 1;
  }
  return r;
}

/* Degree-2 polynomial through (0,g0), (1,g1), (2,g2), evaluated at x by
 * Lagrange interpolation: g0 (x-1)(x-2)/2 - g1 x(x-2) + g2 x(x-1)/2. */
uint64_t or_eval_deg2(uint64_t g0, uint64_t g1, uint64_t g2, uint64_t x) {
  const uint64_t inv2 = (OR_P + 1) / 2;
  uint64_t xm1 = or_sub(x, 1), xm2 = or_sub(x, 2);
  uint64_t l0 = or_mul(or_mul(xm1, xm2), inv2);
  uint64_t l1 = or_mul(x, xm2);
  uint64_t l2 = or_mul(or_mul(x, xm1), inv2);
  return or_add(or_sub(or_mul(g0, l0), or_mul(g1, l1)), or_mul(g2, l2));
}

/* -------------------------------------------------------------- witness -- */
static int64_t floor_div(int64_t a, int64_t b) { /* b > 0 */
  int64_t q = a / b;
  if ((a % b != 0) && (a < 0)) q -= 1;
  return q;
}

/* [HF §2, §3.1] Z = X W^T over the integers (each product is an int8 times
 * an int8), then the rescale by 2^s with its remainder and the clamp.
 * X: [T, d_in] row-major (leading dim ldx); W: [d_out, d_in] (ldw).
 * Returns 0, or -1 if some |Z| >= 2^31 (then Z cannot be stored as int32). */
int or_witness(const int8_t* X, int64_t ldx, const int8_t* W, int64_t ldw, int32_t T, int32_t d_in,
               int32_t d_out, int32_t s, int32_t* Z, int8_t* Y, int8_t* R) {
  int bad = 0;
  const int64_t two_s = (int64_t)1 << s, half = (int64_t)1 << (s - 1);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t o = 0; o < d_out; ++o) {
      const int8_t* xr = X + (int64_t)t * ldx;
      const int8_t* wr = W + (int64_t)o * ldw;
      int64_t acc = 0;
      for (int32_t k = 0; k < d_in; ++k) acc += (int64_t)xr[k] * (int64_t)wr[k];
      if (acc >= ((int64_t)1 << 31) || acc < -((int64_t)1 << 31)) bad = 1;
      int64_t q = floor_div(acc + half, two_s);
      int64_t r = acc - q * two_s;
      int64_t y = q < -128 ? -128 : (q > 127 ? 127 : q);
      int64_t idx = (int64_t)t * d_out + o;
      if (Z) Z[idx] = (int32_t)acc;
      if (Y) Y[idx] = (int8_t)y;
      if (R) R[idx] = (int8_t)r;
    }
  }
  return bad ? -1 : 0;
}

/* Selected witness entries only: Z at (ts[i], os[i]). */
void or_witness_entries(const int8_t* X, int64_t ldx, const int8_t* W, int64_t ldw, int32_t d_in,
                        int64_t n, const int32_t* ts, const int32_t* os, int64_t* Zout) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int8_t* xr = X + (int64_t)ts[i] * ldx;
    const int8_t* wr = W + (int64_t)os[i] * ldw;
    int64_t acc = 0;
    for (int32_t k = 0; k < d_in; ++k) acc += (int64_t)xr[k] * (int64_t)wr[k];
    Zout[i] = acc;
  }
}

/* ------------------------------------------------------------------- eq -- */
/* E[k] = eq(r, k) = prod_j (k_j ? r_j : 1 - r_j), each entry in product form. */
void or_eq_table(const uint64_t* r, int32_t n, uint64_t* E) {
  const int64_t m = (int64_t)1 << n;
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < m; ++k) {
    uint64_t e = 1;
    for (int32_t j = 0; j < n; ++j) e = or_mul(e, ((k >> j) & 1) ? r[j] : or_sub(1, r[j]));
    E[k] = e;
  }
}

/* eq(r, k) for a single index k. */
uint64_t or_eq_at(const uint64_t* r, int32_t n, int64_t k) {
  uint64_t e = 1;
  for (int32_t j = 0; j < n; ++j) e = or_mul(e, ((k >> j) & 1) ? r[j] : or_sub(1, r[j]));
  return e;
}

/* ---------------------------------------------------------------- folds -- */
/* [HF §2] The folded row: out[k] = sum_{t < rows} E[t] * M[t, k] for k < cols,
 * and 0 for cols <= k < cols_pad. Rows at or past `rows` count as zero rows.
 * elem_bytes selects int8 (1) or int32 (4) entries. */
void or_fold_rows(const void* M, int32_t elem_bytes, int64_t ld, int32_t rows, int32_t cols,
                  const uint64_t* E, uint64_t* out, int32_t cols_pad) {
#pragma omp parallel for schedule(static)
  for (int32_t k = 0; k < cols; ++k) {
    uint64_t acc = 0;
    for (int32_t t = 0; t < rows; ++t) {
      int64_t v = elem_bytes == 1 ? (int64_t)((const int8_t*)M)[(int64_t)t * ld + k]
                                  : (int64_t)((const int32_t*)M)[(int64_t)t * ld + k];
      acc = or_add(acc, or_mul(E[t], or_from_int(v)));
    }
    out[k] = acc;
  }
  for (int32_t k = cols; k < cols_pad; ++k) out[k] = 0;
}

/* [HF §2] The folded row of a table whose entries are field elements
 * (committed tables): out[c] = sum_{i < rows} E[i] * M[i, c], c < cols. */
void or_fold_field_rows(const uint64_t* M, int64_t ld, int32_t rows, int32_t cols, const uint64_t* E,
                        uint64_t* out) {
#pragma omp parallel for schedule(static)
  for (int32_t c = 0; c < cols; ++c) {
    uint64_t acc = 0;
    for (int32_t i = 0; i < rows; ++i) acc = or_add(acc, or_mul(E[i], M[(int64_t)i * ld + c] % OR_P));
    out[c] = acc;
  }
}

/* sum_{i < n} a[i] b[i] (an inner product of field vectors). */
uint64_t or_dot(const uint64_t* a, const uint64_t* b, int64_t n) {
  uint64_t acc = 0;
  for (int64_t i = 0; i < n; ++i) acc = or_add(acc, or_mul(a[i] % OR_P, b[i] % OR_P));
  return acc;
}

/* Selected columns of the folded row (for sampled checks at full size). */
void or_fold_cols(const void* M, int32_t elem_bytes, int64_t ld, int32_t rows, const uint64_t* E,
                  int64_t n, const int32_t* ks, uint64_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t acc = 0;
    for (int32_t t = 0; t < rows; ++t) {
      int64_t v = elem_bytes == 1 ? (int64_t)((const int8_t*)M)[(int64_t)t * ld + ks[i]]
                                  : (int64_t)((const int32_t*)M)[(int64_t)t * ld + ks[i]];
      acc = or_add(acc, or_mul(E[t], or_from_int(v)));
    }
    out[i] = acc;
  }
}

/* ------------------------------------------------------------------ MLE -- */
/* Multilinear extension of a table A of 2^n field values, by definition:
 * A~(z) = sum_k eq(z, k) A[k], each eq(z, k) in product form. */
uint64_t or_mle_brute(const uint64_t* A, int32_t n, const uint64_t* z) {
  const int64_t m = (int64_t)1 << n;
  uint64_t acc = 0;
  for (int64_t k = 0; k < m; ++k) acc = or_add(acc, or_mul(or_eq_at(z, n, k), A[k]));
  return acc;
}

/* The same value by binding one variable at a time (LSB first):
 * A[j] <- A[2j] + z_i (A[2j+1] - A[2j]). A second, independent route. */
uint64_t or_mle_seq(const uint64_t* A, int32_t n, const uint64_t* z) {
  const int64_t m = (int64_t)1 << n;
  uint64_t* t = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)(m ? m : 1));
  memcpy(t, A, sizeof(uint64_t) * (size_t)m);
  for (int32_t i = 0; i < n; ++i) {
    int64_t h = m >> (i + 1);
    for (int64_t j = 0; j < h; ++j) t[j] = or_add(t[2 * j], or_mul(z[i], or_sub(t[2 * j + 1], t[2 * j])));
  }
  uint64_t v = t[0];
  free(t);
  return v;
}

/* M~(r_cols || r_rows) for an integer matrix M [rows, cols] padded with
 * zeros to [2^n_rows, 2^n_cols]: sum_t sum_o eq(r_rows,t) eq(r_cols,o) M[t,o].
 * The eq factors come from product-form tables of the two points. */
uint64_t or_mle_matrix(const void* M, int32_t elem_bytes, int64_t ld, int32_t rows, int32_t cols,
                       const uint64_t* r_rows, int32_t n_rows, const uint64_t* r_cols, int32_t n_cols) {
  uint64_t* Er = (uint64_t*)malloc(sizeof(uint64_t) << n_rows);
  uint64_t* Ec = (uint64_t*)malloc(sizeof(uint64_t) << n_cols);
  or_eq_table(r_rows, n_rows, Er);
  or_eq_table(r_cols, n_cols, Ec);
  uint64_t total = 0;
#pragma omp parallel
  {
    uint64_t part = 0;
#pragma omp for schedule(static)
    for (int32_t t = 0; t < rows; ++t) {
      for (int32_t o = 0; o < cols; ++o) {
        int64_t v = elem_bytes == 1 ? (int64_t)((const int8_t*)M)[(int64_t)t * ld + o]
                                    : (int64_t)((const int32_t*)M)[(int64_t)t * ld + o];
        part = or_add(part, or_mul(or_mul(Er[t], Ec[o]), or_from_int(v)));
      }
    }
#pragma omp critical
    total = or_add(total, part);
  }
  free(Er);
  free(Ec);
  return total;
}

/* ------------------------------------------------------------ sum-check -- */
/* [HF §2] Sum-check for the claim sum_j rho_j sum_k A_j[k] B_j[k] over tables
 * of 2^n entries (n_pairs pairs; rho == NULL means every rho_j = 1).
 * Round i (0-based) sends g(c) = sum_j rho_j sum_{q < h} A_c[q] B_c[q] for
 * c = 0, 1, 2, with A_c[q] = A[2q] + c (A[2q+1] - A[2q]), then binds the
 * variable with r[i]: A[q] <- A[2q] + r[i] (A[2q+1] - A[2q]) (B likewise).
 * Outputs: rounds[3i + c], finals[2j] = A_j(z), finals[2j+1] = B_j(z), and
 * the initial claim *claim0. Input tables are not modified. */
void or_sumcheck(int32_t n_pairs, const uint64_t* const* A, const uint64_t* const* B, const uint64_t* rho,
                 int32_t n, const uint64_t* r, uint64_t* rounds, uint64_t* finals, uint64_t* claim0) {
  const int64_t m = (int64_t)1 << n;
  uint64_t** a = (uint64_t**)malloc(sizeof(void*) * (size_t)n_pairs);
  uint64_t** b = (uint64_t**)malloc(sizeof(void*) * (size_t)n_pairs);
  uint64_t c0 = 0;
  for (int32_t j = 0; j < n_pairs; ++j) {
    a[j] = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)m);
    b[j] = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)m);
    memcpy(a[j], A[j], sizeof(uint64_t) * (size_t)m);
    memcpy(b[j], B[j], sizeof(uint64_t) * (size_t)m);
    uint64_t dot = 0;
    for (int64_t k = 0; k < m; ++k) dot = or_add(dot, or_mul(a[j][k], b[j][k]));
    c0 = or_add(c0, or_mul(rho ? rho[j] : 1, dot));
  }
  if (claim0) *claim0 = c0;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t h = m >> (i + 1);
    uint64_t g[3] = {0, 0, 0};
    for (int32_t j = 0; j < n_pairs; ++j) {
      uint64_t gj[3] = {0, 0, 0};
      for (int64_t q = 0; q < h; ++q) {
        uint64_t a0 = a[j][2 * q], a1 = a[j][2 * q + 1], b0 = b[j][2 * q], b1 = b[j][2 * q + 1];
        uint64_t da = or_sub(a1, a0), db = or_sub(b1, b0);
        for (int c = 0; c < 3; ++c) {
          uint64_t ac = or_add(a0, or_mul((uint64_t)c, da));
          uint64_t bc = or_add(b0, or_mul((uint64_t)c, db));
          gj[c] = or_add(gj[c], or_mul(ac, bc));
        }
      }
      for (int c = 0; c < 3; ++c) g[c] = or_add(g[c], or_mul(rho ? rho[j] : 1, gj[c]));
    }
    for (int c = 0; c < 3; ++c) rounds[3 * i + c] = g[c];
    for (int32_t j = 0; j < n_pairs; ++j) {
      for (int64_t q = 0; q < h; ++q) {
        a[j][q] = or_add(a[j][2 * q], or_mul(r[i], or_sub(a[j][2 * q + 1], a[j][2 * q])));
        b[j][q] = or_add(b[j][2 * q], or_mul(r[i], or_sub(b[j][2 * q + 1], b[j][2 * q])));
      }
    }
  }
  for (int32_t j = 0; j < n_pairs; ++j) {
    finals[2 * j] = a[j][0];
    finals[2 * j + 1] = b[j][0];
    free(a[j]);
    free(b[j]);
  }
  free(a);
  free(b);
}

/* ------------------------------------------------------ verifier checks -- */
/* Reason codes of the verifier-side checks. */
enum {
  OR_OK = 0,
  OR_INITIAL_CLAIM = 1,   /* g_1(0) + g_1(1) != claimed c0 */
  OR_ROUND_SUM = 2,       /* g_{i+1}(0) + g_{i+1}(1) != g_i(r_i); *where = i+1 */
  OR_FINAL_CLAIM = 3,     /* g_n(r_n) != sum_j rho_j A_j~(z) B_j~(z) */
  OR_FINAL_OPENING = 4,   /* a final value differs from the table's own MLE at z */
  OR_RESCALE_IDENTITY = 5,/* Z != 2^s Q + R, R out of range, or Y != clamp(Q) */
  OR_WITNESS_MISMATCH = 6 /* Z differs from the naive integer matmul */
};

/* Check a sum-check transcript against the claim c0. If A and B are given,
 * the finals are also checked against brute-force MLEs of the tables at z. */
int or_check_sumcheck(int32_t n_pairs, const uint64_t* const* A, const uint64_t* const* B,
                      const uint64_t* rho, int32_t n, const uint64_t* r, const uint64_t* rounds,
                      const uint64_t* finals, uint64_t c0, int32_t* where) {
  *where = 0;
  uint64_t claim = c0;
  for (int32_t i = 0; i < n; ++i) {
    const uint64_t* g = rounds + 3 * i;
    if (or_add(g[0], g[1]) != claim) {
      *where = i;
      return i == 0 ? OR_INITIAL_CLAIM : OR_ROUND_SUM;
    }
    claim = or_eval_deg2(g[0], g[1], g[2], r[i]);
  }
  uint64_t fin = 0;
  for (int32_t j = 0; j < n_pairs; ++j)
    fin = or_add(fin, or_mul(rho ? rho[j] : 1, or_mul(finals[2 * j], finals[2 * j + 1])));
  if (fin != claim) {
    *where = n;
    return OR_FINAL_CLAIM;
  }
  if (A && B) {
    for (int32_t j = 0; j < n_pairs; ++j) {
      if (or_mle_brute(A[j], n, r) != finals[2 * j] || or_mle_brute(B[j], n, r) != finals[2 * j + 1]) {
        *where = j;
        return OR_FINAL_OPENING;
      }
    }
  }
  return OR_OK;
}

/* Entrywise rescale identity: Z = 2^s Q + R with R in [-2^(s-1), 2^(s-1)),
 * and Y = clamp(Q). Q is recovered as (Z - R) / 2^s. */
int or_check_rescale(const int32_t* Z, const int8_t* Y, const int8_t* R, int64_t n, int32_t s,
                     int64_t* where) {
  const int64_t two_s = (int64_t)1 << s, half = (int64_t)1 << (s - 1);
  for (int64_t i = 0; i < n; ++i) {
    int64_t r = R[i], z = Z[i];
    if (r < -half || r >= half || (z - r) % two_s != 0) {
      *where = i;
      return OR_RESCALE_IDENTITY;
    }
    int64_t q = (z - r) / two_s;
    int64_t y = q < -128 ? -128 : (q > 127 ? 127 : q);
    if (y != Y[i]) {
      *where = i;
      return OR_RESCALE_IDENTITY;
    }
  }
  *where = -1;
  return OR_OK;
}

/* Z against a naive integer matmul, every entry. */
int or_check_witness(const int8_t* X, int64_t ldx, const int8_t* W, int64_t ldw, int32_t T, int32_t d_in,
                     int32_t d_out, const int32_t* Z, int64_t* where) {
  int64_t first = -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t o = 0; o < d_out; ++o) {
      int64_t acc = 0;
      for (int32_t k = 0; k < d_in; ++k) acc += (int64_t)X[(int64_t)t * ldx + k] * (int64_t)W[(int64_t)o * ldw + k];
      if (acc != Z[(int64_t)t * d_out + o]) {
#pragma omp critical
        {
          int64_t idx = (int64_t)t * d_out + o;
          if (first < 0 || idx < first) first = idx;
        }
      }
    }
  }
  *where = first;
  return first >= 0 ? OR_WITNESS_MISMATCH : OR_OK;
}

/* ------------------------------------------------------------ commitment --
 * [HF] §3.1: committing a table Reed-Solomon encodes each row with an NTT and
 * Merkle-hashes each column; values are split into 8-bit limbs packed three to
 * a field element in 20-bit slots. Readings where the page is silent: an int8
 * value is one limb, its byte 0..255; the limbs of A then B fill the rows in
 * order, zero beyond; a row c_0..c_{n-1} is the coefficient vector of a
 * polynomial evaluated at w^j, j < 2n, w = 7^((p-1)/2n) (rate 1/2, natural
 * order). Hashing is done with the host's BLAKE2b in oracle/__init__.py. */

/* msg[e] = l_{3e} + 2^20 l_{3e+1} + 2^40 l_{3e+2} over rows * n_row elements. */
void or_pack_limbs(const int8_t* A, int64_t na, const int8_t* B, int64_t nb, int64_t n_row, int32_t rows,
                   uint64_t* msg) {
  const int64_t total = (int64_t)rows * n_row;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < total; ++e) {
    uint64_t v = 0;
    for (int q = 0; q < 3; ++q) {
      const int64_t l = 3 * e + q;
      uint64_t limb = 0;
      if (l < na) limb = (uint8_t)A[l];
      else if (l - na < nb) limb = (uint8_t)B[l - na];
      v |= limb << (20 * q);
    }
    msg[e] = v;
  }
}

/* A primitive 2^k-th root of unity: 7^((p-1)/2^k) (7 generates the whole group). */
uint64_t or_root_of_unity(int32_t k) { return or_pow(7, (OR_P - 1) >> k); }

/* code[j] = sum_{i<n} msg[i] w^{ij}, j < 2n, w = or_root_of_unity(logn + 1):
 * the row zero-padded to 2n and transformed by textbook iterative radix-2
 * Cooley-Tukey (bit-reversal permutation, then log2(2n) butterfly stages). */
void or_rs_encode(const uint64_t* msg, int32_t logn, uint64_t* code) {
  const int32_t L = logn + 1;
  const int64_t N = (int64_t)1 << L, n = N / 2;
  for (int64_t j = 0; j < N; ++j) {
    int64_t r = 0;
    for (int b = 0; b < L; ++b) r |= ((j >> b) & 1) << (L - 1 - b);
    code[r] = j < n ? msg[j] % OR_P : 0;
  }
  for (int32_t s = 1; s <= L; ++s) {
    const int64_t m = (int64_t)1 << s, h = m / 2;
    const uint64_t wm = or_root_of_unity(s);
    uint64_t* tw = (uint64_t*)malloc(sizeof(uint64_t) * h);
    tw[0] = 1;
    for (int64_t t = 1; t < h; ++t) tw[t] = or_mul(tw[t - 1], wm);
#pragma omp parallel for schedule(static)
    for (int64_t base = 0; base < N; base += m) {
      for (int64_t t = 0; t < h; ++t) {
        const uint64_t u = code[base + t], v = or_mul(code[base + t + h], tw[t]);
        code[base + t] = or_add(u, v);
        code[base + t + h] = or_sub(u, v);
      }
    }
    free(tw);
  }
}

/* One codeword entry by its definition: the row's polynomial at w^j (Horner). */
uint64_t or_rs_eval(const uint64_t* msg, int32_t logn, int64_t j) {
  const int64_t n = (int64_t)1 << logn;
  const uint64_t x = or_pow(or_root_of_unity(logn + 1), (uint64_t)j);
  uint64_t acc = 0;
  for (int64_t i = n - 1; i >= 0; --i) acc = or_add(or_mul(acc, x), msg[i] % OR_P);
  return acc;
}

/* ---------------------------------------------------------------- lookup --
 * [HF] §3.1 (rescale remainders are range-checked by a lookup) and §4 (the
 * lookup is a grand-product argument: the keys' product, formed as a binary
 * tree reduced level by level with sum-check, is matched against the table's
 * product). Readings where the page is
 * silent: keys are int8 values; the tree has 2^L leaves gamma - key_i, padded
 * with gamma - 0 (0 is a row of every remainder table); level d+1 entry i is
 * the product of level d entries 2i and 2i+1; the table side is
 * prod_t (gamma - t)^(m_t) with m_t the multiplicity of t among the padded keys. */

/* tree: level 0 (2^L leaves) first, then each level up, the root last. */
void or_product_tree(const int8_t* keys, int64_t n, int32_t L, uint64_t gamma, uint64_t* tree) {
  const int64_t N = (int64_t)1 << L;
  for (int64_t i = 0; i < N; ++i) tree[i] = or_sub(gamma, i < n ? or_from_int(keys[i]) : 0);
  int64_t off = 0;
  for (int64_t w = N; w > 1; w /= 2) {
    for (int64_t i = 0; i < w / 2; ++i) tree[off + w + i] = or_mul(tree[off + 2 * i], tree[off + 2 * i + 1]);
    off += w;
  }
}

/* The same tree for keys that are field elements (keys[i] for i < n, 0 past n). */
void or_product_tree_field(const uint64_t* keys, int64_t n, int32_t L, uint64_t gamma, uint64_t* tree) {
  const int64_t N = (int64_t)1 << L;
  for (int64_t i = 0; i < N; ++i) tree[i] = or_sub(gamma, i < n ? keys[i] % OR_P : 0);
  int64_t off = 0;
  for (int64_t w = N; w > 1; w /= 2) {
    for (int64_t i = 0; i < w / 2; ++i) tree[off + w + i] = or_mul(tree[off + 2 * i], tree[off + 2 * i + 1]);
    off += w;
  }
}

/* out[i] = A[i] + scale B[i] + offset: a pair of field tables as one key each. */
void or_pair_keys(const uint64_t* A, const uint64_t* B, int64_t n, uint64_t scale, uint64_t offset, uint64_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_add(or_add(A[i] % OR_P, or_mul(scale, B[i] % OR_P)), offset % OR_P);
}

/* Multiplicities of the table values t = -2^(s-1) + i, i < 2^s, among the keys
 * and the 2^L - n padding keys (value 0). Returns the number of keys outside
 * the table. */
int64_t or_lookup_counts(const int8_t* keys, int64_t n, int32_t L, int32_t s, int64_t* counts) {
  const int64_t T = (int64_t)1 << s, lo = -((int64_t)1 << (s - 1));
  int64_t outside = 0;
  for (int64_t t = 0; t < T; ++t) counts[t] = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t k = keys[i] - lo;
    if (k < 0 || k >= T) ++outside;
    else ++counts[k];
  }
  counts[-lo] += ((int64_t)1 << L) - n;
  return outside;
}

/* Degree-3 sum-check of sum_x E[x] A[x] B[x] over m variables, with
 * A[x] = V[2x], B[x] = V[2x+1] (the two children of node x). Round i sends
 * g_i(0), g_i(1), g_i(2), g_i(3) and binds the lowest remaining variable to
 * r[i]; finals are E, A, B at the point. */
void or_sumcheck3(const uint64_t* E, const uint64_t* V, int32_t m, const uint64_t* r, uint64_t* rounds,
                  uint64_t* finals) {
  const int64_t M = (int64_t)1 << m;
  uint64_t* e = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)M);
  uint64_t* a = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)M);
  uint64_t* b = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)M);
  for (int64_t x = 0; x < M; ++x) {
    e[x] = E[x];
    a[x] = V[2 * x];
    b[x] = V[2 * x + 1];
  }
  for (int32_t i = 0; i < m; ++i) {
    const int64_t h = M >> (i + 1);
    uint64_t g[4] = {0, 0, 0, 0};
    for (int64_t q = 0; q < h; ++q) {
      const uint64_t de = or_sub(e[2 * q + 1], e[2 * q]), da = or_sub(a[2 * q + 1], a[2 * q]);
      const uint64_t db = or_sub(b[2 * q + 1], b[2 * q]);
      for (int c = 0; c < 4; ++c) {
        const uint64_t ec = or_add(e[2 * q], or_mul((uint64_t)c, de));
        const uint64_t ac = or_add(a[2 * q], or_mul((uint64_t)c, da));
        const uint64_t bc = or_add(b[2 * q], or_mul((uint64_t)c, db));
        g[c] = or_add(g[c], or_mul(ec, or_mul(ac, bc)));
      }
    }
    for (int c = 0; c < 4; ++c) rounds[4 * i + c] = g[c];
    for (int64_t q = 0; q < h; ++q) {
      e[q] = or_add(e[2 * q], or_mul(r[i], or_sub(e[2 * q + 1], e[2 * q])));
      a[q] = or_add(a[2 * q], or_mul(r[i], or_sub(a[2 * q + 1], a[2 * q])));
      b[q] = or_add(b[2 * q], or_mul(r[i], or_sub(b[2 * q + 1], b[2 * q])));
    }
  }
  finals[0] = e[0];
  finals[1] = a[0];
  finals[2] = b[0];
  free(e);
  free(a);
  free(b);
}

/* A cubic given by its values at 0, 1, 2, 3, evaluated at x (Lagrange form). */
uint64_t or_eval_deg3(const uint64_t* g, uint64_t x) {
  const int64_t den[4] = {-6, 2, -2, 6}; /* prod_{j != i} (i - j) */
  uint64_t acc = 0;
  for (int i = 0; i < 4; ++i) {
    uint64_t num = 1;
    for (int j = 0; j < 4; ++j)
      if (j != i) num = or_mul(num, or_sub(x, (uint64_t)j));
    const uint64_t inv = or_pow(or_from_int(den[i]), OR_P - 2);
    acc = or_add(acc, or_mul(g[i], or_mul(num, inv)));
  }
  return acc;
}
