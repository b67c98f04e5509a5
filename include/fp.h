/*
 * fp.h - C ABI of libfp, the gfx950 prover for fixed-point linear layers.
 *
 * What is proved. For a quantized linear layer the prover computes the integer
 * witness Z = X W^T (int8 x int8 -> int32), the rescaled output
 * Y = clamp(round(Z / 2^s), -128, 127) and the rescale remainders
 * R = Z - 2^s round(Z / 2^s), then runs the sum-check protocol for the matmul
 * claim over the Goldilocks field p = 2^64 - 2^32 + 1.
 * Source: "How fast can FlashProve go", §2 Background (fixed-point model whose
 * products are rescaled and clamped; sum-check reduces each matmul to claims
 * about committed tables and the weights; a table's folded row is the
 * eq-weighted sum of its rows) and §3.1 (rescale g_w = round(g^ / 2^k), the
 * committed remainder r = g^ - 2^k g_w that the matmul's sum-check uses in
 * place of g^; Goldilocks).
 *
 * Conventions (readings where the page is silent):
 *  - rounding ties go up: Q = floor((Z + 2^(s-1)) / 2^s); R = Z - 2^s Q is taken
 *    against the unclamped Q; 1 <= s <= 8 so R fits int8;
 *  - tables are indexed LSB-first: eq(r, k) = prod_j (k_j ? r_j : 1 - r_j) and
 *    the multilinear extension is A~(z) = sum_k eq(z, k) A[k];
 *  - a row-major [rows, cols] matrix flattens with the column index in the low
 *    bits, so M~(r_cols || r_rows) = sum_t sum_c eq(r_rows,t) eq(r_cols,c) M[t,c];
 *    every axis is zero-padded to the next power of two;
 *  - sum-check round i (0-based) binds table bit i (pairs 2q, 2q+1) and sends
 *    the degree-2 round polynomial as its values at 0, 1 and 2.
 *
 * Memory and errors. Unless marked "host", every pointer is a device pointer
 * owned by the caller; inputs are read-only, outputs are fully overwritten.
 * Field elements (fp_elem) are canonical uint64 in [0, p). Integer matrices are
 * row-major with an explicit leading dimension in elements. Calls only enqueue
 * work on `stream` and return; none synchronizes or allocates device memory.
 * Scratch space comes from a caller workspace sized by the matching
 * *_workspace() query (its contents need no initialization, except the
 * FP_FOLD_COUNTER_BYTES of arrival counters at the start of a fp_layer_step
 * workspace: zero them once when the workspace is created; every call leaves
 * them zero). Calls that overlap in time must not share a workspace. Arguments are validated before any launch; a failing
 * call returns a nonzero FP_E* code, launches nothing, and sets a thread-local
 * message readable with fp_last_error(). Faults inside kernels surface at the
 * caller's next stream synchronization. The library keeps no state between
 * calls (thread-safe; calls on one stream run in order).
 */
#ifndef FP_H
#define FP_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint64_t fp_elem;

typedef enum { FP_I8 = 0, FP_I32 = 1 } fp_dtype;

enum {
  FP_OK = 0,
  FP_EARG = 1,       /* null pointer, negative or overflowing size */
  FP_ESHAPE = 2,     /* inconsistent shapes, n > 30, d_in > FP_MAX_DIN, padding too small */
  FP_ERANGE = 3,     /* s outside [1, 8] */
  FP_EWORKSPACE = 4, /* workspace smaller than the *_workspace() size */
  FP_EHIP = 5        /* the HIP runtime reported an error at launch */
};

#define FP_MAX_DIN 131071 /* 128^2 * d_in < 2^31 keeps Z exact in int32 (int8 products reach (-128)^2) */
#define FP_MAX_N 30       /* largest table: 2^30 entries */
#define FP_MAX_GROUPS 256 /* groups in one grouped witness launch */
#define FP_MAX_REQUESTS 4096          /* eq vectors in one multi-request fold */
#define FP_MAX_FOLD_ROWS (1 << 30)    /* rows of a multi-request fold's matrix */
#define FP_MAX_RS_LOGN 23             /* Reed-Solomon rows of up to 2^23 elements (codewords 2^24) */
#define FP_MAX_MERKLE_ROWS (1 << 20)  /* rows hashed into one Merkle leaf */
#define FP_FOLD_COUNTER_BYTES 16384   /* arrival counters at the start of a fp_layer_step workspace */

/* Thread-local message of the last failing call ("" after success). */
const char* fp_last_error(void);

/* ------------------------------------------------------------ witness --- */
/* Witness of one linear layer ("How fast can FlashProve go", §2 and §3.1).
 * X: int8 [T, d_in] (leading dim ldx >= d_in); W: int8 [d_out, d_in] (ldw).
 * Writes Z int32 [T, d_out] (may be NULL: not stored), Y and R int8
 * [T, d_out], all dense row-major. Requires 1 <= s <= 8, d_in <= FP_MAX_DIN.
 * Runs on int8 matrix cores with the rescale/clamp/remainder in the epilogue. */
int fp_witness_linear(const int8_t* X, int64_t ldx, const int8_t* W, int64_t ldw, int32_t T, int32_t d_in,
                      int32_t d_out, int32_t s, int32_t* Z, int8_t* Y, int8_t* R, hipStream_t stream);

/* Grouped witness ("How fast can FlashProve go", §2: in the MoE model each
 * token is sent to one routed expert, so an expert's matmul covers only its
 * tokens; "flashprove-consumer-gpu" README, patch table: every expert's GEMM
 * in one launch): G independent layers sharing d_in, d_out and s in ONE
 * launch (one group per MoE expert). Group g owns rows [row_off[g],
 * row_off[g+1]) of X (int8 [row_off[G], d_in], leading dim ldx) and of the
 * outputs Z/Y/R ([row_off[G], d_out], dense); its weight is W_ptrs[g]
 * (int8 [d_out, d_in], leading dim ldw). row_off (host, G+1 entries,
 * non-decreasing, row_off[0] = 0) and W_ptrs (host array of G device
 * pointers) are read during the call only. Empty groups are allowed.
 * G <= FP_MAX_GROUPS. Z may be NULL. */
int fp_witness_linear_grouped(const int8_t* X, int64_t ldx, const int8_t* const* W_ptrs, int64_t ldw,
                              const int32_t* row_off, int32_t G, int32_t d_in, int32_t d_out, int32_t s,
                              int32_t* Z, int8_t* Y, int8_t* R, hipStream_t stream);

/* Grouped witness from packed weights, each group's claim taken from its
 * accumulators ("How fast can FlashProve go", §2: each token goes to one
 * routed expert, so each expert's matmul covers its own rows; §3.1: the claim
 * is about the product, so Z need not be stored): as fp_witness_linear_grouped
 * (group g owns rows [row_off[g], row_off[g+1]) of X, int8 [row_off[G], d_in]
 * with 16-byte aligned rows and d_in % 16 == 0, and of Y, R (and Z unless
 * NULL), [row_off[G], d_out] dense), with group g's weights packed by
 * fp_witness_pack_weights (Wp: host array of G device pointers, 16-byte
 * aligned). E_t non-NULL (host array of G device pointers, each a table of >=
 * the group's rows): claims[g] = sum_t sum_o E_t[g][t] E_o[g ldeo + o] Z_g[t, o]
 * for every non-empty group (E_o: device, ldeo >= d_out; claims: device [G];
 * the tables complete before the call), with ws of
 * fp_witness_grouped_packed_workspace(row_off, G, d_out) bytes, 256-byte
 * aligned, whose first G * 64 bytes (arrival counters) are zero on entry and
 * left zero. row_off (host, G + 1, non-decreasing, row_off[0] = 0), Wp and E_t
 * are read during the call only. G <= FP_MAX_GROUPS (one launch per 128
 * groups). Empty groups own no tiles and get no claim.
 * w_fold non-NULL (device [G][ld_fold], E_o given): also the weight folds
 * w_fold[g ld_fold + k] = sum_o E_o[g ldeo + o] W_g[o, k] for k < d_in, zero for
 * d_in <= k < fold_cols_pad ("How fast can FlashProve go", §4: the matmuls'
 * sum-checks need a pass over the weights; here it is the witness's own pass),
 * for every non-empty group (empty groups' rows are left alone): the first token
 * tile of each weight panel folds the fragments it streams on the matrix cores,
 * and a second launch of the same call adds the panels. */
int fp_witness_grouped_packed(const int8_t* X, int64_t ldx, const int8_t* const* Wp, const int32_t* row_off,
                              int32_t G, int32_t d_in, int32_t d_out, int32_t s, int32_t* Z, int8_t* Y, int8_t* R,
                              const fp_elem* const* E_t, const fp_elem* E_o, int64_t ldeo, fp_elem* claims,
                              fp_elem* w_fold, int64_t ld_fold, int32_t fold_cols_pad, void* ws, size_t ws_bytes,
                              hipStream_t stream);
/* Bytes of fp_witness_grouped_packed's workspace (with_fold: with weight
 * folds); 0 on bad arguments. */
size_t fp_witness_grouped_packed_workspace(const int32_t* row_off, int32_t G, int32_t d_in, int32_t d_out,
                                           int32_t with_fold);

/* ----------------------------------------------------------- grouping --- */
/* MoE grouping plan, host only (no device work). route (host, T entries in
 * [0, n_experts)) gives each token's expert. Writes counts[e] (host,
 * n_experts), offsets (host, n_experts + 1, offsets[e] = first grouped row of
 * expert e) and perm (host, T: grouped row -> token), grouping stably by
 * expert with tokens ascending within a group ("How fast can FlashProve go",
 * §2: each token goes to one routed expert). */
int fp_moe_plan(const int32_t* route, int32_t T, int32_t n_experts, int32_t* counts, int32_t* offsets,
                int32_t* perm);

/* Xg[i, :] = X[perm[i], :] for i < n_rows (perm: device int32 [n_rows]);
 * X leading dim ldx, Xg dense [n_rows, cols]. */
int fp_gather_rows(const int8_t* X, int64_t ldx, const int32_t* perm, int32_t n_rows, int32_t cols, int8_t* Xg,
                   hipStream_t stream);

/* ------------------------------------------------------------------ eq --- */
/* E[k] = eq(r, k) for k < 2^n (r: n field elements, E: 2^n). n in [0, 30]
 * ("How fast can FlashProve go", §2: the weights of the folded row). */
int fp_eq_table(const fp_elem* r, int32_t n, fp_elem* E, hipStream_t stream);

typedef struct {
  const fp_elem* r; /* device, n elements */
  int32_t n;        /* 0..24 */
  fp_elem* E;       /* device, 2^n elements */
} fp_eq_desc;

/* Several eq tables in as few launches as possible. descs is a HOST array of
 * `count` descriptors, read during the call only; they travel in the kernel
 * arguments, so the call needs no workspace (ws may be NULL; the size query
 * returns 0). */
int fp_eq_table_batched(int32_t count, const fp_eq_desc* descs, void* ws, size_t ws_bytes, hipStream_t stream);
size_t fp_eq_table_batched_workspace(int32_t count);

/* ------------------------------------------------------ packed witness --- */
/* Packed weights: the weights of one layer laid out once in the order the
 * int8 matrix cores read them, for the fp_witness_linear_packed* calls (the
 * weights of a layer are fixed, so one packing serves every proof of it).
 * Fragment (b, c, q) is 1 KiB at byte ((b * nkb + c) * 2 + q) * 1024, nkb =
 * ceil(d_in / 64); its lane l (16 bytes at l * 16) holds
 * W[32 b + l % 32][64 c + 32 (l / 32) + 16 q + 0..15], zero past d_out and
 * d_in. Wp (device, 16-byte aligned) holds
 * fp_witness_packed_weights_bytes(d_out, d_in) =
 * ceil(d_out / 32) * 32 * nkb * 64 bytes; W is int8 [d_out, d_in] (ldw). */
size_t fp_witness_packed_weights_bytes(int32_t d_out, int32_t d_in);
int fp_witness_pack_weights(const int8_t* W, int64_t ldw, int32_t d_out, int32_t d_in, int8_t* Wp,
                            hipStream_t stream);

/* fp_witness_linear with the weights given packed (Wp from
 * fp_witness_pack_weights for this d_out, d_in): the same Z, Y, R. Each wave
 * streams its weight fragments straight into registers and only X passes
 * through LDS. Requires d_in % 16 == 0, ldx % 16 == 0 and X 16-byte aligned
 * (FP_ESHAPE otherwise). The same launch also writes the n_eq eq tables
 * eq[0 .. n_eq) (exactly fp_eq_table_batched(n_eq, eq)) in workgroups beside
 * the GEMM: a proof's eq tables depend only on its challenges, so they are
 * built while its witness runs. n_eq in [0, 8]; the tables must not overlap
 * X, Wp or the outputs. */
int fp_witness_linear_packed(const int8_t* X, int64_t ldx, const int8_t* Wp, int32_t T, int32_t d_in,
                             int32_t d_out, int32_t s, int32_t* Z, int8_t* Y, int8_t* R, int32_t n_eq,
                             const fp_eq_desc* eq, hipStream_t stream);

/* fp_witness_linear_with_sumcheck with packed weights: the witness and eq
 * tables of fp_witness_linear_packed and, in the same launch, the sum-check of
 * another claim (VP * 2^n <= 4096; the conditions of both calls apply; the
 * eq tables must not overlap the sum-check's tables either). */
int fp_witness_linear_packed_with_sumcheck(const int8_t* X, int64_t ldx, const int8_t* Wp, int32_t T,
                                           int32_t d_in, int32_t d_out, int32_t s, int32_t* Z, int8_t* Y,
                                           int8_t* R, int32_t n_pairs, const fp_elem* const* A,
                                           const fp_elem* const* B, const fp_elem* rho, int32_t n,
                                           const fp_elem* r, fp_elem* rounds, fp_elem* finals, fp_elem* claim0,
                                           int32_t n_eq, const fp_eq_desc* eq, hipStream_t stream);

/* --------------------------------------------------------------- folds --- */
/* Folded row of an integer matrix ("How fast can FlashProve go", §2: the
 * weighted sum of all of a table's rows): out[k] = sum_{t<rows} E[t] M[t,k]
 * for k < cols and out[k] = 0 for cols <= k < cols_pad. M is int8 or int32
 * [rows, cols] with leading dim ld; E holds at least `rows` field elements
 * (entries past `rows` are ignored, as if M had zero rows there). With
 * E = eq(r_t, .) over X this is x'[k] = X~(k || r_t); over W with eq(r_o, .)
 * it is w'[k] = W~(k || r_o). Runs on the vector ALUs, bandwidth-bound. */
int fp_fold_matrix(fp_dtype dt, const void* M, int64_t ld, int32_t rows, int32_t cols, const fp_elem* E,
                   fp_elem* out, int32_t cols_pad, void* ws, size_t ws_bytes, hipStream_t stream);
size_t fp_fold_matrix_workspace(fp_dtype dt, int32_t rows, int32_t cols);

typedef struct {
  const void* M;   /* device, int8 or int32 (one dtype per batched call) */
  int64_t ld;
  int32_t rows, cols, cols_pad;
  const fp_elem* E; /* device, >= rows */
  fp_elem* out;     /* device, cols_pad */
  /* Optional, in the step launches' int8 folds only (fp_layer_step,
   * fp_layer_step_multi): a second row-weight vector (device, >= rows) folded
   * from the same read of M into out2 (device, cols_pad), e.g. the weight
   * folds of two proofs of one layer. Both NULL or both set; the other calls
   * that take fold descriptors refuse it (FP_EARG). */
  const fp_elem* E2;
  fp_elem* out2;
} fp_fold_desc;

/* Several folds of one dtype (descs: HOST array read during the call; the
 * descriptors travel in kernel arguments, a dozen per launch). */
int fp_fold_matrix_batched(fp_dtype dt, int32_t count, const fp_fold_desc* descs, void* ws, size_t ws_bytes,
                           hipStream_t stream);
size_t fp_fold_matrix_batched_workspace(fp_dtype dt, int32_t count, const fp_fold_desc* descs);

/* ------------------------------------------------- multi-request folds --- */
/* Request vectors of a batch ("How fast can FlashProve go", §2.1: each request
 * commits the folded row of the weight table before one shared opening):
 * the folds of ONE int8 matrix M [rows, cols] by R eq vectors, with M read once.
 *
 * fp_fold_weights_prepare writes what depends on M alone, once per matrix:
 * Mt [cols, rows] int8 with leading dim ldt (>= rows, a multiple of 16; Mt
 * 16-byte aligned), Mt[k, t] = M[t, k], and colsum [cols] int32,
 * colsum[k] = sum_t M[t, k]. M has leading dim ld >= cols. Bytes of Mt past
 * `rows` in each row are not written. */
int fp_fold_weights_prepare(const int8_t* M, int64_t ld, int32_t rows, int32_t cols, int8_t* Mt, int64_t ldt,
                            int32_t* colsum, hipStream_t stream);

/* out[j*ldo + k] = sum_{t<rows} E[j*lde + t] M[t, k] for j < R, k < cols, and
 * 0 for cols <= k < cols_pad, given Mt and colsum from fp_fold_weights_prepare.
 * Every E entry must be a canonical field element (< p). Each output equals
 * fp_fold_matrix of M by the j-th vector. The eq weights are split into bytes
 * and the sums over t run as one int8 matrix product on the matrix cores
 * (R <= FP_MAX_REQUESTS, rows <= FP_MAX_FOLD_ROWS, lde >= rows, ldo >= cols_pad).
 * ws: fp_fold_matrix_multi_workspace(rows, cols, R) bytes, 256-byte aligned;
 * its contents on entry do not matter. */
int fp_fold_matrix_multi(const int8_t* Mt, int64_t ldt, const int32_t* colsum, int32_t rows, int32_t cols, int32_t R,
                         const fp_elem* E, int64_t lde, fp_elem* out, int64_t ldo, int32_t cols_pad, void* ws,
                         size_t ws_bytes, hipStream_t stream);
size_t fp_fold_matrix_multi_workspace(int32_t rows, int32_t cols, int32_t R);

/* ---------------------------------------------------------- commitment --- */
/* Commitment of committed tables such as Y and R ("How fast can FlashProve
 * go", §3.1: values are cut into 8-bit limbs packed three to a field element in
 * 20-bit slots; each row of the table is Reed-Solomon encoded by an NTT, a row
 * of 2^22 elements into 2^23; each column becomes a salted Merkle leaf hashed
 * with BLAKE2b).
 *
 * fp_commit_pack: msg[e] = l_{3e} + 2^20 l_{3e+1} + 2^40 l_{3e+2} for
 * e < rows * 2^logn, where the limb stream l is the na bytes of A followed by
 * the nb bytes of B (each int8 value is one limb, its byte 0..255) and 0 past
 * them. msg is dense [rows, 2^logn]; rows must hold every limb
 * (FP_ESHAPE otherwise). logn <= FP_MAX_RS_LOGN. */
int fp_commit_pack(const int8_t* A, int64_t na, const int8_t* B, int64_t nb, int32_t logn, int32_t rows,
                   fp_elem* msg, hipStream_t stream);

/* Rate-1/2 Reed-Solomon encoding of each row: for n = 2^logn,
 * code[i*ld_code + j] = sum_{k<n} msg[i*ld_msg + k] w^(jk) for j < 2n, with
 * w = 7^((p-1)/2n) (a primitive 2n-th root of unity; 7 generates the
 * multiplicative group). Natural order. msg entries must be canonical.
 * ws: fp_rs_encode_workspace(rows, logn) bytes, 256-byte aligned (twiddle
 * tables and, for 2n > 256, one intermediate copy of the codewords). */
int fp_rs_encode(const fp_elem* msg, int64_t ld_msg, int32_t rows, int32_t logn, fp_elem* code, int64_t ld_code,
                 void* ws, size_t ws_bytes, hipStream_t stream);
size_t fp_rs_encode_workspace(int32_t rows, int32_t logn);

/* Salted Merkle tree over the 2^log_width columns of code [rows, ld_code]:
 * leaf j = BLAKE2b-256(salt_j || code[0][j] || ... || code[rows-1][j]) with
 * 16-byte salts (salts: 2^log_width x 16 bytes) and elements as 8 little-endian
 * bytes; a parent is BLAKE2b-256(left || right) (RFC 7693, unkeyed, 32-byte
 * digest). tree receives 2^(log_width+1) - 1 digests of 32 bytes: the leaves in
 * column order, then each level above, the root last. salts and tree 8-byte
 * aligned; rows <= FP_MAX_MERKLE_ROWS (rows = 0 hashes the salts alone). */
int fp_merkle_commit(const fp_elem* code, int64_t ld_code, int32_t rows, int32_t log_width, const uint8_t* salts,
                     uint8_t* tree, hipStream_t stream);

/* Committed tables of a layer whose rescale is committed ("How fast can
 * FlashProve go", §3.1: the rescaled value g_w = round(g^ / 2^k) and the
 * remainder r = g^ - 2^k g_w are committed, never g^, and the clamped value
 * is committed too). For each of the count maps (at most FP_MAX_MULTI), with
 * Z int32 [T, ldz] its witness: Q = floor((Z + 2^(s-1)) / 2^s) (before the
 * clamp), R = Z - 2^s Q and Y = clamp(Q, -128, 127), each as a zero-padded
 * [2^n_t, 2^n_o] table of field elements (v < 0 as p + v) flattened with the
 * output index in the low bits, written into rows row_q, row_r, row_y
 * onwards of msg [rows, ld], 2^log_cols elements per row (entry i of a table
 * at row i >> log_cols, column i mod 2^log_cols); each table takes
 * 2^(n_t + n_o - log_cols) whole rows. Needs T <= 2^n_t, d_out <= 2^n_o,
 * n_t + n_o >= log_cols, s in [1, 8]. Errors: FP_EARG, FP_ESHAPE, FP_ERANGE. */
typedef struct {
  const int32_t* Z;
  int64_t ldz;
  int32_t T, d_out, n_o;
  int32_t row_q, row_r, row_y;
} fp_table_desc;
int fp_commit_tables(int32_t count, const fp_table_desc* d, int32_t n_t, int32_t s, int32_t log_cols, fp_elem* msg,
                     int64_t ld, int32_t rows, hipStream_t stream);

/* Folded rows of a committed message matrix over the extension, for
 * openings ("How fast can FlashProve go", §2: an opening sends the folded
 * row, the eq-weighted sum of the table's rows, and opens a few columns; §4
 * footnote 20: over the extension). msg [rows, ld] holds 2^log_cols field
 * elements per row. U [(1 + n_claims)][2][2^log_cols] receives, as 1 and u
 * parts: row 0, the proximity row sum_{i < rows} eq(r_prox, i) msg[i] (r_prox:
 * device [n_prox][2], 2^n_prox >= rows); row 1 + k, claim k's row
 * sum_{i < nrows} eq(z, i) msg[row0 + i], z the n1 coordinates at z1 followed
 * by the n2 at z2 (device [.][2] each), nrows = 2^(n1 + n2). Claims are sorted
 * by row0 and disjoint, at most FP_MAX_OPEN_CLAIMS. Any canonical entries are
 * folded exactly; entries that are 32-bit signed integers (as everywhere in
 * the committed tables) take a cheaper path. ws:
 * fp_commit_fold_ext_workspace(rows) bytes, 256-byte aligned (row weights and
 * the weights' sums). Errors: FP_EARG, FP_ESHAPE, FP_EWORKSPACE. */
#define FP_MAX_OPEN_CLAIMS 16
typedef struct {
  int32_t row0, nrows;
  const fp_elem* z1;
  int32_t n1;
  const fp_elem* z2;
  int32_t n2;
} fp_open_claim;
int fp_commit_fold_ext(const fp_elem* msg, int64_t ld, int32_t rows, int32_t log_cols, const fp_elem* r_prox,
                       int32_t n_prox, int32_t n_claims, const fp_open_claim* claims, fp_elem* U, void* ws,
                       size_t ws_bytes, hipStream_t stream);
size_t fp_commit_fold_ext_workspace(int32_t rows);

/* Openings of nq columns of a committed code [rows, ld_code] with its salts
 * and tree from fp_merkle_commit (2^log_width columns) ("How fast can
 * FlashProve go", §2: an opening opens a few columns; each is checked
 * against the Merkle root): column q is j = chal[2q] mod 2^log_width (chal:
 * device challenges, 2 words each, the first used). Writes cols [nq][rows] =
 * code[.][j], col_salts [nq][16 bytes] = salt_j, paths [nq][log_width][32
 * bytes] = the siblings of j's nodes from the leaf level up (the root
 * excluded) and idx [nq] = j (idx may be NULL). salts, tree, col_salts, paths
 * 8-byte aligned. Errors: FP_EARG, FP_ESHAPE. */
int fp_merkle_open(const fp_elem* code, int64_t ld_code, int32_t rows, int32_t log_width, const uint8_t* salts,
                   const uint8_t* tree, const fp_elem* chal, int32_t nq, fp_elem* cols, uint8_t* col_salts,
                   uint8_t* paths, int32_t* idx, hipStream_t stream);

/* -------------------------------------------------------------- lookup --- */
/* The lookup that shows the remainders R are small ("How fast can FlashProve
 * go", §3.1: the remainders of each rescale are range-checked by a lookup;
 * §4: the lookup is a grand-product argument whose key side is a binary
 * product tree, reduced level by level with sum-check).
 *
 * fp_lookup_tree: tree receives 2^(L+1) - 1 field elements: level 0 = the 2^L
 * leaves gamma - key_i (keys[i] as a field element for i < n, 0 for
 * n <= i < 2^L), level d+1 entry i = (level d entry 2i) * (entry 2i+1), each
 * level after the one below it, the root last. gamma: device pointer to one
 * field element. 0 <= n <= 2^L, L <= FP_MAX_N. */
int fp_lookup_tree(const int8_t* keys, int64_t n, int32_t L, const fp_elem* gamma, fp_elem* tree,
                   hipStream_t stream);

/* The clamp's lookup ("How fast can FlashProve go", §2: a clamp is not a
 * polynomial, so its output is committed and proved by a lookup; §3.1: g_w and
 * the clamped value are committed, 16-bit values). fp_lookup_tree_pairs builds
 * the same tree over the keys A[i] + scale B[i] + offset of two field tables
 * (for the clamp: A = Q, B = Y, scale = 2^16, offset = 2^15 + 2^23, so a key
 * is the table row (q + 2^15) + 2^16 (clamp(q) + 128) of q = Q exactly when
 * Y = clamp(Q)); leaves past n are gamma - 0. fp_lookup_counts_field counts
 * field keys read as signed integers (a > p/2 as a - p): counts[v - lo] for
 * lo <= v < lo + 2^bits (bits <= 24), counts[2^bits] for the others; counts:
 * device, 2^bits + 1 entries, overwritten. Errors: FP_EARG, FP_ESHAPE,
 * FP_ERANGE. */
int fp_lookup_tree_pairs(const fp_elem* A, const fp_elem* B, int64_t n, uint64_t scale, uint64_t offset, int32_t L,
                         const fp_elem* gamma, fp_elem* tree, hipStream_t stream);
int fp_lookup_counts_field(const fp_elem* A, int64_t n, int64_t lo, int32_t bits, uint32_t* counts, hipStream_t stream);

/* Multiplicities of the table values t = -2^(s-1) + i (i < 2^s, 1 <= s <= 8)
 * among the n keys and the 2^L - n padding keys (value 0): counts[i]; keys
 * outside the table are counted in counts[2^s]. counts: device, 2^s + 1
 * entries, overwritten. */
int fp_lookup_counts(const int8_t* keys, int64_t n, int32_t L, int32_t s, uint32_t* counts, hipStream_t stream);

/* Degree-3 sum-check of sum_{x < 2^m} E[x] V[2x] V[2x+1] (0 <= m < FP_MAX_N):
 * round i writes rounds[4i + c] = g_i(c) for c = 0..3 and then binds the
 * lowest remaining variable to r[i] (r_i is applied only after g_i is
 * complete); finals = E, A, B at the point r, with A[x] = V[2x],
 * B[x] = V[2x+1]. E: 2^m, V: 2^(m+1) canonical elements. ws:
 * fp_sumcheck3_workspace(m) bytes, 8-byte aligned. */
int fp_sumcheck3_prove(const fp_elem* E, const fp_elem* V, int32_t m, const fp_elem* r, fp_elem* rounds,
                       fp_elem* finals, void* ws, size_t ws_bytes, hipStream_t stream);
size_t fp_sumcheck3_workspace(int32_t m);

/* The product tree's proof from the root down (1 <= L <= FP_MAX_N): for
 * d = L-1 .. 0 the claim on level d+1 at z_{d+1} is reduced to level d by the
 * degree-3 sum-check with E = eq(z_{d+1}, .) and V = level d of tree. chal holds,
 * for d from L-1 down to 0, the block [lambda_d, rho_1 .. rho_{L-1-d}]
 * (L(L+1)/2 elements): rho are level d's round challenges and the block is
 * z_d (z_L is empty). Outputs in the same level order: rounds (L(L-1)/2
 * rounds of 4 values) and finals (3 per level). ws:
 * fp_lookup_prove_workspace(L) bytes, 256-byte aligned (every level's eq table,
 * built up front from chal in one launch, then each level's own sum-check
 * tables: since chal is an input no level waits for another, and the levels'
 * sum-checks run side by side). */
int fp_lookup_prove(const fp_elem* tree, int32_t L, const fp_elem* chal, fp_elem* rounds, fp_elem* finals, void* ws,
                    size_t ws_bytes, hipStream_t stream);
size_t fp_lookup_prove_workspace(int32_t L);

/* --------------------------------------- soundness-faithful challenges --- */
/* Fiat-Shamir challenges over an extension of Goldilocks ("How fast can
 * FlashProve go", §2: every challenge is a BLAKE2b hash of all the prover has
 * sent so far; §4 footnote 20: challenge arithmetic runs in an extension
 * field). Extension elements are pairs (a, b) = a + u b of canonical base
 * elements with u^2 = 7, stored as two consecutive fp_elem.
 *
 * The transcript state is 32 bytes of device memory (8-byte aligned):
 * fp_fs_init sets it to BLAKE2b-256 of the nbytes (<= 128) host bytes msg
 * (they travel in the kernel arguments); fp_fs_absorb sets
 * state <- BLAKE2b-256(state || data) for nwords device words (8 little-endian
 * bytes each); fp_fs_challenges writes k extension elements to out [k][2]
 * without changing the state: digest 0 is the state, digest j >= 1 is
 * BLAKE2b-256(state || j as 4 little-endian bytes), and digest j's words
 * w0..w3 give challenges 2j = (w0 mod p, w1 mod p) and 2j+1 = (w2 mod p,
 * w3 mod p). */
int fp_fs_init(uint8_t* state, const uint8_t* msg, int32_t nbytes, hipStream_t stream);
int fp_fs_absorb(uint8_t* state, const fp_elem* data, int32_t nwords, hipStream_t stream);
int fp_fs_challenges(const uint8_t* state, int32_t k, fp_elem* out, hipStream_t stream);

/* E0[k] + u E1[k] = prod_j (bit j of k ? r_j : 1 - r_j) for k < 2^n over the
 * extension; r: device [n][2], n <= 24. */
int fp_eq_table_ext(const fp_elem* r, int32_t n, fp_elem* E0, fp_elem* E1, hipStream_t stream);

/* c0 = (c4[0] + 7 c4[1]) + u (c4[2] + c4[3]): the extension claim from the four
 * base claims of (E_t0, E_o0), (E_t1, E_o1), (E_t0, E_o1), (E_t1, E_o0). */
int fp_ext_claim_combine(const fp_elem* c4, fp_elem* c0, hipStream_t stream);

/* Sum-check of sum_{k < 2^n} A(k) B(k) over the extension (A = A0 + u A1,
 * B = B0 + u B1, device arrays of 2^n canonical elements, n <= 12) with the
 * transcript: round i writes rounds[6i .. 6i+5] = g_i(0), g_i(1), g_i(2),
 * absorbs those 6 words, takes r_i = challenge 0 of the new state (written to
 * r[2i], r[2i+1]) and only then binds the lowest remaining variable to r_i.
 * At the end finals = A(r), B(r) (4 words), which are absorbed. One
 * workgroup. */
int fp_sumcheck_ext_fs(const fp_elem* A0, const fp_elem* A1, const fp_elem* B0, const fp_elem* B1, int32_t n,
                       uint8_t* state, fp_elem* rounds, fp_elem* r, fp_elem* finals, hipStream_t stream);

/* The same for sum_j rho_j sum_{k < 2^n} A_j(k) B_j(k) over 1..8 pairs
 * ("How fast can FlashProve go", §2: the maps of a layer share one sum-check
 * when their claims are batched; §4 footnote 20: over the extension). A0, A1,
 * B0, B1 are HOST arrays of n_pairs device pointers (each table 2^n canonical
 * elements as its 1 and u parts); rho: device [n_pairs][2] or NULL (all ones);
 * n <= 24. Round i writes rounds[6i .. 6i+5] = g_i(0), g_i(1), g_i(2) with
 *   g_i(c) = sum_j rho_j sum_q A_j,c[q] B_j,c[q],  A_c[q] = A[2q] + c (A[2q+1] - A[2q]),
 * absorbs those 6 words, takes r_i = challenge 0 of the new state (r[2i],
 * r[2i+1]) and only then binds every table. At the end finals[4j .. 4j+3] =
 * A_j(r), B_j(r) for every pair, absorbed as one message of 4 n_pairs words.
 * The tables stream through ws (fp_sumcheck_ext_fs_multi_workspace(n_pairs, n)
 * bytes, 256-byte aligned; none for n = 0): while the A tables hold more than
 * 1024 entries in all, a round is one launch over many workgroups (each on a
 * run of one pair's entries) for its sums and one for its transcript step;
 * the last rounds run in one workgroup with the tables in LDS. Errors:
 * FP_EARG, FP_ESHAPE (n), FP_EWORKSPACE. */
int fp_sumcheck_ext_fs_multi(int32_t n_pairs, const fp_elem* const* A0, const fp_elem* const* A1,
                             const fp_elem* const* B0, const fp_elem* const* B1, const fp_elem* rho, int32_t n,
                             uint8_t* state, fp_elem* rounds, fp_elem* r, fp_elem* finals, void* ws, size_t ws_bytes,
                             hipStream_t stream);
size_t fp_sumcheck_ext_fs_multi_workspace(int32_t n_pairs, int32_t n);

/* ----------------------------------------------------------------- MLE --- */
/* out[0] = M~(r_cols || r_rows) for an int8/int32 matrix [rows, cols] (leading
 * dim ld) zero-padded to [2^n_rows, 2^n_cols]; rows <= 2^n_rows and
 * cols <= 2^n_cols. Used for the matmul claim c0 = Z~(r_o || r_t)
 * ("How fast can FlashProve go", §3.1: the claim about the rescaled product). */
int fp_mle_eval(fp_dtype dt, const void* M, int64_t ld, int32_t rows, int32_t cols, const fp_elem* r_rows,
                int32_t n_rows, const fp_elem* r_cols, int32_t n_cols, fp_elem* out, void* ws, size_t ws_bytes,
                hipStream_t stream);
size_t fp_mle_eval_workspace(fp_dtype dt, int32_t rows, int32_t cols, int32_t n_rows, int32_t n_cols);

typedef struct {
  const void* M;          /* device, int8 or int32 (one dtype per call) */
  int64_t ld;
  int32_t rows, cols;
  const fp_elem* E_rows;  /* device, >= rows */
  const fp_elem* E_cols;  /* device, >= cols */
  fp_elem* out;           /* device, 1 element */
} fp_claim_desc;

/* Several matmul claims from precomputed eq tables in one pair of launches:
 * out_j = sum_t sum_c E_rows_j[t] E_cols_j[c] M_j[t, c], i.e. M_j~(r_cols ||
 * r_rows) when the tables are eq(r_rows, .) and eq(r_cols, .). descs is a
 * HOST array read during the call (descriptors travel in kernel arguments). */
int fp_claim_eval_batched(fp_dtype dt, int32_t count, const fp_claim_desc* descs, void* ws, size_t ws_bytes,
                          hipStream_t stream);
size_t fp_claim_eval_batched_workspace(fp_dtype dt, int32_t count, const fp_claim_desc* descs);

/* Folds and matmul claims of one layer in a single pass: the fold descriptors
 * (all of dtype fold_dt) and the claim descriptors (all of dtype claim_dt) are
 * processed by one launch of the row-fold kernel and one launch of the
 * cross-chunk sums per dozen descriptors, so the passes over the weights and
 * over Z share the GPU instead of running one after the other ("How fast can
 * FlashProve go", §4 counts these as passes over the tables). Each output is
 * exactly what fp_fold_matrix_batched / fp_claim_eval_batched writes for the
 * same descriptor. Either count may be 0. descs are HOST arrays read during
 * the call. ws: sized by fp_fold_claim_batched_workspace with the same
 * arguments. */
int fp_fold_claim_batched(fp_dtype fold_dt, int32_t n_fold, const fp_fold_desc* folds, fp_dtype claim_dt,
                          int32_t n_claim, const fp_claim_desc* claims, void* ws, size_t ws_bytes, hipStream_t stream);
size_t fp_fold_claim_batched_workspace(fp_dtype fold_dt, int32_t n_fold, const fp_fold_desc* folds, fp_dtype claim_dt,
                                       int32_t n_claim, const fp_claim_desc* claims);

/* ----------------------------------------------------------- layer step --- */
/* One step of a stream of proofs of one layer, in ONE launch: the witness and
 * eq tables of proof k (exactly fp_witness_linear_packed(X, ldx, Wp, T, d_in,
 * d_out, s, Z, Y, R, n_eq, eq)), the folds and claims of proof k-1 (exactly
 * fp_fold_claim_batched(FP_I8, n_fold, folds, FP_I32, n_claim, claims)) and
 * the sum-check of proof k-2 (exactly fp_sumcheck_prove(n_pairs, A, B, rho,
 * n, r, rounds, finals, claim0); n_pairs = 0: none). The three share no data
 * ("How fast can FlashProve go", §2: the witness of every layer, then the
 * folds and each matmul's sum-check), so their workgroups run side by side:
 * the GEMM on most compute units, the folds' workgroups beside it, the
 * sum-check's chain of rounds on one. The folds' cross-chunk sums are done by
 * the last workgroup of each column strip (or claim) to finish, through
 * arrival counters at the start of ws: ws is fp_layer_step_workspace(T, d_out,
 * claim_E_t != NULL, n_fold, folds, n_claim, claims) bytes, 256-byte aligned,
 * and its first FP_FOLD_COUNTER_BYTES must be zero on entry (every call leaves
 * them zero). At most 4 folds and claims, each with rows and columns
 * (FP_ESHAPE otherwise); the conditions of the three calls apply
 * (VP * 2^n <= 4096). Inputs of one part must not be written by another part
 * of the same call.
 *
 * Proof k's own claim (claim_E_t non-NULL; device tables of >= T and >= d_out
 * entries, claim one element): *claim = sum_t sum_o E_t[t] E_o[o] Z[t, o]
 * ("How fast can FlashProve go", §3.1: the claim about the product, the value
 * fp_claim_eval_batched gives for Z), taken from the GEMM's accumulators, so Z
 * need not be stored (Z may be NULL); E_t and E_o must then be complete before
 * the call (not tables that the same call builds). Needs T, d_out > 0
 * (FP_ESHAPE), and claim_E_o and claim with claim_E_t (FP_EARG). */
int fp_layer_step(const int8_t* X, int64_t ldx, const int8_t* Wp, int32_t T, int32_t d_in, int32_t d_out, int32_t s,
                  int32_t* Z, int8_t* Y, int8_t* R, const fp_elem* claim_E_t, const fp_elem* claim_E_o,
                  fp_elem* claim, int32_t n_eq, const fp_eq_desc* eq, int32_t n_fold,
                  const fp_fold_desc* folds, int32_t n_claim, const fp_claim_desc* claims,
                  void* ws, size_t ws_bytes, int32_t n_pairs, const fp_elem* const* A, const fp_elem* const* B,
                  const fp_elem* rho, int32_t n, const fp_elem* r, fp_elem* rounds, fp_elem* finals,
                  fp_elem* claim0, hipStream_t stream);
/* Bytes of fp_layer_step's ws for these folds and claims, with (own_claim != 0)
 * one slot per GEMM wave for the claim of proof k; 0 on bad arguments. */
size_t fp_layer_step_workspace(int32_t T, int32_t d_out, int32_t own_claim, int32_t n_fold,
                               const fp_fold_desc* folds, int32_t n_claim, const fp_claim_desc* claims);

/* ------------------------------------------ all the maps of one layer --- */
/* The witness GEMMs of up to FP_MAX_MULTI linear maps in ONE launch, each
 * map's claim taken from its accumulators ("How fast can FlashProve go", §2:
 * each linear map of the integer model is a matmul whose output is rescaled,
 * clamped and committed with its remainder, and whose claim sum-check reduces
 * to its folded tables; §3.1: that claim is about the product 2^k g_w + r,
 * i.e. about Z, so Z itself need not be stored). For map m (desc mm[m]):
 *   X: int8 [T, d_in] (leading dim ldx >= d_in, rows 16-byte aligned, d_in %
 *   16 == 0); Wp: the map's weights W [d_out, d_in] packed by
 *   fp_witness_pack_weights (16-byte aligned); writes Y, R int8 [T, d_out]
 *   exactly as fp_witness_linear (rescale by 2^s, ties up; R against the
 *   unclamped quotient; Y clamped to [-128, 127]) and Z int32 [T, d_out] when
 *   Z is non-NULL (all dense row-major). With E_t non-NULL (device tables of
 *   >= T and >= d_out entries, complete before the call) it also writes
 *   *claim = sum_t sum_o E_t[t] E_o[o] Z[t, o] mod p (the value
 *   fp_claim_eval_batched gives for Z); such a map needs T, d_out > 0.
 * Maps run in the order given (the longest reduction first balances the
 * launch's end); group_o >= 1 output tiles are walked at a time with the token
 * tiles outermost (1: a weight panel's token tiles one after another). The
 * n_eq eq tables (as fp_eq_table_batched, at most 8) are built by spare
 * workgroups of the same launch: tables of another proof, not ones this
 * launch's claims read. ws: fp_witness_multi_workspace(count, mm) bytes,
 * 256-byte aligned, needed when some map forms a claim (else may be NULL);
 * its first FP_MAX_MULTI * 64 + FP_FOLD_COUNTER_BYTES bytes (arrival counters,
 * the same layout as fp_layer_step_multi's, so one workspace serves both) must
 * be zero on entry and every call leaves them zero. With a workspace and at
 * least 1024 tiles (256 outputs x 128 tokens each), each XCD's last tiles are
 * taken at run time by whichever workgroups get there first (counters in the
 * same first lines); the results do not depend on who takes them. Errors: FP_EARG (count outside [1,
 * FP_MAX_MULTI], null pointers, group_o < 1), FP_ESHAPE (alignment, d_in >
 * FP_MAX_DIN, a claim without outputs), FP_ERANGE (s outside [1, 8]),
 * FP_EWORKSPACE. Maps must not write each other's inputs. */
#define FP_MAX_MULTI 8
typedef struct {
  const int8_t* X;
  int64_t ldx;
  int32_t T, d_in, d_out;
  const int8_t* Wp;
  int32_t* Z;
  int8_t* Y;
  int8_t* R;
  const fp_elem* E_t;
  const fp_elem* E_o;
  fp_elem* claim;
} fp_matmul_desc;
int fp_witness_multi(int32_t count, const fp_matmul_desc* mm, int32_t s, int32_t group_o, int32_t n_eq,
                     const fp_eq_desc* eq, void* ws, size_t ws_bytes, hipStream_t stream);
/* Bytes of fp_witness_multi's workspace for these maps; 0 on bad arguments. */
size_t fp_witness_multi_workspace(int32_t count, const fp_matmul_desc* mm);

/* One step of a stream of proofs of a multi-map layer in ONE launch: the
 * witness GEMMs and claims of proof k (exactly fp_witness_multi(count, mm, s,
 * group_o, n_eq, eq, ...)), the int8 folds of proof k-1 (exactly
 * fp_fold_matrix_batched(FP_I8, n_fold, folds, ...)) and the n_sc sum-check
 * instances of proof k-2 (each exactly fp_sumcheck_prove(n_pairs, A, B, rho,
 * n, r, rounds, finals, claim0)). The three share no data ("How fast can
 * FlashProve go", §2: each map's witness, then its folds and its sum-check),
 * so their workgroups run side by side: each sum-check instance is one
 * workgroup (its first rounds stream the tables through the workspace, the
 * rest run in registers; every round's sums are complete across the
 * workgroup before its challenge is applied), the folds' cross-chunk sums are
 * done by the last workgroup of each column strip, and the GEMM tiles fill
 * the GPU. Inputs of one part must not be written by another part of the
 * same call (the sum-check tables are proof k-2's folds, the folds write
 * proof k-1's). At most FP_STEP_MULTI_MAX_FOLD folds (each with rows and
 * columns) and FP_STEP_MULTI_MAX_SUMCHECK instances of 1..8 pairs with
 * 1 <= n <= FP_STEP_MULTI_MAX_SC_N and 16-byte aligned tables. ws:
 * fp_layer_step_multi_workspace(...) bytes, 256-byte aligned; its first
 * FP_MAX_MULTI * 64 + FP_FOLD_COUNTER_BYTES bytes (arrival counters) must be
 * zero on entry, and every call leaves them zero. Errors as fp_witness_multi,
 * plus FP_EARG/FP_ESHAPE for the folds' and sum-checks' arguments. */
#define FP_STEP_MULTI_MAX_FOLD 12
#define FP_STEP_MULTI_MAX_SUMCHECK 4
#define FP_STEP_MULTI_MAX_SC_N 20
#define FP_SC_DESC_MAX_PAIRS 8
typedef struct {
  int32_t n_pairs, n;
  const fp_elem* A[FP_SC_DESC_MAX_PAIRS]; /* device tables of 2^n entries */
  const fp_elem* B[FP_SC_DESC_MAX_PAIRS];
  const fp_elem* rho; /* device n_pairs weights, or NULL (all ones) */
  const fp_elem* r;   /* device n challenges */
  fp_elem* rounds;    /* device [n][3] */
  fp_elem* finals;    /* device [n_pairs][2] */
  fp_elem* claim0;    /* device 1, or NULL */
} fp_sumcheck_desc;
int fp_layer_step_multi(int32_t count, const fp_matmul_desc* mm, int32_t s, int32_t group_o, int32_t n_eq,
                        const fp_eq_desc* eq, int32_t n_fold, const fp_fold_desc* folds, int32_t n_sc,
                        const fp_sumcheck_desc* sc, void* ws, size_t ws_bytes, hipStream_t stream);
/* Bytes of fp_layer_step_multi's workspace; 0 on bad arguments. */
size_t fp_layer_step_multi_workspace(int32_t count, const fp_matmul_desc* mm, int32_t n_fold,
                                     const fp_fold_desc* folds, int32_t n_sc, const fp_sumcheck_desc* sc);

/* fp_witness_multi without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the arrival counters and claim slots live
 * in a scratch array of FP_WITNESS_MULTI_SCRATCH_BYTES inside the library, one
 * per GPU, held until the process ends. The call allocates nothing; on its
 * first call on a device it looks the array's address up (hipGetSymbolAddress).
 * Arguments, outputs and errors as fp_witness_multi; maps whose
 * fp_witness_multi_workspace exceeds the array are refused with
 * FP_EWORKSPACE. Every call on a GPU shares that GPU's array: the call first
 * clears its counters on the stream, and calls that overlap on one GPU (other
 * streams, other threads) race and must not be issued. */
#define FP_WITNESS_MULTI_SCRATCH_BYTES (1 << 20)
int fp_witness_multi_noalloc(int32_t count, const fp_matmul_desc* mm, int32_t s, int32_t group_o, int32_t n_eq,
                             const fp_eq_desc* eq, hipStream_t stream);

/* ----------------------------------------------------------- sum-check --- */
/* Sum-check of the claim sum_j rho_j sum_k A_j[k] B_j[k] over n_pairs pairs of
 * tables of 2^n entries ("How fast can FlashProve go", §2: sum-check reduces
 * the matmul to claims about the committed tables). A and B are HOST arrays of
 * n_pairs device pointers; rho is a device array of n_pairs field elements or
 * NULL (all ones). r (device, n) are the round challenges. For each round i
 * the prover sends g_i(0), g_i(1), g_i(2) with
 *   g_i(c) = sum_j rho_j sum_q A_j,c[q] B_j,c[q],  A_c[q] = A[2q] + c (A[2q+1] - A[2q]),
 * then binds A[q] <- A[2q] + r_i (A[2q+1] - A[2q]) (B likewise); r_i is
 * applied only after g_i is complete across all of the call's threads (the
 * challenges are inputs and may be loaded earlier). Outputs (device): rounds [n][3],
 * finals [n_pairs][2] = (A_j~(r), B_j~(r)), claim0 (1 element, may be NULL) =
 * the initial claim. Tables are not modified. n in [1, 30]. */
int fp_sumcheck_prove(int32_t n_pairs, const fp_elem* const* A, const fp_elem* const* B, const fp_elem* rho,
                      int32_t n, const fp_elem* r, fp_elem* rounds, fp_elem* finals, fp_elem* claim0, void* ws,
                      size_t ws_bytes, hipStream_t stream);
size_t fp_sumcheck_workspace(int32_t n_pairs, int32_t n);

/* The witness of one linear layer (exactly fp_witness_linear(X, ..., R)) and,
 * in the same launch, the sum-check of another claim (exactly
 * fp_sumcheck_prove(n_pairs, A, B, rho, n, r, rounds, finals, claim0)). For a
 * stream of layer proofs: the sum-check of proof k, a chain of dependent
 * rounds that keeps one compute unit busy, runs beside the GEMM of proof k+1,
 * which has no data in common with it ("How fast can FlashProve go", §2: the
 * witness of every layer, then each matmul's sum-check). The sum-check must fit
 * one workgroup: VP * 2^n <= 4096 (8192 when T > 32 and the output has at
 * least 256 tiles of 256 x 256), VP = n_pairs rounded up to a power of two;
 * FP_ESHAPE otherwise. The sum-check tables must not be written by the
 * witness (they are read while it runs). No workspace. */
int fp_witness_linear_with_sumcheck(const int8_t* X, int64_t ldx, const int8_t* W, int64_t ldw, int32_t T,
                                    int32_t d_in, int32_t d_out, int32_t s, int32_t* Z, int8_t* Y, int8_t* R,
                                    int32_t n_pairs, const fp_elem* const* A, const fp_elem* const* B,
                                    const fp_elem* rho, int32_t n, const fp_elem* r, fp_elem* rounds,
                                    fp_elem* finals, fp_elem* claim0, hipStream_t stream);

/* n_inst independent single-pair sum-checks of 2^n entries in one launch
 * (one MoE expert's claim each: "How fast can FlashProve go", §2, each
 * routed expert's matmul is its own claim, and sum-check reduces each to its
 * folded tables; the round message and binding are fp_sumcheck_prove's). A, B: device [n_inst][2^n]; r: [n_inst][n];
 * rounds: [n_inst][n][3]; finals: [n_inst][2]; claim0: [n_inst] or NULL.
 * n in [1, 13]. */
int fp_sumcheck_prove_multi(int32_t n_inst, int32_t n, const fp_elem* A, const fp_elem* B, const fp_elem* r,
                            fp_elem* rounds, fp_elem* finals, fp_elem* claim0, hipStream_t stream);

/* Random linear combination of finished sum-check claims ("How fast can
 * FlashProve go", §2: claims about the weights are merged into one):
 * out[0] = sum_j rho[j] g_j(x_j), where g_j is the last round polynomial of
 * claim j given by its values at 0, 1, 2 (g_last[j]: device pointer to 3
 * elements) and x_j its last challenge (x_last[j]: device pointer to 1
 * element). g_last and x_last are HOST arrays of `count` device pointers;
 * rho is a device array of `count`. count <= 16. */
int fp_combine_claims(int32_t count, const fp_elem* const* g_last, const fp_elem* const* x_last,
                      const fp_elem* rho, fp_elem* out, hipStream_t stream);

/* out[0] = sum_j rho[j] v_j: the random linear combination of `count`
 * claims ("How fast can FlashProve go", §2: claims are merged), with vals a
 * HOST array of device pointers to one element each; rho device [count];
 * count <= 16. */
int fp_linear_combine(int32_t count, const fp_elem* const* vals, const fp_elem* rho, fp_elem* out,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FP_H */
