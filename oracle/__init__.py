"""CPU oracle for the matmul sum-check prover.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product path never imports this
package, and this package imports nothing from the product.

``oracle.c`` holds the arithmetic (plain C, exact: field products through
unsigned __int128 and ``%``, integer sums in int64). This module marshals numpy
arrays into it and strings the steps of a layer proof together in the order of
"How fast can FlashProve go", §2 (witness, then sum-check claims about the
committed tables and weights) and §3.1 (the remainder of each rescale is
committed beside the rescaled output). Small scalar field arithmetic here uses
Python integers with ``% P``. The commitment of Y and R (§3.1: limbs packed
three to a field element, each row Reed-Solomon encoded by an NTT, each column
a salted BLAKE2b Merkle leaf) uses the C code for packing and encoding and the
host's ``hashlib.blake2b`` for every hash. The lookup that shows the
remainders are small (§3.1, §4: a grand-product argument with the key side as
a binary tree, reduced level by level) is a product tree, a degree-3
sum-check per level in C, and its verifier here. The layer proof with the
rescale committed (§2 and §3.1: Q, R and Y committed, the matmul's claim read as
2^s Q~ + R~ from folded rows of the commitment, columns opened against the root,
challenges from the transcript over F_p[u]/(u^2 - 7)) is strung together here
from those pieces, with a verifier that never forms the witness.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess

import numpy as np

P = 0xFFFFFFFF00000001
INV2 = (P + 1) // 2
REASONS = {0: "OK", 1: "INITIAL_CLAIM", 2: "ROUND_SUM", 3: "FINAL_CLAIM", 4: "FINAL_OPENING",
           5: "RESCALE_IDENTITY", 6: "WITNESS_MISMATCH"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (never hipcc)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        sig = {
            "or_add": (u64, [u64, u64]), "or_sub": (u64, [u64, u64]), "or_mul": (u64, [u64, u64]),
            "or_from_int": (u64, [i64]), "or_pow": (u64, [u64, u64]),
            "or_eval_deg2": (u64, [u64, u64, u64, u64]),
            "or_witness": (ctypes.c_int, [vp, i64, vp, i64, i32, i32, i32, i32, vp, vp, vp]),
            "or_witness_entries": (None, [vp, i64, vp, i64, i32, i64, vp, vp, vp]),
            "or_eq_table": (None, [vp, i32, vp]),
            "or_eq_at": (u64, [vp, i32, i64]),
            "or_fold_rows": (None, [vp, i32, i64, i32, i32, vp, vp, i32]),
            "or_fold_cols": (None, [vp, i32, i64, i32, vp, i64, vp, vp]),
            "or_fold_field_rows": (None, [vp, i64, i32, i32, vp, vp]),
            "or_dot": (u64, [vp, vp, i64]),
            "or_mle_brute": (u64, [vp, i32, vp]),
            "or_mle_seq": (u64, [vp, i32, vp]),
            "or_mle_matrix": (u64, [vp, i32, i64, i32, i32, vp, i32, vp, i32]),
            "or_sumcheck": (None, [i32, vp, vp, vp, i32, vp, vp, vp, vp]),
            "or_check_sumcheck": (ctypes.c_int, [i32, vp, vp, vp, i32, vp, vp, vp, u64, vp]),
            "or_check_rescale": (ctypes.c_int, [vp, vp, vp, i64, i32, vp]),
            "or_check_witness": (ctypes.c_int, [vp, i64, vp, i64, i32, i32, i32, vp, vp]),
            "or_pack_limbs": (None, [vp, i64, vp, i64, i64, i32, vp]),
            "or_root_of_unity": (u64, [i32]),
            "or_rs_encode": (None, [vp, i32, vp]),
            "or_rs_eval": (u64, [vp, i32, i64]),
            "or_product_tree": (None, [vp, i64, i32, u64, vp]),
            "or_lookup_counts": (i64, [vp, i64, i32, i32, vp]),
            "or_product_tree_field": (None, [vp, i64, i32, u64, vp]),
            "or_pair_keys": (None, [vp, vp, i64, u64, u64, vp]),
            "or_sumcheck3": (None, [vp, vp, i32, vp, vp, vp]),
            "or_eval_deg3": (u64, [vp, u64]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous arrays"
    return a.ctypes.data


def _u64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint64))


def log2ceil(v: int) -> int:
    return 0 if v <= 1 else (int(v) - 1).bit_length()


# ------------------------------------------------------------------ field --
def add(a, b): return int(lib().or_add(a, b))
def sub(a, b): return int(lib().or_sub(a, b))
def mul(a, b): return int(lib().or_mul(a, b))
def from_int(v): return int(lib().or_from_int(int(v)))
def power(a, e): return int(lib().or_pow(a, e))
def eval_deg2(g0, g1, g2, x): return int(lib().or_eval_deg2(g0, g1, g2, x))


# ---------------------------------------------------------------- witness --
def witness(X: np.ndarray, W: np.ndarray, s: int):
    """Z = X W^T (int32), Y = clamp(floor((Z + 2^(s-1)) / 2^s)), R = Z - 2^s Q."""
    X, W = np.ascontiguousarray(X, np.int8), np.ascontiguousarray(W, np.int8)
    T, d_in = X.shape
    d_out = W.shape[0]
    assert W.shape[1] == d_in and 1 <= s <= 8
    Z = np.empty((T, d_out), np.int32)
    Y = np.empty((T, d_out), np.int8)
    R = np.empty((T, d_out), np.int8)
    rc = lib().or_witness(_p(X), d_in, _p(W), d_in, T, d_in, d_out, s, _p(Z), _p(Y), _p(R))
    if rc != 0:
        raise OverflowError("|Z| >= 2^31")
    return Z, Y, R


def witness_entries(X, W, ts, os_):
    X, W = np.ascontiguousarray(X, np.int8), np.ascontiguousarray(W, np.int8)
    ts = np.ascontiguousarray(ts, np.int32)
    os_ = np.ascontiguousarray(os_, np.int32)
    out = np.empty(len(ts), np.int64)
    lib().or_witness_entries(_p(X), X.shape[1], _p(W), W.shape[1], X.shape[1], len(ts), _p(ts), _p(os_), _p(out))
    return out


def rescale(Z: np.ndarray, s: int):
    """Q, R, Y of integer values Z, by explicit floor division (no shifts)."""
    Z = np.asarray(Z, np.int64)
    Q = np.floor_divide(Z + (1 << (s - 1)), 1 << s)
    R = Z - Q * (1 << s)
    return Q, R, np.clip(Q, -128, 127)


# --------------------------------------------------------------------- eq --
def eq_table(r) -> np.ndarray:
    r = _u64(r)
    E = np.empty(1 << len(r), np.uint64)
    lib().or_eq_table(_p(r), len(r), _p(E))
    return E


def eq_at(r, k: int) -> int:
    r = _u64(r)
    return int(lib().or_eq_at(_p(r), len(r), k))


# ------------------------------------------------------------------ folds --
def fold_rows(M: np.ndarray, E, cols_pad: int | None = None) -> np.ndarray:
    """out[k] = sum_{t < rows} E[t] M[t, k]; zero for cols <= k < cols_pad."""
    M = np.ascontiguousarray(M)
    assert M.dtype in (np.int8, np.int32)
    rows, cols = M.shape
    E = _u64(E)
    assert len(E) >= rows
    cols_pad = cols if cols_pad is None else cols_pad
    out = np.empty(cols_pad, np.uint64)
    lib().or_fold_rows(_p(M), M.dtype.itemsize, cols, rows, cols, _p(E), _p(out), cols_pad)
    return out


def request_vectors(M: np.ndarray, Es, cols_pad: int | None = None) -> np.ndarray:
    """Folded rows of one weight table for a batch of requests ("How fast can
    FlashProve go", §2.1: each request commits the weight table's folded row,
    its request vector): row j is fold_rows(M, Es[j]). Returns [R, cols_pad]."""
    cols_pad = M.shape[1] if cols_pad is None else cols_pad
    return np.stack([fold_rows(M, E, cols_pad) for E in Es]) if len(Es) else np.zeros((0, cols_pad), np.uint64)


def fold_cols(M: np.ndarray, E, ks) -> np.ndarray:
    M = np.ascontiguousarray(M)
    rows, cols = M.shape
    E = _u64(E)
    ks = np.ascontiguousarray(ks, np.int32)
    out = np.empty(len(ks), np.uint64)
    lib().or_fold_cols(_p(M), M.dtype.itemsize, cols, rows, _p(E), len(ks), _p(ks), _p(out))
    return out


# -------------------------------------------------------------------- MLE --
def mle_brute(A, z) -> int:
    A, z = _u64(A), _u64(z)
    assert len(A) == 1 << len(z)
    return int(lib().or_mle_brute(_p(A), len(z), _p(z)))


def mle_seq(A, z) -> int:
    A, z = _u64(A), _u64(z)
    assert len(A) == 1 << len(z)
    return int(lib().or_mle_seq(_p(A), len(z), _p(z)))


def mle_matrix(M: np.ndarray, r_rows, r_cols) -> int:
    """M~(r_cols || r_rows) of an int8/int32 matrix zero-padded to powers of two."""
    M = np.ascontiguousarray(M)
    rows, cols = M.shape
    r_rows, r_cols = _u64(r_rows), _u64(r_cols)
    assert rows <= 1 << len(r_rows) and cols <= 1 << len(r_cols)
    return int(lib().or_mle_matrix(_p(M), M.dtype.itemsize, cols, rows, cols,
                                   _p(r_rows), len(r_rows), _p(r_cols), len(r_cols)))


# -------------------------------------------------------------- sum-check --
def sumcheck(As, Bs, r, rho=None):
    """Sum-check over pairs (A_j, B_j) of 2^n tables; returns (rounds[n,3],
    finals[n_pairs,2], claim0)."""
    As = [_u64(a) for a in As]
    Bs = [_u64(b) for b in Bs]
    r = _u64(r)
    n = len(r)
    for a, b in zip(As, Bs):
        assert len(a) == len(b) == 1 << n
    k = len(As)
    pa = (ctypes.c_void_p * k)(*[_p(a) for a in As])
    pb = (ctypes.c_void_p * k)(*[_p(b) for b in Bs])
    rho_a = None if rho is None else _u64(rho)
    rounds = np.zeros((max(n, 1), 3), np.uint64)
    finals = np.empty((k, 2), np.uint64)
    c0 = ctypes.c_uint64()
    lib().or_sumcheck(k, pa, pb, _p(rho_a), n, _p(r), _p(rounds), _p(finals), ctypes.byref(c0))
    return rounds[:n], finals, int(c0.value)


def check_sumcheck(rounds, finals, r, c0, rho=None, As=None, Bs=None):
    """Verifier-side checks; returns (reason name, where)."""
    rounds = _u64(rounds).reshape(-1, 3)
    finals = _u64(finals).reshape(-1, 2)
    r = _u64(r)
    k = finals.shape[0]
    pa = pb = None
    if As is not None:
        As = [_u64(a) for a in As]
        Bs = [_u64(b) for b in Bs]
        pa = (ctypes.c_void_p * k)(*[_p(a) for a in As])
        pb = (ctypes.c_void_p * k)(*[_p(b) for b in Bs])
    rho_a = None if rho is None else _u64(rho)
    where = ctypes.c_int32()
    rc = lib().or_check_sumcheck(k, pa, pb, _p(rho_a), len(r), _p(r), _p(rounds), _p(finals),
                                 int(c0) % P, ctypes.byref(where))
    return REASONS[rc], int(where.value)


def check_rescale(Z, Y, R, s):
    Z = np.ascontiguousarray(Z, np.int32)
    Y = np.ascontiguousarray(Y, np.int8)
    R = np.ascontiguousarray(R, np.int8)
    where = ctypes.c_int64()
    rc = lib().or_check_rescale(_p(Z), _p(Y), _p(R), Z.size, s, ctypes.byref(where))
    return REASONS[rc], int(where.value)


def check_witness(X, W, Z):
    X, W = np.ascontiguousarray(X, np.int8), np.ascontiguousarray(W, np.int8)
    Z = np.ascontiguousarray(Z, np.int32)
    where = ctypes.c_int64()
    rc = lib().or_check_witness(_p(X), X.shape[1], _p(W), W.shape[1], X.shape[0], X.shape[1], W.shape[0],
                                _p(Z), ctypes.byref(where))
    return REASONS[rc], int(where.value)


# ------------------------------------------------------------- commitment --
# "How fast can FlashProve go", §3.1: a committed table is Reed-Solomon encoded
# row by row (an NTT) and Merkle-hashed column by column (BLAKE2b); values are
# cut into 8-bit limbs packed three to a field element in 20-bit slots.
SALT_BYTES = 16
DIGEST_BYTES = 32


def pack_limbs(A: np.ndarray, B: np.ndarray, logn: int) -> np.ndarray:
    """The limbs of A then B (int8 values, one limb each: the byte 0..255),
    three per element in 20-bit slots, filling rows of 2^logn elements (as
    many rows as needed, zero beyond). Returns [rows, 2^logn] uint64."""
    A = np.ascontiguousarray(A, np.int8).reshape(-1)
    B = np.ascontiguousarray(B, np.int8).reshape(-1)
    n = 1 << logn
    elems = (A.size + B.size + 2) // 3
    rows = max(1, (elems + n - 1) // n)
    out = np.empty((rows, n), np.uint64)
    lib().or_pack_limbs(_p(A), A.size, _p(B), B.size, n, rows, _p(out))
    return out


def root_of_unity(k: int) -> int:
    return int(lib().or_root_of_unity(k))


def rs_encode(msg: np.ndarray) -> np.ndarray:
    """Rate-1/2 Reed-Solomon codewords of each row of msg [rows, n], n = 2^logn:
    code[i, j] = sum_k msg[i, k] w^(jk) for j < 2n, w a primitive 2n-th root of
    unity (root_of_unity(logn + 1))."""
    msg = np.ascontiguousarray(msg, np.uint64)
    rows, n = msg.shape
    logn = log2ceil(n)
    assert 1 << logn == n
    code = np.empty((rows, 2 * n), np.uint64)
    for i in range(rows):
        lib().or_rs_encode(_p(msg[i]), logn, _p(code[i]))
    return code


def rs_eval(row: np.ndarray, j: int) -> int:
    """One codeword entry of a message row by Horner's rule at w^j."""
    row = np.ascontiguousarray(row, np.uint64)
    return int(lib().or_rs_eval(_p(row), log2ceil(row.size), j))


def blake2b(data: bytes) -> bytes:
    return hashlib.blake2b(data, digest_size=DIGEST_BYTES).digest()


def merkle_leaf(code: np.ndarray, salts: np.ndarray, j: int) -> bytes:
    """Leaf of column j: BLAKE2b-256(salt_j || code[0, j] || ... || code[rows-1, j]),
    field elements as 8 little-endian bytes."""
    col = np.ascontiguousarray(code[:, j], np.uint64)
    return blake2b(bytes(salts[j]) + col.astype("<u8").tobytes())


def merkle_tree(code: np.ndarray, salts: np.ndarray) -> list:
    """All levels of the Merkle tree over the columns of code: level 0 holds the
    leaves, level d+1 holds BLAKE2b-256(left || right) of level d's pairs, the
    last level the root. Returns a list of lists of 32-byte digests."""
    width = code.shape[1]
    levels = [[merkle_leaf(code, salts, j) for j in range(width)]]
    while len(levels[-1]) > 1:
        prev = levels[-1]
        levels.append([blake2b(prev[2 * i] + prev[2 * i + 1]) for i in range(len(prev) // 2)])
    return levels


def merkle_path(levels: list, j: int) -> list:
    """Sibling digests from leaf j up to (not including) the root."""
    path = []
    for lev in levels[:-1]:
        path.append(lev[j ^ 1])
        j >>= 1
    return path


def merkle_verify(root: bytes, leaf: bytes, j: int, path: list) -> bool:
    h = leaf
    for sib in path:
        h = blake2b(h + sib) if j % 2 == 0 else blake2b(sib + h)
        j >>= 1
    return h == root


# ----------------------------------------------------------------- lookup --
# "How fast can FlashProve go", §3.1 (rescale remainders are range-checked by
# a lookup) and §4 (a grand-product argument: the keys' product, built as a
# binary tree and reduced level by level with sum-check, against the table's).
LOOKUP_REASONS = {0: "OK", 1: "LEVEL_SUM", 2: "ROUND_SUM", 3: "LEVEL_FINAL", 4: "LEAF_OPENING", 5: "MULTISET"}


def product_tree(keys: np.ndarray, L: int, gamma: int) -> list:
    """Levels of the keys' product tree: level 0 holds the 2^L leaves
    gamma - key (padded with gamma - 0), level d+1 entry i the product of
    level d entries 2i and 2i+1; the last level is the root."""
    keys = np.ascontiguousarray(keys, np.int8).reshape(-1)
    assert keys.size <= 1 << L
    flat = np.empty((2 << L) - 1, np.uint64)
    lib().or_product_tree(_p(keys), keys.size, L, gamma % P, _p(flat))
    levels, off = [], 0
    for d in range(L + 1):
        w = 1 << (L - d)
        levels.append(flat[off:off + w])
        off += w
    return levels


def product_tree_field(keys: np.ndarray, L: int, gamma: int) -> list:
    """product_tree for keys that are field elements (0 past the keys)."""
    keys = _u64(keys).reshape(-1)
    assert keys.size <= 1 << L
    flat = np.empty((2 << L) - 1, np.uint64)
    lib().or_product_tree_field(_p(keys), keys.size, L, gamma % P, _p(flat))
    levels, off = [], 0
    for d in range(L + 1):
        w = 1 << (L - d)
        levels.append(flat[off:off + w])
        off += w
    return levels


# The clamp's lookup ("How fast can FlashProve go", §2: a clamp is not a
# polynomial, so its output is committed and proved by a lookup; §3.1 and its
# footnote: the rescaled value g_w and the clamped g_k are both committed, each
# a 16-bit value). Readings: the key of an entry is the pair (Q, Y) as
# (Q + 2^15) + 2^16 (Y + 128); the table has one row per 16-bit q,
# (q + 2^15) + 2^16 (clamp(q, -128, 127) + 128); Q and Y are the committed
# tables (zero padded, so the padding keys are the row of q = 0). With Q fixed
# by the matmul (Z = 2^s Q + R, R range-checked) and Y a byte, a key is a row
# only if Y = clamp(Q); a Q outside 16 bits has no row.
CLAMP_BITS = 16
CLAMP_SCALE = 1 << 16
CLAMP_OFFSET = (1 << 15) + (128 << 16)


def pair_keys(A: np.ndarray, B: np.ndarray, scale: int, offset: int) -> np.ndarray:
    """Keys A + scale B + offset of two field tables."""
    A, B = _u64(A).reshape(-1), _u64(B).reshape(-1)
    assert A.size == B.size
    out = np.empty(A.size, np.uint64)
    lib().or_pair_keys(_p(A), _p(B), A.size, scale % P, offset % P, _p(out))
    return out


def clamp_keys(Q: np.ndarray, Y: np.ndarray) -> np.ndarray:
    """Keys Q + 2^16 Y + 2^15 + 2^23 of field tables Q, Y (as field elements)."""
    return pair_keys(Q, Y, CLAMP_SCALE, CLAMP_OFFSET)


def field_signed(a: np.ndarray) -> np.ndarray:
    """Field elements read as signed integers (a > p/2 as a - p)."""
    a = _u64(a)
    return np.where(a > np.uint64(P // 2), (a - np.uint64(P)).view(np.int64), a.view(np.int64))


def clamp_counts(Q: np.ndarray):
    """(multiplicities of q = -2^15 + i among the Q entries, entries outside 16 bits)."""
    q = field_signed(Q).reshape(-1) + (1 << (CLAMP_BITS - 1))
    inside = (q >= 0) & (q < (1 << CLAMP_BITS))
    return np.bincount(q[inside], minlength=1 << CLAMP_BITS).astype(np.int64), int((~inside).sum())


def clamp_row(q: int) -> int:
    return (q + (1 << 15)) + (1 << 16) * (min(max(q, -128), 127) + 128)


def clamp_table_product(counts: np.ndarray, gamma: int) -> int:
    """prod_q (gamma - row(q))^(m_q) over the 16-bit q."""
    acc = 1
    for i in np.nonzero(counts)[0]:
        acc = acc * pow((gamma - clamp_row(int(i) - (1 << 15))) % P, int(counts[i]), P) % P
    return acc


def lookup_counts(keys: np.ndarray, L: int, s: int):
    """(multiplicities of t = -2^(s-1) + i among the padded keys, keys outside)."""
    keys = np.ascontiguousarray(keys, np.int8).reshape(-1)
    counts = np.empty(1 << s, np.int64)
    outside = int(lib().or_lookup_counts(_p(keys), keys.size, L, s, _p(counts)))
    return counts, outside


def table_product(counts: np.ndarray, s: int, gamma: int) -> int:
    """prod_t (gamma - t)^(m_t) over the table t = -2^(s-1) .. 2^(s-1) - 1."""
    acc = 1
    for i, m in enumerate(counts):
        acc = acc * pow((gamma - (i - (1 << (s - 1)))) % P, int(m), P) % P
    return acc


def sumcheck3(E, V, r):
    """Degree-3 sum-check of sum_x E[x] V[2x] V[2x+1]: rounds [m, 4] (values at
    0..3), finals (E, A, B at the point r)."""
    E, V, r = _u64(E), _u64(V), _u64(r)
    m = len(r)
    assert len(E) == 1 << m and len(V) == 2 << m
    rounds = np.empty((max(m, 1), 4), np.uint64)
    finals = np.empty(3, np.uint64)
    lib().or_sumcheck3(_p(E), _p(V), m, _p(r), _p(rounds), _p(finals))
    return rounds[:m], [int(x) for x in finals]


def eval_deg3(g, x: int) -> int:
    return int(lib().or_eval_deg3(_p(_u64(g)), x % P))


def lookup_challenge_offset(L: int, d: int) -> int:
    """Start of level d's challenges [lambda_d, rho_1 .. rho_(L-1-d)] in the
    challenge array: levels are proved from d = L-1 down to 0."""
    return (L - 1 - d) * (L - d) // 2


def lookup_challenges_len(L: int) -> int:
    return L * (L + 1) // 2


def grand_product_prove(levels: list, chal) -> list:
    """The product tree's proof, level by level from the root down: for level d
    (2^(L-d) entries) the claim on level d+1 at z_(d+1) is reduced by a
    degree-3 sum-check of eq(z_(d+1), x) V_d(0, x) V_d(1, x) with challenges
    rho; z_d = (lambda_d, rho) is the next point. Returns per level (rounds,
    finals)."""
    L = len(levels) - 1
    chal = _u64(chal)
    proof = []
    z = []  # point of the claim on level d+1
    for d in range(L - 1, -1, -1):
        off = lookup_challenge_offset(L, d)
        m = L - 1 - d
        rho = chal[off + 1: off + 1 + m]
        E = eq_table(z) if m else np.ones(1, np.uint64)
        rounds, finals = sumcheck3(E, levels[d], rho)
        proof.append((rounds, finals))
        z = [int(chal[off])] + [int(x) for x in rho]
    return proof


def grand_product_verify(root: int, proof: list, chal, L: int, keys: np.ndarray, gamma: int, counts=None, s=None,
                         table_prod=None):
    """Verifier of the lookup: each level's round sums, the final
    eq(z, rho) a b, the leaf claim against the keys (int8 keys, or field
    elements given as uint64), and (with counts) the root against the table's
    product, or against table_prod when given. Returns (reason, level)."""
    chal = _u64(chal)
    claim = root % P
    z = []
    for idx, d in enumerate(range(L - 1, -1, -1)):
        rounds, finals = proof[idx]
        off = lookup_challenge_offset(L, d)
        m = L - 1 - d
        rho = [int(x) for x in chal[off + 1: off + 1 + m]]
        for i in range(m):
            g = [int(x) for x in rounds[i]]
            if (g[0] + g[1]) % P != claim:
                return (1 if i == 0 else 2), d
            claim = eval_deg3(g, rho[i])
        e, a, b = finals
        ez = 1
        for zj, rj in zip(z, rho):
            ez = ez * ((zj * rj + (1 - zj) * (1 - rj)) % P) % P
        if e != ez or claim != ez * a % P * b % P:
            return 3, d
        lam = int(chal[off])
        claim = (a + lam * (b - a)) % P
        z = [lam] + rho
    E0 = eq_table(z)
    if isinstance(keys, np.ndarray) and keys.dtype == np.uint64:
        keys = np.ascontiguousarray(keys).reshape(-1)
        kz = int(lib().or_dot(_p(np.ascontiguousarray(E0[:keys.size])), _p(keys), keys.size)) if keys.size else 0
    else:
        keys = np.ascontiguousarray(keys, np.int8).reshape(-1)
        kz = int(fold_rows(keys.reshape(-1, 1), E0[:keys.size])[0]) if keys.size else 0  # sum_i eq(z, i) key_i
    leaf = (gamma - kz) % P
    if leaf != claim:
        return 4, 0
    if table_prod is not None:
        if table_prod % P != root % P:
            return 5, L
    elif counts is not None and table_product(counts, s, gamma) != root % P:
        return 5, L
    return 0, -1


# ----------------------------------------------------------- layer proofs --
def pad_to(v: np.ndarray, size: int) -> np.ndarray:
    out = np.zeros(size, np.uint64)
    out[:len(v)] = v
    return out


def prove_matmul(X, W, s, r_t, r_o, r_rounds, witness_full=True, n_pad=None, x_fold=None):
    """One matmul claim: witness, eq tables, folds, claim and sum-check.

    The claim is c0 = Z~(r_o || r_t); the sum-check runs over k on
    x'[k] = X~(k || r_t) and w'[k] = W~(k || r_o), zero-padded to 2^n.
    With ``witness_full`` False the witness is skipped and c0 is the
    sum-check's own initial claim sum_k x'[k] w'[k] (equal to Z~ because
    Z = X W^T); callers use this at sizes where the full matmul is too slow.
    """
    T, d_in = X.shape
    d_out = W.shape[0]
    n = log2ceil(d_in) if n_pad is None else n_pad
    assert len(r_rounds) == n and len(r_t) == log2ceil(T) and len(r_o) == log2ceil(d_out)
    out = {}
    E_t, E_o = eq_table(r_t), eq_table(r_o)
    out["E_t"], out["E_o"] = E_t, E_o
    out["x_fold"] = fold_rows(X, E_t, 1 << n) if x_fold is None else x_fold
    out["w_fold"] = fold_rows(W, E_o, 1 << n)
    rounds, finals, claim0 = sumcheck([out["x_fold"]], [out["w_fold"]], r_rounds)
    out["rounds"], out["finals"], out["claim0"] = rounds, finals, claim0
    if witness_full:
        Z, Y, R = witness(X, W, s)
        out["Z"], out["Y"], out["R"] = Z, Y, R
        out["c0"] = mle_matrix(Z, r_t, r_o)
    else:
        out["c0"] = claim0
    return out


def group_tokens(route: np.ndarray, n_experts: int):
    """Tokens of each expert in ascending token order (stable by expert)."""
    order = np.argsort(route, kind="stable")
    counts = np.bincount(route, minlength=n_experts)
    offs = np.concatenate([[0], np.cumsum(counts)])
    return [order[offs[e]:offs[e + 1]] for e in range(n_experts)]


def prove_config(cfg, inp: dict, ch: dict, witness_full=True, experts=None):
    """The whole layer proof for one workload description (see synth)."""
    s = cfg.s
    if cfg.kind == "single":
        m = cfg.matmuls[0]
        return {m.name: prove_matmul(inp[m.x], inp[m.w], s, ch["r_t"], ch["r_o"], ch["rounds"], witness_full)}
    if cfg.kind == "rlc_out":
        res, xf = {}, {}
        E_t = eq_table(ch["r_t"])
        for m in cfg.matmuls:
            key = (m.x, m.n)
            if key not in xf:
                xf[key] = fold_rows(inp[m.x], E_t, 1 << m.n)
            res[m.name] = prove_matmul(inp[m.x], inp[m.w], s, ch["r_t"], ch["r_o/" + m.name],
                                       ch["rounds/" + m.name], witness_full, x_fold=xf[key])
        C = 0
        for m in cfg.matmuls:
            g = res[m.name]["rounds"][-1]
            gn = eval_deg2(int(g[0]), int(g[1]), int(g[2]), int(ch["rounds/" + m.name][-1]))
            C = (C + int(ch["rho/" + m.name][0]) * gn) % P
        res["rlc"] = C
        return res
    if cfg.kind == "batched":
        res, xf = {}, {}
        n = cfg.batched_n
        E_t = eq_table(ch["r_t"])
        As, Bs, rho = [], [], []
        c0 = 0
        for m in cfg.matmuls:
            if m.x not in xf:
                xf[m.x] = fold_rows(inp[m.x], E_t, 1 << n)
            E_o = eq_table(ch["r_o/" + m.name])
            wf = fold_rows(inp[m.w], E_o, 1 << n)
            one = {"E_o": E_o, "x_fold": xf[m.x], "w_fold": wf}
            if witness_full:
                Z, Y, R = witness(inp[m.x], inp[m.w], s)
                one.update(Z=Z, Y=Y, R=R, c0=mle_matrix(Z, ch["r_t"], ch["r_o/" + m.name]))
            res[m.name] = one
            As.append(xf[m.x])
            Bs.append(wf)
            rho.append(int(ch["rho/" + m.name][0]))
        rounds, finals, claim0 = sumcheck(As, Bs, ch["rounds"], rho=rho)
        res["E_t"] = E_t
        res["batch"] = {"rounds": rounds, "finals": finals, "claim0": claim0, "rho": rho}
        if witness_full:
            for m, rj in zip(cfg.matmuls, rho):
                c0 = (c0 + rj * res[m.name]["c0"]) % P
            res["batch"]["c0"] = c0
        return res
    if cfg.kind == "moe":
        route = inp["route"]
        groups = group_tokens(route, cfg.n_experts)
        res = {}
        for e in range(cfg.n_experts):
            toks = groups[e]
            if len(toks) == 0 or (experts is not None and e not in experts):
                continue
            Xe = np.ascontiguousarray(inp["X"][toks])
            He = np.ascontiguousarray(inp["H"][toks])
            r_t = ch["r_t/%d" % e]
            up = prove_matmul(Xe, inp["W1_%d" % e], s, r_t, ch["r_o_up/%d" % e], ch["rounds_up/%d" % e],
                              witness_full)
            dn = prove_matmul(He, inp["W2_%d" % e], s, r_t, ch["r_o_down/%d" % e], ch["rounds_down/%d" % e],
                              witness_full)
            res[e] = {"tokens": toks, "up": up, "down": dn}
        return res
    raise ValueError(cfg.kind)


# ------------------------------------------- soundness-faithful challenges --
# "How fast can FlashProve go", §2 (every challenge is a BLAKE2b hash of all
# the prover has sent so far) and §4 footnote 20 (challenge and lookup
# arithmetic runs in an extension of Goldilocks). Readings: the extension is
# F_p[u]/(u^2 - 7) (7 generates F_p*, so it is not a square); the transcript
# state is a 32-byte BLAKE2b-256 digest, s <- BLAKE2b-256(s || message) per
# message; challenges come from s and, beyond the first two, from
# BLAKE2b-256(s || j) for j = 1, 2, ... (32-bit little-endian j), each digest's
# four little-endian words giving two elements (w0 mod p) + u (w1 mod p) and
# (w2 mod p) + u (w3 mod p).
EXT_W = 7
FS_LABEL = b"zkp-matmul-sumcheck-fs-v1"


def e2(a, b=0):
    return (a % P, b % P)


def e2_add(x, y):
    return ((x[0] + y[0]) % P, (x[1] + y[1]) % P)


def e2_sub(x, y):
    return ((x[0] - y[0]) % P, (x[1] - y[1]) % P)


def e2_mul(x, y):
    return ((x[0] * y[0] + EXT_W * x[1] * y[1]) % P, (x[0] * y[1] + x[1] * y[0]) % P)


def e2_inv(x):
    n = (x[0] * x[0] - EXT_W * x[1] * x[1]) % P  # norm: x * conj(x)
    ni = pow(n, P - 2, P)
    return (x[0] * ni % P, (-x[1]) * ni % P)


def e2_pow(x, e: int):
    r = (1, 0)
    while e:
        if e & 1:
            r = e2_mul(r, x)
        x = e2_mul(x, x)
        e >>= 1
    return r


def e2_words(x) -> bytes:
    return int(x[0]).to_bytes(8, "little") + int(x[1]).to_bytes(8, "little")


class Transcript:
    def __init__(self, params: bytes, label: bytes = FS_LABEL):
        self.s = blake2b(label + params)

    def absorb(self, msg: bytes):
        self.s = blake2b(self.s + msg)

    def challenges(self, k: int) -> list:
        out, j = [], 0
        while len(out) < k:
            d = self.s if j == 0 else blake2b(self.s + j.to_bytes(4, "little"))
            w = [int.from_bytes(d[8 * i: 8 * i + 8], "little") for i in range(4)]
            out += [(w[0] % P, w[1] % P), (w[2] % P, w[3] % P)]
            j += 1
        return out[:k]


def layer_params(T: int, d_in: int, d_out: int, s: int) -> bytes:
    return b"".join(int(v).to_bytes(4, "little") for v in (T, d_in, d_out, s))


def eq_table_e2(r) -> list:
    """eq(r, k) over the extension, k < 2^len(r), bit j of k picking r_j."""
    E = [(1, 0)]
    for j, rj in enumerate(r):
        one_m = e2_sub((1, 0), rj)
        E = [e2_mul(e, one_m) for e in E] + [e2_mul(e, rj) for e in E]
    return E


def e2_split(E) -> tuple:
    return np.array([e[0] for e in E], np.uint64), np.array([e[1] for e in E], np.uint64)


def e2_join(a, b) -> list:
    return [(int(x), int(y)) for x, y in zip(a, b)]


def fold_rows_e2(M: np.ndarray, E, cols_pad: int) -> list:
    """sum_t E[t] M[t, :] with extension weights: the two base folds."""
    E0, E1 = e2_split(E)
    return e2_join(fold_rows(M, E0, cols_pad), fold_rows(M, E1, cols_pad))


def sumcheck_e2(A: list, B: list, tr: Transcript):
    """Sum-check of sum_k A[k] B[k] over the extension with the transcript:
    round i absorbs g_i(0), g_i(1), g_i(2) and takes r_i from the transcript,
    then binds the lowest remaining variable. Returns (rounds, r, finals)."""
    a, b = list(A), list(B)
    rounds, rs = [], []
    while len(a) > 1:
        h = len(a) // 2
        g = [(0, 0)] * 3
        for q in range(h):
            da, db = e2_sub(a[2 * q + 1], a[2 * q]), e2_sub(b[2 * q + 1], b[2 * q])
            ac, bc = a[2 * q], b[2 * q]
            for c in range(3):
                g[c] = e2_add(g[c], e2_mul(ac, bc))
                ac, bc = e2_add(ac, da), e2_add(bc, db)
        rounds.append(g)
        tr.absorb(b"".join(e2_words(x) for x in g))
        r = tr.challenges(1)[0]
        rs.append(r)
        a = [e2_add(a[2 * q], e2_mul(r, e2_sub(a[2 * q + 1], a[2 * q]))) for q in range(h)]
        b = [e2_add(b[2 * q], e2_mul(r, e2_sub(b[2 * q + 1], b[2 * q]))) for q in range(h)]
    return rounds, rs, (a[0], b[0])


def e2_eval_deg2(g, x):
    """The quadratic through (0, g0), (1, g1), (2, g2) at x (Lagrange)."""
    inv2 = (P + 1) // 2
    l0 = e2_mul(e2_mul(e2_sub(x, (1, 0)), e2_sub(x, (2, 0))), (inv2, 0))
    l1 = e2_mul(e2_mul(x, e2_sub(x, (2, 0))), (P - 1, 0))
    l2 = e2_mul(e2_mul(x, e2_sub(x, (1, 0))), (inv2, 0))
    return e2_add(e2_add(e2_mul(g[0], l0), e2_mul(g[1], l1)), e2_mul(g[2], l2))


def sumcheck_e2_multi(As: list, Bs: list, rho, tr: Transcript):
    """Sum-check of sum_j rho_j sum_k A_j[k] B_j[k] over the extension with the
    transcript (rho None: all ones): round i sends g_i(c) = sum_j rho_j
    sum_q A_j,c[q] B_j,c[q] for c = 0, 1, 2, absorbs them, takes r_i as the
    first challenge of the new state and binds every table; at the end the
    finals (A_j(r), B_j(r)) of all pairs are absorbed as one message.
    Returns (rounds, r, finals)."""
    a = [list(x) for x in As]
    b = [list(x) for x in Bs]
    rho = [(1, 0)] * len(a) if rho is None else [tuple(x) for x in rho]
    rounds, rs = [], []
    while len(a[0]) > 1:
        h = len(a[0]) // 2
        g = [(0, 0)] * 3
        for j in range(len(a)):
            gj = [(0, 0)] * 3
            for q in range(h):
                da, db = e2_sub(a[j][2 * q + 1], a[j][2 * q]), e2_sub(b[j][2 * q + 1], b[j][2 * q])
                ac, bc = a[j][2 * q], b[j][2 * q]
                for c in range(3):
                    gj[c] = e2_add(gj[c], e2_mul(ac, bc))
                    ac, bc = e2_add(ac, da), e2_add(bc, db)
            g = [e2_add(g[c], e2_mul(rho[j], gj[c])) for c in range(3)]
        rounds.append(g)
        tr.absorb(b"".join(e2_words(x) for x in g))
        r = tr.challenges(1)[0]
        rs.append(r)
        for j in range(len(a)):
            a[j] = [e2_add(a[j][2 * q], e2_mul(r, e2_sub(a[j][2 * q + 1], a[j][2 * q]))) for q in range(h)]
            b[j] = [e2_add(b[j][2 * q], e2_mul(r, e2_sub(b[j][2 * q + 1], b[j][2 * q]))) for q in range(h)]
    finals = [(a[j][0], b[j][0]) for j in range(len(a))]
    tr.absorb(b"".join(e2_words(x) + e2_words(y) for x, y in finals))
    return rounds, rs, finals


# ------------------------------ layer proof with the rescale committed --
# "How fast can FlashProve go", §2 (the prover commits intermediate values and
# sum-check reduces each matmul to claims about the committed tables and the
# weights, settled by openings; an opening sends a table's folded row, the
# eq-weighted sum of its rows, and opens a few columns; every challenge hashes
# all the prover has sent so far) and §3.1 (the rescaled value g_w and the
# remainder r are committed, never g^ itself, and the matmul's sum-check uses
# 2^k g_w + r in its place; the clamped value is committed too). Readings where
# the pages are silent:
#   - each map's Q (the rounded value before the clamp), R and Y are
#     [2^n_t, 2^n_o] tables of field elements (v < 0 as p + v), zero padded and
#     flattened with the output index in the low bits; rows hold 2^L elements,
#     L = min(18, min over maps of n_t + n_o); the tables follow each other in
#     the order Q_0, R_0, Y_0, Q_1, ..., each a run of whole rows; the rows are
#     Reed-Solomon encoded and the columns Merkle hashed exactly as in the
#     commitment above (one value per element here, no limb packing, so that a
#     claim about a table is a claim about the committed rows);
#   - the transcript starts from the label and the layer's shape (T, s, the
#     number of maps M, the mode, L, the number of opened columns, then every
#     map's d_in and d_out, as 32-bit little-endian words), absorbs the Merkle
#     root, and yields r_t, each map's r_o and a point r_prox of
#     log2ceil(rows) coordinates;
#   - the prover sends 2M + 1 folded rows: the proximity row (row i weighted by
#     eq(r_prox, i), every row of the commitment) and, per map, the rows of Q
#     and of R weighted by eq(z_hi, .), where z = (r_o || r_t) splits into its
#     first L coordinates z_lo and the rest z_hi; the transcript absorbs the
#     Merkle root (zero salts) of these rows laid out as 2(2M + 1) base rows,
#     each extension row as its 1 part then its u part;
#   - the verifier reads Q~(z) = sum_c eq(z_lo, c) u_Q[c] and R~(z) from the
#     rows, and the matmul's claim is c0 = 2^s Q~(z) + R~(z);
#   - batched mode: rho (M challenges) and one sum-check of
#     sum_m rho_m sum_k x'_m[k] w'_m[k] over 2^n, n the largest log2ceil(d_in),
#     against sum_m rho_m c0_m; separate mode: each map's own sum-check over
#     2^log2ceil(d_in) against c0_m, then rho and the combination
#     C = sum_m rho_m x'_m(r_m) w'_m(r_m);
#   - then 64 column indices, j = (challenge's first part) mod 2^(L+1); each
#     is opened with its salt, its column of the code and its Merkle path; the
#     verifier checks the path and that the codeword of every folded row at j
#     equals the same weighted sum of the column's entries;
#   - the finals x'_m(r) = X~(r || r_t) and w'_m(r) = W~(r || r_o) are claims
#     about the layer's input and weights, whose commitments are outside this
#     proof: the verifier evaluates them from X and W.
LAYER_LABEL = b"zkp-layer-committed-rescale-v1"
LAYER_LOG_ROW = 18
LAYER_OPEN_COLUMNS = 64
LAYER_REASONS = ("OK", "ROUND_SUM", "FINAL_CLAIM", "FINAL_OPENING", "COLUMN_PATH", "COLUMN_CODE", "STATE")


class LayerLayout:
    """Where each map's Q, R and Y rows sit in the commitment."""

    def __init__(self, T: int, d_outs):
        self.n_t = log2ceil(T)
        self.n_o = [log2ceil(d) for d in d_outs]
        self.L = min(LAYER_LOG_ROW, min(self.n_t + n for n in self.n_o))
        self.base, self.table_rows = [], []
        row = 0
        for n in self.n_o:
            k = 1 << (self.n_t + n - self.L)
            self.base.append((row, row + k, row + 2 * k))
            self.table_rows.append(k)
            row += 3 * k
        self.rows = row
        self.n_prox = log2ceil(row)


def layer_params_committed(T, s, maps_shape, batched, L, nq) -> bytes:
    words = [T, s, len(maps_shape), int(bool(batched)), L, nq]
    for d_in, d_out in maps_shape:
        words += [d_in, d_out]
    return b"".join(int(v).to_bytes(4, "little") for v in words)


def field_embed(v: np.ndarray) -> np.ndarray:
    """Signed integers as field elements (v < 0 as p + v)."""
    v = np.asarray(v, np.int64)
    w = v.astype(np.uint64)  # 2^64 + v for v < 0
    return np.where(v < 0, w - np.uint64((1 << 32) - 1), w)


def fold_field_rows(M: np.ndarray, E) -> np.ndarray:
    """sum_i E[i] M[i, :] for a field-valued [rows, cols] matrix."""
    M = np.ascontiguousarray(M, np.uint64)
    rows, cols = M.shape
    E = _u64(E)
    assert len(E) >= rows
    out = np.empty(cols, np.uint64)
    lib().or_fold_field_rows(_p(M), cols, rows, cols, _p(E), _p(out))
    return out


def dot(a, b) -> int:
    a, b = _u64(a), _u64(b)
    assert len(a) == len(b)
    return int(lib().or_dot(_p(a), _p(b), len(a)))


def e2_dot(u, E) -> tuple:
    """sum_c u[c] E[c] with u given as its parts (u0, u1) and E a list of e2."""
    E0, E1 = e2_split(E)
    a00, a11 = dot(u[0], E0), dot(u[1], E1)
    a01, a10 = dot(u[0], E1), dot(u[1], E0)
    return ((a00 + EXT_W * a11) % P, (a01 + a10) % P)


def e2_fold_rows(M: np.ndarray, E) -> np.ndarray:
    """Extension-weighted folded row of field rows: [2, cols] (1 part, u part)."""
    E0, E1 = e2_split(E)
    return np.stack([fold_field_rows(M, E0), fold_field_rows(M, E1)])


def layer_tables(Z: np.ndarray, s: int, n_t: int, n_o: int):
    """The committed Q, R, Y of one map: zero-padded [2^n_t, 2^n_o] field tables."""
    T, d_out = Z.shape
    out = []
    for v in rescale(Z, s):
        t = np.zeros((1 << n_t, 1 << n_o), np.int64)
        t[:T, :d_out] = v
        out.append(field_embed(t).reshape(-1))
    return out  # Q, R, Y


def _layer_points(lay: LayerLayout, ch):
    r_t = ch[:lay.n_t]
    off = lay.n_t
    r_o = []
    for n in lay.n_o:
        r_o.append(ch[off:off + n])
        off += n
    return r_t, r_o, ch[off:off + lay.n_prox]


def _row_weights(lay: LayerLayout, r_o, r_t, r_prox):
    """Row weights of the 2M + 1 folded rows (lists of e2 per commitment row,
    zeros outside a claim's table) and each claim's column point z_lo."""
    prox = eq_table_e2(r_prox)[:lay.rows]
    rows_w, z_lo = [prox], []
    zero = (0, 0)
    for m, n in enumerate(lay.n_o):
        z = list(r_o[m]) + list(r_t)
        z_lo.append(z[:lay.L])
        Eh = eq_table_e2(z[lay.L:])
        for which in (0, 1):  # Q, R
            w = [zero] * lay.rows
            b = lay.base[m][which]
            w[b:b + lay.table_rows[m]] = Eh
            rows_w.append(w)
    return rows_w, z_lo


def _merkle_root_rows(U: np.ndarray) -> bytes:
    """Merkle root (zero salts) over the columns of the folded rows U [K, 2, 2^L]."""
    K, _, n = U.shape
    return merkle_tree(U.reshape(2 * K, n), np.zeros((n, 16), np.uint8))[-1][0]


def prove_layer_committed(maps, s: int, batched: bool, salts: np.ndarray, tamper: str | None = None) -> dict:
    """The layer's proof with the rescale committed (steps and readings above).
    maps: list of (X, W), every X with the same T rows. tamper names a
    deliberate mistake of a cheating prover, for the verifier's negative
    controls: "Q" commits Q + 1 at one entry and proves honestly otherwise;
    "Q_rows" commits that Q but folds the true one; "prox_row" sends a wrong
    proximity row and proves consistently with it; "column" sends a wrong
    entry in the first opened column."""
    T = maps[0][0].shape[0]
    shapes = [(X.shape[1], W.shape[0]) for X, W in maps]
    lay = LayerLayout(T, [d for _, d in shapes])
    n_cols = 1 << lay.L
    msg = np.zeros((lay.rows, n_cols), np.uint64)
    true_msg = None
    out = {"layout": lay, "Z": [], "tables": []}
    for m, (X, W) in enumerate(maps):
        Z = witness(X, W, s)[0]
        Q, R, Y = layer_tables(Z, s, lay.n_t, lay.n_o[m])
        out["Z"].append(Z)
        out["tables"].append((Q, R, Y))
        for which, tab in enumerate((Q, R, Y)):
            b = lay.base[m][which]
            msg[b:b + lay.table_rows[m]] = tab.reshape(-1, n_cols)
    if tamper in ("Q", "Q_rows"):
        true_msg = msg.copy()
        msg[lay.base[0][0], 0] = (int(msg[lay.base[0][0], 0]) + 1) % P
    code = rs_encode(msg)
    assert salts.shape == (2 * n_cols, 16)
    levels = merkle_tree(code, salts)
    root = levels[-1][0]
    nq = LAYER_OPEN_COLUMNS
    tr = Transcript(layer_params_committed(T, s, shapes, batched, lay.L, nq), LAYER_LABEL)
    tr.absorb(root)
    ch = tr.challenges(lay.n_t + sum(lay.n_o) + lay.n_prox)
    r_t, r_o, r_prox = _layer_points(lay, ch)
    rows_w, z_lo = _row_weights(lay, r_o, r_t, r_prox)
    fold_src = true_msg if tamper == "Q_rows" else msg
    U = np.stack([e2_fold_rows(fold_src, w) for w in rows_w])  # [2M+1, 2, 2^L]
    if tamper == "prox_row":
        U[0, 0, 0] = (int(U[0, 0, 0]) + 1) % P
    tr.absorb(_merkle_root_rows(U))
    Et = eq_table_e2(r_t)
    xf, wf, c0 = [], [], []
    n_all = max(log2ceil(d) for d, _ in shapes)
    for m, (X, W) in enumerate(maps):
        n = n_all if batched else log2ceil(shapes[m][0])
        xf.append(fold_rows_e2(X, Et[:T], 1 << n))
        wf.append(fold_rows_e2(W, eq_table_e2(r_o[m])[:shapes[m][1]], 1 << n))
        Ez = eq_table_e2(z_lo[m])
        q, e = e2_dot(U[1 + 2 * m], Ez), e2_dot(U[2 + 2 * m], Ez)
        c0.append(e2_add(e2_mul((1 << s, 0), q), e))
    sumchecks = []
    if batched:
        rho = tr.challenges(len(maps))
        rounds, rs, finals = sumcheck_e2_multi(xf, wf, rho, tr)
        sumchecks.append({"rounds": rounds, "r": rs, "finals": finals})
        C = None
    else:
        for m in range(len(maps)):
            rounds, rs, finals = sumcheck_e2_multi([xf[m]], [wf[m]], None, tr)
            sumchecks.append({"rounds": rounds, "r": rs, "finals": finals})
        rho = tr.challenges(len(maps))
        C = (0, 0)
        for m, sc in enumerate(sumchecks):
            a, b = sc["finals"][0]
            C = e2_add(C, e2_mul(rho[m], e2_mul(a, b)))
    state = tr.s
    idx = [int(c[0]) % (2 * n_cols) for c in tr.challenges(nq)]
    columns = np.stack([code[:, j] for j in idx])
    if tamper == "column":
        columns[0, 0] = (int(columns[0, 0]) + 1) % P
    out.update(root=root, U=U, c0=c0, rho=rho, C=C, sumchecks=sumchecks, state=state, idx=idx, columns=columns,
               col_salts=np.stack([salts[j] for j in idx]), paths=[merkle_path(levels, j) for j in idx],
               r_t=r_t, r_o=r_o, r_prox=r_prox, x_fold=xf, w_fold=wf, msg=msg, code=code)
    return out


def verify_layer_committed(maps, s: int, batched: bool, proof: dict) -> str:
    """Checks a proof from prove_layer_committed without the witness: replays
    the transcript, reads the claims from the folded rows, checks every
    sum-check, the finals against X~ and W~ at the point, and every opened
    column against the root and the folded rows. Returns a name from
    LAYER_REASONS."""
    T = maps[0][0].shape[0]
    shapes = [(X.shape[1], W.shape[0]) for X, W in maps]
    lay = LayerLayout(T, [d for _, d in shapes])
    n_cols = 1 << lay.L
    nq = LAYER_OPEN_COLUMNS
    U = np.asarray(proof["U"], np.uint64)
    assert U.shape == (1 + 2 * len(maps), 2, n_cols)
    tr = Transcript(layer_params_committed(T, s, shapes, batched, lay.L, nq), LAYER_LABEL)
    tr.absorb(proof["root"])
    ch = tr.challenges(lay.n_t + sum(lay.n_o) + lay.n_prox)
    r_t, r_o, r_prox = _layer_points(lay, ch)
    rows_w, z_lo = _row_weights(lay, r_o, r_t, r_prox)
    tr.absorb(_merkle_root_rows(U))
    c0 = []
    for m in range(len(maps)):
        Ez = eq_table_e2(z_lo[m])
        q, e = e2_dot(U[1 + 2 * m], Ez), e2_dot(U[2 + 2 * m], Ez)
        c0.append(e2_add(e2_mul((1 << s, 0), q), e))

    def run(claim, sc, n_pairs, rho, n):
        rs = []
        if len(sc["rounds"]) != n:
            return "ROUND_SUM", None
        for g in sc["rounds"]:
            g = [tuple(int(v) for v in x) for x in g]
            if e2_add(g[0], g[1]) != claim:
                return "ROUND_SUM", None
            tr.absorb(b"".join(e2_words(x) for x in g))
            r = tr.challenges(1)[0]
            rs.append(r)
            claim = e2_eval_deg2(g, r)
        fin = [(tuple(int(v) for v in a), tuple(int(v) for v in b)) for a, b in sc["finals"]]
        if len(fin) != n_pairs:
            return "FINAL_CLAIM", None
        tot = (0, 0)
        for j, (a, b) in enumerate(fin):
            tot = e2_add(tot, e2_mul(rho[j] if rho else (1, 0), e2_mul(a, b)))
        if tot != claim:
            return "FINAL_CLAIM", None
        tr.absorb(b"".join(e2_words(a) + e2_words(b) for a, b in fin))
        return None, (rs, fin)

    Et = eq_table_e2(r_t)
    n_all = max(log2ceil(d) for d, _ in shapes)

    def opening(m, rs, a, b, n):
        X, W = maps[m]
        if len(rs) != n:
            return False
        Er = eq_table_e2(rs)
        xa = e2_dot(np.stack(e2_split(fold_rows_e2(X, Et[:T], 1 << n))), Er)
        wa = e2_dot(np.stack(e2_split(fold_rows_e2(W, eq_table_e2(r_o[m])[:shapes[m][1]], 1 << n))), Er)
        return (xa, wa) == (a, b)

    scs = proof["sumchecks"]
    if batched:
        rho = tr.challenges(len(maps))
        claim = (0, 0)
        for m in range(len(maps)):
            claim = e2_add(claim, e2_mul(rho[m], c0[m]))
        if len(scs) != 1:
            return "ROUND_SUM"
        why, res = run(claim, scs[0], len(maps), rho, n_all)
        if why:
            return why
        rs, fin = res
        for m in range(len(maps)):
            if not opening(m, rs, fin[m][0], fin[m][1], n_all):
                return "FINAL_OPENING"
    else:
        if len(scs) != len(maps):
            return "ROUND_SUM"
        for m in range(len(maps)):
            why, res = run(c0[m], scs[m], 1, None, log2ceil(shapes[m][0]))
            if why:
                return why
            rs, fin = res
            if not opening(m, rs, fin[0][0], fin[0][1], log2ceil(shapes[m][0])):
                return "FINAL_OPENING"
        tr.challenges(len(maps))  # rho: drawn from the state, nothing absorbed
    if proof.get("state") is not None and bytes(proof["state"]) != tr.s:
        return "STATE"
    idx = [int(c[0]) % (2 * n_cols) for c in tr.challenges(nq)]
    columns = np.asarray(proof["columns"], np.uint64)
    if columns.shape != (nq, lay.rows):
        return "COLUMN_PATH"
    for q, j in enumerate(idx):
        leaf = blake2b(bytes(np.asarray(proof["col_salts"][q], np.uint8)) + columns[q].astype("<u8").tobytes())
        if not merkle_verify(proof["root"], leaf, j, proof["paths"][q]):
            return "COLUMN_PATH"
        for k, w in enumerate(rows_w):
            got = (rs_eval(U[k, 0], j), rs_eval(U[k, 1], j))
            W0, W1 = e2_split(w)
            want = (dot(W0, columns[q]), dot(W1, columns[q]))
            if got != want:
                return "COLUMN_CODE"
    return "OK"
