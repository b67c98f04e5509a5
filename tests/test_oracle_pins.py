"""Pins for the CPU oracle: closed forms, worked cases, invariants and brute
force, chosen so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them. CPU only."""
import itertools
import os
import random

import numpy as np
import pytest

import oracle as O
import synth

P = O.P
HERE = os.path.dirname(os.path.abspath(__file__))


# ------------------------------------------------------------------ field --
def test_field_closed_forms():
    # 2^64 = 2^32 - 1 and 2^96 = -1 (mod p), so 2 has multiplicative order 192.
    assert O.power(2, 64) == 2**32 - 1
    assert O.power(2, 96) == P - 1
    assert O.power(2, 192) == 1
    assert O.mul(2, O.INV2) == 1
    assert O.INV2 == 0x7FFFFFFF80000001
    # p - 1 = 2^32 (2^32 - 1): Fermat and the 2-adic part of the group order.
    rng = random.Random(7)
    for _ in range(200):
        a = rng.randrange(1, P)
        assert O.power(a, P - 1) == 1
        assert O.power(a, (P - 1) // 2) in (1, P - 1)  # Euler's criterion
    # 7 generates the multiplicative group: 7^((p-1)/q) != 1 for each prime q | p-1
    for q in (2, 3, 5, 17, 257, 65537):
        assert (P - 1) % q == 0
        assert O.power(7, (P - 1) // q) != 1
    assert O.from_int(-1) == P - 1 and O.from_int(-128) == P - 128 and O.from_int(5) == 5


def test_field_against_bigint_and_ring_laws():
    rng = random.Random(11)
    edges = [0, 1, 2, P - 1, P - 2, 2**32, 2**32 - 1, 2**63, 2**63 - 1, P // 2, P // 2 + 1]
    vals = edges + [rng.randrange(P) for _ in range(3000)]
    for a in vals[:200]:
        for b in edges:
            assert O.add(a, b) == (a + b) % P
            assert O.sub(a, b) == (a - b) % P
            assert O.mul(a, b) == (a * b) % P
    for _ in range(3000):
        a, b, c = rng.choice(vals), rng.choice(vals), rng.choice(vals)
        assert O.mul(a, O.add(b, c)) == O.add(O.mul(a, b), O.mul(a, c))
        assert O.mul(O.mul(a, b), c) == O.mul(a, O.mul(b, c))
        assert O.add(O.sub(a, b), b) == a
        assert O.mul(a, b) == O.mul(b, a)


def test_eval_deg2_interpolates():
    rng = random.Random(3)
    for _ in range(300):
        c0, c1, c2 = rng.randrange(P), rng.randrange(P), rng.randrange(P)
        f = lambda x: (c0 + c1 * x + c2 * x * x) % P
        g0, g1, g2 = f(0), f(1), f(2)
        x = rng.randrange(P)
        assert O.eval_deg2(g0, g1, g2, x) == f(x)
        assert O.eval_deg2(g0, g1, g2, 0) == g0 and O.eval_deg2(g0, g1, g2, 2) == g2
        # degree <= 2 extrapolation at 3
        assert O.eval_deg2(g0, g1, g2, 3) == (g0 - 3 * g1 + 3 * g2) % P


# -------------------------------------------------------------- SplitMix64 --
def test_splitmix64_known_outputs():
    for line in open(os.path.join(HERE, "golden", "splitmix64.txt")):
        if line.startswith("#") or not line.strip():
            continue
        seed, idx, val = line.split()
        assert int(synth.raw(int(seed), 1, start=int(idx))[0]) == int(val, 16)


def test_challenge_stream_is_output_mod_p():
    x = synth.raw(1, 64)
    c = synth.challenges(1, 64)
    assert all(int(a) % P == int(b) for a, b in zip(x, c))
    assert int(c[0]) == 10451216379200822465


def test_generator_distributions():
    g = synth.matrix(123, (400000,), "gauss32").astype(np.float64)
    assert abs(g.mean()) < 0.5 and 30.5 < g.std() < 33.5
    lp = synth.matrix(124, (400000,), "laplace16").astype(np.float64)
    assert abs(lp.mean()) < 0.3 and abs(np.abs(lp).mean() - 16.0) < 0.6
    u = synth.matrix(125, (400000,), "uniform127")
    assert u.min() == -127 and u.max() == 127
    q = synth.matrix(126, (100000,), "int4")
    assert q.min() == -7 and q.max() == 7
    z = synth.zipf(127, 200000, 128, 1.1)
    cnt = np.bincount(z, minlength=128)
    ratio = cnt[0] / cnt[1]
    assert abs(ratio - 2 ** 1.1) < 0.1


# ---------------------------------------------------------------- witness --
def test_rescale_worked_cases():
    for line in open(os.path.join(HERE, "golden", "rescale_edges.txt")):
        if line.startswith("#") or not line.strip():
            continue
        s, Z, Q, R, Y = map(int, line.split())
        q, r, y = O.rescale(np.array([Z]), s)
        assert (int(q[0]), int(r[0]), int(y[0])) == (Q, R, Y)
        # the C witness on a 1x1 "matmul" producing Z where representable
        if abs(Z) <= 127 * 127:
            for a in range(1, 128):
                if Z % a == 0 and abs(Z // a) <= 127:
                    z, yy, rr = O.witness(np.array([[a]], np.int8), np.array([[Z // a]], np.int8), s)
                    assert (int(z[0, 0]), int(yy[0, 0]), int(rr[0, 0])) == (Z, Y, R)
                    break


def test_witness_against_numpy_matmul_and_rounding():
    rng = np.random.default_rng(1)
    for (T, d_in, d_out, s) in [(1, 1, 1, 8), (3, 17, 5, 7), (16, 256, 33, 8), (40, 300, 70, 1)]:
        X = rng.integers(-128, 128, size=(T, d_in), dtype=np.int8)
        W = rng.integers(-128, 128, size=(d_out, d_in), dtype=np.int8)
        Z, Y, R = O.witness(X, W, s)
        Zref = X.astype(np.int64) @ W.astype(np.int64).T
        assert np.array_equal(Z.astype(np.int64), Zref)
        # round-to-nearest property: |Z/2^s - Q| <= 1/2, ties up
        Q = (Z.astype(np.int64) - R) // (1 << s)
        assert np.array_equal(Q * (1 << s) + R, Zref)
        diff = Zref - Q * (1 << s)  # = R
        assert np.all(np.abs(2 * diff) <= (1 << s))
        tie = 2 * diff == -(1 << s)
        assert np.all(~(2 * diff == (1 << s)))  # a tie never rounds down
        assert np.all(Y == np.clip(Q, -128, 127))
        assert O.check_rescale(Z, Y, R, s) == ("OK", -1)
        _ = tie


def test_witness_entries_against_numpy_matmul():
    # the sampled-entry witness (the checker of every full-size Z sample) against
    # numpy's int64 matmul: rows and columns of different counts and lengths, so a
    # swapped (t, o) pair, a transposed operand or a dropped k term fails
    rng = np.random.default_rng(11)
    for (T, d_in, d_out) in [(1, 1, 1), (5, 3, 7), (33, 257, 19), (64, 4096, 48), (3, 14336, 5)]:
        X = rng.integers(-128, 128, size=(T, d_in), dtype=np.int8)
        W = rng.integers(-128, 128, size=(d_out, d_in), dtype=np.int8)
        Zref = X.astype(np.int64) @ W.astype(np.int64).T
        ts = np.concatenate([[0, T - 1], rng.integers(0, T, 200)]).astype(np.int32)
        os_ = np.concatenate([[d_out - 1, 0], rng.integers(0, d_out, 200)]).astype(np.int32)
        got = O.witness_entries(X, W, ts, os_)
        assert got.dtype == np.int64
        assert np.array_equal(got, Zref[ts, os_])
    # extremes: every product (-128)(-128), the largest |Z| the int32 witness allows
    X = np.full((2, 131071), -128, np.int8)
    W = np.full((3, 131071), -128, np.int8)
    assert list(O.witness_entries(X, W, [1, 0], [2, 1])) == [16384 * 131071] * 2
    # agrees with the full witness on a small case
    X = rng.integers(-128, 128, size=(9, 40), dtype=np.int8)
    W = rng.integers(-128, 128, size=(11, 40), dtype=np.int8)
    Z, _, _ = O.witness(X, W, 8)
    tt, oo = np.meshgrid(np.arange(9), np.arange(11), indexing="ij")
    assert np.array_equal(O.witness_entries(X, W, tt.ravel(), oo.ravel()), Z.astype(np.int64).ravel())


def test_witness_extremes_and_overflow():
    X = np.full((2, 4096), -128, np.int8)
    W = np.full((3, 4096), -128, np.int8)
    Z, Y, R = O.witness(X, W, 8)
    assert np.all(Z == 128 * 128 * 4096)
    X = np.full((1, 131073), -128, np.int8)
    W = np.full((1, 131073), -128, np.int8)
    with pytest.raises(OverflowError):
        O.witness(X, W, 8)


# --------------------------------------------------------------------- eq --
def _eq_doubling(r):
    """eq table by doubling (a second routine): E_{j+1}[k + b 2^j] = E_j[k] (b ? r_j : 1 - r_j)."""
    E = [1]
    for rj in r:
        E = [e * ((1 - rj) % P) % P for e in E] + [e * rj % P for e in E]
    return E


def test_eq_identities():
    rng = random.Random(5)
    assert list(O.eq_table([])) == [1]
    for n in range(0, 9):
        r = [rng.randrange(P) for _ in range(n)]
        E = O.eq_table(r)
        assert sum(int(e) for e in E) % P == 1
        assert [int(e) for e in E] == _eq_doubling(r)
        # Boolean point -> one-hot at sum_j r_j 2^j
        bits = [rng.randrange(2) for _ in range(n)]
        Eb = O.eq_table(bits)
        idx = sum(b << j for j, b in enumerate(bits))
        assert [int(e) for e in Eb] == [1 if k == idx else 0 for k in range(1 << n)]
        if n:
            k = rng.randrange(1 << n)
            assert O.eq_at(r, k) == int(E[k])


# ------------------------------------------------------------------ folds --
def test_fold_boolean_point_selects_row_and_linearity():
    rng = np.random.default_rng(2)
    M = rng.integers(-128, 128, size=(13, 37), dtype=np.int8)
    for t in range(13):
        bits = [(t >> j) & 1 for j in range(4)]
        f = O.fold_rows(M, O.eq_table(bits), 64)
        assert [int(v) for v in f[:37]] == [O.from_int(int(v)) for v in M[t]]
        assert np.all(f[37:] == 0)
    r = [int(v) for v in synth.challenges(99, 4)]
    E = O.eq_table(r)
    A = rng.integers(-2**30, 2**30, size=(13, 37), dtype=np.int32)
    B = rng.integers(-2**30, 2**30, size=(13, 37), dtype=np.int32)
    fa, fb, fab = O.fold_rows(A, E), O.fold_rows(B, E), O.fold_rows((A.astype(np.int64) + B).astype(np.int32), E)
    assert all(O.add(int(x), int(y)) == int(z) for x, y, z in zip(fa, fb, fab))
    # definition by hand on one column, with Python integers
    k = 5
    want = sum(int(E[t]) * (int(A[t, k]) % P) for t in range(13)) % P
    assert int(fa[k]) == want
    # rows past `rows` are ignored: a 13-row fold equals a 16-row fold with zero rows
    Apad = np.zeros((16, 37), np.int32)
    Apad[:13] = A
    assert np.array_equal(O.fold_rows(Apad, E), fa)
    assert np.array_equal(O.fold_cols(A, E, [0, 5, 36]), fa[[0, 5, 36]])


def test_request_vectors_open_the_weight_table():
    # A request vector is the weight table's folded row at the request's point
    # r_o: its MLE over the columns at r_k is W~(r_k || r_o) (the opening the
    # batch shares), and at a Boolean r_o it is that row of W itself.
    rng = np.random.default_rng(11)
    W = rng.integers(-128, 128, size=(6, 5), dtype=np.int8)
    pts = [[int(v) for v in synth.challenges(40 + j, 3)] for j in range(3)]
    Es = [O.eq_table(r) for r in pts] + [O.eq_table([1, 0, 1])]
    V = O.request_vectors(W, Es, 8)
    assert V.shape == (4, 8) and np.all(V[:, 5:] == 0)
    r_k = [int(v) for v in synth.challenges(50, 3)]
    for j, r in enumerate(pts):
        assert O.mle_seq(V[j], r_k) == O.mle_matrix(W, r, r_k)
    assert [int(v) for v in V[3, :5]] == [O.from_int(int(v)) for v in W[5]]
    # Freivalds' view of the same projection: <v_j, x> = <E_j, W x> for any x
    x = [int(v) for v in synth.challenges(51, 5)]
    Wx = [sum(O.from_int(int(W[t, k])) * x[k] for k in range(5)) % P for t in range(6)]
    for j in range(3):
        lhs = sum(int(V[j, k]) * x[k] for k in range(5)) % P
        assert lhs == sum(int(Es[j][t]) * Wx[t] for t in range(6)) % P
    assert O.request_vectors(W, [], 8).shape == (0, 8)


def test_mle_two_routes_and_boolean_points():
    rng = random.Random(8)
    for n in range(0, 9):
        A = [rng.randrange(P) for _ in range(1 << n)]
        z = [rng.randrange(P) for _ in range(n)]
        assert O.mle_brute(A, z) == O.mle_seq(A, z)
        k = rng.randrange(1 << n)
        zb = [(k >> j) & 1 for j in range(n)]
        assert O.mle_brute(A, zb) == A[k] == O.mle_seq(A, zb)
    # multilinearity in the first variable: A~(x, ...) is affine in x
    n = 5
    A = [rng.randrange(P) for _ in range(1 << n)]
    z = [rng.randrange(P) for _ in range(n)]
    f = lambda x: O.mle_seq(A, [x] + z[1:])
    assert (f(0) + 2 * (f(1) - f(0))) % P == f(2)


def test_mle_matrix_layout_and_boolean_points():
    rng = np.random.default_rng(3)
    Z = rng.integers(-2**31, 2**31, size=(5, 6), dtype=np.int32)
    r_rows = [int(v) for v in synth.challenges(5, 3)]
    r_cols = [int(v) for v in synth.challenges(6, 3)]
    # flatten with the column in the low bits, zero-padded to [8, 8]
    flat = np.zeros(64, np.uint64)
    for t in range(5):
        for o in range(6):
            flat[t * 8 + o] = O.from_int(int(Z[t, o]))
    assert O.mle_matrix(Z, r_rows, r_cols) == O.mle_brute(flat, r_cols + r_rows)
    # a transposed operand gives a different value
    assert O.mle_matrix(Z, r_rows, r_cols) != O.mle_brute(flat, r_rows + r_cols)
    for t, o in [(0, 0), (4, 5), (2, 3)]:
        rb = [(t >> j) & 1 for j in range(3)]
        cb = [(o >> j) & 1 for j in range(3)]
        assert O.mle_matrix(Z, rb, cb) == O.from_int(int(Z[t, o]))


# -------------------------------------------------------------- sum-check --
def _brute_round_values(A, B, r, i, n):
    """g_i(c) by enumerating the hypercube: sum over b in {0,1}^(n-i-1) of
    A~(r_0..r_{i-1}, c, b) B~(r_0..r_{i-1}, c, b), evaluated from the
    multilinear extensions by definition."""
    out = []
    for c in (0, 1, 2):
        tot = 0
        for b in itertools.product((0, 1), repeat=n - i - 1):
            pt = list(r[:i]) + [c] + list(b)
            tot = (tot + O.mle_brute(A, pt) * O.mle_brute(B, pt)) % P
        out.append(tot)
    return out


@pytest.mark.parametrize("n", [0, 1, 2, 3, 4])
def test_sumcheck_against_hypercube_enumeration(n):
    rng = random.Random(100 + n)
    A = [rng.randrange(P) for _ in range(1 << n)]
    B = [rng.randrange(P) for _ in range(1 << n)]
    r = [rng.randrange(P) for _ in range(n)]
    rounds, finals, c0 = O.sumcheck([A], [B], r)
    assert c0 == sum(a * b for a, b in zip(A, B)) % P
    for i in range(n):
        assert [int(v) for v in rounds[i]] == _brute_round_values(A, B, r, i, n)
    assert int(finals[0, 0]) == O.mle_brute(A, r) and int(finals[0, 1]) == O.mle_brute(B, r)
    assert O.check_sumcheck(rounds, finals, r, c0, As=[A], Bs=[B])[0] == "OK"


def test_sumcheck_batched_is_rho_combination():
    rng = random.Random(21)
    n, k = 5, 3
    As = [[rng.randrange(P) for _ in range(1 << n)] for _ in range(k)]
    Bs = [[rng.randrange(P) for _ in range(1 << n)] for _ in range(k)]
    r = [rng.randrange(P) for _ in range(n)]
    rho = [rng.randrange(P) for _ in range(k)]
    rounds, finals, c0 = O.sumcheck(As, Bs, r, rho=rho)
    single = [O.sumcheck([a], [b], r) for a, b in zip(As, Bs)]
    assert c0 == sum(rj * s[2] for rj, s in zip(rho, single)) % P
    for i in range(n):
        for c in range(3):
            assert int(rounds[i, c]) == sum(rj * int(s[0][i, c]) for rj, s in zip(rho, single)) % P
    assert O.check_sumcheck(rounds, finals, r, c0, rho=rho, As=As, Bs=Bs)[0] == "OK"


def test_sumcheck_boolean_challenges_reduce_to_dot_product():
    rng = np.random.default_rng(4)
    X = rng.integers(-127, 128, size=(8, 16), dtype=np.int8)
    W = rng.integers(-127, 128, size=(4, 16), dtype=np.int8)
    t, o = 5, 2
    r_t = [(t >> j) & 1 for j in range(3)]
    r_o = [(o >> j) & 1 for j in range(2)]
    res = O.prove_matmul(X, W, 8, r_t, r_o, [int(v) for v in synth.challenges(9, 4)])
    textbook = int(np.dot(X[t].astype(np.int64), W[o].astype(np.int64)))
    assert res["c0"] == O.from_int(textbook) == res["claim0"]


# ------------------------------------------------------- negative controls --
def _proof(n=6, seed=31):
    rng = random.Random(seed)
    A = [rng.randrange(P) for _ in range(1 << n)]
    B = [rng.randrange(P) for _ in range(1 << n)]
    r = [rng.randrange(P) for _ in range(n)]
    rounds, finals, c0 = O.sumcheck([A], [B], r)
    return A, B, r, rounds, finals, c0


def test_negative_controls_sumcheck():
    A, B, r, rounds, finals, c0 = _proof()
    assert O.check_sumcheck(rounds, finals, r, c0, As=[A], Bs=[B])[0] == "OK"
    assert O.check_sumcheck(rounds, finals, r, (c0 + 1) % P)[0] == "INITIAL_CLAIM"
    for i in range(len(r)):
        for c in range(3):
            bad = rounds.copy()
            bad[i, c] = (int(bad[i, c]) + 1) % P
            reason, where = O.check_sumcheck(bad, finals, r, c0)
            if c < 2:
                assert (reason, where) == (("INITIAL_CLAIM", 0) if i == 0 else ("ROUND_SUM", i))
            else:  # g_i(2) only enters through g_i(r_i)
                assert (reason, where) == (("ROUND_SUM", i + 1) if i + 1 < len(r) else ("FINAL_CLAIM", len(r)))
    bad = finals.copy()
    bad[0, 1] = (int(bad[0, 1]) + 1) % P
    assert O.check_sumcheck(rounds, bad, r, c0)[0] == "FINAL_CLAIM"
    # a tampered table: finals no longer open to the committed table's MLE
    A2 = list(A)
    A2[3] = (A2[3] + 1) % P
    assert O.check_sumcheck(rounds, finals, r, c0, As=[A2], Bs=[B])[0] == "FINAL_OPENING"
    # a challenge the prover did not use
    r2 = list(r)
    r2[2] = (r2[2] + 1) % P
    assert O.check_sumcheck(rounds, finals, r2, c0)[0] in ("ROUND_SUM", "FINAL_CLAIM")
    # MSB-first binding gives a transcript this verifier rejects
    n = len(r)
    perm = lambda T: [T[int(format(k, "0%db" % n)[::-1], 2)] for k in range(1 << n)]
    rr, ff, cc = O.sumcheck([perm(A)], [perm(B)], r)
    assert cc == c0
    assert O.check_sumcheck(rr, ff, r, c0, As=[A], Bs=[B])[0] == "FINAL_OPENING"


def test_negative_controls_witness():
    rng = np.random.default_rng(6)
    X = rng.integers(-127, 128, size=(9, 40), dtype=np.int8)
    W = rng.integers(-127, 128, size=(11, 40), dtype=np.int8)
    Z, Y, R = O.witness(X, W, 8)
    assert O.check_witness(X, W, Z) == ("OK", -1)
    Z2 = Z.copy()
    Z2[4, 7] += 1
    assert O.check_witness(X, W, Z2) == ("WITNESS_MISMATCH", 4 * 11 + 7)
    assert O.check_rescale(Z2, Y, R, 8)[0] == "RESCALE_IDENTITY"
    R2 = R.copy()
    R2[1, 1] ^= 1
    assert O.check_rescale(Z, Y, R2, 8) == ("RESCALE_IDENTITY", 1 * 11 + 1)
    Y2 = Y.copy()
    Y2[0, 0] = Y2[0, 0] + 1 if Y2[0, 0] < 127 else 126
    assert O.check_rescale(Z, Y2, R, 8) == ("RESCALE_IDENTITY", 0)
    # the wrong shift: Y and R of s = 8 fail the s = 7 identity somewhere
    assert O.check_rescale(Z, Y, R, 7)[0] == "RESCALE_IDENTITY"
    # the claim follows Z: one changed entry changes Z~ at a random point
    r_t = [int(v) for v in synth.challenges(1, 4)]
    r_o = [int(v) for v in synth.challenges(2, 4)]
    assert O.mle_matrix(Z, r_t, r_o) != O.mle_matrix(Z2, r_t, r_o)


# ------------------------------------------------------------- commitment --
def test_pack_limbs_worked_example_and_unpacking():
    A = np.array([1, -1, 127, -128], np.int8)
    B = np.array([5], np.int8)
    msg = O.pack_limbs(A, B, 2)  # rows of 4 elements
    # limbs 1, 255, 127 | 128, 5 (then zeros), 20-bit slots
    assert msg.shape == (1, 4)
    assert [int(v) for v in msg[0]] == [1 + 255 * 2**20 + 127 * 2**40, 128 + 5 * 2**20, 0, 0]
    rng = np.random.default_rng(1)
    A = rng.integers(-128, 128, 1000).astype(np.int8)
    B = rng.integers(-128, 128, 777).astype(np.int8)
    msg = O.pack_limbs(A, B, 6)
    assert msg.shape == (10, 64)  # ceil(ceil(1777 / 3) / 64) rows
    limbs = [(int(v) >> (20 * q)) & 0xFFFFF for v in msg.reshape(-1) for q in range(3)]
    want = [int(x) & 0xFF for x in np.concatenate([A, B])]
    assert limbs[:len(want)] == want and not any(limbs[len(want):])
    assert all(int(v) < 2**60 for v in msg.reshape(-1))  # three slots fit below p


def test_roots_of_unity():
    for k in (1, 2, 5, 12, 23, 32):
        w = O.root_of_unity(k)
        assert O.power(w, 2**k) == 1 and O.power(w, 2**(k - 1)) == P - 1
    # 2 has order 192, so the primitive 64th roots are the powers 2^(3u), u odd;
    # the one this generator gives is 2^39 (small-radix twiddles become shifts)
    assert O.root_of_unity(6) == pow(2, 39, P)
    assert O.power(O.root_of_unity(23), 2**17) == O.root_of_unity(6)


def test_rs_encode_is_the_polynomial_on_the_subgroup():
    rng = random.Random(21)
    for logn in range(0, 6):
        n = 1 << logn
        msg = np.array([[rng.randrange(P) for _ in range(n)] for _ in range(2)], np.uint64)
        msg[0, 0] = P - 1
        code = O.rs_encode(msg)
        w = O.root_of_unity(logn + 1)
        for i in range(2):
            want = [sum(int(msg[i, k]) * pow(w, j * k, P) for k in range(n)) % P for j in range(2 * n)]
            assert [int(v) for v in code[i]] == want
    # larger rows: entries by Horner's rule at sampled points
    logn = 12
    n = 1 << logn
    msg = np.array([[rng.randrange(P) for _ in range(n)]], np.uint64)
    code = O.rs_encode(msg)
    for j in [0, 1, 2, 777, 4096, 8191]:
        assert int(code[0, j]) == O.rs_eval(msg[0], j)
    # folding: with P = Lo + x^(n/2) Hi, at the n-th roots x^(n/2) = (-1)^j, so
    # code[4j] and code[4j + 2] come from the half-length rows Lo + Hi and Lo - Hi
    lo, hi = msg[0, : n // 2].astype(object), msg[0, n // 2:].astype(object)
    plus = np.array([[(a + b) % P for a, b in zip(lo, hi)]], np.uint64)
    minus = np.array([[(a - b) % P for a, b in zip(lo, hi)]], np.uint64)
    cp, cm = O.rs_encode(plus)[0], O.rs_encode(minus)[0]
    assert np.array_equal(code[0, 0::4], cp[0::2]) and np.array_equal(code[0, 2::4], cm[1::2])
    # a constant row gives a constant codeword; the row (0, 1, 0, ...) gives w^j
    c = O.rs_encode(np.array([[9] + [0] * 7], np.uint64))
    assert np.all(c == 9)
    x = O.rs_encode(np.array([[0, 1] + [0] * 6], np.uint64))
    w = O.root_of_unity(4)
    assert [int(v) for v in x[0]] == [pow(w, j, P) for j in range(16)]


def test_rs_encode_convolution_theorem():
    # codewords multiply pointwise: the product of two rows' polynomials
    # (schoolbook, degree < 2n - 1) evaluated on the same 2n points
    rng = random.Random(22)
    n = 32
    a = [rng.randrange(P) for _ in range(n)]
    b = [rng.randrange(P) for _ in range(n)]
    c = [0] * (2 * n)
    for i in range(n):
        for j in range(n):
            c[i + j] = (c[i + j] + a[i] * b[j]) % P
    ca, cb = O.rs_encode(np.array([a, b], np.uint64))
    cc = O.rs_encode(np.array([c], np.uint64))[0]  # evaluations on 4n points
    assert all(int(x) * int(y) % P == int(z) for x, y, z in zip(ca, cb, cc[::2]))


def test_blake2b_published_vector():
    import hashlib
    for line in open(os.path.join(HERE, "golden", "blake2b.txt")):
        if line.startswith("#") or not line.strip():
            continue
        msg, nbytes, hexd = line.split()
        assert hashlib.blake2b(msg.encode(), digest_size=int(nbytes)).hexdigest() == hexd


def test_merkle_tree_by_hand_and_paths():
    import hashlib
    rng = np.random.default_rng(23)
    code = rng.integers(0, 2**63, size=(3, 2), dtype=np.uint64)
    salts = rng.integers(0, 256, size=(2, O.SALT_BYTES), dtype=np.uint8)
    lv = O.merkle_tree(code, salts)
    leaf = [hashlib.blake2b(bytes(salts[j]) + b"".join(int(code[i, j]).to_bytes(8, "little") for i in range(3)),
                            digest_size=32).digest() for j in range(2)]
    assert lv[0] == leaf and lv[1] == [hashlib.blake2b(leaf[0] + leaf[1], digest_size=32).digest()]
    code = rng.integers(0, 2**63, size=(2, 16), dtype=np.uint64)
    salts = rng.integers(0, 256, size=(16, O.SALT_BYTES), dtype=np.uint8)
    lv = O.merkle_tree(code, salts)
    assert [len(x) for x in lv] == [16, 8, 4, 2, 1]
    root = lv[-1][0]
    for j in range(16):
        assert O.merkle_verify(root, lv[0][j], j, O.merkle_path(lv, j))
        assert not O.merkle_verify(root, lv[0][j], j ^ 1, O.merkle_path(lv, j))
    code2 = code.copy()
    code2[1, 5] ^= np.uint64(1)
    lv2 = O.merkle_tree(code2, salts)
    assert lv2[0][5] != lv[0][5] and lv2[-1][0] != root and lv2[0][4] == lv[0][4]


# ----------------------------------------------------------------- lookup --
def test_product_tree_by_hand():
    keys = np.array([3, -1, 0], np.int8)
    g = 1000
    lev = O.product_tree(keys, 2, g)
    leaves = [g - 3, g + 1, g, g]  # padded with the key 0
    assert [int(v) for v in lev[0]] == leaves
    assert [int(v) for v in lev[1]] == [leaves[0] * leaves[1] % P, leaves[2] * leaves[3] % P]
    assert int(lev[2][0]) == (g - 3) * (g + 1) * g * g % P


def test_eval_deg3_interpolates_a_cubic():
    f = lambda x: (5 * x**3 + 7 * x**2 + (P - 2) * x + 11) % P
    g = [f(x) for x in range(4)]
    for x in (4, 9, P - 1, 123456789):
        assert O.eval_deg3(g, x) == f(x)


def _brute_round_values3(E, A, B, r, i, m):
    """g_i(c), c = 0..3, by enumerating the hypercube over the multilinear
    extensions of E, A and B by definition."""
    out = []
    for c in range(4):
        tot = 0
        for b in itertools.product((0, 1), repeat=m - i - 1):
            pt = list(r[:i]) + [c] + list(b)
            tot = (tot + O.mle_brute(E, pt) * O.mle_brute(A, pt) * O.mle_brute(B, pt)) % P
        out.append(tot)
    return out


@pytest.mark.parametrize("m", [0, 1, 2, 3, 4])
def test_sumcheck3_against_hypercube_enumeration(m):
    rng = random.Random(300 + m)
    E = [rng.randrange(P) for _ in range(1 << m)]
    V = [rng.randrange(P) for _ in range(2 << m)]
    A, B = V[0::2], V[1::2]
    r = [rng.randrange(P) for _ in range(m)]
    rounds, finals = O.sumcheck3(E, V, r)
    total = sum(e * a * b for e, a, b in zip(E, A, B)) % P
    if m:
        assert (int(rounds[0][0]) + int(rounds[0][1])) % P == total
    for i in range(m):
        assert [int(v) for v in rounds[i]] == _brute_round_values3(E, A, B, r, i, m)
    assert finals == [O.mle_brute(E, r), O.mle_brute(A, r), O.mle_brute(B, r)]


def test_lookup_proof_verifies_and_negative_controls():
    L, s = 6, 4
    rng = np.random.default_rng(31)
    keys = rng.integers(-8, 8, 50).astype(np.int8)
    keys[:2] = [-8, 7]
    gamma = int(synth.challenges(77, 1)[0])
    chal = synth.challenges(78, O.lookup_challenges_len(L))
    lev = O.product_tree(keys, L, gamma)
    root = int(lev[-1][0])
    counts, outside = O.lookup_counts(keys, L, s)
    assert outside == 0 and counts.sum() == 1 << L and counts[8] >= (1 << L) - 50
    # the two products agree exactly when every key is a table row
    assert O.table_product(counts, s, gamma) == root
    proof = O.grand_product_prove(lev, chal)
    assert len(proof) == L and [len(r) for r, _ in proof] == list(range(L))
    assert O.grand_product_verify(root, proof, chal, L, keys, gamma, counts, s) == (0, -1)
    # a changed round value, a changed final, a different key, a key off the table
    bad = [(r.copy(), list(f)) for r, f in proof]
    bad[3][0][1, 2] = (int(bad[3][0][1, 2]) + 1) % P
    assert O.grand_product_verify(root, bad, chal, L, keys, gamma)[0] == 2
    bad = [(r.copy(), list(f)) for r, f in proof]
    bad[2][0][0, 0] = (int(bad[2][0][0, 0]) + 1) % P
    assert O.grand_product_verify(root, bad, chal, L, keys, gamma)[0] == 1
    bad = [(r.copy(), list(f)) for r, f in proof]
    bad[4][1][1] = (bad[4][1][1] + 1) % P
    assert O.grand_product_verify(root, bad, chal, L, keys, gamma)[0] == 3
    k2 = keys.copy()
    k2[10] ^= 1
    assert O.grand_product_verify(root, proof, chal, L, k2, gamma)[0] == 4
    k3 = keys.copy()
    k3[5] = 100  # outside [-8, 8)
    lev3 = O.product_tree(k3, L, gamma)
    c3, out3 = O.lookup_counts(k3, L, s)
    assert out3 == 1
    p3 = O.grand_product_prove(lev3, chal)
    assert O.grand_product_verify(int(lev3[-1][0]), p3, chal, L, k3, gamma, c3, s) == (5, L)


# ------------------------------------------- soundness-faithful challenges --
def test_extension_field():
    # 7 is not a square mod p (Euler's criterion), so F_p[u]/(u^2 - 7) is a field
    assert pow(7, (P - 1) // 2, P) == P - 1
    rng = random.Random(41)
    u = (0, 1)
    assert O.e2_mul(u, u) == (7, 0)
    for _ in range(50):
        a, b, c = [(rng.randrange(P), rng.randrange(P)) for _ in range(3)]
        assert O.e2_mul(O.e2_mul(a, b), c) == O.e2_mul(a, O.e2_mul(b, c))
        assert O.e2_mul(a, O.e2_add(b, c)) == O.e2_add(O.e2_mul(a, b), O.e2_mul(a, c))
        assert O.e2_mul(a, O.e2_inv(a)) == (1, 0)
    # Frobenius: a^p is the conjugate, since u^p = u 7^((p-1)/2) = -u
    a = (rng.randrange(P), rng.randrange(P))
    assert O.e2_pow(a, P) == (a[0], (P - a[1]) % P)
    # the multiplicative group has order p^2 - 1
    assert O.e2_pow(a, P * P - 1) == (1, 0)


def test_transcript_derivation_and_sensitivity():
    import hashlib
    h = lambda b: hashlib.blake2b(b, digest_size=32).digest()
    tr = O.Transcript(b"params")
    s0 = h(O.FS_LABEL + b"params")
    assert tr.s == s0
    tr.absorb(b"root")
    s1 = h(s0 + b"root")
    assert tr.s == s1
    ch = tr.challenges(3)
    w = [int.from_bytes(s1[8 * i: 8 * i + 8], "little") for i in range(4)]
    assert ch[0] == (w[0] % P, w[1] % P) and ch[1] == (w[2] % P, w[3] % P)
    d1 = h(s1 + (1).to_bytes(4, "little"))
    assert ch[2] == (int.from_bytes(d1[:8], "little") % P, int.from_bytes(d1[8:16], "little") % P)
    # another label starts another transcript
    assert O.Transcript(b"params", O.LAYER_LABEL).s == h(O.LAYER_LABEL + b"params") != s0
    # any change to an absorbed byte changes every later challenge
    tr2 = O.Transcript(b"params")
    tr2.absorb(b"rooT")
    assert all(a != b for a, b in zip(tr2.challenges(3), ch))


def _mle_e2(A, pt):
    E = O.eq_table_e2(pt)
    acc = (0, 0)
    for e, a in zip(E, A):
        acc = O.e2_add(acc, O.e2_mul(e, a))
    return acc


def test_sumcheck_e2_against_hypercube_enumeration():
    rng = random.Random(42)
    n = 3
    A = [(rng.randrange(P), rng.randrange(P)) for _ in range(1 << n)]
    B = [(rng.randrange(P), rng.randrange(P)) for _ in range(1 << n)]
    rounds, rs, finals = O.sumcheck_e2(A, B, O.Transcript(b"t"))
    total = (0, 0)
    for a, b in zip(A, B):
        total = O.e2_add(total, O.e2_mul(a, b))
    assert O.e2_add(rounds[0][0], rounds[0][1]) == total
    for i in range(n):
        for c in range(3):
            tot = (0, 0)
            for bits in itertools.product((0, 1), repeat=n - i - 1):
                pt = list(rs[:i]) + [(c, 0)] + [(x, 0) for x in bits]
                tot = O.e2_add(tot, O.e2_mul(_mle_e2(A, pt), _mle_e2(B, pt)))
            assert rounds[i][c] == tot
    assert finals == (_mle_e2(A, rs), _mle_e2(B, rs))


def test_sumcheck_e2_multi_one_pair_and_rho_weights():
    rng = random.Random(43)
    n = 3
    rnd = lambda: [(rng.randrange(P), rng.randrange(P)) for _ in range(1 << n)]
    A, B = rnd(), rnd()
    # one pair without weights: sumcheck_e2's rounds, then the finals absorbed
    t1, t2 = O.Transcript(b"x"), O.Transcript(b"x")
    r1, s1, f1 = O.sumcheck_e2(A, B, t1)
    t1.absorb(O.e2_words(f1[0]) + O.e2_words(f1[1]))
    r2, s2, f2 = O.sumcheck_e2_multi([A], [B], None, t2)
    assert (r1, s1, [f1]) == (r2, s2, f2) and t1.s == t2.s
    # three pairs: every round is the rho combination of the pairs' own round
    # values at the shared challenges (by enumeration), the finals the MLEs at r
    As, Bs = [rnd() for _ in range(3)], [rnd() for _ in range(3)]
    rho = [(rng.randrange(P), rng.randrange(P)) for _ in range(3)]
    rounds, rs, finals = O.sumcheck_e2_multi(As, Bs, rho, O.Transcript(b"y"))
    for i in range(n):
        for c in range(3):
            tot = (0, 0)
            for j in range(3):
                for bits in itertools.product((0, 1), repeat=n - i - 1):
                    pt = list(rs[:i]) + [(c, 0)] + [(x, 0) for x in bits]
                    tot = O.e2_add(tot, O.e2_mul(rho[j], O.e2_mul(_mle_e2(As[j], pt), _mle_e2(Bs[j], pt))))
            assert rounds[i][c] == tot
    assert finals == [(_mle_e2(As[j], rs), _mle_e2(Bs[j], rs)) for j in range(3)]


def test_field_embed_and_field_fold():
    v = np.array([0, 1, -1, 127, -128, (1 << 31) - 1, -(1 << 31)], np.int64)
    assert [int(x) for x in O.field_embed(v)] == [int(x) % P for x in v]
    rng = np.random.default_rng(44)
    M = rng.integers(0, P, size=(5, 7), dtype=np.uint64)
    E = [int(x) for x in rng.integers(0, P, size=5, dtype=np.uint64)]
    got = O.fold_field_rows(M, E)
    assert [int(x) for x in got] == [sum(E[i] * int(M[i, c]) for i in range(5)) % P for c in range(7)]
    assert O.dot(M[0], M[1]) == sum(int(a) * int(b) for a, b in zip(M[0], M[1])) % P


def test_layer_layout_of_the_seven_map_layer():
    # T = 4096; outputs of Q, K, V, O, gate, up, down (14336 pads to 2^14)
    lay = O.LayerLayout(4096, [4096, 1024, 1024, 4096, 14336, 14336, 4096])
    assert lay.L == 18 and lay.n_t == 12
    assert lay.table_rows == [64, 16, 16, 64, 256, 256, 64]
    assert lay.rows == 3 * 736 and lay.n_prox == 12
    assert lay.base[1] == (192, 208, 224) and lay.base[6][2] == lay.rows - 64
    # a small layer: rows as short as the smallest table
    lay = O.LayerLayout(24, [48, 20, 40])
    assert (lay.L, lay.rows) == (5 + 5, 3 * (2 + 1 + 2)) and lay.base[1] == (6, 7, 8)


def _small_layer(seed=45):
    rng = np.random.default_rng(seed)
    r8 = lambda *sh: rng.integers(-127, 128, size=sh).astype(np.int8)
    T = 24
    X, H = r8(T, 40), r8(T, 72)
    maps = [(X, r8(48, 40)), (X, r8(20, 40)), (H, r8(40, 72))]
    lay = O.LayerLayout(T, [48, 20, 40])
    salts = rng.integers(0, 256, size=(2 << lay.L, 16), dtype=np.uint8)
    return maps, salts


@pytest.mark.parametrize("batched", [True, False])
def test_layer_committed_claims_by_enumeration(batched):
    """The claims read from the folded rows are the witness's MLE at (r_o || r_t)
    (summed over every (t, o) with extension eq weights, independently of the
    layout), and each folded row is the weighted sum of its rows."""
    maps, salts = _small_layer()
    s = 7
    pr = O.prove_layer_committed(maps, s, batched, salts)
    lay = pr["layout"]
    for m, (X, W) in enumerate(maps):
        Z = X.astype(np.int64) @ W.astype(np.int64).T
        Et, Eo = O.eq_table_e2(pr["r_t"]), O.eq_table_e2(pr["r_o"][m])
        want = (0, 0)
        for t in range(Z.shape[0]):
            for o in range(Z.shape[1]):
                want = O.e2_add(want, O.e2_mul(O.e2_mul(Et[t], Eo[o]), (int(Z[t, o]) % P, 0)))
        assert pr["c0"][m] == want
        # the Q table is the rounded value before the clamp, element by element
        Q = pr["tables"][m][0].reshape(1 << lay.n_t, 1 << lay.n_o[m])
        q_int = np.floor_divide(Z + (1 << (s - 1)), 1 << s)
        assert all(int(Q[t, o]) == int(q_int[t, o]) % P for t in range(Z.shape[0]) for o in range(Z.shape[1]))
        assert not Q[Z.shape[0]:].any() and not Q[:, Z.shape[1]:].any()
    # the R row of map 2: its weights put eq(z_hi, i) on the table's rows only
    z = list(pr["r_o"][2]) + list(pr["r_t"])
    Eh = O.eq_table_e2(z[lay.L:])
    b = lay.base[2][1]
    for c in (0, 5, (1 << lay.L) - 1):
        acc = (0, 0)
        for i in range(lay.table_rows[2]):
            acc = O.e2_add(acc, O.e2_mul(Eh[i], (int(pr["msg"][b + i, c]), 0)))
        assert acc == (int(pr["U"][2 + 2 * 2][0][c]), int(pr["U"][2 + 2 * 2][1][c]))


@pytest.mark.parametrize("batched", [True, False])
def test_layer_committed_proof_and_negative_controls(batched):
    maps, salts = _small_layer()
    s = 7
    pr = O.prove_layer_committed(maps, s, batched, salts)
    V = lambda proof, mp=maps: O.verify_layer_committed(mp, s, batched, proof)
    assert V(pr) == "OK"
    assert len(pr["sumchecks"]) == (1 if batched else 3) and len(pr["idx"]) == O.LAYER_OPEN_COLUMNS
    # the challenges live in the extension, not in F_p
    assert any(r[1] != 0 for sc in pr["sumchecks"] for r in sc["r"])
    # a committed Q off by one at one entry: the claim 2^s Q~ + R~ is no longer Z~
    assert V(O.prove_layer_committed(maps, s, batched, salts, tamper="Q")) == "ROUND_SUM"
    # the same commitment with the true Q's folded rows: the columns disagree
    assert V(O.prove_layer_committed(maps, s, batched, salts, tamper="Q_rows")) == "COLUMN_CODE"
    assert V(O.prove_layer_committed(maps, s, batched, salts, tamper="prox_row")) == "COLUMN_CODE"
    assert V(O.prove_layer_committed(maps, s, batched, salts, tamper="column")) == "COLUMN_PATH"
    # a message changed after the fact
    bad = dict(pr, sumchecks=[dict(sc, rounds=[list(g) for g in sc["rounds"]]) for sc in pr["sumchecks"]])
    g = bad["sumchecks"][-1]["rounds"][1]
    g[2] = O.e2_add(g[2], (1, 0))
    assert V(bad) == "ROUND_SUM"
    bad = dict(pr, sumchecks=[dict(sc, finals=list(sc["finals"])) for sc in pr["sumchecks"]])
    a, b = bad["sumchecks"][0]["finals"][0]
    bad["sumchecks"][0]["finals"][0] = (O.e2_add(a, (0, 1)), b)
    assert V(bad) == "FINAL_CLAIM"
    bad = dict(pr, root=O.blake2b(b"other"))
    assert V(bad) == "ROUND_SUM"
    bad = dict(pr, state=O.blake2b(b"other"))
    assert V(bad) == "STATE"
    # other weights than the proof's: the finals are not W~ at the point
    W2 = maps[1][1].copy()
    W2[3, 7] ^= 1
    assert V(pr, [maps[0], (maps[1][0], W2), maps[2]]) == "FINAL_OPENING"


def test_layer_committed_single_map_and_tiny_rows():
    rng = np.random.default_rng(46)
    X = rng.integers(-127, 128, size=(2, 3)).astype(np.int8)
    W = rng.integers(-127, 128, size=(3, 3)).astype(np.int8)
    lay = O.LayerLayout(2, [3])
    assert (lay.L, lay.rows) == (3, 3)
    salts = rng.integers(0, 256, size=(2 << lay.L, 16), dtype=np.uint8)
    pr = O.prove_layer_committed([(X, W)], 1, False, salts)
    assert O.verify_layer_committed([(X, W)], 1, False, pr) == "OK"


# ------------------------------------------------------------- clamp lookup --
def test_clamp_rows_and_keys():
    # the row of q encodes (q, clamp(q)) without overlap: q + 2^15 in the low 16 bits, clamp(q) + 128 above
    for q in (-(1 << 15), -129, -128, -1, 0, 1, 127, 128, (1 << 15) - 1):
        row = O.clamp_row(q)
        assert row & 0xFFFF == q + (1 << 15) and row >> 16 == min(max(q, -128), 127) + 128
    rows = {O.clamp_row(q) for q in range(-(1 << 15), 1 << 15)}
    assert len(rows) == 1 << 16
    # a key of committed (Q, Y) tables is the row of Q exactly when Y = clamp(Q)
    Q = np.array([0, 5, -5, 127, 128, 3000, -129, -3000], np.int64)
    Y = np.clip(Q, -128, 127)
    keys = O.clamp_keys(O.field_embed(Q), O.field_embed(Y))
    assert [int(k) for k in keys] == [O.clamp_row(int(q)) for q in Q]
    bad = O.clamp_keys(O.field_embed(Q), O.field_embed(Y + np.array([0, 0, 0, 0, -1, 0, 0, 0])))
    assert int(bad[4]) not in rows and all(int(b) in rows for i, b in enumerate(bad) if i != 4)
    assert list(O.field_signed(O.field_embed(Q))) == list(Q)


def _clamp_case(seed, L, lo=-300, hi=300):
    rng = np.random.default_rng(seed)
    q = rng.integers(lo, hi, size=1 << L)
    q[: 1 << (L - 2)] = 0  # padding-like zeros
    return O.field_embed(q), O.field_embed(np.clip(q, -128, 127))


def test_clamp_lookup_proof_and_negative_controls():
    L = 9
    Qf, Yf = _clamp_case(50, L)
    gamma = 0x1234567890ABCDEF % P
    chal = synth.challenges(77, O.lookup_challenges_len(L))
    keys = O.clamp_keys(Qf, Yf)
    levels = O.product_tree_field(keys, L, gamma)
    # the root is the product of gamma - key over the keys (big integers)
    acc = 1
    for k in keys:
        acc = acc * (gamma - int(k)) % P
    assert int(levels[-1][0]) == acc
    counts, outside = O.clamp_counts(Qf)
    assert outside == 0 and counts.sum() == 1 << L
    tp = O.clamp_table_product(counts, gamma)
    assert tp == acc
    proof = O.grand_product_prove(levels, chal)
    assert O.grand_product_verify(int(levels[-1][0]), proof, chal, L, keys, gamma, table_prod=tp) == (0, -1)
    # one clamped output off by one: the key is no row, and the multiset differs
    Y2 = Yf.copy()
    j = int(np.nonzero(O.field_signed(Qf) > 127)[0][0])
    Y2[j] = O.field_embed(np.array([126]))[0]
    keys2 = O.clamp_keys(Qf, Y2)
    lev2 = O.product_tree_field(keys2, L, gamma)
    p2 = O.grand_product_prove(lev2, chal)
    assert O.grand_product_verify(int(lev2[-1][0]), p2, chal, L, keys2, gamma, table_prod=tp) == (5, L)
    # keys other than the tree's leaves fail the leaf opening
    assert O.grand_product_verify(int(levels[-1][0]), proof, chal, L, keys2, gamma, table_prod=tp) == (4, 0)
    # a Q outside 16 bits has no row
    Q3 = O.field_embed(np.array([1 << 15, -(1 << 15) - 1, 7]))
    assert O.clamp_counts(Q3)[1] == 2
