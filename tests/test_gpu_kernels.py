"""GPU parity of each libfp entry point against the CPU oracle, element by
element and bit-exact, on seeded inputs that span several tiles and ragged
tails, plus the degenerate cases (empty, single row/column, n = 0 or 1,
challenges 0, 1, p-1, extreme int8 values, rounding ties)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu
P = O.P


def _rng(seed):
    return np.random.default_rng(seed)


def _field(rng, n, specials=True):
    v = rng.integers(0, 2**63, size=n, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, size=n, dtype=np.uint64)
    v = np.where(v >= np.uint64(P), v - np.uint64(P), v).astype(np.uint64)
    if specials and n >= 4:
        v[:3] = [0, 1, P - 1]
    return v


def _i8(rng, shape, lo=-128, hi=127):
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int8)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ------------------------------------------------------------------- eq ---
@pytest.mark.parametrize("n", [0, 1, 2, 7, 8, 9, 11, 12, 13, 16, 22])
def test_eq_table(fp, n):
    rng = _rng(100 + n)
    r = _field(rng, n, specials=(n >= 4))
    E = fp.eq_table(fp.to_field_tensor(r) if n else torch.empty(0, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(fp.field_numpy(E), O.eq_table(r))


def test_eq_table_batched(fp):
    rng = _rng(7)
    ns = [0, 3, 8, 9, 12, 1]
    rs = [_field(rng, n, specials=False) for n in ns]
    Es = fp.eq_table_batched([fp.to_field_tensor(r) if len(r) else torch.empty(0, dtype=torch.int64, device="cuda")
                              for r in rs])
    torch.cuda.synchronize()
    for r, E in zip(rs, Es):
        assert np.array_equal(fp.field_numpy(E), O.eq_table(r))


# ---------------------------------------------------------------- folds ---
FOLD_SHAPES = [(1, 1, 1), (3, 5, 8), (17, 37, 64), (300, 256, 256), (1000, 300, 512), (2500, 1030, 2048),
               (4, 4, 4), (1025, 257, 512)]


@pytest.mark.parametrize("rows,cols,cols_pad", FOLD_SHAPES)
def test_fold_int8(fp, rows, cols, cols_pad):
    rng = _rng(rows * 7 + cols)
    M = _i8(rng, (rows, cols))
    E = _field(rng, rows)
    out = fp.fold_matrix(_dev(M), fp.to_field_tensor(E), cols_pad)
    torch.cuda.synchronize()
    assert np.array_equal(fp.field_numpy(out), O.fold_rows(M, E, cols_pad))


@pytest.mark.parametrize("rows,cols,cols_pad", FOLD_SHAPES)
def test_fold_int32(fp, rows, cols, cols_pad):
    rng = _rng(rows * 11 + cols)
    M = rng.integers(-2**31, 2**31, size=(rows, cols), dtype=np.int64).astype(np.int32)
    M.flat[:3] = [-2**31, 2**31 - 1, 0][:min(3, M.size)]
    E = _field(rng, rows)
    out = fp.fold_matrix(_dev(M), fp.to_field_tensor(E), cols_pad)
    torch.cuda.synchronize()
    assert np.array_equal(fp.field_numpy(out), O.fold_rows(M, E, cols_pad))


def test_fold_strided_and_extremes(fp):
    rng = _rng(5)
    base = _i8(rng, (700, 333))
    base[:, 0] = -128
    base[:, 1] = 127
    M = base[:, 3:300]  # leading dim 333, unaligned start
    E = _field(rng, 700)
    E[5:] = P - 1
    Mt = _dev(base)[:, 3:300]
    out = fp.fold_matrix(Mt, fp.to_field_tensor(E), 512)
    torch.cuda.synchronize()
    assert np.array_equal(fp.field_numpy(out), O.fold_rows(np.ascontiguousarray(M), E, 512))


def test_fold_batched(fp):
    rng = _rng(9)
    shapes = [(5, 7, 8), (0, 9, 16), (600, 300, 512), (33, 1, 4)]
    jobs, want = [], []
    for rows, cols, cp in shapes:
        M = _i8(rng, (rows, cols))
        E = _field(rng, max(rows, 1))
        jobs.append((_dev(M), fp.to_field_tensor(E), cp, torch.empty(cp, dtype=torch.int64, device="cuda")))
        want.append(O.fold_rows(M, E, cp) if rows else np.zeros(cp, np.uint64))
    outs = fp.fold_matrix_batched(jobs)
    torch.cuda.synchronize()
    for o, w in zip(outs, want):
        assert np.array_equal(fp.field_numpy(o), w)



def test_fold_claim_batched(fp):
    """Folds (int8) and claims (int32) in one pass, more jobs than one launch
    carries, with ragged, unaligned and empty matrices among them."""
    rng = _rng(31)
    folds, fwant = [], []
    for rows, cols, cp in [(5, 7, 8), (0, 9, 16), (1500, 300, 512), (33, 1, 4), (700, 1030, 2048), (64, 256, 256)] * 2:
        base = _i8(rng, (rows, cols + 3))
        M = base[:, 3:]  # unaligned start, leading dim cols + 3
        E = _field(rng, max(rows, 1))
        Mt = _dev(base)[:, 3:]
        folds.append((Mt, fp.to_field_tensor(E), cp, torch.empty(cp, dtype=torch.int64, device="cuda")))
        fwant.append(O.fold_rows(np.ascontiguousarray(M), E, cp) if rows else np.zeros(cp, np.uint64))
    claims, cwant = [], []
    for rows, cols in [(16, 256), (7, 9), (300, 1000), (0, 5), (513, 260), (1, 1), (40, 4096)]:
        M = rng.integers(-2**31, 2**31, size=(rows, cols), dtype=np.int64).astype(np.int32)
        r_rows, r_cols = _field(rng, O.log2ceil(max(rows, 1)), False), _field(rng, O.log2ceil(cols), False)
        claims.append((_dev(M), fp.to_field_tensor(O.eq_table(r_rows)), fp.to_field_tensor(O.eq_table(r_cols)),
                       torch.empty(1, dtype=torch.int64, device="cuda")))
        cwant.append(O.mle_matrix(M, r_rows, r_cols) if rows else 0)
    fo, co = fp.fold_claim_batched(folds, claims)
    torch.cuda.synchronize()
    for o, w in zip(fo, fwant):
        assert np.array_equal(fp.field_numpy(o), w)
    assert [int(fp.field_numpy(o)[0]) for o in co] == cwant


def test_fold_wide_and_many_jobs(fp):
    """Calls of different shapes on one workspace: 65536-column folds of several chunks, more jobs than one
    launch carries, and a claim beside them, all equal to the oracle."""
    rng = _rng(77)
    def fold_case(rows, cols, cp):
        M = _i8(rng, (rows, cols))
        E = _field(rng, rows)
        return (_dev(M), fp.to_field_tensor(E), cp, torch.empty(cp, dtype=torch.int64, device="cuda")), \
            O.fold_rows(M, E, cp)
    big = [fold_case(3000, 65536, 65536), fold_case(2000, 60000, 65536)]  # 256 + 235 strips of 2-3 chunks
    small = [fold_case(900, 700, 1024) for _ in range(40)]               # > 32 jobs: several launches
    # 17 folds of one 1025 x 65536 matrix (2 chunks, 256 strips each)
    Mw = _i8(rng, (1025, 65536))
    Mw_d = _dev(Mw)
    wide = []
    for _ in range(17):
        E = _field(rng, 1025)
        wide.append(((Mw_d, fp.to_field_tensor(E), 65536, torch.empty(65536, dtype=torch.int64, device="cuda")),
                     O.fold_rows(Mw, E, 65536)))
    M = rng.integers(-2**31, 2**31, size=(700, 3000), dtype=np.int64).astype(np.int32)
    rr, rc = _field(rng, 10, False), _field(rng, 12, False)
    claim = (_dev(M), fp.to_field_tensor(O.eq_table(rr)), fp.to_field_tensor(O.eq_table(rc)),
             torch.empty(1, dtype=torch.int64, device="cuda"))
    for jobs in (big, small, wide, big + small[:5]):
        fo, co = fp.fold_claim_batched([j for j, _ in jobs], [claim])
        torch.cuda.synchronize()
        for o, (_, w) in zip(fo, jobs):
            assert np.array_equal(fp.field_numpy(o), w)
        assert int(fp.field_numpy(co[0])[0]) == O.mle_matrix(M, rr, rc)


# ------------------------------------------------------------------ MLE ---
@pytest.mark.parametrize("rows,cols", [(1, 1), (5, 6), (16, 256), (100, 300), (513, 1030)])
@pytest.mark.parametrize("dt", [np.int8, np.int32])
def test_mle_eval(fp, rows, cols, dt):
    rng = _rng(rows + 3 * cols)
    if dt == np.int8:
        M = _i8(rng, (rows, cols))
    else:
        M = rng.integers(-2**31, 2**31, size=(rows, cols), dtype=np.int64).astype(np.int32)
    nr, nc = O.log2ceil(rows), O.log2ceil(cols)
    r_rows, r_cols = _field(rng, nr, False), _field(rng, nc, False)
    z = torch.empty(0, dtype=torch.int64, device="cuda")
    out = fp.mle_eval(_dev(M), fp.to_field_tensor(r_rows) if nr else z, fp.to_field_tensor(r_cols) if nc else z)
    torch.cuda.synchronize()
    assert int(fp.field_numpy(out)[0]) == O.mle_matrix(M, r_rows, r_cols)


def test_claim_eval_batched(fp):
    rng = _rng(12)
    jobs, want = [], []
    for rows, cols in [(16, 256), (7, 9), (300, 1000)]:
        M = rng.integers(-2**31, 2**31, size=(rows, cols), dtype=np.int64).astype(np.int32)
        r_rows, r_cols = _field(rng, O.log2ceil(rows), False), _field(rng, O.log2ceil(cols), False)
        jobs.append((_dev(M), fp.to_field_tensor(O.eq_table(r_rows)), fp.to_field_tensor(O.eq_table(r_cols)),
                     torch.empty(1, dtype=torch.int64, device="cuda")))
        want.append(O.mle_matrix(M, r_rows, r_cols))
    outs = fp.claim_eval_batched(jobs)
    torch.cuda.synchronize()
    assert [int(fp.field_numpy(o)[0]) for o in outs] == want


# ------------------------------------------------------------ sum-check ---
@pytest.mark.parametrize("n", [1, 2, 5, 12, 13, 14, 15])
def test_sumcheck_single(fp, n):
    rng = _rng(200 + n)
    A, B = _field(rng, 1 << n), _field(rng, 1 << n)
    r = _field(rng, n, specials=(n >= 4))
    rounds, finals, c0 = fp.sumcheck_prove([fp.to_field_tensor(A)], [fp.to_field_tensor(B)], fp.to_field_tensor(r))
    torch.cuda.synchronize()
    wr, wf, wc = O.sumcheck([A], [B], r)
    assert np.array_equal(fp.field_numpy(rounds), wr)
    assert np.array_equal(fp.field_numpy(finals), wf)
    assert int(fp.field_numpy(c0)[0]) == wc


@pytest.mark.parametrize("k,n", [(2, 3), (3, 11), (7, 14), (7, 10)])
def test_sumcheck_batched_rho(fp, k, n):
    rng = _rng(300 + 17 * k + n)
    As = [_field(rng, 1 << n, False) for _ in range(k)]
    Bs = [_field(rng, 1 << n, False) for _ in range(k)]
    rho = _field(rng, k, False)
    r = _field(rng, n, False)
    rounds, finals, c0 = fp.sumcheck_prove([fp.to_field_tensor(a) for a in As], [fp.to_field_tensor(b) for b in Bs],
                                           fp.to_field_tensor(r), rho=fp.to_field_tensor(rho))
    torch.cuda.synchronize()
    wr, wf, wc = O.sumcheck(As, Bs, r, rho=rho)
    assert np.array_equal(fp.field_numpy(rounds), wr)
    assert np.array_equal(fp.field_numpy(finals), wf)
    assert int(fp.field_numpy(c0)[0]) == wc


@pytest.mark.parametrize("n_inst,n", [(1, 1), (5, 6), (40, 13)])
def test_sumcheck_multi(fp, n_inst, n):
    rng = _rng(400 + n_inst + n)
    A = np.stack([_field(rng, 1 << n, False) for _ in range(n_inst)])
    B = np.stack([_field(rng, 1 << n, False) for _ in range(n_inst)])
    r = np.stack([_field(rng, n, False) for _ in range(n_inst)])
    rounds, finals, c0 = fp.sumcheck_prove_multi(fp.to_field_tensor(A.reshape(-1)).view(n_inst, -1),
                                                 fp.to_field_tensor(B.reshape(-1)).view(n_inst, -1),
                                                 fp.to_field_tensor(r.reshape(-1)).view(n_inst, n))
    torch.cuda.synchronize()
    R, F, C = fp.field_numpy(rounds), fp.field_numpy(finals), fp.field_numpy(c0)
    for i in range(n_inst):
        wr, wf, wc = O.sumcheck([A[i]], [B[i]], r[i])
        assert np.array_equal(R[i], wr) and np.array_equal(F[i], wf[0]) and int(C[i]) == wc



@pytest.mark.parametrize("T,d_in,d_out,k,n", [(100, 300, 700, 1, 12), (16, 64, 48, 1, 1), (600, 256, 300, 3, 9),
                                             (0, 64, 64, 2, 10), (40, 96, 0, 1, 5)])
def test_witness_with_sumcheck(fp, T, d_in, d_out, k, n):
    """One launch: a witness and an unrelated sum-check, each against the oracle."""
    rng = _rng(500 + T + n + k)
    X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
    As = [_field(rng, 1 << n, False) for _ in range(k)]
    Bs = [_field(rng, 1 << n, False) for _ in range(k)]
    r = _field(rng, n, specials=(n >= 4))
    rho = _field(rng, k, False) if k > 1 else None
    Z = torch.empty((T, d_out), dtype=torch.int32, device="cuda")
    Y = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    R = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    _, (rounds, finals, c0) = fp.witness_linear_with_sumcheck(
        _dev(X), _dev(W), 8, Z, Y, R, [fp.to_field_tensor(a) for a in As], [fp.to_field_tensor(b) for b in Bs],
        fp.to_field_tensor(r), rho=None if rho is None else fp.to_field_tensor(rho))
    torch.cuda.synchronize()
    if T and d_out:
        wz, wy, wr = O.witness(X, W, 8)
        assert np.array_equal(Z.cpu().numpy(), wz)
        assert np.array_equal(Y.cpu().numpy(), wy)
        assert np.array_equal(R.cpu().numpy(), wr)
    grs, gfs, gc = O.sumcheck(As, Bs, r, rho=rho)
    assert np.array_equal(fp.field_numpy(rounds), grs)
    assert np.array_equal(fp.field_numpy(finals), gfs)
    assert int(fp.field_numpy(c0)[0]) == gc


def test_witness_with_sumcheck_too_large(fp):
    X = torch.zeros((16, 64), dtype=torch.int8, device="cuda")
    W = torch.zeros((64, 64), dtype=torch.int8, device="cuda")
    A = torch.zeros(1 << 13, dtype=torch.int64, device="cuda")
    r = torch.zeros(13, dtype=torch.int64, device="cuda")
    Z = torch.empty((16, 64), dtype=torch.int32, device="cuda")
    Y = torch.empty((16, 64), dtype=torch.int8, device="cuda")
    with pytest.raises(fp.FPError, match="exceed one"):
        fp.witness_linear_with_sumcheck(X, W, 8, Z, Y, Y.clone(), [A], [A], r)


def test_combine_and_linear_combine(fp):
    rng = _rng(13)
    g = [_field(rng, 3, False) for _ in range(3)]
    x = [_field(rng, 1, False) for _ in range(3)]
    rho = _field(rng, 3, False)
    gd = [fp.to_field_tensor(v) for v in g]
    xd = [fp.to_field_tensor(v) for v in x]
    out = fp.combine_claims(gd, xd, fp.to_field_tensor(rho))
    lin = fp.linear_combine([fp.to_field_tensor(v[:1]) for v in g], fp.to_field_tensor(rho))
    torch.cuda.synchronize()
    want = sum(int(rho[j]) * O.eval_deg2(*[int(v) for v in g[j]], int(x[j][0])) for j in range(3)) % P
    assert int(fp.field_numpy(out)[0]) == want
    assert int(fp.field_numpy(lin)[0]) == sum(int(rho[j]) * int(g[j][0]) for j in range(3)) % P


# -------------------------------------------------------------- witness ---
WIT_SHAPES = [(1, 1, 1, 8), (5, 17, 7, 7), (16, 256, 256, 7), (33, 64, 129, 8), (130, 300, 300, 1),
              (200, 1000, 260, 8), (257, 128, 513, 4)]


@pytest.mark.parametrize("T,d_in,d_out,s", WIT_SHAPES)
def test_witness(fp, T, d_in, d_out, s):
    rng = _rng(T * 1000 + d_in + d_out)
    X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
    Z, Y, R = fp.witness_linear(_dev(X), _dev(W), s)
    torch.cuda.synchronize()
    wz, wy, wr = O.witness(X, W, s)
    assert np.array_equal(Z.cpu().numpy(), wz)
    assert np.array_equal(Y.cpu().numpy(), wy)
    assert np.array_equal(R.cpu().numpy(), wr)


def test_witness_extremes_and_ties(fp):
    # |Z| at its largest (all -128), all +127 rows, and exact rounding ties
    T, d_in, d_out = 40, 4096, 70
    X = np.full((T, d_in), -128, np.int8)
    X[1::2] = 127
    W = np.full((d_out, d_in), -128, np.int8)
    W[3::3] = 127
    W[5, :] = 0
    W[5, 0] = 1                # Z = X[t, 0] exactly: -128 or 127
    X[7, :] = 0
    X[7, :128] = 1
    W[6, :] = 0
    W[6, :128] = 1             # Z[7, 6] = 128: a tie at s = 8
    for s in (8, 7, 1):
        Z, Y, R = fp.witness_linear(_dev(X), _dev(W), s)
        torch.cuda.synchronize()
        wz, wy, wr = O.witness(X, W, s)
        assert np.array_equal(Z.cpu().numpy(), wz)
        assert np.array_equal(Y.cpu().numpy(), wy) and np.array_equal(R.cpu().numpy(), wr)


def test_witness_strided_inputs(fp):
    rng = _rng(21)
    Xb, Wb = _i8(rng, (50, 320)), _i8(rng, (90, 330))
    X, W = Xb[:, 5:305], Wb[:, 7:307]
    Z, Y, R = fp.witness_linear(_dev(Xb)[:, 5:305], _dev(Wb)[:, 7:307], 8)
    torch.cuda.synchronize()
    wz, wy, wr = O.witness(np.ascontiguousarray(X), np.ascontiguousarray(W), 8)
    assert np.array_equal(Z.cpu().numpy(), wz) and np.array_equal(Y.cpu().numpy(), wy)
    assert np.array_equal(R.cpu().numpy(), wr)


# ------------------------------------------------------- packed weights ---
def _pack_ref(W):
    """The packed layout include/fp.h documents, built in numpy: fragment (b, c, q), lane l holds
    W[32 b + l % 32][64 c + 32 (l // 32) + 16 q + 0..15], zero past the matrix."""
    d_out, d_in = W.shape
    nrb, nkb = -(-d_out // 32), -(-d_in // 64)
    Wz = np.zeros((nrb * 32, nkb * 64), np.int8)
    Wz[:d_out, :d_in] = W
    A = Wz.reshape(nrb, 32, nkb, 2, 2, 16)  # [b][row][c][half][q][byte]
    return A.transpose(0, 2, 4, 3, 1, 5).reshape(-1)  # [b][c][q][lane = 32 half + row][byte]


@pytest.mark.parametrize("d_out,d_in", [(1, 1), (7, 17), (33, 64), (100, 300), (64, 4096)])
def test_pack_weights(fp, d_out, d_in):
    rng = _rng(d_out * 7 + d_in)
    W = _i8(rng, (d_out, d_in))
    Wp = fp.pack_weights(_dev(W))
    torch.cuda.synchronize()
    want = _pack_ref(W)
    assert Wp.data.numel() == max(want.size, 16)
    assert np.array_equal(Wp.data.cpu().numpy()[:want.size], want)


PACK_SHAPES = [(1, 16, 1, 8), (5, 48, 7, 7), (33, 64, 129, 8), (130, 304, 300, 1), (200, 1008, 260, 8),
               (257, 128, 513, 4), (64, 4096, 256, 8), (300, 80, 70, 3), (4, 0, 9, 8),
               (1000, 208, 6100, 8), (1030, 64, 6144, 5)]  # the last two: 256x128 tiles (>= 192 of them)


@pytest.mark.parametrize("T,d_in,d_out,s", PACK_SHAPES)
def test_witness_packed(fp, T, d_in, d_out, s):
    """The witness from packed weights equals the oracle's (256x64 tiles: ragged in T, d_out and d_in)."""
    rng = _rng(T * 1000 + d_in + d_out + 7)
    X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
    Z, Y, R = fp.witness_linear_packed(_dev(X), fp.pack_weights(_dev(W)), s)
    torch.cuda.synchronize()
    wz, wy, wr = O.witness(X, W, s)
    assert np.array_equal(Z.cpu().numpy(), wz)
    assert np.array_equal(Y.cpu().numpy(), wy)
    assert np.array_equal(R.cpu().numpy(), wr)


def test_witness_packed_extremes_strided_and_no_z(fp):
    # |Z| at its largest, rounding ties, X rows with a 16-byte aligned stride, and Z not stored
    T, d_in, d_out = 40, 4096, 70
    X = np.full((T, d_in), -128, np.int8)
    X[1::2] = 127
    W = np.full((d_out, d_in), -128, np.int8)
    W[3::3] = 127
    W[5, :] = 0
    W[5, 0] = 1
    X[7, :] = 0
    X[7, :128] = 1
    W[6, :] = 0
    W[6, :128] = 1  # Z[7, 6] = 128: a tie at s = 8
    Wp = fp.pack_weights(_dev(W))
    for s in (8, 7, 1):
        Z, Y, R = fp.witness_linear_packed(_dev(X), Wp, s)
        torch.cuda.synchronize()
        wz, wy, wr = O.witness(X, W, s)
        assert np.array_equal(Z.cpu().numpy(), wz)
        assert np.array_equal(Y.cpu().numpy(), wy) and np.array_equal(R.cpu().numpy(), wr)
    rng = _rng(22)
    Xb, W2 = _i8(rng, (50, 352)), _i8(rng, (90, 304))
    _, Y, R = fp.witness_linear_packed(_dev(Xb)[:, 32:336], fp.pack_weights(_dev(W2)), 8, with_z=False)
    torch.cuda.synchronize()
    _, wy, wr = O.witness(np.ascontiguousarray(Xb[:, 32:336]), W2, 8)
    assert np.array_equal(Y.cpu().numpy(), wy) and np.array_equal(R.cpu().numpy(), wr)


def test_witness_rescale_at_the_int32_limit(fp):
    """The rescale forms Z + 2^(s-1) in int32 before its shift: with d_in at its largest (131071 for the row-major
    kernel, 131056 = the largest multiple of 16 for the packed one) and every product 128 * 128, |Z| is within
    2^14 of 2^31, and every s in [1, 8] must still match the oracle's floor division."""
    for d_in, kinds in ((131056, (True, False)), (131071, (False,))):
        X = np.full((3, d_in), -128, np.int8)
        X[1] = 127
        X[2, ::2] = 5
        W = np.full((5, d_in), -128, np.int8)
        W[1] = 127
        W[3, 1::3] = -7
        Wp = fp.pack_weights(_dev(W)) if True in kinds else None
        for s in (1, 2, 7, 8):
            wz, wy, wr = O.witness(X, W, s)
            assert int(np.abs(wz.astype(np.int64)).max()) == 128 * 128 * d_in
            for packed in kinds:
                if packed:
                    Z, Y, R = fp.witness_linear_packed(_dev(X), Wp, s)
                else:
                    Z, Y, R = fp.witness_linear(_dev(X), _dev(W), s)
                torch.cuda.synchronize()
                assert np.array_equal(Z.cpu().numpy(), wz), (d_in, s, packed)
                assert np.array_equal(Y.cpu().numpy(), wy) and np.array_equal(R.cpu().numpy(), wr), (d_in, s, packed)


@pytest.mark.parametrize("T,d_out", [(200, 260), (0, 64)])
def test_witness_packed_with_eq_tables(fp, T, d_out):
    """eq tables built by spare workgroups of the packed witness launch (one per 256 x 2^min(n - 8, 6) entries)
    equal the oracle's, and the witness beside them is unchanged; with no tokens only the tables are built."""
    rng = _rng(31 + T)
    d_in = 320
    X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
    ns = [0, 1, 8, 9, 14, 15, 20, 3]
    rs = [_field(rng, n, specials=(n >= 4)) for n in ns]
    rt = [fp.to_field_tensor(r) if len(r) else torch.empty(0, dtype=torch.int64, device="cuda") for r in rs]
    Es = [torch.empty(1 << n, dtype=torch.int64, device="cuda") for n in ns]
    Z, Y, R = fp.witness_linear_packed(_dev(X), fp.pack_weights(_dev(W)), 8, eq=list(zip(rt, Es)))
    torch.cuda.synchronize()
    for r, E in zip(rs, Es):
        assert np.array_equal(fp.field_numpy(E), O.eq_table(r))
    wz, wy, wr = O.witness(X, W, 8)
    assert np.array_equal(Z.cpu().numpy(), wz)
    assert np.array_equal(Y.cpu().numpy(), wy) and np.array_equal(R.cpu().numpy(), wr)


@pytest.mark.parametrize("T,d_in,d_out,k", [(100, 320, 700, 1), (1000, 96, 6100, 2), (16, 64, 48, 0)])
def test_layer_step(fp, T, d_in, d_out, k):
    """One launch with a witness and its eq tables, the folds and claim of an unrelated proof and the sum-check of
    a third: each part equals the oracle's; the arrival counters are zero again after every call."""
    rng = _rng(1200 + T + k)
    X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
    # another proof's tables: int8 folds of two matrices and an int32 claim, several chunks each
    X2, W2 = _i8(rng, (700, 300)), _i8(rng, (3000, 260))
    Z2 = rng.integers(-2**31, 2**31, size=(700, 3000), dtype=np.int64).astype(np.int32)
    E1, E2 = _field(rng, 700), _field(rng, 3000)
    rr, rc = _field(rng, 10, False), _field(rng, 12, False)
    n = 9
    As = [_field(rng, 1 << n, False) for _ in range(k)]
    Bs = [_field(rng, 1 << n, False) for _ in range(k)]
    r = _field(rng, n)
    rho = _field(rng, k, False) if k > 1 else None
    re_t, re_o = _field(rng, 10), _field(rng, 13)
    Et = torch.empty(1 << 10, dtype=torch.int64, device="cuda")
    Eo = torch.empty(1 << 13, dtype=torch.int64, device="cuda")
    Z = torch.empty((T, d_out), dtype=torch.int32, device="cuda")
    Y = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    R = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    xo = torch.empty(512, dtype=torch.int64, device="cuda")
    wo = torch.empty(512, dtype=torch.int64, device="cuda")
    co = torch.empty(1, dtype=torch.int64, device="cuda")
    rounds = torch.empty((n, 3), dtype=torch.int64, device="cuda")
    finals = torch.empty((max(k, 1), 2), dtype=torch.int64, device="cuda")
    c0 = torch.empty(1, dtype=torch.int64, device="cuda")
    ws = fp.StepWorkspace()
    for rep in range(2):
        fp.layer_step(_dev(X), fp.pack_weights(_dev(W)), 8, Z, Y, R,
                      eq=[(fp.to_field_tensor(re_t), Et), (fp.to_field_tensor(re_o), Eo)],
                      folds=[(_dev(X2), fp.to_field_tensor(E1), 512, xo), (_dev(W2), fp.to_field_tensor(E2), 512, wo)],
                      claims=[(_dev(Z2), fp.to_field_tensor(O.eq_table(rr)), fp.to_field_tensor(O.eq_table(rc)), co)],
                      As=[fp.to_field_tensor(a) for a in As], Bs=[fp.to_field_tensor(b) for b in Bs],
                      r=fp.to_field_tensor(r), rho=None if rho is None else fp.to_field_tensor(rho),
                      rounds=rounds, finals=finals, claim0=c0, ws=ws)
        torch.cuda.synchronize()
        wz, wy, wr = O.witness(X, W, 8)
        assert np.array_equal(Z.cpu().numpy(), wz)
        assert np.array_equal(Y.cpu().numpy(), wy) and np.array_equal(R.cpu().numpy(), wr)
        assert np.array_equal(fp.field_numpy(Et), O.eq_table(re_t))
        assert np.array_equal(fp.field_numpy(Eo), O.eq_table(re_o))
        assert np.array_equal(fp.field_numpy(xo), O.fold_rows(X2, E1, 512))
        assert np.array_equal(fp.field_numpy(wo), O.fold_rows(W2, E2, 512))
        assert int(fp.field_numpy(co)[0]) == O.mle_matrix(Z2, rr, rc)
        if k:
            grs, gfs, gc = O.sumcheck(As, Bs, r, rho=rho)
            assert np.array_equal(fp.field_numpy(rounds), grs)
            assert np.array_equal(fp.field_numpy(finals), gfs)
            assert int(fp.field_numpy(c0)[0]) == gc
        assert int(ws.buf[:16384].count_nonzero()) == 0


@pytest.mark.parametrize("T,d_in,d_out,keep_z,tables,fold", [
    (100, 320, 700, True, "eq", True), (1000, 96, 6100, False, "rand", True), (1000, 96, 6100, True, "eq", False),
    (16, 64, 48, False, "rand", False), (1, 16, 1, True, "rand", True), (4, 0, 9, True, "eq", False),
    (512, 512, 2048, False, "eq", True)])
def test_layer_step_own_claim(fp, T, d_in, d_out, keep_z, tables, fold):
    """The witness's own claim sum_t sum_o E_t[t] E_o[o] Z[t, o] taken from the GEMM's accumulators (both tile
    configurations, ragged edges, Z stored or not, eq tables or arbitrary field tables with 0, 1 and p - 1),
    beside another proof's fold: the claim, Y, R (and Z) equal the oracle's on two calls in a row, and the
    arrival counters are zero again."""
    rng = _rng(1300 + T + d_out + d_in)
    X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
    if tables == "eq":
        rt, ro = _field(rng, max(1, (T - 1).bit_length())), _field(rng, max(1, (d_out - 1).bit_length()))
        Et_h, Eo_h = O.eq_table(rt), O.eq_table(ro)
    else:
        Et_h, Eo_h = _field(rng, T), _field(rng, d_out)
    Et, Eo = fp.to_field_tensor(Et_h), fp.to_field_tensor(Eo_h)
    X2, E1 = _i8(rng, (300, 200)), _field(rng, 300)
    xo = torch.empty(256, dtype=torch.int64, device="cuda")
    Z = torch.empty((T, d_out), dtype=torch.int32, device="cuda") if keep_z else None
    Y = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    R = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    c = torch.empty(1, dtype=torch.int64, device="cuda")
    ws = fp.StepWorkspace()
    Wp = fp.pack_weights(_dev(W))
    wz, wy, wr = O.witness(X, W, 8)
    if tables == "eq":
        want = O.mle_matrix(wz, rt, ro)
    else:
        u = O.fold_rows(wz, Et_h)
        want = 0
        for o in range(d_out):
            want = O.add(want, O.mul(int(Eo_h[o]), int(u[o])))
    for rep in range(2):
        c.fill_(-1)
        fp.layer_step(_dev(X), Wp, 8, Z, Y, R, own_claim=(Et, Eo, c),
                      folds=[(_dev(X2), fp.to_field_tensor(E1), 256, xo)] if fold else (), ws=ws)
        torch.cuda.synchronize()
        assert int(fp.field_numpy(c)[0]) == want
        assert np.array_equal(Y.cpu().numpy(), wy) and np.array_equal(R.cpu().numpy(), wr)
        if keep_z:
            assert np.array_equal(Z.cpu().numpy(), wz)
        if fold:
            assert np.array_equal(fp.field_numpy(xo), O.fold_rows(X2, E1, 256))
        assert int(ws.buf[:16384].count_nonzero()) == 0


def test_layer_step_own_claim_errors(fp):
    """The own claim needs both tables and an output, and tokens and outputs."""
    X = torch.zeros((8, 16), dtype=torch.int8, device="cuda")
    Wp = fp.pack_weights(torch.zeros((8, 16), dtype=torch.int8, device="cuda"))
    Y = torch.empty((8, 8), dtype=torch.int8, device="cuda")
    R = torch.empty((8, 8), dtype=torch.int8, device="cuda")
    E = torch.zeros(8, dtype=torch.int64, device="cuda")
    with pytest.raises(RuntimeError):
        fp.layer_step(X, Wp, 8, None, Y, R, own_claim=(E, None, torch.empty(1, dtype=torch.int64, device="cuda")))
    with pytest.raises(RuntimeError):
        fp.layer_step(X[:0], Wp, 8, None, Y[:0], R[:0], own_claim=(E, E, torch.empty(1, dtype=torch.int64, device="cuda")))


@pytest.mark.parametrize("T,d_in,d_out,k,n", [(100, 320, 700, 1, 12), (16, 64, 48, 1, 1), (600, 256, 300, 3, 9),
                                             (0, 64, 64, 2, 10), (40, 96, 0, 1, 5), (1000, 96, 6100, 2, 11)])
def test_witness_packed_with_sumcheck(fp, T, d_in, d_out, k, n):
    """One launch: a packed-weight witness and an unrelated sum-check, each against the oracle."""
    rng = _rng(900 + T + n + k)
    X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
    As = [_field(rng, 1 << n, False) for _ in range(k)]
    Bs = [_field(rng, 1 << n, False) for _ in range(k)]
    r = _field(rng, n, specials=(n >= 4))
    rho = _field(rng, k, False) if k > 1 else None
    Z = torch.empty((T, d_out), dtype=torch.int32, device="cuda")
    Y = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    R = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    re = _field(rng, 11, specials=True)
    E = torch.empty(1 << 11, dtype=torch.int64, device="cuda")
    _, (rounds, finals, c0) = fp.witness_linear_packed_with_sumcheck(
        _dev(X), fp.pack_weights(_dev(W)), 8, Z, Y, R, [fp.to_field_tensor(a) for a in As],
        [fp.to_field_tensor(b) for b in Bs], fp.to_field_tensor(r),
        rho=None if rho is None else fp.to_field_tensor(rho), eq=[(fp.to_field_tensor(re), E)])
    torch.cuda.synchronize()
    assert np.array_equal(fp.field_numpy(E), O.eq_table(re))
    if T and d_out:
        wz, wy, wr = O.witness(X, W, 8)
        assert np.array_equal(Z.cpu().numpy(), wz)
        assert np.array_equal(Y.cpu().numpy(), wy)
        assert np.array_equal(R.cpu().numpy(), wr)
    grs, gfs, gc = O.sumcheck(As, Bs, r, rho=rho)
    assert np.array_equal(fp.field_numpy(rounds), grs)
    assert np.array_equal(fp.field_numpy(finals), gfs)
    assert int(fp.field_numpy(c0)[0]) == gc


def test_witness_grouped(fp):
    rng = _rng(22)
    sizes = [3, 0, 40, 1, 0, 65, 17]
    d_in, d_out = 200, 150
    row_off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    Xg = _i8(rng, (int(row_off[-1]), d_in))
    Ws = [_i8(rng, (d_out, d_in)) for _ in sizes]
    Z, Y, R = fp.witness_linear_grouped(_dev(Xg), [_dev(w) for w in Ws], row_off, 8)
    torch.cuda.synchronize()
    Z, Y, R = Z.cpu().numpy(), Y.cpu().numpy(), R.cpu().numpy()
    for g, w in enumerate(Ws):
        a, b = row_off[g], row_off[g + 1]
        if a == b:
            continue
        wz, wy, wr = O.witness(Xg[a:b], w, 8)
        assert np.array_equal(Z[a:b], wz) and np.array_equal(Y[a:b], wy) and np.array_equal(R[a:b], wr)


def test_gather_rows(fp):
    rng = _rng(23)
    X = _i8(rng, (50, 96))
    perm = rng.permutation(50).astype(np.int32)[:31]
    out = fp.gather_rows(_dev(X), _dev(perm))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), X[perm])
