"""fp_witness_multi: the witness GEMMs of several linear maps in one launch, each
map's claim sum_t sum_o E_t[t] E_o[o] Z[t, o] taken from its accumulators,
against the CPU oracle (witness, rescale, MLE of Z or the claim's definition),
bit-exact, on ragged shapes spanning several tiles, with Z stored or not, eq
tables and arbitrary field tables (0, 1, p - 1), several tile walks, eq tables
of another proof in the same launch, two calls in a row on one workspace, and
the error cases."""
import zlib

import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu
P = O.P


def _rng(seed):
    return np.random.default_rng(seed)


def _field(rng, n):
    v = rng.integers(0, 2**63, size=n, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, size=n, dtype=np.uint64)
    v = np.where(v >= np.uint64(P), v - np.uint64(P), v).astype(np.uint64)
    if n >= 4:
        v[:3] = [0, 1, P - 1]
    return v


def _i8(rng, shape):
    return rng.integers(-128, 128, size=shape, dtype=np.int8)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _claim_def(Z, Et, Eo):
    """sum_t sum_o E_t[t] E_o[o] Z[t, o] mod p by its definition (the oracle's fold of Z's rows by E_t, then the
    E_o-weighted sum of the folded row)."""
    u = O.fold_rows(Z, Et)
    want = 0
    for o in range(Z.shape[1]):
        want = O.add(want, O.mul(int(Eo[o]), int(u[o])))
    return want


# (T, d_in, d_out, keep_z, claim): claim "eq" (eq tables of random points: the oracle's MLE of Z), "rand"
# (arbitrary field tables: the claim's definition) or None
CASES = {
    "layer": [(300, 1024, 700, False, "eq"), (300, 1024, 256, True, "eq"), (300, 4096, 130, False, "rand"),
              (300, 64, 1000, True, None)],
    "ragged": [(1, 16, 1, True, "rand"), (33, 48, 257, False, "eq"), (129, 2000, 31, True, "eq"),
               (257, 96, 513, False, "rand"), (5, 0, 40, True, "eq")],
    "one": [(700, 512, 900, False, "eq")],
}


@pytest.mark.parametrize("case,group_o,with_eq", [("layer", 1, False), ("layer", 3, True), ("ragged", 1, True),
                                                   ("ragged", 2, False), ("one", 5, False)])
def test_witness_multi(fp, case, group_o, with_eq):
    rng = _rng(zlib.crc32(('%s/%d' % (case, group_o)).encode()))
    maps, jobs = [], []
    for (T, d_in, d_out, keep_z, claim) in CASES[case]:
        X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
        want = {}
        want["Z"], want["Y"], want["R"] = O.witness(X, W, 7)
        Et = Eo = c = None
        if claim == "eq":
            rt = _field(rng, max(1, (T - 1).bit_length()))
            ro = _field(rng, max(1, (d_out - 1).bit_length()))
            want["c"] = O.mle_matrix(want["Z"], rt, ro)
            Et, Eo = fp.to_field_tensor(O.eq_table(rt)), fp.to_field_tensor(O.eq_table(ro))
        elif claim == "rand":
            Et_h, Eo_h = _field(rng, T), _field(rng, d_out)
            want["c"] = _claim_def(want["Z"], Et_h, Eo_h)
            Et, Eo = fp.to_field_tensor(Et_h), fp.to_field_tensor(Eo_h)
        if claim:
            c = torch.empty(1, dtype=torch.int64, device="cuda")
        Z = torch.empty((T, d_out), dtype=torch.int32, device="cuda") if keep_z else None
        Y = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
        R = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
        jobs.append(fp.MatmulJob(_dev(X), fp.pack_weights(_dev(W)), Y, R, Z, Et, Eo, c))
        maps.append(want)
    eq, eq_want = None, []
    if with_eq:
        rs = [_field(rng, n) for n in (0, 5, 13)]
        Es = [torch.empty(1 << len(r), dtype=torch.int64, device="cuda") for r in rs]
        eq = [(fp.to_field_tensor(r) if len(r) else torch.empty(0, dtype=torch.int64, device="cuda"), E)
              for r, E in zip(rs, Es)]
        eq_want = [O.eq_table(r) for r in rs]
    ws = fp.StepWorkspace()
    for rep in range(2):
        for j in jobs:
            j.Y.fill_(3)
            j.R.fill_(3)
            if j.claim is not None:
                j.claim.fill_(-1)
        fp.witness_multi(jobs, 7, group_o=group_o, eq=eq, ws=ws)
        torch.cuda.synchronize()
        for j, want in zip(jobs, maps):
            assert np.array_equal(j.Y.cpu().numpy(), want["Y"]) and np.array_equal(j.R.cpu().numpy(), want["R"])
            if j.Z is not None:
                assert np.array_equal(j.Z.cpu().numpy(), want["Z"])
            if j.claim is not None:
                assert int(fp.field_numpy(j.claim)[0]) == want["c"]
        for (r, E), w in zip(eq or [], eq_want):
            assert np.array_equal(fp.field_numpy(E), w)
        assert ws.buf is None or int(ws.buf[:512].count_nonzero()) == 0


@pytest.mark.parametrize("group_o", [1, 4])
def test_witness_multi_tile_pool(fp, group_o):
    """Launches of more than two full waves of tiles hand each XCD's last tiles to workgroups that take them at
    run time (from their own XCD's pool or another's): with ragged tokens and outputs, claims of eq tables and of
    arbitrary tables, Z kept on one map, every output and claim equals the oracle's on three calls in a row, and
    the pool's counters (in the workspace's first 512 bytes) are zero after each."""
    rng = _rng(1201 + group_o)
    T = 1000
    jobs, wants = [], []
    for i, (d_in, d_out, claim) in enumerate([(64, 12900, "eq"), (48, 12800, "rand"), (96, 12544, "eq")]):
        X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
        Z, Y, R = O.witness(X, W, 8)
        if claim == "eq":
            rt, ro = _field(rng, 10), _field(rng, (d_out - 1).bit_length())
            c = O.mle_matrix(Z, rt, ro)
            Et, Eo = fp.to_field_tensor(O.eq_table(rt)), fp.to_field_tensor(O.eq_table(ro))
        else:
            Et_h, Eo_h = _field(rng, T), _field(rng, d_out)
            c = _claim_def(Z, Et_h, Eo_h)
            Et, Eo = fp.to_field_tensor(Et_h), fp.to_field_tensor(Eo_h)
        Zd = torch.empty((T, d_out), dtype=torch.int32, device="cuda") if i == 1 else None
        jobs.append(fp.MatmulJob(_dev(X), fp.pack_weights(_dev(W)), torch.empty((T, d_out), dtype=torch.int8,
                                 device="cuda"), torch.empty((T, d_out), dtype=torch.int8, device="cuda"), Zd, Et, Eo,
                                 torch.empty(1, dtype=torch.int64, device="cuda")))
        wants.append((Z, Y, R, c))
    assert sum(((T + 127) // 128) * ((j.Y.shape[1] + 255) // 256) for j in jobs) >= 1024  # the pool is used
    ws = fp.StepWorkspace()
    for rep in range(3):
        for j in jobs:
            j.Y.fill_(3)
            j.R.fill_(3)
            j.claim.fill_(-1)
        fp.witness_multi(jobs, 8, group_o=group_o, ws=ws)
        torch.cuda.synchronize()
        for j, (Z, Y, R, c) in zip(jobs, wants):
            assert np.array_equal(j.Y.cpu().numpy(), Y) and np.array_equal(j.R.cpu().numpy(), R)
            if j.Z is not None:
                assert np.array_equal(j.Z.cpu().numpy(), Z)
            assert int(fp.field_numpy(j.claim)[0]) == c
        assert int(ws.buf[:512].count_nonzero()) == 0


def test_witness_multi_seven_maps_one_token_axis(fp):
    """Seven maps over one token axis and shared inputs, in the layer's order (longest reduction first), the
    claims of eq tables sharing E_t: every output and claim is the oracle's."""
    rng = _rng(77)
    T = 200
    Xa, Xo, Xm, H = _i8(rng, (T, 256)), _i8(rng, (T, 256)), _i8(rng, (T, 256)), _i8(rng, (T, 640))
    shapes = [("down", H, 256), ("q", Xa, 256), ("k", Xa, 64), ("v", Xa, 64), ("o", Xo, 256), ("gate", Xm, 640),
              ("up", Xm, 640)]
    rt = _field(rng, 8)
    Et_h = O.eq_table(rt)
    Et = fp.to_field_tensor(Et_h)
    jobs, wants = [], []
    for name, X, d_out in shapes:
        W = _i8(rng, (d_out, X.shape[1]))
        ro = _field(rng, (d_out - 1).bit_length())
        Z, Y, R = O.witness(X, W, 8)
        wants.append((Y, R, O.mle_matrix(Z, rt, ro)))
        jobs.append(fp.MatmulJob(_dev(X), fp.pack_weights(_dev(W)), torch.empty((T, d_out), dtype=torch.int8,
                                 device="cuda"), torch.empty((T, d_out), dtype=torch.int8, device="cuda"), None, Et,
                                 fp.to_field_tensor(O.eq_table(ro)), torch.empty(1, dtype=torch.int64, device="cuda")))
    fp.witness_multi(jobs, 8)
    torch.cuda.synchronize()
    for j, (Y, R, c) in zip(jobs, wants):
        assert np.array_equal(j.Y.cpu().numpy(), Y) and np.array_equal(j.R.cpu().numpy(), R)
        assert int(fp.field_numpy(j.claim)[0]) == c


def test_witness_multi_errors(fp):
    """Bad counts, a claim without its E_o or without outputs, unaligned X, s and group_o out of range, a
    short workspace: each is refused before any launch."""
    X = torch.zeros((8, 16), dtype=torch.int8, device="cuda")
    Wp = fp.pack_weights(torch.zeros((8, 16), dtype=torch.int8, device="cuda"))
    Y = torch.empty((8, 8), dtype=torch.int8, device="cuda")
    R = torch.empty((8, 8), dtype=torch.int8, device="cuda")
    E = torch.zeros(8, dtype=torch.int64, device="cuda")
    c = torch.empty(1, dtype=torch.int64, device="cuda")
    ok = fp.MatmulJob(X, Wp, Y, R, None, E, E, c)
    fp.witness_multi([ok], 8)
    with pytest.raises(AssertionError):
        fp.witness_multi([], 8)
    with pytest.raises(RuntimeError):
        fp.witness_multi([ok] * 9, 8)
    with pytest.raises(RuntimeError):
        fp.witness_multi([ok], 9)
    with pytest.raises(RuntimeError):
        fp.witness_multi([ok], 8, group_o=0)
    bad = fp.MatmulJob(X, Wp, Y, R, None, E, None, c)
    with pytest.raises((RuntimeError, ValueError)):
        fp.witness_multi([bad], 8)
    Xu = torch.zeros(8 * 16 + 1, dtype=torch.int8, device="cuda")[1:].view(8, 16)
    with pytest.raises(RuntimeError):
        fp.witness_multi([fp.MatmulJob(Xu, Wp, Y, R)], 8)
    lib = fp.lib()
    arr = fp._multi_descs([ok])
    with pytest.raises(RuntimeError):
        fp._check(lib.fp_witness_multi(1, arr, 8, 1, 0, None, None, 0, fp._stream()), "fp_witness_multi")


# ------------------------------------------------- fp_layer_step_multi ---
def _small_map(fp, rng, T=64, d_in=64, d_out=96):
    X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
    Z, Y, R = O.witness(X, W, 8)
    Y_d = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    R_d = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    return fp.MatmulJob(_dev(X), fp.pack_weights(_dev(W)), Y_d, R_d), (Y, R)


@pytest.mark.parametrize("insts", [[(1, 1)], [(1, 12)], [(1, 13)], [(1, 14)], [(3, 12), (2, 9)], [(7, 14)],
                                   [(8, 16), (1, 5), (5, 13), (2, 3)], [(2, 18)]])
def test_layer_step_multi_sumchecks(fp, insts):
    """Whole sum-check instances run by single workgroups of the step launch (streamed rounds, then the register
    tail; i0 from 0 to 9), with and without rho, beside a GEMM: rounds, finals and the initial claim equal the
    oracle's sum-check, on two calls in a row."""
    rng = _rng(zlib.crc32(repr(insts).encode()))
    job, (Y, R) = _small_map(fp, rng)
    scs, wants = [], []
    for idx, (k, n) in enumerate(insts):
        As = [_field(rng, 1 << n) for _ in range(k)]
        Bs = [_field(rng, 1 << n) for _ in range(k)]
        r = _field(rng, n)
        rho = [int(v) for v in _field(rng, k)] if idx % 2 == 0 else None
        wants.append(O.sumcheck(As, Bs, r, rho=rho))
        scs.append(fp.SumcheckJob([fp.to_field_tensor(a) for a in As], [fp.to_field_tensor(b) for b in Bs],
                                  fp.to_field_tensor(r), torch.empty((n, 3), dtype=torch.int64, device="cuda"),
                                  torch.empty((k, 2), dtype=torch.int64, device="cuda"),
                                  torch.empty(1, dtype=torch.int64, device="cuda"),
                                  rho=fp.to_field_tensor(np.array(rho, np.uint64)) if rho else None))
    ws = fp.StepWorkspace()
    for rep in range(2):
        for j in scs:
            j.rounds.fill_(-1)
            j.claim0.fill_(-1)
        fp.layer_step_multi([job], 8, sumchecks=scs, ws=ws)
        torch.cuda.synchronize()
        for j, (rounds, finals, claim0) in zip(scs, wants):
            assert np.array_equal(fp.field_numpy(j.rounds), rounds)
            assert np.array_equal(fp.field_numpy(j.finals).reshape(-1, 2), finals)
            assert int(fp.field_numpy(j.claim0)[0]) == claim0
        assert np.array_equal(job.Y.cpu().numpy(), Y) and np.array_equal(job.R.cpu().numpy(), R)
        assert int(ws.buf[:512 + 16384].count_nonzero()) == 0


def test_layer_step_multi_folds_claims_and_eq(fp):
    """All the parts in one launch: two maps' GEMMs with claims from the accumulators, eleven folds of other
    tables (int8, ragged, padded columns) in arrival mode, eq tables and a sum-check: every output equals the
    oracle's, and the arrival counters are zero after each of two calls."""
    rng = _rng(909)
    T = 300
    maps, wants = [], []
    rt = _field(rng, 9)
    Et = fp.to_field_tensor(O.eq_table(rt))
    for d_in, d_out in ((1024, 700), (512, 256)):
        X, W = _i8(rng, (T, d_in)), _i8(rng, (d_out, d_in))
        ro = _field(rng, (d_out - 1).bit_length())
        Z, Y, R = O.witness(X, W, 8)
        wants.append((Y, R, O.mle_matrix(Z, rt, ro)))
        maps.append(fp.MatmulJob(_dev(X), fp.pack_weights(_dev(W)), torch.empty((T, d_out), dtype=torch.int8,
                                 device="cuda"), torch.empty((T, d_out), dtype=torch.int8, device="cuda"), None, Et,
                                 fp.to_field_tensor(O.eq_table(ro)), torch.empty(1, dtype=torch.int64, device="cuda")))
    folds, fwant = [], []
    for (rows, cols, cp) in [(300, 1000, 1024), (1, 16, 16), (4100, 96, 128), (77, 4096, 4096), (2048, 5120, 8192),
                             (700, 200, 256), (33, 1024, 1024), (14336, 256, 256), (5, 5, 8), (64, 64, 128),
                             (1000, 300, 512)]:
        M = _i8(rng, (rows, cols))
        E = _field(rng, rows)
        out = torch.full((cp,), -1, dtype=torch.int64, device="cuda")
        folds.append((_dev(M), fp.to_field_tensor(E), cp, out))
        fwant.append(O.fold_rows(M, E, cp))
    re = [_field(rng, 12), _field(rng, 3)]
    Es = [torch.empty(1 << 12, dtype=torch.int64, device="cuda"), torch.empty(8, dtype=torch.int64, device="cuda")]
    As, Bs, r = [_field(rng, 1 << 13)], [_field(rng, 1 << 13)], _field(rng, 13)
    sc = fp.SumcheckJob([fp.to_field_tensor(As[0])], [fp.to_field_tensor(Bs[0])], fp.to_field_tensor(r),
                        torch.empty((13, 3), dtype=torch.int64, device="cuda"),
                        torch.empty((1, 2), dtype=torch.int64, device="cuda"))
    swant = O.sumcheck(As, Bs, r)
    ws = fp.StepWorkspace()
    for rep in range(2):
        for (_, _, _, out) in folds:
            out.fill_(-1)
        fp.layer_step_multi(maps, 8, group_o=2, eq=[(fp.to_field_tensor(x), E) for x, E in zip(re, Es)],
                            folds=folds, sumchecks=[sc], ws=ws)
        torch.cuda.synchronize()
        for j, (Y, R, c) in zip(maps, wants):
            assert np.array_equal(j.Y.cpu().numpy(), Y) and np.array_equal(j.R.cpu().numpy(), R)
            assert int(fp.field_numpy(j.claim)[0]) == c
        for (_, _, _, out), w in zip(folds, fwant):
            assert np.array_equal(fp.field_numpy(out), w)
        for x, E in zip(re, Es):
            assert np.array_equal(fp.field_numpy(E), O.eq_table(x))
        assert np.array_equal(fp.field_numpy(sc.rounds), swant[0])
        assert np.array_equal(fp.field_numpy(sc.finals).reshape(-1, 2), swant[1])
        assert int(ws.buf[:512 + 16384].count_nonzero()) == 0


def test_layer_step_two_vector_folds(fp):
    """Folds of one int8 matrix by two row-weight vectors from one read (the weight folds of two proofs of a
    layer): mixed with one-vector folds in the step launches (fp_layer_step_multi and fp_layer_step), ragged
    and padded, one chunk and many, unaligned rows; both folded rows equal the oracle's on two calls in a row
    with the arrival counters zero after each; the other fold calls and a half-given pair are refused."""
    rng = _rng(4242)
    job, (Y, R) = _small_map(fp, rng)
    folds, fwant = [], []
    for idx, (rows, cols, cp) in enumerate([(300, 1000, 1024), (1, 16, 16), (4100, 96, 128), (77, 4096, 4096),
                                            (14336, 256, 256), (5, 5, 8), (2048, 5120, 8192), (1000, 300, 512)]):
        M = _i8(rng, (rows, cols))
        E, E2 = _field(rng, rows), _field(rng, rows)
        out = torch.full((cp,), -1, dtype=torch.int64, device="cuda")
        f = (_dev(M), fp.to_field_tensor(E), cp, out)
        w = [O.fold_rows(M, E, cp)]
        if idx != 3:
            f += (fp.to_field_tensor(E2), torch.full((cp,), -1, dtype=torch.int64, device="cuda"))
            w.append(O.fold_rows(M, E2, cp))
        folds.append(f)
        fwant.append(w)
    # one workspace per entry point: their arrival counters sit at different offsets
    wss = [fp.StepWorkspace(), fp.StepWorkspace()]
    for call in range(4):
        ws = wss[call % 2]
        for f in folds:
            for o in f[3::2]:
                o.fill_(-1)
        if call % 2 == 0:
            fp.layer_step_multi([job], 8, folds=folds, ws=ws)
        else:
            Z = torch.empty((job.X.shape[0], job.Wp.d_out), dtype=torch.int32, device="cuda")
            fp.layer_step(job.X, job.Wp, 8, Z, job.Y, job.R, folds=folds[:4], ws=ws)  # at most four jobs
        torch.cuda.synchronize()
        for f, w in zip(folds if call % 2 == 0 else folds[:4], fwant):
            assert np.array_equal(fp.field_numpy(f[3]), w[0])
            if len(f) > 4:
                assert np.array_equal(fp.field_numpy(f[5]), w[1])
        assert np.array_equal(job.Y.cpu().numpy(), Y) and np.array_equal(job.R.cpu().numpy(), R)
        # the arrival counters: the multi launch's map counters and then the folds', or the folds' alone
        assert int(ws.buf[:(512 if call % 2 == 0 else 0) + 16384].count_nonzero()) == 0
    with pytest.raises(RuntimeError):
        fp.fold_matrix_batched([folds[0]])
    with pytest.raises(RuntimeError):
        fp.fold_claim_batched([folds[0]], [])
    M, E, cp, out, E2, out2 = folds[0]
    half = fp._FoldDesc(M.data_ptr(), fp._ld(M), M.shape[0], M.shape[1], cp, E.data_ptr(), out.data_ptr(),
                        E2.data_ptr(), None)
    arr = fp._multi_descs([job])
    fd = (fp._FoldDesc * 1)(half)
    sd = (fp._SumcheckDesc * 1)()
    with pytest.raises(RuntimeError):
        fp._check(fp.lib().fp_layer_step_multi(1, arr, 8, 1, 0, None, 1, fd, 0, sd, wss[0].buf.data_ptr(),
                                               wss[0].buf.numel(), fp._stream()), "fp_layer_step_multi")


# ------------------------------------------------ fp_witness_grouped_packed ---
@pytest.mark.parametrize("rows,d_in,d_out,claims,keep_z,fold", [
    ([5, 0, 40, 1, 300, 33], 96, 700, True, False, True), ([1, 2, 3], 64, 256, True, True, False),
    ([0, 0, 129], 2000, 31, True, True, True), ([32, 64, 17], 512, 300, False, True, True),
    ([0, 0], 64, 64, True, False, True), ([7, 40], 5120, 8192, True, False, True)])
def test_witness_grouped_packed(fp, rows, d_in, d_out, claims, keep_z, fold):
    """Groups of rows (empty ones included) each with their own packed weights: Y, R (and Z) of every group,
    every non-empty group's claim from the accumulators and its weight fold sum_o E_o[o] W[o, k] from the same
    pass (ragged panels, padded columns) against the oracle, on two calls in a row; the counters are zero after
    each call."""
    rng = _rng(zlib.crc32(repr((rows, d_in, d_out)).encode()))
    G = len(rows)
    row_off = [0]
    for r in rows:
        row_off.append(row_off[-1] + r)
    T = row_off[-1]
    X = _i8(rng, (T, d_in))
    Ws = [_i8(rng, (d_out, d_in)) for _ in range(G)]
    Wps = [fp.pack_weights(_dev(w)) for w in Ws]
    E_ts, Eo_h, want_c = [], [], []
    for g in range(G):
        a, b = row_off[g], row_off[g + 1]
        Et_h = _field(rng, max(1, b - a))
        Eo = _field(rng, d_out)
        E_ts.append(fp.to_field_tensor(Et_h))
        Eo_h.append(Eo)
        if b > a:
            Z, _, _ = O.witness(X[a:b], Ws[g], 8)
            want_c.append(_claim_def(Z, Et_h[:b - a], Eo))
        else:
            want_c.append(None)
    E_o = fp.to_field_tensor(np.stack(Eo_h)).reshape(G, d_out)
    c = torch.full((G,), -1, dtype=torch.int64, device="cuda")
    cols_pad = 1 << max(0, (d_in - 1).bit_length())
    wf = torch.full((G, cols_pad), -1, dtype=torch.int64, device="cuda") if fold else None
    Y = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    R = torch.empty((T, d_out), dtype=torch.int8, device="cuda")
    Z = torch.empty((T, d_out), dtype=torch.int32, device="cuda") if keep_z else None
    ws = fp.StepWorkspace()
    for rep in range(2):
        Y.fill_(3)
        R.fill_(3)
        fp.witness_grouped_packed(_dev(X), Wps, row_off, 8, Y, R, Z, E_ts if claims else None,
                                  E_o if (claims or fold) else None, c if claims else None, w_fold=wf, ws=ws)
        torch.cuda.synchronize()
        if fold:
            got = fp.field_numpy(wf).reshape(G, cols_pad)
            for g in range(G):
                if row_off[g + 1] > row_off[g]:
                    assert np.array_equal(got[g], O.fold_rows(Ws[g], Eo_h[g], cols_pad)), g
                else:
                    assert np.all(got[g] == np.uint64(2**64 - 1))  # left alone
        for g in range(G):
            a, b = row_off[g], row_off[g + 1]
            if b == a:
                continue
            wz, wy, wr = O.witness(X[a:b], Ws[g], 8)
            assert np.array_equal(Y[a:b].cpu().numpy(), wy) and np.array_equal(R[a:b].cpu().numpy(), wr)
            if keep_z:
                assert np.array_equal(Z[a:b].cpu().numpy(), wz)
            if claims:
                assert int(fp.field_numpy(c[g:g + 1])[0]) == want_c[g]
        if claims:
            assert ws.buf is None or int(ws.buf[:G * 64].count_nonzero()) == 0
