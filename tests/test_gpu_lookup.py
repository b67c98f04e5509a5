"""GPU parity of the remainder lookup: the keys' product tree, the
multiplicities, the degree-3 sum-check on both sides of the single-workgroup
threshold, and the level-by-level proof of the tree, bit-exact against the
oracle (and accepted by its verifier), up to the up-projection's 7.3 M
remainders."""
import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu
P = O.P


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _f(a):
    return _dev(np.ascontiguousarray(a, np.uint64).view(np.int64))


def _u64(t):
    return t.detach().cpu().numpy().view(np.uint64)


def _field(rng, n):
    v = rng.integers(0, 2**63, size=n, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, size=n, dtype=np.uint64)
    return np.where(v >= np.uint64(P), v - np.uint64(P), v).astype(np.uint64)


def _keys(rng, n, s):
    k = rng.integers(-(1 << (s - 1)), 1 << (s - 1), n).astype(np.int8)
    if n >= 2:
        k[:2] = [-(1 << (s - 1)), (1 << (s - 1)) - 1]
    return k


def _kdev(k):
    return _dev(k) if k.size else torch.empty(0, dtype=torch.int8, device="cuda")


@pytest.mark.parametrize("n,L", [(0, 0), (1, 0), (3, 2), (27, 5), (1000, 10), (4096, 12), (70000, 17)])
def test_lookup_tree(fp, n, L):
    rng = np.random.default_rng(n + L)
    keys = _keys(rng, n, 8)
    gamma = int(_field(rng, 1)[0])
    tree = fp.lookup_tree(_kdev(keys), L, _f([gamma]))
    torch.cuda.synchronize()
    want = np.concatenate(O.product_tree(keys, L, gamma))
    assert np.array_equal(_u64(tree), want)


@pytest.mark.parametrize("n,L,s", [(0, 3, 4), (50, 6, 4), (1000, 10, 1), (100000, 17, 7), (300000, 19, 8)])
def test_lookup_counts(fp, n, L, s):
    rng = np.random.default_rng(n + s)
    keys = rng.integers(-128, 128, n).astype(np.int8)  # some keys fall outside small tables
    got = fp.lookup_counts(_kdev(keys), L, s).cpu().numpy().view(np.uint32)
    want, outside = O.lookup_counts(keys, L, s)
    assert np.array_equal(got[:-1].astype(np.int64), want) and int(got[-1]) == outside


@pytest.mark.parametrize("m", [0, 1, 2, 5, 10, 11, 12, 13, 14, 16])
def test_sumcheck3(fp, m):
    rng = np.random.default_rng(500 + m)
    E = _field(rng, 1 << m)
    V = _field(rng, 2 << m)
    V[: min(3, V.size)] = [0, 1, P - 1][: min(3, V.size)]
    r = _field(rng, m)
    rounds, finals = fp.sumcheck3_prove(_f(E), _f(V), _f(r) if m else torch.empty(0, dtype=torch.int64,
                                                                                    device="cuda"))
    torch.cuda.synchronize()
    want_r, want_f = O.sumcheck3(E, V, r)
    assert np.array_equal(_u64(rounds).reshape(-1, 4), np.asarray(want_r, np.uint64).reshape(-1, 4))
    assert [int(x) for x in _u64(finals)] == want_f


def _split(rounds, finals, L):
    out, off = [], 0
    for k in range(L):
        out.append((rounds[off:off + k], [int(x) for x in finals[k]]))
        off += k
    return out


@pytest.mark.parametrize("n,L,s", [(1, 1, 8), (3, 2, 4), (40, 6, 4), (3000, 12, 8), (50000, 16, 7)])
def test_lookup_prove(fp, n, L, s):
    rng = np.random.default_rng(n + 7 * L)
    keys = _keys(rng, n, s)
    gamma = int(synth.challenges(900 + L, 1)[0])
    chal = synth.challenges(901 + L, O.lookup_challenges_len(L))
    tree = fp.lookup_tree(_kdev(keys), L, _f([gamma]))
    rounds, finals = fp.lookup_prove(tree, L, _f(chal))
    torch.cuda.synchronize()
    lev = O.product_tree(keys, L, gamma)
    want = O.grand_product_prove(lev, chal)
    got = _split(_u64(rounds).reshape(-1, 4), _u64(finals).reshape(L, 3), L)
    for (gr, gf), (wr, wf) in zip(got, want):
        assert np.array_equal(gr, np.asarray(wr, np.uint64).reshape(-1, 4)) and gf == wf
    counts, outside = O.lookup_counts(keys, L, s)
    assert outside == 0
    assert O.grand_product_verify(int(lev[-1][0]), got, chal, L, keys, gamma, counts, s) == (0, -1)


def test_lookup_full_remainders(fp):
    # the up-projection's 512 x 14336 remainders (s = 8): 2^23 leaves
    rng = np.random.default_rng(11)
    n, L, s = 512 * 14336, 23, 8
    keys = _keys(rng, n, s)
    gamma = int(synth.challenges(1000, 1)[0])
    chal = synth.challenges(1001, O.lookup_challenges_len(L))
    kd = _dev(keys)
    tree = fp.lookup_tree(kd, L, _f([gamma]))
    rounds, finals = fp.lookup_prove(tree, L, _f(chal))
    counts = fp.lookup_counts(kd, L, s)
    torch.cuda.synchronize()
    lev = O.product_tree(keys, L, gamma)
    assert np.array_equal(_u64(tree), np.concatenate(lev))
    want_c, outside = O.lookup_counts(keys, L, s)
    assert np.array_equal(counts.cpu().numpy().view(np.uint32)[:-1].astype(np.int64), want_c) and outside == 0
    got = _split(_u64(rounds).reshape(-1, 4), _u64(finals).reshape(L, 3), L)
    assert O.grand_product_verify(int(lev[-1][0]), got, chal, L, keys, gamma, want_c, s) == (0, -1)
    # the biggest levels against the oracle's own rounds
    want = O.grand_product_prove(lev, chal)
    for k in (L - 1, L - 2):
        assert np.array_equal(got[k][0], np.asarray(want[k][0], np.uint64).reshape(-1, 4)) and got[k][1] == want[k][1]


def test_lookup_prove_many_levels(fp):
    # 2^25 leaves, ragged: 13 levels take wide launches and 25 take tails, more
    # than one launch holds of either, so both are split over two launches;
    # every level's rounds and finals against the oracle's
    rng = np.random.default_rng(25)
    L, s = 25, 8
    n = (1 << L) - 12345
    keys = _keys(rng, n, s)
    gamma = int(synth.challenges(1100, 1)[0])
    chal = synth.challenges(1101, O.lookup_challenges_len(L))
    tree = fp.lookup_tree(_dev(keys), L, _f([gamma]))
    rounds, finals = fp.lookup_prove(tree, L, _f(chal))
    torch.cuda.synchronize()
    got = _split(_u64(rounds).reshape(-1, 4), _u64(finals).reshape(L, 3), L)
    del tree, rounds, finals
    lev = O.product_tree(keys, L, gamma)
    want = O.grand_product_prove(lev, chal)
    for (gr, gf), (wr, wf) in zip(got, want):
        assert np.array_equal(gr, np.asarray(wr, np.uint64).reshape(-1, 4)) and gf == wf


# ------------------------------------------------------------- clamp lookup --
@pytest.mark.parametrize("n,L", [(0, 0), (1, 0), (5, 3), (1000, 10), (70000, 17)])
def test_lookup_tree_pairs(fp, n, L):
    rng = np.random.default_rng(400 + L)
    A, B = _field(rng, n), _field(rng, n)
    scale, offset, gamma = (int(x) for x in _field(rng, 3))
    tree = fp.lookup_tree_pairs(_f(A), _f(B), L, _f([gamma]), scale=scale, offset=offset)
    torch.cuda.synchronize()
    want = O.product_tree_field(O.pair_keys(A, B, scale, offset), L, gamma)
    assert np.array_equal(_u64(tree), np.concatenate(want))


@pytest.mark.parametrize("bits,lo", [(16, -(1 << 15)), (8, -128), (20, -(1 << 19))])
def test_lookup_counts_field(fp, bits, lo):
    rng = np.random.default_rng(410 + bits)
    n = 300000
    v = rng.integers(-300, 300, size=n)
    v[:1000] = rng.integers(lo, lo + (1 << bits), size=1000)      # anywhere in the table, past the LDS window
    v[1000:1100] = rng.integers(1 << 21, 1 << 30, size=100)       # outside it
    v[1100:1110] = -rng.integers(1 << 21, 1 << 30, size=10)
    v[1110:1112] = [lo, lo + (1 << bits) - 1]
    A = O.field_embed(v)
    A[1112] = np.uint64(P // 2 + 3)                                # a field element far from any integer key
    counts = fp.lookup_counts_field(_f(A), lo=lo, bits=bits)
    torch.cuda.synchronize()
    got = counts.cpu().numpy().view(np.uint32).astype(np.int64)
    sv = O.field_signed(A)
    k = sv - lo
    inside = (k >= 0) & (k < (1 << bits))
    assert np.array_equal(got[:-1], np.bincount(k[inside], minlength=1 << bits)) and got[-1] == int((~inside).sum())


@pytest.mark.parametrize("cid,shape", [(2, dict(T=24, d_in=1024, d_out=200)), (2, {})])
def test_clamp_lookup_layer(fp, cid, shape):
    """The clamp's lookup over a layer's committed Q and Y (the padded [2^n_t, 2^n_o] tables from the GPU
    witness): the whole tree and the multiplicities against the oracle's from its own witness, the proof
    accepted by its verifier with the table's product, and a clamped output changed on the device refused."""
    cfg = synth.config(cid, **shape)
    inp = synth.make_inputs(cfg)
    m = cfg.matmuls[0]
    X, W = _dev(inp[m.x]), _dev(inp[m.w])
    Z, _, _ = fp.witness_linear(X, W, cfg.s)
    n_t, n_o = synth.log2ceil(cfg.T), synth.log2ceil(m.d_out)
    L = n_t + n_o
    msg = torch.empty((3, 1 << L), dtype=torch.int64, device="cuda")  # one row per table: Q, R, Y
    fp.commit_tables([(Z, n_o, 0, 1, 2)], n_t, cfg.s, msg)
    Q, Y = msg[0], msg[2]
    gamma = int(synth.challenges(1200 + L, 1)[0])
    chal = synth.challenges(1201 + L, O.lookup_challenges_len(L))
    tree = fp.lookup_tree_pairs(Q, Y, L, _f([gamma]))
    counts = fp.lookup_counts_field(Q)
    rounds, finals = fp.lookup_prove(tree, L, _f(chal))
    torch.cuda.synchronize()
    Zo = O.witness(inp[m.x], inp[m.w], cfg.s)[0]
    Qo, _, Yo = O.layer_tables(Zo, cfg.s, n_t, n_o)
    keys = O.clamp_keys(Qo, Yo)
    lev = O.product_tree_field(keys, L, gamma)
    assert np.array_equal(_u64(tree), np.concatenate(lev))
    want_c, outside = O.clamp_counts(Qo)
    got_c = counts.cpu().numpy().view(np.uint32).astype(np.int64)
    assert outside == 0 and got_c[-1] == 0 and np.array_equal(got_c[:-1], want_c)
    tp = O.clamp_table_product(want_c, gamma)
    got = _split(_u64(rounds).reshape(-1, 4), _u64(finals).reshape(L, 3), L)
    assert O.grand_product_verify(int(lev[-1][0]), got, chal, L, keys, gamma, table_prod=tp) == (0, -1)
    if L <= 16:
        want = O.grand_product_prove(lev, chal)
        for (gr, gf), (wr, wf) in zip(got, want):
            assert np.array_equal(gr, np.asarray(wr, np.uint64).reshape(-1, 4)) and gf == wf
    # a clamped output moved by one on the device: its key is no row of the table
    j = int(np.nonzero(O.field_signed(Qo) > 127)[0][0])
    Y[j] = int(O.field_embed(np.array([126]))[0])
    tree2 = fp.lookup_tree_pairs(Q, Y, L, _f([gamma]))
    rounds2, finals2 = fp.lookup_prove(tree2, L, _f(chal))
    torch.cuda.synchronize()
    keys2 = keys.copy()
    keys2[j] = O.clamp_keys(Qo[j:j + 1], O.field_embed(np.array([126])))[0]
    got2 = _split(_u64(rounds2).reshape(-1, 4), _u64(finals2).reshape(L, 3), L)
    root2 = int(_u64(tree2)[-1])
    assert O.grand_product_verify(root2, got2, chal, L, keys2, gamma, table_prod=tp) == (5, L)
