"""GPU parity of the commitment of Y and R: limb packing, Reed-Solomon
encoding by NTT (one, two and three passes; several rows; the full 2^22 -> 2^23
rows) and the salted BLAKE2b Merkle tree (leaves of one and several
compression blocks, whole small trees, the full-size tree on sampled nodes),
bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu
P = O.P


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _u64(t):
    return t.detach().cpu().numpy().view(np.uint64)


def _field(rng, shape):
    v = rng.integers(0, 2**63, size=shape, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, size=shape,
                                                                                            dtype=np.uint64)
    return np.where(v >= np.uint64(P), v - np.uint64(P), v).astype(np.uint64)


@pytest.mark.parametrize("na,nb,logn,extra", [(0, 0, 0, 0), (1, 0, 0, 0), (5, 4, 2, 1), (1000, 777, 6, 0),
                                              (3 * 4096, 3 * 4096 + 1, 12, 2), (70000, 1, 10, 0)])
def test_commit_pack(fp, na, nb, logn, extra):
    rng = np.random.default_rng(na + nb + logn)
    A = rng.integers(-128, 128, na).astype(np.int8)
    B = rng.integers(-128, 128, nb).astype(np.int8)
    if na:
        A[0] = -128
    want = O.pack_limbs(A, B, logn)
    rows = want.shape[0] + extra
    got = fp.commit_pack(_dev(A) if na else torch.empty(0, dtype=torch.int8, device="cuda"),
                         _dev(B) if nb else torch.empty(0, dtype=torch.int8, device="cuda"), logn, rows)
    torch.cuda.synchronize()
    g = _u64(got)
    assert np.array_equal(g[: want.shape[0]], want) and not g[want.shape[0]:].any()


@pytest.mark.parametrize("rows,logn", [(1, 0), (1, 1), (2, 3), (3, 7), (1, 8), (2, 9), (1, 11), (3, 12), (2, 15),
                                       (1, 16), (3, 16), (2, 17), (2, 18), (1, 19)])
def test_rs_encode(fp, rows, logn):
    rng = np.random.default_rng(100 + logn)
    msg = _field(rng, (rows, 1 << logn))
    msg[0, 0] = P - 1
    if rows > 1:
        msg[1] = P - 1
    code = fp.rs_encode(_dev(msg.view(np.int64)))
    torch.cuda.synchronize()
    assert np.array_equal(_u64(code), O.rs_encode(msg))


def test_rs_encode_strided(fp):
    rng = np.random.default_rng(7)
    logn, rows = 10, 3
    big = _field(rng, (rows, (1 << logn) + 40))
    msg_d = _dev(big.view(np.int64))[:, : 1 << logn]
    code_big = torch.full((rows, (2 << logn) + 24), -1, dtype=torch.int64, device="cuda")
    fp.rs_encode(msg_d, code=code_big[:, : 2 << logn])
    torch.cuda.synchronize()
    cb = code_big.cpu().numpy()
    assert np.array_equal(cb[:, : 2 << logn].view(np.uint64), O.rs_encode(big[:, : 1 << logn]))
    assert np.all(cb[:, 2 << logn:] == -1)


def test_rs_encode_full_rows(fp):
    # rows of 2^22 elements into 2^23, as the pages size them
    rng = np.random.default_rng(8)
    msg = _field(rng, (2, 1 << 22))
    code = _u64(fp.rs_encode(_dev(msg.view(np.int64))))
    torch.cuda.synchronize()
    assert np.array_equal(code[0], O.rs_encode(msg[:1])[0])
    for j in [0, 1, (1 << 22) + 5, (1 << 23) - 1, 3333333]:
        assert int(code[1, j]) == O.rs_eval(msg[1], j)


def _salts(rng, W):
    return rng.integers(0, 256, size=(W, O.SALT_BYTES), dtype=np.uint8)


@pytest.mark.parametrize("rows,logw", [(0, 0), (1, 0), (1, 1), (2, 4), (3, 9), (14, 5), (15, 5), (30, 3), (2, 10),
                                       (1, 12), (1, 17), (2, 18)])
def test_merkle_tree(fp, rows, logw):
    """Every node of the tree against the oracle's: widths up to 2^16 climb near the root only (up to nine levels
    per launch), 2^17 and 2^18 first take three levels per launch while a level holds 2^17 nodes or more."""
    rng = np.random.default_rng(rows * 31 + logw)
    W = 1 << logw
    code = _field(rng, (max(rows, 1), W))[:rows]
    salts = _salts(rng, W)
    code_d = _dev(code.view(np.int64)) if rows else torch.empty((0, W), dtype=torch.int64, device="cuda")
    tree = fp.merkle_commit(code_d, _dev(salts))
    torch.cuda.synchronize()
    t = tree.cpu().numpy()
    want = O.merkle_tree(code.reshape(rows, W), salts)
    flat = [d for lev in want for d in lev]
    assert len(flat) == t.shape[0]
    for i, d in enumerate(flat):
        assert bytes(t[i]) == d, i


def test_commit_layer_outputs(fp):
    # Y and R of the up-projection's shape: pack, encode (2 rows of 2^22), tree
    rng = np.random.default_rng(9)
    T, d_out = 512, 14336
    Y = rng.integers(-128, 128, size=(T, d_out), dtype=np.int8)
    R = rng.integers(-128, 128, size=(T, d_out), dtype=np.int8)
    logn = 22
    msg = fp.commit_pack(_dev(Y), _dev(R), logn)
    code = fp.rs_encode(msg)
    W = code.shape[1]
    salts = _salts(rng, W)
    tree = fp.merkle_commit(code, _dev(salts))
    torch.cuda.synchronize()
    want_msg = O.pack_limbs(Y, R, logn)
    assert np.array_equal(_u64(msg), want_msg)
    c = _u64(code)
    want_code = O.rs_encode(want_msg)
    assert np.array_equal(c, want_code)
    t = tree.cpu().numpy()
    # every leaf: the oracle's leaf message of each column (salt, then the column's elements as 8 little-endian
    # bytes), hashed by the oracle's BLAKE2b-256, against the GPU's whole leaf level
    assert bytes(t[1234567]) == O.merkle_leaf(want_code, salts, 1234567)
    msgs = np.concatenate([salts.astype(np.uint8), np.ascontiguousarray(c.T).astype("<u8").view(np.uint8)], axis=1)
    leaves = [O.blake2b(row.tobytes()) for row in msgs]
    assert leaves == [bytes(x) for x in t[:W]]
    # every level above, from the oracle's own leaves, against the GPU's whole tree
    level, off = leaves, W
    while len(level) > 1:
        level = [O.blake2b(level[2 * i] + level[2 * i + 1]) for i in range(len(level) // 2)]
        assert level == [bytes(x) for x in t[off:off + len(level)]], len(level)
        off += len(level)
