"""GPU parity of the multi-request weight fold (request vectors of a batch):
fp_fold_weights_prepare against the transpose and column sums it defines,
fp_fold_matrix_multi against the oracle's request vectors, bit-exact, over
ragged shapes, split reductions, extreme weights and eq entries, strided
operands, the empty cases, and the up-projection's full weight matrix, on both
of its kernels (row-major digit rows below 16 requests, packed from 16 on)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu
P = O.P


def _rng(seed):
    return np.random.default_rng(seed)


def _field(rng, n):
    v = rng.integers(0, 2**63, size=n, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, size=n, dtype=np.uint64)
    return np.where(v >= np.uint64(P), v - np.uint64(P), v).astype(np.uint64)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _fields(fp, a):
    return _dev(np.ascontiguousarray(a, np.uint64).view(np.int64))


@pytest.mark.parametrize("rows,cols", [(1, 1), (17, 37), (300, 256), (1000, 333), (70, 4100)])
def test_fold_weights_prepare(fp, rows, cols):
    rng = _rng(rows + cols)
    M = rng.integers(-128, 128, size=(rows, cols), dtype=np.int8)
    M[0, :] = -128
    Mt, c = fp.fold_weights_prepare(_dev(M))
    torch.cuda.synchronize()
    Mt = Mt.cpu().numpy()
    assert np.array_equal(Mt[:, :rows], M.T)
    assert np.array_equal(c.cpu().numpy(), M.astype(np.int64).sum(0))


MULTI = [  # rows, cols, cols_pad, R (from 16 requests on the digit rows go through the packed-weight kernel)
    (1, 1, 1, 1), (3, 5, 8, 2), (17, 37, 64, 3), (300, 256, 256, 1), (1000, 300, 512, 8), (2500, 1030, 2048, 5),
    (1025, 257, 512, 64), (4096, 640, 1024, 64), (4097, 100, 128, 33), (70000, 64, 64, 1), (20, 2049, 4096, 70),
    (100, 96, 128, 15), (70000, 130, 256, 16),
]


@pytest.mark.parametrize("rows,cols,cols_pad,R", MULTI)
def test_fold_multi(fp, rows, cols, cols_pad, R):
    rng = _rng(rows * 13 + cols * 7 + R)
    M = rng.integers(-128, 128, size=(rows, cols), dtype=np.int8)
    M.flat[: min(5, M.size)] = [-128, 127, -128, 127, 0][: min(5, M.size)]
    Es = [_field(rng, rows) for _ in range(R)]
    Es[0][: min(3, rows)] = [P - 1, 0, 1][: min(3, rows)]  # bytes 0xFF.. and 0x00..
    if R > 1:
        Es[1][:] = P - 1
    Mt, c = fp.fold_weights_prepare(_dev(M))
    out = fp.fold_matrix_multi(Mt, c, rows, _fields(fp, np.stack(Es)), cols_pad)
    torch.cuda.synchronize()
    got = fp.field_numpy(out)
    if rows * cols * R <= 4_000_000:
        assert np.array_equal(got, O.request_vectors(M, Es, cols_pad))
    else:  # every request, a sample of columns and the padding
        ks = sorted(set([0, 1, cols - 1] + list(rng.integers(0, cols, size=24))))
        for j in range(R):
            assert np.array_equal(got[j, ks], O.fold_cols(M, Es[j], ks)), j
        assert np.all(got[:, cols:] == 0)


def test_fold_multi_eq_vectors_strided(fp):
    # eq vectors of real points, E and out with leading dims past their rows
    rng = _rng(4)
    rows, cols, R = 1 << 10, 520, 6
    M = rng.integers(-128, 128, size=(rows, cols), dtype=np.int8)
    pts = [[int(v) for v in synth.challenges(300 + j, 10)] for j in range(R)]
    Es = np.stack([O.eq_table(r) for r in pts])
    Ebig = np.zeros((R, rows + 24), np.uint64)
    Ebig[:, :rows] = Es
    Ed = _fields(fp, Ebig)[:, :rows]
    outbig = torch.full((R, 1024 + 8), -1, dtype=torch.int64, device="cuda")
    Mt, c = fp.fold_weights_prepare(_dev(M))
    fp.fold_matrix_multi(Mt, c, rows, Ed, 1024, out=outbig[:, :1024])
    torch.cuda.synchronize()
    got = fp.field_numpy(outbig)
    assert np.array_equal(got[:, :1024], O.request_vectors(M, list(Es), 1024))
    assert np.all(outbig[:, 1024:].cpu().numpy() == -1)  # nothing written past cols_pad


def test_fold_multi_empty(fp):
    M = np.zeros((0, 40), np.int8)
    Mt, c = fp.fold_weights_prepare(torch.empty((0, 40), dtype=torch.int8, device="cuda"))
    out = torch.full((3, 64), -1, dtype=torch.int64, device="cuda")
    fp.fold_matrix_multi(Mt, c, 0, torch.empty((3, 0), dtype=torch.int64, device="cuda"), 64, out=out)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0)
    # no requests, and no columns with padding
    fp.fold_matrix_multi(Mt, c, 0, torch.empty((0, 0), dtype=torch.int64, device="cuda"), 64,
                         out=torch.empty((0, 64), dtype=torch.int64, device="cuda"))
    W = _dev(np.ones((5, 0), np.int8))
    Mt2, c2 = fp.fold_weights_prepare(W)
    out2 = fp.fold_matrix_multi(Mt2, c2, 5, _fields(fp, np.ones((2, 5), np.uint64)), 4)
    torch.cuda.synchronize()
    assert np.all(out2.cpu().numpy() == 0)
    del M


def test_fold_multi_full_up_projection(fp):
    # the up-projection's weights [14336, 4096] folded by 64 requests' eq vectors
    rows, cols, R = 14336, 4096, 64
    g = torch.Generator(device="cuda").manual_seed(17)
    W = torch.randint(-128, 128, (rows, cols), dtype=torch.int8, device="cuda", generator=g)
    rng = _rng(18)
    Es = [O.eq_table([int(v) for v in synth.challenges(500 + j, 14)])[:rows] for j in range(R)]
    Mt, c = fp.fold_weights_prepare(W)
    out = fp.fold_matrix_multi(Mt, c, rows, _fields(fp, np.stack(Es)), cols)
    torch.cuda.synchronize()
    got = fp.field_numpy(out)
    Wn = W.cpu().numpy()
    ks = sorted(set([0, cols - 1] + list(rng.integers(0, cols, size=14))))
    for j in range(0, R, 7):
        assert np.array_equal(got[j, ks], O.fold_cols(Wn, Es[j], ks)), j
    # every output against the one-request fold, request by request
    for j in range(R):
        one = fp.fold_matrix(W, _fields(fp, Es[j]), cols)
        assert torch.equal(one, out[j]), j
