"""fp_witness_multi_noalloc (the allocation-free variant of fp_witness_multi,
its claim slots and counters in the library's scratch array) against
fp_witness_multi with a caller workspace, through the C ABI: Y, R, Z and every
claim equal on two calls in a row, the second with a smaller input; maps that
need more scratch than the array holds are refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu
P = O.P


def _field(rng, n):
    v = rng.integers(0, 2**63, size=n, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, size=n, dtype=np.uint64)
    return np.where(v >= np.uint64(P), v - np.uint64(P), v).astype(np.uint64)


def _maps(fp, rng, specs):
    """Inputs of each map and two sets of outputs (for the two entry points)."""
    out = []
    for (T, d_in, d_out, keep_z) in specs:
        X = torch.from_numpy(rng.integers(-128, 128, size=(T, d_in), dtype=np.int8)).cuda()
        W = torch.from_numpy(rng.integers(-128, 128, size=(d_out, d_in), dtype=np.int8)).cuda()
        Et = fp.to_field_tensor(_field(rng, T))
        Eo = fp.to_field_tensor(_field(rng, d_out))
        Wp = fp.pack_weights(W)
        sets = []
        for _ in range(2):
            Z = torch.full((T, d_out), 7, dtype=torch.int32, device="cuda") if keep_z else None
            Y = torch.full((T, d_out), 7, dtype=torch.int8, device="cuda")
            R = torch.full((T, d_out), 7, dtype=torch.int8, device="cuda")
            c = torch.full((1,), -1, dtype=torch.int64, device="cuda")
            sets.append(fp.MatmulJob(X, Wp, Y, R, Z, Et, Eo, c))
        out.append(sets)
    return out


def test_noalloc_matches_the_workspace_call(fp):
    rng = np.random.default_rng(4242)
    big = [(1100, 2048, 1500, False), (1100, 512, 700, True), (1100, 4096, 300, False)]
    small = [(100, 256, 96, True), (33, 64, 40, False)]
    lib = fp.lib()
    for specs in (big, small):
        maps = _maps(fp, rng, specs)
        ref = [m[0] for m in maps]
        new = [m[1] for m in maps]
        fp.witness_multi(ref, 8, group_o=2)
        arr = fp._multi_descs(new)
        fp._check(lib.fp_witness_multi_noalloc(len(new), arr, 8, 2, 0, None, fp._stream()), "fp_witness_multi_noalloc")
        torch.cuda.synchronize()
        for a, b in zip(ref, new):
            assert torch.equal(a.Y, b.Y) and torch.equal(a.R, b.R)
            if a.Z is not None:
                assert torch.equal(a.Z, b.Z)
            assert int(a.claim.item()) == int(b.claim.item())


def test_noalloc_refuses_maps_beyond_its_scratch(fp):
    """2 maps of 16384 x 65536 outputs need 2 MiB of claim slots: refused (the pointers are never read)."""
    lib = fp.lib()
    buf = torch.zeros(1 << 12, dtype=torch.int64, device="cuda")
    p = buf.data_ptr()
    d = fp._MatmulDesc(p, 16, 16384, 16, 65536, p, None, p, p, p, p, p)
    arr = (fp._MatmulDesc * 2)(d, d)
    rc = lib.fp_witness_multi_noalloc(2, arr, 8, 1, 0, None, fp._stream())
    assert rc != 0 and b"scratch" in lib.fp_last_error()
    torch.cuda.synchronize()
