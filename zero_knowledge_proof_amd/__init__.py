"""MI355X (gfx950) prover for fixed-point linear layers: the witness of each
quantized matmul and the sum-check proof of its claim over Goldilocks.

This module is the thin binding over ``libfp.so`` (declared in
``include/fp.h``): it marshals torch tensors into device pointers and the
current HIP stream, and nothing else. Every step runs in the library's HIP
kernels; there is no CPU fallback. Field elements travel as int64 tensors
holding the raw 64-bit patterns of canonical values in [0, p).
"""
from __future__ import annotations

import ctypes
import os

import torch

P = 0xFFFFFFFF00000001
FP_I8, FP_I32 = 0, 1
HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp.so")
EXPORTS = [
    "fp_last_error", "fp_witness_linear", "fp_witness_linear_grouped", "fp_moe_plan", "fp_gather_rows",
    "fp_eq_table", "fp_eq_table_batched", "fp_eq_table_batched_workspace",
    "fp_fold_matrix", "fp_fold_matrix_workspace", "fp_fold_matrix_batched", "fp_fold_matrix_batched_workspace",
    "fp_mle_eval", "fp_mle_eval_workspace", "fp_sumcheck_prove", "fp_sumcheck_workspace",
    "fp_sumcheck_prove_multi", "fp_combine_claims", "fp_claim_eval_batched", "fp_claim_eval_batched_workspace",
    "fp_linear_combine", "fp_fold_claim_batched", "fp_fold_claim_batched_workspace",
    "fp_witness_linear_with_sumcheck", "fp_fold_weights_prepare", "fp_fold_matrix_multi",
    "fp_fold_matrix_multi_workspace", "fp_commit_pack", "fp_rs_encode", "fp_rs_encode_workspace",
    "fp_merkle_commit", "fp_lookup_tree", "fp_lookup_counts", "fp_sumcheck3_prove", "fp_sumcheck3_workspace",
    "fp_lookup_prove", "fp_lookup_prove_workspace", "fp_fs_init", "fp_fs_absorb", "fp_fs_challenges",
    "fp_eq_table_ext", "fp_ext_claim_combine", "fp_sumcheck_ext_fs", "fp_witness_packed_weights_bytes",
    "fp_witness_pack_weights", "fp_witness_linear_packed", "fp_witness_linear_packed_with_sumcheck",
    "fp_layer_step", "fp_layer_step_workspace", "fp_witness_multi", "fp_witness_multi_workspace",
    "fp_witness_multi_noalloc", "fp_layer_step_multi", "fp_layer_step_multi_workspace",
    "fp_witness_grouped_packed", "fp_witness_grouped_packed_workspace",
    "fp_sumcheck_ext_fs_multi", "fp_sumcheck_ext_fs_multi_workspace", "fp_commit_tables", "fp_commit_fold_ext",
    "fp_commit_fold_ext_workspace", "fp_merkle_open", "fp_lookup_tree_pairs", "fp_lookup_counts_field",
]

_lib = None


class FPError(RuntimeError):
    pass


class _EqDesc(ctypes.Structure):
    _fields_ = [("r", ctypes.c_void_p), ("n", ctypes.c_int32), ("E", ctypes.c_void_p)]


class _ClaimDesc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_void_p), ("ld", ctypes.c_int64), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("E_rows", ctypes.c_void_p), ("E_cols", ctypes.c_void_p), ("out", ctypes.c_void_p)]


class _TableDesc(ctypes.Structure):
    _fields_ = [("Z", ctypes.c_void_p), ("ldz", ctypes.c_int64), ("T", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("n_o", ctypes.c_int32), ("row_q", ctypes.c_int32), ("row_r", ctypes.c_int32),
                ("row_y", ctypes.c_int32)]


class _OpenClaim(ctypes.Structure):
    _fields_ = [("row0", ctypes.c_int32), ("nrows", ctypes.c_int32), ("z1", ctypes.c_void_p), ("n1", ctypes.c_int32),
                ("z2", ctypes.c_void_p), ("n2", ctypes.c_int32)]


class _MatmulDesc(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("T", ctypes.c_int32), ("d_in", ctypes.c_int32),
                ("d_out", ctypes.c_int32), ("Wp", ctypes.c_void_p), ("Z", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("R", ctypes.c_void_p), ("E_t", ctypes.c_void_p), ("E_o", ctypes.c_void_p), ("claim", ctypes.c_void_p)]


class _SumcheckDesc(ctypes.Structure):
    _fields_ = [("n_pairs", ctypes.c_int32), ("n", ctypes.c_int32), ("A", ctypes.c_void_p * 8),
                ("B", ctypes.c_void_p * 8), ("rho", ctypes.c_void_p), ("r", ctypes.c_void_p),
                ("rounds", ctypes.c_void_p), ("finals", ctypes.c_void_p), ("claim0", ctypes.c_void_p)]


class _FoldDesc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_void_p), ("ld", ctypes.c_int64), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("cols_pad", ctypes.c_int32), ("E", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("E2", ctypes.c_void_p), ("out2", ctypes.c_void_p)]


def _fold_desc(f):
    """(M, E, cols_pad, out) or, in the step launches, (M, E, cols_pad, out, E2, out2): M folded by E into
    out and by E2 into out2 from one read."""
    M, E, cp, out = f[:4]
    E2, out2 = f[4:6] if len(f) > 4 else (None, None)
    return _FoldDesc(M.data_ptr(), _ld(M), M.shape[0], M.shape[1], cp, E.data_ptr(), out.data_ptr(), _ptr(E2),
                     _ptr(out2))


def lib():
    """Load libfp.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FPError("libfp.so is not built (run __graft_entry__.build()): %s" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint64
        sig = {
            "fp_last_error": (ctypes.c_char_p, []),
            "fp_witness_linear": (ctypes.c_int, [vp, i64, vp, i64, i32, i32, i32, i32, vp, vp, vp, vp]),
            "fp_witness_linear_grouped": (ctypes.c_int, [vp, i64, vp, i64, vp, i32, i32, i32, i32, vp, vp, vp, vp]),
            "fp_moe_plan": (ctypes.c_int, [vp, i32, i32, vp, vp, vp]),
            "fp_gather_rows": (ctypes.c_int, [vp, i64, vp, i32, i32, vp, vp]),
            "fp_eq_table": (ctypes.c_int, [vp, i32, vp, vp]),
            "fp_eq_table_batched": (ctypes.c_int, [i32, vp, vp, sz, vp]),
            "fp_eq_table_batched_workspace": (sz, [i32]),
            "fp_fold_matrix": (ctypes.c_int, [i32, vp, i64, i32, i32, vp, vp, i32, vp, sz, vp]),
            "fp_fold_matrix_workspace": (sz, [i32, i32, i32]),
            "fp_fold_matrix_batched": (ctypes.c_int, [i32, i32, vp, vp, sz, vp]),
            "fp_fold_matrix_batched_workspace": (sz, [i32, i32, vp]),
            "fp_mle_eval": (ctypes.c_int, [i32, vp, i64, i32, i32, vp, i32, vp, i32, vp, vp, sz, vp]),
            "fp_mle_eval_workspace": (sz, [i32, i32, i32, i32, i32]),
            "fp_sumcheck_prove": (ctypes.c_int, [i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
            "fp_sumcheck_workspace": (sz, [i32, i32]),
            "fp_sumcheck_prove_multi": (ctypes.c_int, [i32, i32, vp, vp, vp, vp, vp, vp, vp]),
            "fp_combine_claims": (ctypes.c_int, [i32, vp, vp, vp, vp, vp]),
            "fp_claim_eval_batched": (ctypes.c_int, [i32, i32, vp, vp, sz, vp]),
            "fp_claim_eval_batched_workspace": (sz, [i32, i32, vp]),
            "fp_linear_combine": (ctypes.c_int, [i32, vp, vp, vp, vp]),
            "fp_fold_claim_batched": (ctypes.c_int, [i32, i32, vp, i32, i32, vp, vp, sz, vp]),
            "fp_fold_claim_batched_workspace": (sz, [i32, i32, vp, i32, i32, vp]),
            "fp_witness_linear_with_sumcheck": (ctypes.c_int, [vp, i64, vp, i64, i32, i32, i32, i32, vp, vp, vp,
                                                               i32, vp, vp, vp, i32, vp, vp, vp, vp, vp]),
            "fp_fold_weights_prepare": (ctypes.c_int, [vp, i64, i32, i32, vp, i64, vp, vp]),
            "fp_fold_matrix_multi": (ctypes.c_int, [vp, i64, vp, i32, i32, i32, vp, i64, vp, i64, i32, vp, sz, vp]),
            "fp_fold_matrix_multi_workspace": (sz, [i32, i32, i32]),
            "fp_commit_pack": (ctypes.c_int, [vp, i64, vp, i64, i32, i32, vp, vp]),
            "fp_rs_encode": (ctypes.c_int, [vp, i64, i32, i32, vp, i64, vp, sz, vp]),
            "fp_rs_encode_workspace": (sz, [i32, i32]),
            "fp_merkle_commit": (ctypes.c_int, [vp, i64, i32, i32, vp, vp, vp]),
            "fp_lookup_tree": (ctypes.c_int, [vp, i64, i32, vp, vp, vp]),
            "fp_lookup_counts": (ctypes.c_int, [vp, i64, i32, i32, vp, vp]),
            "fp_sumcheck3_prove": (ctypes.c_int, [vp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "fp_sumcheck3_workspace": (sz, [i32]),
            "fp_lookup_prove": (ctypes.c_int, [vp, i32, vp, vp, vp, vp, sz, vp]),
            "fp_lookup_prove_workspace": (sz, [i32]),
            "fp_fs_init": (ctypes.c_int, [vp, ctypes.c_char_p, i32, vp]),
            "fp_fs_absorb": (ctypes.c_int, [vp, vp, i32, vp]),
            "fp_fs_challenges": (ctypes.c_int, [vp, i32, vp, vp]),
            "fp_eq_table_ext": (ctypes.c_int, [vp, i32, vp, vp, vp]),
            "fp_ext_claim_combine": (ctypes.c_int, [vp, vp, vp]),
            "fp_sumcheck_ext_fs": (ctypes.c_int, [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]),
            "fp_witness_packed_weights_bytes": (sz, [i32, i32]),
            "fp_witness_pack_weights": (ctypes.c_int, [vp, i64, i32, i32, vp, vp]),
            "fp_witness_linear_packed": (ctypes.c_int, [vp, i64, vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp]),
            "fp_witness_linear_packed_with_sumcheck": (ctypes.c_int, [vp, i64, vp, i32, i32, i32, i32, vp, vp, vp,
                                                                      i32, vp, vp, vp, i32, vp, vp, vp, vp, i32, vp,
                                                                      vp]),
            "fp_layer_step": (ctypes.c_int, [vp, i64, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, i32, vp,
                                             i32, vp, vp, sz, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp]),
            "fp_witness_multi": (ctypes.c_int, [i32, vp, i32, i32, i32, vp, vp, sz, vp]),
            "fp_witness_multi_workspace": (sz, [i32, vp]),
            "fp_witness_multi_noalloc": (ctypes.c_int, [i32, vp, i32, i32, i32, vp, vp]),
            "fp_layer_step_multi": (ctypes.c_int, [i32, vp, i32, i32, i32, vp, i32, vp, i32, vp, vp, sz, vp]),
            "fp_layer_step_multi_workspace": (sz, [i32, vp, i32, vp, i32, vp]),
            "fp_witness_grouped_packed": (ctypes.c_int, [vp, i64, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, i64,
                                                         vp, vp, i64, i32, vp, sz, vp]),
            "fp_witness_grouped_packed_workspace": (sz, [vp, i32, i32, i32, i32]),
            "fp_layer_step_workspace": (sz, [i32, i32, i32, i32, vp, i32, vp]),
            "fp_sumcheck_ext_fs_multi": (ctypes.c_int, [i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
            "fp_sumcheck_ext_fs_multi_workspace": (sz, [i32, i32]),
            "fp_commit_tables": (ctypes.c_int, [i32, vp, i32, i32, i32, vp, i64, i32, vp]),
            "fp_commit_fold_ext": (ctypes.c_int, [vp, i64, i32, i32, vp, i32, i32, vp, vp, vp, sz, vp]),
            "fp_commit_fold_ext_workspace": (sz, [i32]),
            "fp_merkle_open": (ctypes.c_int, [vp, i64, i32, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp]),
            "fp_lookup_tree_pairs": (ctypes.c_int, [vp, vp, i64, u64, u64, i32, vp, vp, vp]),
            "fp_lookup_counts_field": (ctypes.c_int, [vp, i64, i64, i32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def require_gpu():
    """Raise unless a GPU and the built library are both present."""
    if not torch.cuda.is_available():
        raise FPError("no GPU visible: the prover runs only on the GPU")
    lib()


def _check(rc: int, name: str):
    if rc != 0:
        raise FPError("%s failed (code %d): %s" % (name, rc, lib().fp_last_error().decode()))


def _ptr(t) -> int | None:
    if t is None:
        return None
    assert t.is_cuda, "device tensor expected"
    return t.data_ptr()


def _need(t, dtype, numel: int, name: str):
    """Check a buffer handed to the library: its dtype, contiguity and at least
    numel elements (a short buffer would be written past its end on the device)."""
    if t is None:
        raise ValueError("%s: missing buffer" % name)
    if t.dtype != dtype:
        raise ValueError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.numel() and not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % name)
    if t.numel() < numel:
        raise ValueError("%s: %d elements, at least %d needed" % (name, t.numel(), numel))


def _ld(M) -> int:
    """Leading dimension of a row-major 2-D tensor (any value >= cols when it has <= 1 row)."""
    return M.stride(0) if M.shape[0] > 1 else max(M.stride(0), M.shape[1])


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev():
    return torch.device("cuda", torch.cuda.current_device())


class Workspace:
    """A growable device scratch buffer; each entry-point family keeps its own
    (calls on one stream run in order, so a family may reuse its buffer)."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=_dev())
        return self.buf.data_ptr(), self.buf.numel()


_ws_fold, _ws_claim, _ws_mle, _ws_sc = Workspace(), Workspace(), Workspace(), Workspace()
_ws_multi, _ws_rs, _ws_lookup = Workspace(), Workspace(), Workspace()
_ws_open, _ws_scx = Workspace(), Workspace()


def to_field_tensor(vals, device=None) -> torch.Tensor:
    """Field values (ints or a uint64 array) as a device int64 tensor."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(vals, dtype=np.uint64)).view(np.int64)
    return torch.from_numpy(a.copy()).to(device or _dev())


def field_numpy(t: torch.Tensor):
    """A device int64 field tensor as a numpy uint64 array."""
    return t.detach().cpu().numpy().view("uint64")


# ------------------------------------------------------------------ witness --
def witness_linear(X, W, s: int, Z=None, Y=None, R=None, with_z: bool = True):
    T, d_in = X.shape
    d_out = W.shape[0]
    assert X.dtype == torch.int8 and W.dtype == torch.int8
    assert (X.numel() == 0 or X.stride(1) == 1) and (W.numel() == 0 or W.stride(1) == 1), "rows must be contiguous"
    if with_z and Z is None:
        Z = torch.empty((T, d_out), dtype=torch.int32, device=X.device)
    Y = torch.empty((T, d_out), dtype=torch.int8, device=X.device) if Y is None else Y
    R = torch.empty((T, d_out), dtype=torch.int8, device=X.device) if R is None else R
    _check(lib().fp_witness_linear(_ptr(X), _ld(X), _ptr(W), _ld(W), T, d_in, d_out, s,
                                   _ptr(Z) if with_z else None, _ptr(Y), _ptr(R), _stream()),
           "fp_witness_linear")
    return Z, Y, R


def witness_linear_with_sumcheck(X, W, s: int, Z, Y, R, As, Bs, r, rho=None, rounds=None, finals=None, claim0=None):
    """witness_linear(X, W, s, Z, Y, R) and sumcheck_prove(As, Bs, r, rho, ...) in one launch."""
    T, d_in = X.shape
    d_out = W.shape[0]
    assert X.dtype == torch.int8 and W.dtype == torch.int8
    assert (X.numel() == 0 or X.stride(1) == 1) and (W.numel() == 0 or W.stride(1) == 1), "rows must be contiguous"
    k = len(As)
    n = r.numel()
    dev = r.device
    rounds = torch.empty((n, 3), dtype=torch.int64, device=dev) if rounds is None else rounds
    finals = torch.empty((k, 2), dtype=torch.int64, device=dev) if finals is None else finals
    claim0 = torch.empty(1, dtype=torch.int64, device=dev) if claim0 is None else claim0
    pa = (ctypes.c_void_p * k)(*[a.data_ptr() for a in As])
    pb = (ctypes.c_void_p * k)(*[b.data_ptr() for b in Bs])
    _check(lib().fp_witness_linear_with_sumcheck(_ptr(X), _ld(X), _ptr(W), _ld(W), T, d_in, d_out, s, _ptr(Z),
                                                 _ptr(Y), _ptr(R), k, pa, pb, _ptr(rho), n, _ptr(r), _ptr(rounds),
                                                 _ptr(finals), _ptr(claim0), _stream()),
           "fp_witness_linear_with_sumcheck")
    return (Z, Y, R), (rounds, finals, claim0)


class PackedWeights:
    """The weights of one layer packed for the matrix cores (fp_witness_pack_weights):
    ``data`` is the packed int8 buffer, ``d_out`` and ``d_in`` the shape of W."""

    def __init__(self, data: torch.Tensor, d_out: int, d_in: int):
        self.data, self.d_out, self.d_in = data, d_out, d_in


def pack_weights(W, out: PackedWeights | None = None) -> PackedWeights:
    d_out, d_in = W.shape
    assert W.dtype == torch.int8 and (W.numel() == 0 or W.stride(1) == 1), "rows must be contiguous"
    nbytes = lib().fp_witness_packed_weights_bytes(d_out, d_in)
    if out is not None:
        assert (out.d_out, out.d_in) == (d_out, d_in) and out.data.numel() >= nbytes
        Wp = out.data
    else:
        Wp = torch.empty(max(nbytes, 16), dtype=torch.int8, device=W.device)
    _check(lib().fp_witness_pack_weights(_ptr(W), _ld(W), d_out, d_in, _ptr(Wp), _stream()),
           "fp_witness_pack_weights")
    return PackedWeights(Wp, d_out, d_in)


def _eq_descs(eq):
    """fp_eq_desc array of (r, E) pairs (None: no tables)."""
    eq = list(eq or [])
    return len(eq), (_EqDesc * max(len(eq), 1))(*[_EqDesc(r.data_ptr() if r.numel() else None, r.numel(),
                                                          E.data_ptr()) for r, E in eq])


def witness_linear_packed(X, Wp: PackedWeights, s: int, Z=None, Y=None, R=None, with_z: bool = True, eq=None):
    """witness_linear(X, W, s) with W given packed (pack_weights(W)); eq: (r, E) pairs of eq tables
    written by the same launch (eq_table_batched of them)."""
    T, d_in = X.shape
    assert X.dtype == torch.int8 and d_in == Wp.d_in
    assert X.numel() == 0 or X.stride(1) == 1, "rows must be contiguous"
    d_out = Wp.d_out
    if with_z and Z is None:
        Z = torch.empty((T, d_out), dtype=torch.int32, device=X.device)
    Y = torch.empty((T, d_out), dtype=torch.int8, device=X.device) if Y is None else Y
    R = torch.empty((T, d_out), dtype=torch.int8, device=X.device) if R is None else R
    ne, descs = _eq_descs(eq)
    _check(lib().fp_witness_linear_packed(_ptr(X), _ld(X), _ptr(Wp.data), T, d_in, d_out, s,
                                          _ptr(Z) if with_z else None, _ptr(Y), _ptr(R), ne, descs, _stream()),
           "fp_witness_linear_packed")
    return Z, Y, R


def witness_linear_packed_with_sumcheck(X, Wp: PackedWeights, s: int, Z, Y, R, As, Bs, r, rho=None, rounds=None,
                                        finals=None, claim0=None, eq=None):
    """witness_linear_packed(X, Wp, s, Z, Y, R, eq=eq) and sumcheck_prove(As, Bs, r, rho, ...) in one launch."""
    T, d_in = X.shape
    assert X.dtype == torch.int8 and d_in == Wp.d_in
    assert X.numel() == 0 or X.stride(1) == 1, "rows must be contiguous"
    k = len(As)
    n = r.numel()
    dev = r.device
    rounds = torch.empty((n, 3), dtype=torch.int64, device=dev) if rounds is None else rounds
    finals = torch.empty((k, 2), dtype=torch.int64, device=dev) if finals is None else finals
    claim0 = torch.empty(1, dtype=torch.int64, device=dev) if claim0 is None else claim0
    pa = (ctypes.c_void_p * k)(*[a.data_ptr() for a in As])
    pb = (ctypes.c_void_p * k)(*[b.data_ptr() for b in Bs])
    _check(lib().fp_witness_linear_packed_with_sumcheck(_ptr(X), _ld(X), _ptr(Wp.data), T, d_in, Wp.d_out, s,
                                                        _ptr(Z), _ptr(Y), _ptr(R), k, pa, pb, _ptr(rho), n, _ptr(r),
                                                        _ptr(rounds), _ptr(finals), _ptr(claim0), *_eq_descs(eq),
                                                        _stream()),
           "fp_witness_linear_packed_with_sumcheck")
    return (Z, Y, R), (rounds, finals, claim0)


class StepWorkspace:
    """Workspace of fp_layer_step: arrival counters (zeroed once, here) and the
    folds' partial values."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=_dev())
        return self.buf.data_ptr(), self.buf.numel()


_ws_step = StepWorkspace()


def layer_step(X, Wp: PackedWeights, s: int, Z, Y, R, eq=None, folds=(), claims=(), As=(), Bs=(), r=None, rho=None,
               rounds=None, finals=None, claim0=None, ws: StepWorkspace | None = None, own_claim=None):
    """One launch: the witness and eq tables of a proof (as witness_linear_packed), the int8 folds
    (M, E, cols_pad, out[, E2, out2]) and int32 claims (M, E_rows, E_cols, out) of another (as fold_claim_batched), and
    the sum-check of a third (as sumcheck_prove over As, Bs, r; none when As is empty). own_claim =
    (E_t, E_o, out): the witness's own claim sum E_t[t] E_o[o] Z[t, o] from the accumulators (Z may then
    be None; E_t and E_o must be finished before the call)."""
    T, d_in = X.shape
    assert X.dtype == torch.int8 and d_in == Wp.d_in
    assert X.numel() == 0 or X.stride(1) == 1, "rows must be contiguous"
    ne, eqd = _eq_descs(eq)
    nf, nc = len(folds), len(claims)
    fd = (_FoldDesc * max(nf, 1))(*[_fold_desc(f) for f in folds])
    cd = (_ClaimDesc * max(nc, 1))(*[_ClaimDesc(M.data_ptr(), _ld(M), M.shape[0], M.shape[1], Er.data_ptr(),
                                                Ec.data_ptr(), out.data_ptr()) for (M, Er, Ec, out) in claims])
    ws = _ws_step if ws is None else ws
    cEt, cEo, cout = own_claim if own_claim is not None else (None, None, None)
    p, nb = ws.get(lib().fp_layer_step_workspace(T, Wp.d_out, int(own_claim is not None), nf, fd, nc, cd))
    k = len(As)
    pa = (ctypes.c_void_p * max(k, 1))(*[a.data_ptr() for a in As])
    pb = (ctypes.c_void_p * max(k, 1))(*[b.data_ptr() for b in Bs])
    n = r.numel() if r is not None else 0
    _check(lib().fp_layer_step(_ptr(X), _ld(X), _ptr(Wp.data), T, d_in, Wp.d_out, s, _ptr(Z), _ptr(Y), _ptr(R),
                               _ptr(cEt), _ptr(cEo), _ptr(cout),
                               ne, eqd, nf, fd, nc, cd, p, nb, k, pa, pb, _ptr(rho), n, _ptr(r), _ptr(rounds),
                               _ptr(finals), _ptr(claim0), _stream()), "fp_layer_step")


class MatmulJob:
    """One linear map of fp_witness_multi: X int8 [T, d_in], its packed weights, the outputs Y, R
    (and Z, or None) int8/int32 [T, d_out], and for the claim from the accumulators the eq tables
    E_t, E_o and the one-element claim output (all None: no claim)."""

    def __init__(self, X, Wp: PackedWeights, Y, R, Z=None, E_t=None, E_o=None, claim=None):
        self.X, self.Wp, self.Y, self.R, self.Z = X, Wp, Y, R, Z
        self.E_t, self.E_o, self.claim = E_t, E_o, claim


def _multi_descs(jobs):
    """fp_matmul_desc array of MatmulJobs (buffers checked)."""
    assert len(jobs) > 0, "no maps"
    descs = []
    for j in jobs:
        T, d_in = j.X.shape
        assert j.X.dtype == torch.int8 and d_in == j.Wp.d_in and (j.X.numel() == 0 or j.X.stride(1) == 1)
        d_out = j.Wp.d_out
        _need(j.Y, torch.int8, T * d_out, "Y")
        _need(j.R, torch.int8, T * d_out, "R")
        if j.Z is not None:
            _need(j.Z, torch.int32, T * d_out, "Z")
        if j.E_t is not None:
            _need(j.E_t, torch.int64, T, "E_t")
            _need(j.E_o, torch.int64, d_out, "E_o")
            _need(j.claim, torch.int64, 1, "claim")
        descs.append(_MatmulDesc(_ptr(j.X), _ld(j.X), T, d_in, d_out, _ptr(j.Wp.data), _ptr(j.Z), _ptr(j.Y),
                                 _ptr(j.R), _ptr(j.E_t), _ptr(j.E_o), _ptr(j.claim)))
    return (_MatmulDesc * len(descs))(*descs)


def witness_multi(jobs, s: int, group_o: int = 1, eq=None, ws: StepWorkspace | None = None):
    """The witness GEMMs of several linear maps (MatmulJob) in one launch, each map's claim
    sum_t sum_o E_t[t] E_o[o] Z[t, o] taken from its accumulators; eq: (r, E) tables of another
    proof built by the same launch."""
    arr = _multi_descs(jobs)
    ne, eqd = _eq_descs(eq)
    ws = _ws_step if ws is None else ws
    p, nb = ws.get(lib().fp_witness_multi_workspace(len(jobs), arr))
    _check(lib().fp_witness_multi(len(jobs), arr, s, group_o, ne, eqd, p, nb, _stream()), "fp_witness_multi")


class SumcheckJob:
    """One sum-check instance of layer_step_multi: pairs of tables As[j], Bs[j] (int64 [2^n]), the round
    challenges r [n], weights rho [n_pairs] or None, outputs rounds [n, 3], finals [n_pairs, 2] and claim0 [1]
    (or None)."""

    def __init__(self, As, Bs, r, rounds, finals, claim0=None, rho=None):
        self.As, self.Bs, self.r, self.rounds, self.finals, self.claim0, self.rho = As, Bs, r, rounds, finals, claim0, rho


def _sc_descs(scs):
    out = []
    for j in scs:
        n, k = j.r.numel(), len(j.As)
        assert 1 <= k <= 8 and len(j.Bs) == k
        for t in list(j.As) + list(j.Bs):
            _need(t, torch.int64, 1 << n, "sum-check table")
        _need(j.r, torch.int64, n, "r")
        _need(j.rounds, torch.int64, 3 * n, "rounds")
        _need(j.finals, torch.int64, 2 * k, "finals")
        if j.rho is not None:
            _need(j.rho, torch.int64, k, "rho")
        d = _SumcheckDesc()
        d.n_pairs, d.n = k, n
        for i in range(k):
            d.A[i], d.B[i] = j.As[i].data_ptr(), j.Bs[i].data_ptr()
        d.rho, d.r, d.rounds, d.finals, d.claim0 = _ptr(j.rho), _ptr(j.r), _ptr(j.rounds), _ptr(j.finals), _ptr(j.claim0)
        out.append(d)
    return len(out), (_SumcheckDesc * max(len(out), 1))(*out)


def _fold_descs(folds):
    nf = len(folds)
    return nf, (_FoldDesc * max(nf, 1))(*[_fold_desc(f) for f in folds])


def layer_step_multi(jobs, s: int, group_o: int = 1, eq=None, folds=(), sumchecks=(), ws: StepWorkspace | None = None):
    """One launch: the witness GEMMs and claims of a proof's maps (as witness_multi), the int8 folds
    (M, E, cols_pad, out) of another proof (as fold_matrix_batched; (M, E, cols_pad, out, E2, out2) also
    folds M by E2 into out2 from the same read) and whole sum-check instances (SumcheckJob) of a third, side
    by side."""
    arr = _multi_descs(jobs)
    ne, eqd = _eq_descs(eq)
    nf, fd = _fold_descs(folds)
    ns, sd = _sc_descs(sumchecks)
    ws = _ws_step if ws is None else ws
    p, nb = ws.get(lib().fp_layer_step_multi_workspace(len(jobs), arr, nf, fd, ns, sd))
    _check(lib().fp_layer_step_multi(len(jobs), arr, s, group_o, ne, eqd, nf, fd, ns, sd, p, nb, _stream()),
           "fp_layer_step_multi")


def witness_multi_noalloc(jobs, s: int, group_o: int = 1, eq=None):
    """witness_multi without a workspace: the library's own scratch array holds the claims' slots and
    counters (calls that overlap on one GPU race)."""
    arr = _multi_descs(jobs)
    ne, eqd = _eq_descs(eq)
    _check(lib().fp_witness_multi_noalloc(len(jobs), arr, s, group_o, ne, eqd, _stream()), "fp_witness_multi_noalloc")


def witness_grouped_packed(Xg, Wps, row_off, s: int, Y, R, Z=None, E_ts=None, E_o=None, claims=None, w_fold=None,
                           ws: StepWorkspace | None = None):
    """Grouped witness from packed weights (Wps: PackedWeights per group), rows row_off (host ints, G + 1);
    with E_ts (per-group tables), E_o (int64 [G, >= d_out]) and claims (int64 [G]) every non-empty group's
    claim sum_t sum_o E_t[t] E_o[o] Z[t, o] from the accumulators; with w_fold (int64 [G, cols_pad], E_o
    given) every non-empty group's weight fold sum_o E_o[o] W[o, k] from the same pass over the weights."""
    G = len(Wps)
    T, d_in = Xg.shape
    d_out = Wps[0].d_out if G else 0
    assert Xg.dtype == torch.int8 and (Xg.numel() == 0 or Xg.stride(1) == 1) and len(row_off) == G + 1
    assert all(w.d_in == d_in and w.d_out == d_out for w in Wps) and row_off[-1] <= T
    _need(Y, torch.int8, row_off[-1] * d_out, "Y")
    _need(R, torch.int8, row_off[-1] * d_out, "R")
    if Z is not None:
        _need(Z, torch.int32, row_off[-1] * d_out, "Z")
    ro = (ctypes.c_int32 * (G + 1))(*row_off)
    wp = (ctypes.c_void_p * max(G, 1))(*[w.data.data_ptr() for w in Wps])
    et = None
    ldeo = 0
    p, nb = None, 0
    ld_fold, cols_pad = 0, 0
    if E_o is not None:
        assert E_o.dim() == 2 and E_o.shape[0] >= G and E_o.stride(1) == 1 and E_o.dtype == torch.int64
        assert E_o.shape[1] >= d_out
        ldeo = E_o.stride(0)
    if E_ts is not None:
        for g in range(G):
            if row_off[g + 1] > row_off[g]:
                _need(E_ts[g], torch.int64, row_off[g + 1] - row_off[g], "E_t")
        _need(claims, torch.int64, G, "claims")
        et = (ctypes.c_void_p * max(G, 1))(*[e.data_ptr() for e in E_ts])
    if w_fold is not None:
        assert w_fold.dim() == 2 and w_fold.shape[0] >= G and w_fold.stride(1) == 1 and w_fold.dtype == torch.int64
        ld_fold, cols_pad = w_fold.stride(0), w_fold.shape[1]
    if E_ts is not None or w_fold is not None:
        ws = _ws_step if ws is None else ws
        p, nb = ws.get(lib().fp_witness_grouped_packed_workspace(ro, G, d_in, d_out, int(w_fold is not None)))
    _check(lib().fp_witness_grouped_packed(_ptr(Xg), _ld(Xg), wp, ro, G, d_in, d_out, s, _ptr(Z), _ptr(Y), _ptr(R),
                                           et, _ptr(E_o), ldeo, _ptr(claims), _ptr(w_fold), ld_fold, cols_pad, p, nb,
                                           _stream()), "fp_witness_grouped_packed")


def witness_linear_grouped(Xg, Ws, row_off, s: int, Z=None, Y=None, R=None, with_z: bool = True):
    """Xg: int8 [row_off[-1], d_in]; Ws: list of int8 [d_out, d_in]; row_off: host ints (G+1)."""
    G = len(Ws)
    d_in = Xg.shape[1]
    d_out = Ws[0].shape[0]
    total = int(row_off[-1])
    if with_z and Z is None:
        Z = torch.empty((total, d_out), dtype=torch.int32, device=Xg.device)
    Y = torch.empty((total, d_out), dtype=torch.int8, device=Xg.device) if Y is None else Y
    R = torch.empty((total, d_out), dtype=torch.int8, device=Xg.device) if R is None else R
    wp = (ctypes.c_void_p * G)(*[w.data_ptr() for w in Ws])
    ro = (ctypes.c_int32 * (G + 1))(*[int(v) for v in row_off])
    _check(lib().fp_witness_linear_grouped(_ptr(Xg), _ld(Xg), wp, _ld(Ws[0]), ro, G, d_in, d_out, s,
                                           _ptr(Z) if with_z else None, _ptr(Y), _ptr(R), _stream()),
           "fp_witness_linear_grouped")
    return Z, Y, R


def moe_plan(route, n_experts: int):
    """Host-only grouping plan: (counts, offsets, perm) as numpy int32 arrays."""
    import numpy as np
    route = np.ascontiguousarray(route, dtype=np.int32)
    T = len(route)
    counts = np.empty(n_experts, np.int32)
    offsets = np.empty(n_experts + 1, np.int32)
    perm = np.empty(max(T, 1), np.int32)
    _check(lib().fp_moe_plan(route.ctypes.data, T, n_experts, counts.ctypes.data, offsets.ctypes.data,
                             perm.ctypes.data), "fp_moe_plan")
    return counts, offsets, perm[:T]


def gather_rows(X, perm_dev, out=None):
    n = perm_dev.numel()
    cols = X.shape[1]
    out = torch.empty((n, cols), dtype=X.dtype, device=X.device) if out is None else out
    _check(lib().fp_gather_rows(_ptr(X), _ld(X), _ptr(perm_dev), n, cols, _ptr(out), _stream()),
           "fp_gather_rows")
    return out


# ----------------------------------------------------------------------- eq --
def eq_table(r, E=None):
    n = r.numel()
    E = torch.empty(1 << n, dtype=torch.int64, device=_dev()) if E is None else E
    _check(lib().fp_eq_table(_ptr(r) if n else None, n, _ptr(E), _stream()), "fp_eq_table")
    return E


def eq_table_batched(rs, Es=None):
    k = len(rs)
    if Es is None:
        Es = [torch.empty(1 << r.numel(), dtype=torch.int64, device=_dev()) for r in rs]
    descs = (_EqDesc * k)(*[_EqDesc(r.data_ptr() if r.numel() else None, r.numel(), E.data_ptr())
                            for r, E in zip(rs, Es)])
    _check(lib().fp_eq_table_batched(k, descs, None, 0, _stream()), "fp_eq_table_batched")
    return Es


# -------------------------------------------------------------------- folds --
def _dt(M):
    if M.dtype == torch.int8:
        return FP_I8
    if M.dtype == torch.int32:
        return FP_I32
    raise TypeError(M.dtype)


def fold_matrix(M, E, cols_pad: int | None = None, rows: int | None = None, out=None):
    rows = M.shape[0] if rows is None else rows
    cols = M.shape[1]
    cols_pad = cols if cols_pad is None else cols_pad
    out = torch.empty(cols_pad, dtype=torch.int64, device=M.device) if out is None else out
    need = lib().fp_fold_matrix_workspace(_dt(M), rows, cols)
    p, nb = _ws_fold.get(need)
    _check(lib().fp_fold_matrix(_dt(M), _ptr(M), _ld(M), rows, cols, _ptr(E), _ptr(out), cols_pad, p, nb,
                                _stream()), "fp_fold_matrix")
    return out


def fold_matrix_batched(jobs):
    """jobs: list of (M, E, cols_pad, out); all M of one dtype."""
    k = len(jobs)
    dt = _dt(jobs[0][0])
    descs = (_FoldDesc * k)(*[_fold_desc(f) for f in jobs])
    need = lib().fp_fold_matrix_batched_workspace(dt, k, descs)
    p, nb = _ws_fold.get(need)
    _check(lib().fp_fold_matrix_batched(dt, k, descs, p, nb, _stream()), "fp_fold_matrix_batched")
    return [j[3] for j in jobs]


def fold_weights_prepare(M, Mt=None, colsum=None):
    """Transposed copy Mt [cols, ldt] (ldt = rows rounded up to 16) and column
    sums [cols] int32 of an int8 matrix M [rows, cols], for fold_matrix_multi."""
    rows, cols = M.shape
    ldt = max(16, (rows + 15) // 16 * 16)
    Mt = torch.empty((cols, ldt), dtype=torch.int8, device=M.device) if Mt is None else Mt
    colsum = torch.empty(cols, dtype=torch.int32, device=M.device) if colsum is None else colsum
    assert Mt.dtype == torch.int8 and Mt.shape[0] == cols and Mt.stride(1) == 1
    _check(lib().fp_fold_weights_prepare(_ptr(M) if M.numel() else None, _ld(M), rows, cols,
                                         _ptr(Mt) if Mt.numel() else None, Mt.stride(0), _ptr(colsum), _stream()),
           "fp_fold_weights_prepare")
    return Mt, colsum


def fold_matrix_multi(Mt, colsum, rows: int, E, cols_pad: int | None = None, out=None):
    """out[j, k] = sum_t E[j, t] M[t, k] for every row j of E [R, >= rows]
    (int64 field tensor), from fold_weights_prepare's Mt and colsum."""
    cols = Mt.shape[0]
    R = E.shape[0]
    cols_pad = cols if cols_pad is None else cols_pad
    out = torch.empty((R, cols_pad), dtype=torch.int64, device=Mt.device) if out is None else out
    assert E.dtype == torch.int64 and E.stride(1) == 1 and out.stride(1) == 1
    lde = E.stride(0) if R > 1 else max(E.stride(0), rows)
    ldo = out.stride(0) if R > 1 else max(out.stride(0), cols_pad)
    need = lib().fp_fold_matrix_multi_workspace(rows, cols, R)
    p, nb = _ws_multi.get(need)
    _check(lib().fp_fold_matrix_multi(_ptr(Mt) if Mt.numel() else None, Mt.stride(0), _ptr(colsum), rows, cols, R,
                                      _ptr(E) if E.numel() else None, lde, _ptr(out) if out.numel() else None, ldo,
                                      cols_pad, p, nb, _stream()), "fp_fold_matrix_multi")
    return out


# --------------------------------------------------------------- commitment --
SALT_BYTES, DIGEST_BYTES = 16, 32


def commit_rows(na: int, nb: int, logn: int) -> int:
    """Rows of 2^logn elements that hold na + nb limbs, three per element."""
    elems = (na + nb + 2) // 3
    return max(1, (elems + (1 << logn) - 1) >> logn)


def commit_pack(A, B, logn: int, rows: int | None = None, out=None):
    """Limbs of the int8 tensors A then B, three per field element in 20-bit
    slots, as [rows, 2^logn] (zero past the limbs)."""
    na, nb = A.numel(), B.numel()
    rows = commit_rows(na, nb, logn) if rows is None else rows
    dev = A.device if na else B.device
    out = torch.empty((rows, 1 << logn), dtype=torch.int64, device=dev) if out is None else out
    assert out.is_contiguous() and A.is_contiguous() and B.is_contiguous()
    _check(lib().fp_commit_pack(_ptr(A) if na else None, na, _ptr(B) if nb else None, nb, logn, rows, _ptr(out),
                                _stream()), "fp_commit_pack")
    return out


def rs_encode(msg, code=None):
    """Rate-1/2 Reed-Solomon codewords [rows, 2n] of the rows of msg [rows, n]."""
    rows, n = msg.shape
    logn = n.bit_length() - 1
    assert 1 << logn == n and msg.stride(1) == 1
    code = torch.empty((rows, 2 * n), dtype=torch.int64, device=msg.device) if code is None else code
    need = lib().fp_rs_encode_workspace(rows, logn)
    p, nbytes = _ws_rs.get(need)
    _check(lib().fp_rs_encode(_ptr(msg), msg.stride(0) if rows > 1 else n, rows, logn, _ptr(code),
                              code.stride(0) if rows > 1 else 2 * n, p, nbytes, _stream()), "fp_rs_encode")
    return code


def merkle_commit(code, salts, tree=None):
    """Salted BLAKE2b-256 Merkle tree over the columns of code [rows, W]
    (W a power of 2); salts: uint8 [W, 16]. Returns the tree as uint8
    [2W - 1, 32]: the W leaves, then each level up, the root last."""
    rows, W = code.shape
    logw = W.bit_length() - 1
    assert 1 << logw == W and salts.shape == (W, SALT_BYTES) and salts.is_contiguous()
    tree = torch.empty((2 * W - 1, DIGEST_BYTES), dtype=torch.uint8, device=code.device) if tree is None else tree
    _check(lib().fp_merkle_commit(_ptr(code), code.stride(0) if rows > 1 else W, rows, logw, _ptr(salts),
                                  _ptr(tree), _stream()), "fp_merkle_commit")
    return tree


# ------------------------------------------------------------------- lookup --
def lookup_tree(keys, L: int, gamma, tree=None):
    """Product tree [2^(L+1) - 1] of the leaves gamma - key (int8 keys, padded
    with 0 to 2^L), levels from the leaves up; gamma: device int64 [1]."""
    n = keys.numel()
    _need(keys, torch.int8, n, "keys")
    assert 0 <= L <= 30 and n <= (1 << L), "keys must fit the 2^L leaves"
    _need(gamma, torch.int64, 1, "gamma")
    tree = torch.empty((2 << L) - 1, dtype=torch.int64, device=gamma.device) if tree is None else tree
    _need(tree, torch.int64, (2 << L) - 1, "tree")
    _check(lib().fp_lookup_tree(_ptr(keys) if n else None, n, L, _ptr(gamma), _ptr(tree), _stream()),
           "fp_lookup_tree")
    return tree


CLAMP_SCALE, CLAMP_OFFSET, CLAMP_BITS = 1 << 16, (1 << 15) + (128 << 16), 16


def lookup_tree_pairs(A, B, L: int, gamma, scale: int = CLAMP_SCALE, offset: int = CLAMP_OFFSET, tree=None):
    """Product tree [2^(L+1) - 1] of the leaves gamma - (A + scale B + offset) of two field tables of 2^L
    entries (by default the clamp's keys of Q = A and Y = B)."""
    n = A.numel()
    _need(A, torch.int64, n, "A")
    _need(B, torch.int64, n, "B")
    assert n <= (1 << L) and B.numel() == n
    _need(gamma, torch.int64, 1, "gamma")
    tree = torch.empty((2 << L) - 1, dtype=torch.int64, device=A.device) if tree is None else tree
    _need(tree, torch.int64, (2 << L) - 1, "tree")
    _check(lib().fp_lookup_tree_pairs(_ptr(A), _ptr(B), n, scale % P, offset % P, L, _ptr(gamma), _ptr(tree),
                                      _stream()), "fp_lookup_tree_pairs")
    return tree


def lookup_counts_field(A, lo: int = -(1 << 15), bits: int = CLAMP_BITS, counts=None):
    """Multiplicities [2^bits + 1] of the field values A read as signed integers over [lo, lo + 2^bits) (the
    last entry: values outside)."""
    n = A.numel()
    _need(A, torch.int64, n, "A")
    counts = torch.empty((1 << bits) + 1, dtype=torch.int32, device=A.device) if counts is None else counts
    _need(counts, torch.int32, (1 << bits) + 1, "counts")
    _check(lib().fp_lookup_counts_field(_ptr(A), n, lo, bits, _ptr(counts), _stream()), "fp_lookup_counts_field")
    return counts


def lookup_counts(keys, L: int, s: int, counts=None):
    """Multiplicities [2^s + 1] (int32 holding uint32) of the table values
    -2^(s-1) + i among the padded keys; the last entry counts keys outside."""
    n = keys.numel()
    dev = keys.device if n else _dev()
    _need(keys, torch.int8, n, "keys")
    assert 1 <= s <= 8, "s outside [1, 8]"
    counts = torch.empty((1 << s) + 1, dtype=torch.int32, device=dev) if counts is None else counts
    _need(counts, torch.int32, (1 << s) + 1, "counts")
    _check(lib().fp_lookup_counts(_ptr(keys) if n else None, n, L, s, _ptr(counts), _stream()), "fp_lookup_counts")
    return counts


def sumcheck3_prove(E, V, r, rounds=None, finals=None):
    """Degree-3 sum-check of sum_x E[x] V[2x] V[2x+1]: rounds [m, 4], finals [3]."""
    m = r.numel()
    dev = E.device
    rounds = torch.empty((max(m, 1), 4), dtype=torch.int64, device=dev) if rounds is None else rounds
    finals = torch.empty(3, dtype=torch.int64, device=dev) if finals is None else finals
    _need(E, torch.int64, 1 << m, "E")
    _need(V, torch.int64, 2 << m, "V")
    _need(r, torch.int64, m, "r")
    _need(rounds, torch.int64, 4 * m, "rounds")
    _need(finals, torch.int64, 3, "finals")
    need = lib().fp_sumcheck3_workspace(m)
    p, nbytes = _ws_lookup.get(need)
    _check(lib().fp_sumcheck3_prove(_ptr(E), _ptr(V), m, _ptr(r) if m else None, _ptr(rounds), _ptr(finals), p,
                                    nbytes, _stream()), "fp_sumcheck3_prove")
    return rounds[:m], finals


def lookup_prove(tree, L: int, chal, rounds=None, finals=None):
    """The product tree's proof: rounds [L(L-1)/2, 4] and finals [L, 3], levels
    from the root down; chal: device int64 [L(L+1)/2]."""
    dev = tree.device
    nr = L * (L - 1) // 2
    rounds = torch.empty((max(nr, 1), 4), dtype=torch.int64, device=dev) if rounds is None else rounds
    finals = torch.empty((L, 3), dtype=torch.int64, device=dev) if finals is None else finals
    _need(tree, torch.int64, (2 << L) - 1, "tree")
    _need(chal, torch.int64, L * (L + 1) // 2, "chal")
    _need(rounds, torch.int64, 4 * nr, "rounds")
    _need(finals, torch.int64, 3 * L, "finals")
    need = lib().fp_lookup_prove_workspace(L)
    p, nbytes = _ws_lookup.get(need)
    _check(lib().fp_lookup_prove(_ptr(tree), L, _ptr(chal), _ptr(rounds), _ptr(finals), p, nbytes, _stream()),
           "fp_lookup_prove")
    return rounds[:nr], finals


# ---------------------------------------------- soundness-faithful challenges --
def fs_init(state, msg: bytes):
    """state (device uint8 [32], 8-byte aligned) <- BLAKE2b-256(msg), msg <= 128 bytes."""
    _check(lib().fp_fs_init(_ptr(state), msg, len(msg), _stream()), "fp_fs_init")
    return state


def fs_absorb(state, data):
    """state <- BLAKE2b-256(state || data), data a device int64 tensor of words."""
    _check(lib().fp_fs_absorb(_ptr(state), _ptr(data) if data.numel() else None, data.numel(), _stream()),
           "fp_fs_absorb")
    return state


def fs_challenges(state, k: int, out=None):
    """k extension challenges [k, 2] read from the state."""
    out = torch.empty((max(k, 1), 2), dtype=torch.int64, device=state.device) if out is None else out
    _check(lib().fp_fs_challenges(_ptr(state), k, _ptr(out), _stream()), "fp_fs_challenges")
    return out[:k]


def eq_table_ext(r, E0=None, E1=None):
    """(E0, E1): eq over the extension at r [n, 2]."""
    n = r.shape[0]
    dev = r.device
    E0 = torch.empty(1 << n, dtype=torch.int64, device=dev) if E0 is None else E0
    E1 = torch.empty(1 << n, dtype=torch.int64, device=dev) if E1 is None else E1
    _check(lib().fp_eq_table_ext(_ptr(r) if n else None, n, _ptr(E0), _ptr(E1), _stream()), "fp_eq_table_ext")
    return E0, E1


def ext_claim_combine(c4, c0=None):
    c0 = torch.empty(2, dtype=torch.int64, device=c4.device) if c0 is None else c0
    _check(lib().fp_ext_claim_combine(_ptr(c4), _ptr(c0), _stream()), "fp_ext_claim_combine")
    return c0


def sumcheck_ext_fs(A0, A1, B0, B1, state, rounds=None, r=None, finals=None):
    """Extension sum-check with the transcript: rounds [n, 3, 2], r [n, 2], finals [2, 2]."""
    n = A0.numel().bit_length() - 1
    dev = A0.device
    rounds = torch.empty((max(n, 1), 3, 2), dtype=torch.int64, device=dev) if rounds is None else rounds
    r = torch.empty((max(n, 1), 2), dtype=torch.int64, device=dev) if r is None else r
    finals = torch.empty((2, 2), dtype=torch.int64, device=dev) if finals is None else finals
    _check(lib().fp_sumcheck_ext_fs(_ptr(A0), _ptr(A1), _ptr(B0), _ptr(B1), n, _ptr(state), _ptr(rounds), _ptr(r),
                                    _ptr(finals), _stream()), "fp_sumcheck_ext_fs")
    return rounds[:n], r[:n], finals


def sumcheck_ext_fs_multi(A0s, A1s, B0s, B1s, state, rho=None, rounds=None, r=None, finals=None):
    """Extension sum-check of sum_j rho_j sum_k A_j[k] B_j[k] (A_j = A0s[j] + u A1s[j], 1..8 pairs of int64
    [2^n] tables; rho device [n_pairs, 2] or None) with the transcript: rounds [n, 3, 2], r [n, 2],
    finals [n_pairs, 2, 2]."""
    k = len(A0s)
    assert 1 <= k <= 8 and len(A1s) == len(B0s) == len(B1s) == k
    N = A0s[0].numel()
    n = N.bit_length() - 1
    assert N == 1 << n
    for t in list(A0s) + list(A1s) + list(B0s) + list(B1s):
        _need(t, torch.int64, N, "sum-check table")
    dev = A0s[0].device
    rounds = torch.empty((max(n, 1), 3, 2), dtype=torch.int64, device=dev) if rounds is None else rounds
    r = torch.empty((max(n, 1), 2), dtype=torch.int64, device=dev) if r is None else r
    finals = torch.empty((k, 2, 2), dtype=torch.int64, device=dev) if finals is None else finals
    _need(rounds, torch.int64, 6 * n, "rounds")
    _need(r, torch.int64, 2 * n, "r")
    _need(finals, torch.int64, 4 * k, "finals")
    assert state.is_contiguous() and state.numel() * state.element_size() >= 32, "state: 32 bytes"
    if rho is not None:
        _need(rho, torch.int64, 2 * k, "rho")
    arr = lambda ts: (ctypes.c_void_p * k)(*[t.data_ptr() for t in ts])
    p, nb = _ws_scx.get(lib().fp_sumcheck_ext_fs_multi_workspace(k, n))
    _check(lib().fp_sumcheck_ext_fs_multi(k, arr(A0s), arr(A1s), arr(B0s), arr(B1s), _ptr(rho), n, _ptr(state),
                                          _ptr(rounds), _ptr(r), _ptr(finals), p, nb, _stream()),
           "fp_sumcheck_ext_fs_multi")
    return rounds[:n], r[:n], finals


def commit_tables(maps, n_t: int, s: int, msg):
    """Each map's Q (before the clamp), R and Y as zero-padded [2^n_t, 2^n_o] field tables in whole rows of
    msg [rows, 2^L]; maps: (Z int32 [T, d_out], n_o, row_q, row_r, row_y)."""
    rows, cols = msg.shape
    L = cols.bit_length() - 1
    assert 1 << L == cols and msg.is_contiguous() and msg.dtype == torch.int64
    descs = []
    for Z, n_o, rq, rr, ry in maps:
        T, d_out = Z.shape
        _need(Z, torch.int32, T * d_out, "Z")
        descs.append(_TableDesc(_ptr(Z) if Z.numel() else None, max(d_out, 1), T, d_out, n_o, rq, rr, ry))
    arr = (_TableDesc * len(descs))(*descs)
    _check(lib().fp_commit_tables(len(descs), arr, n_t, s, L, _ptr(msg), cols, rows, _stream()), "fp_commit_tables")
    return msg


def commit_fold_ext(msg, r_prox, claims, U):
    """Folded rows over the extension of msg [rows, 2^L]: U [1 + len(claims), 2, 2^L] receives the proximity row
    (row weights eq(r_prox, i); r_prox [n_prox, 2]) and each claim's row; claims: (row0, z1 [n1, 2], z2 [n2, 2])
    with 2^(n1 + n2) rows from row0, sorted and disjoint."""
    rows, cols = msg.shape
    L = cols.bit_length() - 1
    assert 1 << L == cols and msg.is_contiguous() and msg.dtype == torch.int64
    _need(U, torch.int64, (1 + len(claims)) * 2 * cols, "U")
    cs = []
    for row0, z1, z2 in claims:
        n1, n2 = z1.shape[0], z2.shape[0]
        for z in (z1, z2):
            assert z.dtype == torch.int64 and (z.numel() == 0 or z.is_contiguous())
        cs.append(_OpenClaim(row0, 1 << (n1 + n2), _ptr(z1) if n1 else None, n1, _ptr(z2) if n2 else None, n2))
    arr = (_OpenClaim * max(1, len(cs)))(*cs)
    n_prox = r_prox.shape[0]
    assert r_prox.dtype == torch.int64 and r_prox.is_contiguous()
    p, nb = _ws_open.get(lib().fp_commit_fold_ext_workspace(rows))
    _check(lib().fp_commit_fold_ext(_ptr(msg), cols, rows, L, _ptr(r_prox) if n_prox else None, n_prox, len(cs), arr,
                                    _ptr(U), p, nb, _stream()), "fp_commit_fold_ext")
    return U


def merkle_open(code, salts, tree, chal, cols=None, col_salts=None, paths=None, idx=None):
    """Columns j = chal[q, 0] mod W of code [rows, W] with their salts and Merkle paths: cols [nq, rows] int64,
    col_salts [nq, 16] uint8, paths [nq, log2 W, 32] uint8, idx [nq] int32."""
    rows, W = code.shape
    logw = W.bit_length() - 1
    nq = chal.shape[0]
    assert 1 << logw == W and code.is_contiguous() and chal.dtype == torch.int64 and chal.is_contiguous()
    _need(salts, torch.uint8, W * SALT_BYTES, "salts")
    _need(tree, torch.uint8, (2 * W - 1) * DIGEST_BYTES, "tree")
    dev = code.device
    cols = torch.empty((nq, rows), dtype=torch.int64, device=dev) if cols is None else cols
    col_salts = torch.empty((nq, SALT_BYTES), dtype=torch.uint8, device=dev) if col_salts is None else col_salts
    paths = torch.empty((nq, logw, DIGEST_BYTES), dtype=torch.uint8, device=dev) if paths is None else paths
    idx = torch.empty(nq, dtype=torch.int32, device=dev) if idx is None else idx
    _need(cols, torch.int64, nq * rows, "cols")
    _need(col_salts, torch.uint8, nq * SALT_BYTES, "col_salts")
    _need(paths, torch.uint8, nq * logw * DIGEST_BYTES, "paths")
    _need(idx, torch.int32, nq, "idx")
    _check(lib().fp_merkle_open(_ptr(code), W, rows, logw, _ptr(salts), _ptr(tree), _ptr(chal), nq, _ptr(cols),
                                _ptr(col_salts), _ptr(paths), _ptr(idx), _stream()), "fp_merkle_open")
    return cols, col_salts, paths, idx


def mle_eval(M, r_rows, r_cols, out=None):
    rows, cols = M.shape
    out = torch.empty(1, dtype=torch.int64, device=M.device) if out is None else out
    nr, nc = r_rows.numel(), r_cols.numel()
    need = lib().fp_mle_eval_workspace(_dt(M), rows, cols, nr, nc)
    p, nb = _ws_mle.get(need)
    _check(lib().fp_mle_eval(_dt(M), _ptr(M), _ld(M), rows, cols, _ptr(r_rows) if nr else None, nr,
                             _ptr(r_cols) if nc else None, nc, _ptr(out), p, nb, _stream()), "fp_mle_eval")
    return out


# ---------------------------------------------------------------- sum-check --
def sumcheck_prove(As, Bs, r, rho=None, rounds=None, finals=None, claim0=None):
    k = len(As)
    n = r.numel()
    dev = r.device
    rounds = torch.empty((n, 3), dtype=torch.int64, device=dev) if rounds is None else rounds
    finals = torch.empty((k, 2), dtype=torch.int64, device=dev) if finals is None else finals
    claim0 = torch.empty(1, dtype=torch.int64, device=dev) if claim0 is None else claim0
    pa = (ctypes.c_void_p * k)(*[a.data_ptr() for a in As])
    pb = (ctypes.c_void_p * k)(*[b.data_ptr() for b in Bs])
    need = lib().fp_sumcheck_workspace(k, n)
    p, nb = _ws_sc.get(need)
    _check(lib().fp_sumcheck_prove(k, pa, pb, _ptr(rho), n, _ptr(r), _ptr(rounds), _ptr(finals), _ptr(claim0),
                                   p, nb, _stream()), "fp_sumcheck_prove")
    return rounds, finals, claim0


def sumcheck_prove_multi(A, B, r, rounds=None, finals=None, claim0=None):
    n_inst, m = A.shape
    n = r.shape[1]
    assert m == 1 << n
    dev = A.device
    rounds = torch.empty((n_inst, n, 3), dtype=torch.int64, device=dev) if rounds is None else rounds
    finals = torch.empty((n_inst, 2), dtype=torch.int64, device=dev) if finals is None else finals
    claim0 = torch.empty(n_inst, dtype=torch.int64, device=dev) if claim0 is None else claim0
    _check(lib().fp_sumcheck_prove_multi(n_inst, n, _ptr(A), _ptr(B), _ptr(r), _ptr(rounds), _ptr(finals),
                                         _ptr(claim0), _stream()), "fp_sumcheck_prove_multi")
    return rounds, finals, claim0


def combine_claims(g_last, x_last, rho, out=None):
    """out = sum_j rho[j] g_j(x_j); g_last[j]: device view of 3 values, x_last[j]: view of 1."""
    k = len(g_last)
    out = torch.empty(1, dtype=torch.int64, device=rho.device) if out is None else out
    pg = (ctypes.c_void_p * k)(*[g.data_ptr() for g in g_last])
    px = (ctypes.c_void_p * k)(*[x.data_ptr() for x in x_last])
    _check(lib().fp_combine_claims(k, pg, px, _ptr(rho), _ptr(out), _stream()), "fp_combine_claims")
    return out


def claim_eval_batched(jobs):
    """jobs: list of (M, E_rows, E_cols, out); out_j = sum E_rows[t] E_cols[c] M[t, c]."""
    k = len(jobs)
    dt = _dt(jobs[0][0])
    descs = (_ClaimDesc * k)(*[_ClaimDesc(M.data_ptr(), _ld(M), M.shape[0], M.shape[1], Er.data_ptr(),
                                          Ec.data_ptr(), out.data_ptr()) for (M, Er, Ec, out) in jobs])
    need = lib().fp_claim_eval_batched_workspace(dt, k, descs)
    p, nb = _ws_claim.get(need)
    _check(lib().fp_claim_eval_batched(dt, k, descs, p, nb, _stream()), "fp_claim_eval_batched")
    return [j[3] for j in jobs]


def fold_claim_batched(fold_jobs, claim_jobs):
    """One pass over fold jobs (M, E, cols_pad, out) of one dtype and claim jobs
    (M, E_rows, E_cols, out) of one dtype; outputs as fold_matrix_batched and
    claim_eval_batched."""
    nf, nc = len(fold_jobs), len(claim_jobs)
    fdt = _dt(fold_jobs[0][0]) if nf else FP_I8
    cdt = _dt(claim_jobs[0][0]) if nc else FP_I32
    fd = (_FoldDesc * max(nf, 1))(*[_fold_desc(f) for f in fold_jobs])
    cd = (_ClaimDesc * max(nc, 1))(*[_ClaimDesc(M.data_ptr(), _ld(M), M.shape[0], M.shape[1], Er.data_ptr(),
                                                Ec.data_ptr(), out.data_ptr()) for (M, Er, Ec, out) in claim_jobs])
    need = lib().fp_fold_claim_batched_workspace(fdt, nf, fd, cdt, nc, cd)
    p, nb = _ws_fold.get(need)
    _check(lib().fp_fold_claim_batched(fdt, nf, fd, cdt, nc, cd, p, nb, _stream()), "fp_fold_claim_batched")
    return [j[3] for j in fold_jobs], [j[3] for j in claim_jobs]


def linear_combine(vals, rho, out=None):
    k = len(vals)
    out = torch.empty(1, dtype=torch.int64, device=rho.device) if out is None else out
    pv = (ctypes.c_void_p * k)(*[v.data_ptr() for v in vals])
    _check(lib().fp_linear_combine(k, pv, _ptr(rho), _ptr(out), _stream()), "fp_linear_combine")
    return out
