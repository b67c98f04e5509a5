"""The C ABI: libfp.so loads and exports every function include/fp.h
declares; argument errors are reported without any launch. CPU only."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_hot_path():
    names = _declared()
    for f in ("fp_witness_linear", "fp_eq_table", "fp_fold_matrix", "fp_mle_eval", "fp_sumcheck_prove"):
        assert f in names


def test_library_exports_every_declared_symbol():
    import zero_knowledge_proof_amd as fp
    L = fp.lib()
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(fp.EXPORTS) == _declared()


def test_argument_errors_without_gpu():
    import zero_knowledge_proof_amd as fp
    L = fp.lib()
    # s outside [1, 8]
    assert L.fp_witness_linear(None, 16, None, 16, 4, 16, 4, 9, None, None, None, None) == 3
    assert b"s=9" in L.fp_last_error()
    # d_in too large for an exact int32 witness
    assert L.fp_witness_linear(None, 200000, None, 200000, 1, 131073, 1, 8, None, None, None, None) == 2
    # 128^2 * 131072 = 2^31 would overflow int32 when every product is (-128)^2
    assert L.fp_witness_linear(None, 131072, None, 131072, 1, 131072, 1, 8, None, None, None, None) == 2
    # eq table size
    assert L.fp_eq_table(None, 31, None, None) == 2
    # sum-check sizes
    assert L.fp_sumcheck_prove(0, None, None, None, 4, None, None, None, None, None, 0, None) == 1
    assert L.fp_sumcheck_prove_multi(1, 14, None, None, None, None, None, None, None) == 2
    # a fold with ld < cols
    assert L.fp_fold_matrix(0, None, 3, 4, 5, None, None, 5, None, 0, None) == 2
    # workspace too small for a multi-chunk fold
    need = L.fp_fold_matrix_workspace(0, 100000, 4096)
    assert need > 0
    dummy = ctypes.c_void_p(16)
    assert L.fp_fold_matrix(0, dummy, 4096, 100000, 4096, dummy, dummy, 4096, dummy, need - 1, None) == 4
    # grouped witness row offsets must start at 0 and not decrease
    ro = (ctypes.c_int32 * 3)(1, 2, 3)
    wp = (ctypes.c_void_p * 2)(16, 16)
    assert L.fp_witness_linear_grouped(dummy, 16, wp, 16, ro, 2, 16, 16, 8, None, dummy, dummy, None) == 1
    # witness + sum-check in one launch: pair count, and tables too large for one workgroup
    pa = (ctypes.c_void_p * 1)(16)
    assert L.fp_witness_linear_with_sumcheck(None, 16, None, 16, 0, 16, 4, 8, None, None, None, 0, pa, pa, None, 4,
                                             dummy, dummy, dummy, None, None) == 1
    assert L.fp_witness_linear_with_sumcheck(None, 16, None, 16, 0, 16, 4, 8, None, None, None, 1, pa, pa, None, 13,
                                             dummy, dummy, dummy, None, None) == 2
    assert b"exceed one" in L.fp_last_error()
    # packed weights: ceil(d_out / 32) * 32 rows of ceil(d_in / 64) * 64 bytes; the packed witness needs
    # d_in % 16 == 0 and 16-byte aligned X rows
    assert L.fp_witness_packed_weights_bytes(100, 100) == 128 * 128
    assert L.fp_witness_packed_weights_bytes(14336, 4096) == 14336 * 4096
    assert L.fp_witness_packed_weights_bytes(-1, 4) == 0
    assert L.fp_witness_pack_weights(dummy, 8, 4, 16, dummy, None) == 2
    assert L.fp_witness_linear_packed(dummy, 40, dummy, 4, 40, 4, 8, None, dummy, dummy, 0, None, None) == 2
    assert b"d_in % 16" in L.fp_last_error()
    assert L.fp_witness_linear_packed(ctypes.c_void_p(24), 48, dummy, 4, 48, 4, 8, None, dummy, dummy, 0, None,
                                      None) == 2
    assert L.fp_witness_linear_packed(dummy, 48, dummy, 4, 48, 4, 0, None, dummy, dummy, 0, None, None) == 3
    assert L.fp_witness_linear_packed_with_sumcheck(dummy, 48, dummy, 4, 48, 4, 8, None, dummy, dummy, 1, pa, pa, None,
                                                    13, dummy, dummy, dummy, None, 0, None, None) == 2
    assert b"exceed one" in L.fp_last_error()
    # the layer step: at most 4 folds and claims, none empty, and a large enough workspace
    fd = (fp._FoldDesc * 5)(*[fp._FoldDesc(16, 64, 10, 64, 64, 16, 16) for _ in range(5)])
    assert L.fp_layer_step(dummy, 48, dummy, 4, 48, 4, 8, None, dummy, dummy, None, None, None, 0, None, 5, fd, 0,
                           None, dummy, 1 << 20, 0, None, None, None, 0, None, None, None, None, None) == 1
    fd0 = (fp._FoldDesc * 1)(fp._FoldDesc(16, 64, 0, 64, 64, 16, 16))
    assert L.fp_layer_step(dummy, 48, dummy, 4, 48, 4, 8, None, dummy, dummy, None, None, None, 0, None, 1, fd0, 0,
                           None, dummy, 1 << 20, 0, None, None, None, 0, None, None, None, None, None) == 2
    fd1 = (fp._FoldDesc * 1)(fp._FoldDesc(16, 64, 5000, 64, 64, 16, 16))
    need = L.fp_layer_step_workspace(4, 4, 0, 1, fd1, 0, None)
    assert need > 16384
    # the witness's own claim: one more slot per GEMM wave, both tables and an output, tokens and outputs
    assert L.fp_layer_step_workspace(4, 4, 1, 1, fd1, 0, None) > need
    assert L.fp_layer_step_workspace(4, 4, 1, 0, None, 0, None) > 16384
    assert L.fp_layer_step_workspace(-1, 4, 1, 0, None, 0, None) == 0
    assert L.fp_layer_step(dummy, 48, dummy, 4, 48, 4, 8, None, dummy, dummy, dummy, None, dummy, 0, None, 0, None, 0,
                           None, dummy, 1 << 20, 0, None, None, None, 0, None, None, None, None, None) == 1
    assert L.fp_layer_step(dummy, 48, dummy, 0, 48, 4, 8, None, dummy, dummy, dummy, dummy, dummy, 0, None, 0, None,
                           0, None, dummy, 1 << 20, 0, None, None, None, 0, None, None, None, None, None) == 2
    assert L.fp_layer_step(ctypes.c_void_p(256), 48, dummy, 4, 48, 4, 8, None, dummy, dummy, None, None, None, 0,
                           None, 1, fd1, 0, None, ctypes.c_void_p(256), need - 1, 0, None, None, None, 0, None, None,
                           None, None, None) == 4
    # eq tables built beside the packed witness: at most 8, each n in [0, 30] with non-null pointers
    assert L.fp_witness_linear_packed(dummy, 48, dummy, 4, 48, 4, 8, None, dummy, dummy, 9, dummy, None) == 1
    eqd = (fp._EqDesc * 2)(fp._EqDesc(16, 3, 16), fp._EqDesc(16, 31, 16))
    assert L.fp_witness_linear_packed(dummy, 48, dummy, 4, 48, 4, 8, None, dummy, dummy, 2, eqd, None) == 2
    assert b"n=31" in L.fp_last_error()
    eqd = (fp._EqDesc * 1)(fp._EqDesc(None, 3, 16))
    assert L.fp_witness_linear_packed(dummy, 48, dummy, 4, 48, 4, 8, None, dummy, dummy, 1, eqd, None) == 1
    # multi-request fold: Mt's leading dim must be a multiple of 16, R bounded, workspace checked
    assert L.fp_fold_weights_prepare(dummy, 64, 100, 64, dummy, 104, dummy, None) == 2
    assert L.fp_fold_matrix_multi(dummy, 112, dummy, 100, 64, 5000, dummy, 100, dummy, 64, 64, dummy, 0, None) == 2
    need = L.fp_fold_matrix_multi_workspace(14336, 4096, 64)
    assert need >= 8 * 64 * 14336  # the digit rows at least
    assert L.fp_fold_matrix_multi_workspace(14336, 4096, 1) < need
    assert L.fp_fold_matrix_multi(dummy, 14336, dummy, 14336, 4096, 64, dummy, 14336, dummy, 4096, 4096, dummy,
                                  need - 1, None) == 4
    # commitment: sizes, limbs that do not fit, workspace, null salts
    assert L.fp_commit_pack(dummy, 10, dummy, 0, 24, 1, dummy, None) == 2
    assert L.fp_commit_pack(dummy, 100, dummy, 0, 2, 2, dummy, None) == 2  # 34 elements > 2 rows of 4
    assert L.fp_rs_encode(dummy, 1 << 24, 1, 24, dummy, 1 << 25, dummy, 1 << 30, None) == 2
    need = L.fp_rs_encode_workspace(2, 22)
    assert need >= 2 * (1 << 23) * 8
    assert L.fp_rs_encode(dummy, 1 << 22, 2, 22, dummy, 1 << 23, dummy, need - 1, None) == 4
    assert L.fp_merkle_commit(dummy, 1 << 26, 1, 26, dummy, dummy, None) == 2
    assert L.fp_merkle_commit(dummy, 16, 1, 4, None, dummy, None) == 1
    # lookup: sizes, s, workspace
    assert L.fp_lookup_tree(dummy, 10, 31, dummy, dummy, None) == 2
    assert L.fp_lookup_tree(dummy, 17, 4, dummy, dummy, None) == 2  # n > 2^L
    assert L.fp_lookup_counts(dummy, 10, 4, 9, dummy, None) == 3
    assert L.fp_sumcheck3_prove(dummy, dummy, 30, dummy, dummy, dummy, dummy, 1 << 40, None) == 2
    need = L.fp_lookup_prove_workspace(23)
    assert need >= (1 << 22) * 8
    assert L.fp_lookup_prove(dummy, 23, dummy, dummy, dummy, dummy, need - 1, None) == 4
    # transcript and extension sum-check: message size, table size, null state
    assert L.fp_fs_init(dummy, b"x" * 200, 200, None) == 1
    assert L.fp_sumcheck_ext_fs(dummy, dummy, dummy, dummy, 13, dummy, dummy, dummy, dummy, None) == 2
    assert L.fp_fs_absorb(None, dummy, 4, None) == 1
    assert L.fp_eq_table_ext(dummy, 25, dummy, dummy, None) == 2
    # committed-rescale proof: tables, folded rows, column openings, the streamed extension sum-check
    td = (fp._TableDesc * 1)(fp._TableDesc(16, 100, 10, 100, 7, 0, 8, 16))  # d_out = 100 > 2^7 fits; T > 2^n_t?
    assert L.fp_commit_tables(1, td, 3, 8, 7, dummy, 128, 24, None) == 2  # T = 10 > 2^3
    assert b"map 0" in L.fp_last_error()
    td = (fp._TableDesc * 1)(fp._TableDesc(16, 100, 8, 100, 7, 0, 8, 16))
    assert L.fp_commit_tables(1, td, 3, 9, 7, dummy, 128, 24, None) == 3  # s = 9
    assert L.fp_commit_tables(1, td, 3, 8, 7, dummy, 128, 23, None) == 2  # Y's 8 rows end past 23 rows
    assert L.fp_commit_tables(1, td, 3, 8, 11, dummy, 2048, 24, None) == 2  # rows of 2^11 > the table's 2^10
    assert L.fp_commit_tables(9, td, 3, 8, 7, dummy, 128, 24, None) == 1
    td = (fp._TableDesc * 1)(fp._TableDesc(None, 100, 8, 100, 7, 0, 8, 16))
    assert L.fp_commit_tables(1, td, 3, 8, 7, dummy, 128, 24, None) == 1  # null Z with entries
    cl = (fp._OpenClaim * 2)(fp._OpenClaim(0, 8, dummy, 2, dummy, 1), fp._OpenClaim(4, 4, dummy, 2, None, 0))
    ws = 256  # a 256-byte aligned (never dereferenced) workspace address
    need = L.fp_commit_fold_ext_workspace(16)
    assert need >= 16 * 32
    assert L.fp_commit_fold_ext(dummy, 64, 16, 6, dummy, 4, 2, cl, dummy, ws, need, None) == 2  # overlap
    assert b"claim 1" in L.fp_last_error()
    cl = (fp._OpenClaim * 1)(fp._OpenClaim(0, 8, dummy, 2, dummy, 2))
    assert L.fp_commit_fold_ext(dummy, 64, 16, 6, dummy, 4, 1, cl, dummy, ws, need, None) == 2  # 8 != 2^4
    cl = (fp._OpenClaim * 1)(fp._OpenClaim(0, 8, dummy, 2, dummy, 1))
    assert L.fp_commit_fold_ext(dummy, 64, 16, 6, dummy, 3, 1, cl, dummy, ws, need, None) == 2  # 2^3 < 16 rows
    assert L.fp_commit_fold_ext(dummy, 64, 16, 6, dummy, 4, 1, cl, dummy, ws, need - 1, None) == 4
    assert L.fp_commit_fold_ext(dummy, 64, 16, 6, dummy, 4, 17, cl, dummy, ws, need, None) == 1
    assert L.fp_merkle_open(dummy, 64, 4, 7, dummy, dummy, dummy, 3, dummy, dummy, dummy, None, None) == 2  # ld < 2^7
    assert L.fp_merkle_open(dummy, 128, 4, 7, dummy, dummy, None, 3, dummy, dummy, dummy, None, None) == 1
    assert L.fp_merkle_open(dummy, 128, 4, 7, dummy, dummy, dummy, 0, dummy, dummy, dummy, None, None) == 0
    arr = (ctypes.c_void_p * 9)(*([dummy] * 9))
    assert L.fp_sumcheck_ext_fs_multi(9, arr, arr, arr, arr, None, 4, dummy, dummy, dummy, dummy, None, 0, None) == 1
    assert L.fp_sumcheck_ext_fs_multi(2, arr, arr, arr, arr, None, 25, dummy, dummy, dummy, dummy, None, 0, None) == 2
    need = L.fp_sumcheck_ext_fs_multi_workspace(7, 14)
    assert need >= 7 * (1 << 19)
    assert L.fp_sumcheck_ext_fs_multi(7, arr, arr, arr, arr, None, 14, dummy, dummy, dummy, dummy, ws, need - 1,
                                      None) == 4
    assert L.fp_sumcheck_ext_fs_multi_workspace(7, 0) == 0
    # the clamp lookup: sizes and table bits
    assert L.fp_lookup_tree_pairs(dummy, dummy, 17, 1 << 16, 0, 4, dummy, dummy, None) == 2  # n > 2^L
    assert L.fp_lookup_tree_pairs(None, dummy, 16, 1 << 16, 0, 4, dummy, dummy, None) == 1
    assert L.fp_lookup_counts_field(dummy, 100, -(1 << 15), 25, dummy, None) == 3
    assert L.fp_lookup_counts_field(dummy, 100, -(1 << 15), 16, None, None) == 1
    # moe plan is host-only and runs here
    import numpy as np
    counts, offsets, perm = fp.moe_plan(np.array([2, 0, 2, 1, 0], np.int32), 4)
    assert list(counts) == [2, 1, 2, 0] and list(offsets) == [0, 2, 3, 5, 5] and list(perm) == [1, 4, 3, 0, 2]
    route = np.array([0, 5], np.int32)
    with pytest.raises(fp.FPError):
        fp.moe_plan(route, 4)
