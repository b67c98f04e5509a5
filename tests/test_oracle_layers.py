"""The oracle's layer proofs on the five workload descriptions (full size for
the 256x256 layer, reduced shapes for the others), checked by the verifier-side
invariants: round sums, the final claim against independent brute-force MLEs
of X and W over their flattened padded tables, the initial claim against a
brute-force MLE of Z, the witness against a naive matmul, and each random
linear combination recomputed from per-claim values. CPU only."""
import numpy as np
import pytest

import oracle as O
import synth

P = O.P


def _flat_padded(M, n_rows, n_cols):
    """Field values of M zero-padded to [2^n_rows, 2^n_cols], column in the low bits."""
    out = np.zeros((1 << n_rows, 1 << n_cols), np.uint64)
    for t in range(M.shape[0]):
        out[t, :M.shape[1]] = [O.from_int(int(v)) for v in M[t]]
    return out.reshape(-1)


def _check_claim(X, W, res, r_t, r_o, r_rounds, n, s, witness=True):
    x_f, w_f = res["x_fold"], res["w_fold"]
    # invariant 1: the initial claim
    dot = sum(int(a) * int(b) for a, b in zip(x_f, w_f)) % P
    assert res["claim0"] == dot
    reason, where = O.check_sumcheck(res["rounds"], res["finals"], r_rounds, dot, As=[x_f], Bs=[w_f])
    assert reason == "OK", (reason, where)
    # invariant 3 against independent MLEs of X and W at (z || r_t), (z || r_o)
    z = [int(v) for v in r_rounds]
    n_t, n_o = len(r_t), len(r_o)
    Xf = _flat_padded(X, n_t, n)
    Wf = _flat_padded(W, n_o, n)
    xz = O.mle_seq(Xf, z + [int(v) for v in r_t])
    wz = O.mle_seq(Wf, z + [int(v) for v in r_o])
    assert int(res["finals"][0, 0]) == xz and int(res["finals"][0, 1]) == wz
    g = res["rounds"][-1] if n else None
    if n:
        assert O.eval_deg2(int(g[0]), int(g[1]), int(g[2]), z[-1]) == xz * wz % P
    if witness:
        # invariant 4: c0 = Z~(r_o || r_t) by a brute-force MLE of flattened padded Z
        Zf = _flat_padded(res["Z"], n_t, len(r_o))
        assert res["c0"] == O.mle_seq(Zf, [int(v) for v in r_o] + [int(v) for v in r_t]) == dot
        # invariant 5: the witness against a naive matmul; the rescale identity
        assert O.check_witness(X, W, res["Z"]) == ("OK", -1)
        assert O.check_rescale(res["Z"], res["Y"], res["R"], s) == ("OK", -1)


def test_layer_cfg1_full():
    cfg = synth.config(1)
    inp = synth.make_inputs(cfg)
    ch = synth.draw_challenges(cfg)
    assert [len(ch[k]) for k in ("r_t", "r_o", "rounds")] == [4, 8, 8]
    res = O.prove_config(cfg, inp, ch)["main"]
    _check_claim(inp["X"], inp["W"], res, ch["r_t"], ch["r_o"], ch["rounds"], 8, cfg.s)


def test_layer_cfg2_reduced():
    cfg = synth.config(2, T=12, d_in=40, d_out=23)
    inp = synth.make_inputs(cfg)
    ch = synth.draw_challenges(cfg)
    res = O.prove_config(cfg, inp, ch)["up"]
    _check_claim(inp["X"], inp["W"], res, ch["r_t"], ch["r_o"], ch["rounds"], 6, cfg.s)


def test_layer_cfg3_reduced_rlc():
    cfg = synth.config(3, T=6, d=20, d_ff=36)
    inp = synth.make_inputs(cfg)
    ch = synth.draw_challenges(cfg)
    res = O.prove_config(cfg, inp, ch)
    C = 0
    for m in cfg.matmuls:
        r = res[m.name]
        _check_claim(inp[m.x], inp[m.w], r, ch["r_t"], ch["r_o/" + m.name], ch["rounds/" + m.name], m.n, cfg.s)
        z = [int(v) for v in ch["rounds/" + m.name]]
        C = (C + int(ch["rho/" + m.name][0]) * O.mle_seq(r["x_fold"], z) * O.mle_seq(r["w_fold"], z)) % P
    assert res["rlc"] == C
    # gate and up share X_mlp and r_t, so they share x'
    assert np.array_equal(res["gate"]["x_fold"], res["up"]["x_fold"])


def test_layer_cfg4_reduced_moe():
    cfg = synth.config(4, T=40, d=24, d_ff=40, n_experts=6)
    inp = synth.make_inputs(cfg)
    route = inp["route"]
    ch = synth.draw_challenges(cfg, route)
    res = O.prove_config(cfg, inp, ch)
    counts = np.bincount(route, minlength=6)
    assert set(res.keys()) == {e for e in range(6) if counts[e] > 0}
    for e, r in res.items():
        toks = r["tokens"]
        assert list(toks) == sorted(np.nonzero(route == e)[0])
        Xe, He = inp["X"][toks], inp["H"][toks]
        _check_claim(Xe, inp["W1_%d" % e], r["up"], ch["r_t/%d" % e], ch["r_o_up/%d" % e],
                     ch["rounds_up/%d" % e], 5, cfg.s)
        _check_claim(He, inp["W2_%d" % e], r["down"], ch["r_t/%d" % e], ch["r_o_down/%d" % e],
                     ch["rounds_down/%d" % e], 6, cfg.s)


def test_layer_cfg5_reduced_batched():
    cfg = synth.config(5, T=8, d=16, d_kv=8, d_ff=28)
    inp = synth.make_inputs(cfg)
    ch = synth.draw_challenges(cfg)
    res = O.prove_config(cfg, inp, ch)
    b = res["batch"]
    n = cfg.batched_n
    assert n == 5
    As = [res[m.name]["x_fold"] for m in cfg.matmuls]
    Bs = [res[m.name]["w_fold"] for m in cfg.matmuls]
    rho = b["rho"]
    assert O.check_sumcheck(b["rounds"], b["finals"], ch["rounds"], b["c0"], rho=rho, As=As, Bs=Bs)[0] == "OK"
    # the batched claim is the rho-combination of the seven Z~ claims
    assert b["c0"] == b["claim0"]
    z = [int(v) for v in ch["rounds"]]
    for j, m in enumerate(cfg.matmuls):
        X, W = inp[m.x], inp[m.w]
        Wf = _flat_padded(W, m.n_o, n)
        assert int(b["finals"][j, 1]) == O.mle_seq(Wf, z + [int(v) for v in ch["r_o/" + m.name]])
        Xf = _flat_padded(X, cfg.n_t, n)
        assert int(b["finals"][j, 0]) == O.mle_seq(Xf, z + [int(v) for v in ch["r_t"]])
        assert O.check_witness(X, W, res[m.name]["Z"]) == ("OK", -1)
