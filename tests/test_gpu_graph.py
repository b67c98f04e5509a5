"""A whole layer step recorded as one HIP graph gives, on every replay, the
same bytes as the eager step, with eager work and synchronizations between
replays (outputs are cleared by a fill kernel before each replay)."""
import numpy as np
import pytest
import torch

import synth
from zero_knowledge_proof_amd.prover import make_prover

pytestmark = pytest.mark.gpu


def _same(a, b, path=""):
    if isinstance(a, dict):
        assert a.keys() == b.keys(), path
        for k in a:
            _same(a[k], b[k], path + "/" + str(k))
    else:
        assert np.array_equal(np.asarray(a), np.asarray(b)), path


@pytest.mark.parametrize("cid,shape", [(1, {}), (2, dict(T=100, d_in=1000, d_out=700)),
                                       (3, dict(T=40, d=320, d_ff=600)),
                                       (5, dict(T=24, d=96, d_kv=40, d_ff=300)),
                                       (4, dict(T=200, d=96, d_ff=128, n_experts=12))])
def test_graph_replays_match_eager(fp, cid, shape):
    cfg = synth.config(cid, **shape)
    inp = synth.make_inputs(cfg)
    ch = synth.draw_challenges(cfg, inp.get("route"))
    prover = make_prover(cfg, inp, ch)
    prover.run()
    torch.cuda.synchronize()
    want = prover.results()
    prover.capture()
    for rep in range(3):
        for t in prover.output_tensors():
            t.zero_()             # a fill kernel, outside the graph
        torch.cuda.synchronize()
        prover.replay()
        torch.cuda.synchronize()
        _same(prover.results(), want, "replay%d" % rep)
        prover.run()              # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("cid,shape", [(1, {}), (2, dict(T=100, d_in=1000, d_out=700))])
def test_pipelined_graph_replays(fp, cid, shape):
    """Pipelined proofs recorded as a graph: replays followed by the drain give
    the eager pipelined outputs, with outputs cleared between replays."""
    cfg = synth.config(cid, **shape)
    inp = synth.make_inputs(cfg)
    ch = synth.draw_challenges(cfg, inp.get("route"))
    prover = make_prover(cfg, inp, ch, pipelined=True)
    prover.run()
    prover.drain()
    torch.cuda.synchronize()
    want = prover.results()
    prover.capture(steps=2)       # two consecutive proofs per graph
    for rep in range(3):
        for t in prover.output_tensors():
            t.zero_()
        torch.cuda.synchronize()
        prover.replay()           # proofs 1 and 2 (proof 1's sum-check runs inside proof 2's witness launch)
        prover.drain()
        torch.cuda.synchronize()
        _same(prover.results(), want, "replay%d" % rep)
        prover.run()              # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("cid,shape,steps,keep_z", [(1, {}, 6, False), (2, dict(T=100, d_in=1008, d_out=700), 6, True),
                                                    (3, dict(T=300, d=256, d_ff=1024), 6, False),
                                                    (5, dict(T=200, d=128, d_kv=64, d_ff=320), 6, False)])
def test_overlapped_graph_replays(fp, cid, shape, steps, keep_z):
    """Three proofs in flight recorded as a graph (one launch per step; single layers and multi-map layers):
    replays followed by the drain give the eager outputs for each of the last three proofs (each keeps its own
    outputs, its sum-check's included), with every buffer cleared between replays and eager steps in between; a
    graph of a number of steps that is not a multiple of the prover's period (three sets of buffers; six steps
    for the multi-map layers, whose weight folds of two proofs run every other step) is refused."""
    cfg = synth.config(cid, **shape)
    inp = synth.make_inputs(cfg)
    ch = synth.draw_challenges(cfg, inp.get("route"))
    prover = make_prover(cfg, inp, ch, pipelined=True, overlapped=True, keep_z=keep_z)
    with pytest.raises(ValueError):
        prover.capture(steps=4)
    prover.run()
    prover.run()
    prover.drain()
    torch.cuda.synchronize()
    want = prover.results()
    prover.capture(steps=steps)
    for rep in range(3):
        for t in prover.output_tensors():
            t.zero_()
        torch.cuda.synchronize()
        prover.replay()
        prover.replay()
        prover.drain()
        torch.cuda.synchronize()
        for k in range(prover.k - 3, prover.k):
            _same(prover.results(k), want, "replay%d proof %d" % (rep, k))
        prover.run()              # eager work between replays
        torch.cuda.synchronize()
