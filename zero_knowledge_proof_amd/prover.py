"""Layer proofs strung together from the libfp entry points.

"How fast can FlashProve go", §2: for each linear map the prover commits the
rescaled output and the remainder (§3.1), and sum-check reduces the matmul
claim about Z to claims about the committed activations and the weights. One
``run()`` of a layer prover performs, on one stream and in protocol order:

  witness  Z = X W^T, Y, R                     (fp_witness_linear_packed from weights packed once by
                                               fp_witness_pack_weights; fp_witness_linear[_grouped])
  eq       E_t = eq(r_t, .), E_o = eq(r_o, .)  (fp_eq_table_batched)
  folds    x' = X~(. || r_t), w' = W~(. || r_o) (fp_fold_claim_batched: the
  claim    c0 = Z~(r_o || r_t)                   folds and the claims in one pass)
  rounds   sum-check over k on (x', w')         (fp_sumcheck_prove[_multi])
  merge    random linear combinations           (fp_combine_claims, fp_linear_combine)

The challenges (drawn before the run and passed in) follow the witness in the
stream order; each round challenge is applied on the device only after its
round polynomial is complete. Every buffer is allocated at construction, so ``run``
only enqueues kernels. Inputs are host numpy arrays uploaded once.
"""
from __future__ import annotations

import itertools

import numpy as np
import torch

from . import (MatmulJob, StepWorkspace, SumcheckJob, combine_claims, commit_fold_ext, commit_tables,
               eq_table_batched, eq_table_ext, field_numpy, fold_claim_batched, fold_matrix_batched, fs_absorb,
               fs_challenges, fs_init, gather_rows, layer_step, layer_step_multi, linear_combine, merkle_commit,
               merkle_open, moe_plan, pack_weights, rs_encode, sumcheck_ext_fs_multi, sumcheck_prove,
               sumcheck_prove_multi, to_field_tensor, witness_linear, witness_linear_grouped, witness_grouped_packed,
               witness_linear_packed, witness_linear_packed_with_sumcheck, witness_linear_with_sumcheck,
               witness_multi)


def _nomark(name):
    pass


def log2ceil(v: int) -> int:
    return 0 if v <= 1 else (int(v) - 1).bit_length()


def _i8(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _f(n, dev):
    return torch.empty(n, dtype=torch.int64, device=dev)


def _packed(W: torch.Tensor):
    """The weights packed for the matrix cores (fp_witness_pack_weights, once per layer) when the
    packed witness applies to them (d_in % 16 == 0), else None."""
    return pack_weights(W) if W.shape[1] % 16 == 0 else None


def _witness(X, W, Wp, s, Z, Y, R):
    if Wp is not None:
        witness_linear_packed(X, Wp, s, Z, Y, R)
    else:
        witness_linear(X, W, s, Z, Y, R)


class _Prover:
    """Common driver: ``phases()`` lists the protocol steps in order; ``run``
    enqueues them eagerly; ``capture`` records them into one HIP graph."""

    graph = None

    def phases(self):
        raise NotImplementedError

    def run(self, mark=_nomark):
        for name, fn in self.phases():
            mark(name)
            fn()
        mark("end")

    def capture(self, steps: int = 1):
        """Record `steps` consecutive whole steps into one HIP graph (run once
        eagerly first so that every workspace has its final size). Several
        steps per graph spread the fixed cost of a graph launch."""
        self.run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                self.run()
        torch.cuda.synchronize()
        self.graph = g
        self.graph_steps = steps
        return g

    def replay(self):
        self.graph.replay()

    def drain(self):
        """Finish work a pipelined prover leaves for the next run (none here)."""

    # tensors the step writes (for tests that clear them between runs)
    OUTPUTS = ()

    def output_tensors(self):
        out = []
        for name in self.OUTPUTS:
            v = getattr(self, name)
            out.extend(t for t in (v if isinstance(v, list) else [v]) if t is not None)
        return out


class _Challenges:
    """All challenges of a workload in one device buffer, with named views."""

    def __init__(self, ch: dict, dev):
        keys = list(ch.keys())
        flat = np.concatenate([np.asarray(ch[k], np.uint64) for k in keys]) if keys else np.zeros(0, np.uint64)
        self.buf = to_field_tensor(flat, dev) if len(flat) else _f(0, dev)
        self.views, pos = {}, 0
        for k in keys:
            n = len(ch[k])
            self.views[k] = self.buf[pos:pos + n]
            pos += n

    def __getitem__(self, k):
        return self.views[k]


# tables of at most this many entries fit the sum-check workgroup that runs
# inside a witness launch
OVERLAP_ENTRIES = 4096


class SingleLayerProver(_Prover):
    """One linear map: witness, claim and sum-check over d_in.

    With packed weights (d_in % 16 == 0) the witness launch also builds the
    proof's eq tables (they depend on its challenges only).

    pipelined: for a stream of proofs of the layer. ``run()`` then launches the
    witness of this proof together with the sum-check of the previous one
    (fp_witness_linear[_packed]_with_sumcheck), followed by this proof's folds
    and claim; ``drain()`` runs the sum-check of the last proof. The outputs
    of a proof are complete after the next ``run()`` or ``drain()``."""

    OUTPUTS = ("Z", "Y", "R", "E_t", "E_o", "xf", "wf", "c0", "rounds", "finals", "claim0")

    def __init__(self, X: np.ndarray, W: np.ndarray, s: int, ch: dict, dev=None, with_z: bool = True,
                 pipelined: bool = False):
        dev = dev or torch.device("cuda")
        self.pipelined = pipelined
        self.s = s
        self.X, self.W = _i8(X, dev), _i8(W, dev)
        self.Wp = _packed(self.W)
        T, d_in = X.shape
        d_out = W.shape[0]
        self.n = log2ceil(d_in)
        self.ch = _Challenges({"r_t": ch["r_t"], "r_o": ch["r_o"], "rounds": ch["rounds"]}, dev)
        self.Z = torch.empty((T, d_out), dtype=torch.int32, device=dev)
        self.Y = torch.empty((T, d_out), dtype=torch.int8, device=dev)
        self.R = torch.empty((T, d_out), dtype=torch.int8, device=dev)
        self.E_t, self.E_o = _f(1 << log2ceil(T), dev), _f(1 << log2ceil(d_out), dev)
        if pipelined and (1 << self.n) > OVERLAP_ENTRIES:
            raise ValueError("pipelined proofs need d_in <= %d" % OVERLAP_ENTRIES)
        # zeros: the first pipelined run proves the all-zero claim of no layer
        self.xf = torch.zeros(1 << self.n, dtype=torch.int64, device=dev)
        self.wf = torch.zeros(1 << self.n, dtype=torch.int64, device=dev)
        self.c0 = _f(1, dev)
        self.rounds = torch.empty((self.n, 3), dtype=torch.int64, device=dev)
        self.finals = torch.empty((1, 2), dtype=torch.int64, device=dev)
        self.claim0 = _f(1, dev)

    def _sumcheck(self):
        sumcheck_prove([self.xf], [self.wf], self.ch["rounds"], rounds=self.rounds, finals=self.finals,
                       claim0=self.claim0)

    def _eq_pairs(self):
        return [(self.ch["r_t"], self.E_t), (self.ch["r_o"], self.E_o)]

    def _witness_and_previous_sumcheck(self):
        if self.Wp is not None:
            # this proof's eq tables are built by the same launch
            witness_linear_packed_with_sumcheck(self.X, self.Wp, self.s, self.Z, self.Y, self.R, [self.xf], [self.wf],
                                                self.ch["rounds"], rounds=self.rounds, finals=self.finals,
                                                claim0=self.claim0, eq=self._eq_pairs())
        else:
            witness_linear_with_sumcheck(self.X, self.W, self.s, self.Z, self.Y, self.R, [self.xf], [self.wf],
                                         self.ch["rounds"], rounds=self.rounds, finals=self.finals,
                                         claim0=self.claim0)

    def drain(self):
        """Pipelined mode: the sum-check of the last proof."""
        if self.pipelined:
            self._sumcheck()

    def phases(self):
        n = self.n
        fold = ("fold+claim", lambda: fold_claim_batched([(self.X, self.E_t, 1 << n, self.xf),
                                                          (self.W, self.E_o, 1 << n, self.wf)],
                                                         [(self.Z, self.E_t, self.E_o, self.c0)]))
        eq = ("eq", lambda: eq_table_batched([self.ch["r_t"], self.ch["r_o"]], [self.E_t, self.E_o]))
        if self.Wp is not None:
            # packed weights: the witness launch also builds the eq tables
            if self.pipelined:
                return [("witness+eq+sumcheck", self._witness_and_previous_sumcheck), fold]
            return [("witness+eq", lambda: witness_linear_packed(self.X, self.Wp, self.s, self.Z, self.Y, self.R,
                                                                 eq=self._eq_pairs())), fold,
                    ("sumcheck", self._sumcheck)]
        if self.pipelined:
            return [("witness+sumcheck", self._witness_and_previous_sumcheck), eq, fold]
        return [("witness", lambda: _witness(self.X, self.W, self.Wp, self.s, self.Z, self.Y, self.R)), eq, fold,
                ("sumcheck", self._sumcheck)]

    def results(self) -> dict:
        return {"Z": self.Z.cpu().numpy(), "Y": self.Y.cpu().numpy(), "R": self.R.cpu().numpy(),
                "E_t": field_numpy(self.E_t), "E_o": field_numpy(self.E_o),
                "x_fold": field_numpy(self.xf), "w_fold": field_numpy(self.wf),
                "c0": int(field_numpy(self.c0)[0]), "rounds": field_numpy(self.rounds),
                "finals": field_numpy(self.finals), "claim0": int(field_numpy(self.claim0)[0])}


class OverlappedLayerProver(SingleLayerProver):
    """Single-layer proofs three deep, for a stream of proofs of one layer with
    packed weights: step k is ONE launch (fp_layer_step) that runs proof k's
    witness together with its claim c0 = Z~(r_o || r_t), taken from the GEMM's
    accumulators (so Z never has to be stored and read back), proof k+1's eq
    tables, proof k-1's folds and proof k-2's sum-check side by side. A proof's
    eq tables depend on its challenges alone, so they are built one step ahead
    and are complete when its GEMM's epilogue weights the claim with them;
    proof k-1's folds read only its own tables (likewise finished), and proof
    k-2's sum-check only its own folds, so each proof still follows the
    protocol order. The buffers of a proof (Y, R, tables, folds, c0) live from
    the step that builds its eq tables to the one that runs its sum-check, so
    they rotate over three sets, and a captured graph holds a multiple of three
    steps. ``drain()`` finishes the last two proofs. Each set also holds its
    proof's rounds, finals and initial claim, so the last three proofs can be
    read back (``results(k)``). keep_z: also write Z (which the proof never
    reads back)."""

    PER_PROOF = ("Z", "Y", "R", "E_t", "E_o", "xf", "wf", "c0", "rounds", "finals", "claim0")
    SETS = 3
    GRAPH_QUANTUM = 3  # steps per captured graph must be a multiple of this

    def __init__(self, X: np.ndarray, W: np.ndarray, s: int, ch: dict, dev=None, keep_z: bool = False):
        super().__init__(X, W, s, ch, dev, pipelined=True)
        if self.Wp is None:
            raise ValueError("overlapped proofs need packed weights (d_in % 16 == 0)")
        self.keep_z = keep_z
        first = {k: getattr(self, k) for k in self.PER_PROOF}
        if not keep_z:
            first["Z"] = None
        self.bufs = [first] + [
            {k: (None if v is None else torch.zeros_like(v) if k in ("xf", "wf") else torch.empty_like(v))
             for k, v in first.items()} for _ in range(self.SETS - 1)]
        # the sum-check outputs of a proof stay with its set (read after the step that finishes it)
        self.k = 0
        self.ws = StepWorkspace()

    def _buf(self, k):
        return self.bufs[k % self.SETS]

    def _eq_jobs(self, b):
        return [(self.ch["r_t"], b["E_t"]), (self.ch["r_o"], b["E_o"])]

    def _folds(self, b):
        n = self.n
        return [(self.X, b["E_t"], 1 << n, b["xf"]), (self.W, b["E_o"], 1 << n, b["wf"])]

    def _step(self, k, fold: bool, tail: bool):
        cur, nxt, prev, old = self._buf(k), self._buf(k + 1), self._buf(k - 1), self._buf(k - 2)
        layer_step(self.X, self.Wp, self.s, cur["Z"], cur["Y"], cur["R"], own_claim=(cur["E_t"], cur["E_o"], cur["c0"]),
                   eq=self._eq_jobs(nxt), folds=self._folds(prev) if fold else (),
                   As=[old["xf"]] if tail else (), Bs=[old["wf"]] if tail else (), r=self.ch["rounds"],
                   rounds=old["rounds"], finals=old["finals"], claim0=old["claim0"], ws=self.ws)

    def run(self, mark=_nomark):
        mark("step")
        if self.k == 0:  # the first proof's eq tables (later ones are built a step ahead)
            b = self._buf(0)
            eq_table_batched([self.ch["r_t"], self.ch["r_o"]], [b["E_t"], b["E_o"]])
        # proof k's witness and claim; proof k+1's eq tables; proof k-1's folds; proof k-2's sum-check
        self._step(self.k, self.k >= 1, self.k >= 2)
        mark("end")
        self.k += 1

    def phases(self):
        # the whole step is one launch
        wit = "witness" if self.keep_z else "witness(Y,R)"
        return [(wit + "+claim(acc)+eq+fold+sumcheck", lambda: self._step(2, True, True))]

    def capture(self, steps: int = 1):
        if steps % self.GRAPH_QUANTUM:
            raise ValueError("a captured graph holds a multiple of %d steps" % self.GRAPH_QUANTUM)
        while self.k < 2:  # every captured step then has all its parts
            self.run()
        self.run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                self.run()
        torch.cuda.synchronize()
        self.graph = g
        self.graph_steps = steps
        self.k_graph = self.k
        return g

    def replay(self):
        """The captured steps again (with their buffers: a multiple of three
        steps leaves every set where the graph expects it); drain() then
        finishes the replay's last two proofs."""
        self.graph.replay()
        self.k = self.k_graph

    def drain(self):
        """The sum-check of the next-to-last proof, then the folds and
        sum-check of the last one (its claim came with its witness)."""
        last = self.k - 1
        if last < 0:
            return
        if last >= 1:
            prev = self._buf(last - 1)
            sumcheck_prove([prev["xf"]], [prev["wf"]], self.ch["rounds"], rounds=prev["rounds"],
                           finals=prev["finals"], claim0=prev["claim0"])
        cur = self._buf(last)
        fold_claim_batched(self._folds(cur), [])
        sumcheck_prove([cur["xf"]], [cur["wf"]], self.ch["rounds"], rounds=cur["rounds"], finals=cur["finals"],
                       claim0=cur["claim0"])

    def output_tensors(self):
        return [t for b in self.bufs for t in b.values() if t is not None]

    def results(self, k: int | None = None) -> dict:
        """Outputs of proof k (default: the last one; the last three are held)."""
        b = self._buf(self.k - 1 if k is None else k)
        out = {"Y": b["Y"].cpu().numpy(), "R": b["R"].cpu().numpy(),
               "E_t": field_numpy(b["E_t"]), "E_o": field_numpy(b["E_o"]),
               "x_fold": field_numpy(b["xf"]), "w_fold": field_numpy(b["wf"]),
               "c0": int(field_numpy(b["c0"])[0]), "rounds": field_numpy(b["rounds"]),
               "finals": field_numpy(b["finals"]), "claim0": int(field_numpy(b["claim0"])[0])}
        if b["Z"] is not None:
            out["Z"] = b["Z"].cpu().numpy()
        return out


class MultiMatmulProver(_Prover):
    """Several linear maps of one layer sharing the token axis (one r_t).

    mode "rlc_out": each claim gets its own sum-check; the finished claims are
    merged by a random linear combination (the dense MLP's gate/up/down).
    mode "batched": the claims are merged first (rho-weighted) and proved by
    one batched sum-check over tables padded to 2^batched_n (all seven maps of
    a transformer layer).

    Maps whose d_in is a multiple of 16 (every map of the full-size layers)
    run their witness GEMMs in ONE launch (fp_witness_multi, longest reduction
    first) that also forms each map's claim c0 = Z~(r_o || r_t) from the GEMM's
    accumulators, so Z is neither stored nor read back; the eq tables are built
    first, since that launch's claims read them. Other maps take the row-major
    witness and their claims are taken from the stored Z in the fold launch.
    keep_z: also store Z (for tests)."""

    def output_tensors(self):
        out = [self.E_t]
        for d in self.mm:
            out += [d[k] for k in ("Z", "Y", "R", "E_o", "xf", "wf", "c0", "rounds", "finals", "claim0")
                    if d.get(k) is not None]
        for k in ("rlc", "c0_batch", "rounds", "finals", "claim0"):
            if hasattr(self, k):
                out.append(getattr(self, k))
        return out

    def __init__(self, cfg, inp: dict, ch: dict, dev=None, keep_z: bool = False, group_o: int = 1):
        dev = dev or torch.device("cuda")
        self.cfg = cfg
        self.mode = cfg.kind
        self.keep_z = keep_z
        self.group_o = group_o
        s = cfg.s
        self.s = s
        self.tens = {}
        for m in cfg.matmuls:
            for nm in (m.x, m.w):
                if nm not in self.tens:
                    self.tens[nm] = _i8(inp[nm], dev)
        self.ch = _Challenges(ch, dev)
        T = cfg.T
        self.E_t = _f(1 << cfg.n_t, dev)
        self.mm = []
        nb = cfg.batched_n if self.mode == "batched" else None
        xf = {}
        self.packed = {m.w: _packed(self.tens[m.w]) for m in cfg.matmuls}
        for m in cfg.matmuls:
            n = nb if nb is not None else m.n
            key = (m.x, n)
            if key not in xf:
                xf[key] = _f(1 << n, dev)
            fused = self.packed[m.w] is not None
            d = {"m": m, "n": n, "xf": xf[key], "wf": _f(1 << n, dev), "E_o": _f(1 << m.n_o, dev),
                 "fused": fused,
                 "Z": torch.empty((T, m.d_out), dtype=torch.int32, device=dev) if (keep_z or not fused) else None,
                 "Y": torch.empty((T, m.d_out), dtype=torch.int8, device=dev),
                 "R": torch.empty((T, m.d_out), dtype=torch.int8, device=dev), "c0": _f(1, dev)}
            if self.mode == "rlc_out":
                d.update(rounds=torch.empty((n, 3), dtype=torch.int64, device=dev),
                         finals=torch.empty((1, 2), dtype=torch.int64, device=dev), claim0=_f(1, dev))
            self.mm.append(d)
        self.x_jobs = [(self.tens[x], None, 1 << n, buf) for (x, n), buf in xf.items()]
        # the maps of the one-launch witness, longest reduction first
        fused = sorted((d for d in self.mm if d["fused"]), key=lambda d: -d["m"].d_in)
        self.jobs = [MatmulJob(self.tens[d["m"].x], self.packed[d["m"].w], d["Y"], d["R"], d["Z"], self.E_t, d["E_o"],
                               d["c0"]) for d in fused]
        self.ws = StepWorkspace()
        self.rho = torch.cat([self.ch["rho/" + m.name] for m in cfg.matmuls]).contiguous()
        if self.mode == "rlc_out":
            self.rlc = _f(1, dev)
        else:
            self.c0_batch = _f(1, dev)
            self.rounds = torch.empty((nb, 3), dtype=torch.int64, device=dev)
            self.finals = torch.empty((len(cfg.matmuls), 2), dtype=torch.int64, device=dev)
            self.claim0 = _f(1, dev)

    def _eq(self):
        eq_table_batched([self.ch["r_t"]] + [self.ch["r_o/" + d["m"].name] for d in self.mm],
                         [self.E_t] + [d["E_o"] for d in self.mm])

    def _witness(self):
        if self.jobs:
            witness_multi(self.jobs, self.s, group_o=self.group_o, ws=self.ws)
        for d in self.mm:
            if not d["fused"]:
                m = d["m"]
                witness_linear(self.tens[m.x], self.tens[m.w], self.s, d["Z"], d["Y"], d["R"])

    def _fold_claim(self):
        jobs = [(M, self.E_t, cp, out) for (M, _, cp, out) in self.x_jobs]
        jobs += [(self.tens[d["m"].w], d["E_o"], 1 << d["n"], d["wf"]) for d in self.mm]
        fold_claim_batched(jobs, [(d["Z"], self.E_t, d["E_o"], d["c0"]) for d in self.mm if not d["fused"]])

    def _sumcheck(self):
        if self.mode == "rlc_out":
            for d in self.mm:
                sumcheck_prove([d["xf"]], [d["wf"]], self.ch["rounds/" + d["m"].name], rounds=d["rounds"],
                               finals=d["finals"], claim0=d["claim0"])
        else:
            linear_combine([d["c0"] for d in self.mm], self.rho, out=self.c0_batch)
            sumcheck_prove([d["xf"] for d in self.mm], [d["wf"] for d in self.mm], self.ch["rounds"], rho=self.rho,
                           rounds=self.rounds, finals=self.finals, claim0=self.claim0)

    def _merge(self):
        combine_claims([d["rounds"][-1] for d in self.mm],
                       [self.ch["rounds/" + d["m"].name][-1:] for d in self.mm], self.rho, out=self.rlc)

    def phases(self):
        all_fused = all(d["fused"] for d in self.mm)
        wname = "witness(Y,R)+claim(acc)" if all_fused and not self.keep_z else "witness+claim(acc)"
        ph = [("eq", self._eq), (wname, self._witness), ("fold" if all_fused else "fold+claim", self._fold_claim),
              ("sumcheck", self._sumcheck)]
        if self.mode == "rlc_out":
            ph.append(("merge", self._merge))
        return ph

    def results(self) -> dict:
        out = {"E_t": field_numpy(self.E_t)}
        for d in self.mm:
            r = {"Y": d["Y"].cpu().numpy(), "R": d["R"].cpu().numpy(),
                 "E_o": field_numpy(d["E_o"]), "x_fold": field_numpy(d["xf"]), "w_fold": field_numpy(d["wf"]),
                 "c0": int(field_numpy(d["c0"])[0])}
            if d["Z"] is not None:
                r["Z"] = d["Z"].cpu().numpy()
            if self.mode == "rlc_out":
                r.update(rounds=field_numpy(d["rounds"]), finals=field_numpy(d["finals"]),
                         claim0=int(field_numpy(d["claim0"])[0]))
            out[d["m"].name] = r
        if self.mode == "rlc_out":
            out["rlc"] = int(field_numpy(self.rlc)[0])
        else:
            out["batch"] = {"rounds": field_numpy(self.rounds), "finals": field_numpy(self.finals),
                            "claim0": int(field_numpy(self.claim0)[0]), "c0": int(field_numpy(self.c0_batch)[0])}
        return out


class OverlappedMultiProver(MultiMatmulProver):
    """A stream of proofs of a multi-map layer (the dense MLP, the seven-map
    layer), three in flight: step k is ONE launch (fp_layer_step_multi) that runs
    proof k's witness GEMMs with every map's claim taken from the accumulators,
    proof k+1's eq tables, proof k-1's folds of X, and proof k-2's
    sum-check(s), each instance one workgroup; on even k the same launch folds
    the weights for proofs k-1 and k together, from one read of each weight
    matrix (the proofs of a layer share its weights, and a weight fold needs
    only its proof's eq tables). A proof's eq tables depend on its challenges
    alone, so they are built a step ahead; its folds read only its own tables
    and its sum-check only its own folds, so each proof keeps the protocol
    order. Then a small launch merges proof k-2's claims (the RLC of the three
    output claims, or the rho-combination of the seven input claims that the
    batched sum-check starts from). A proof's buffers (Y, R, tables, folds,
    claims, rounds, finals) live from the step that builds its eq tables to the
    one that merges it, so they rotate over three sets; with the weight folds'
    two-step period a captured graph holds a multiple of six steps.
    ``drain()`` finishes the last two proofs. Needs every map's d_in % 16 == 0."""

    SETS = 3
    GRAPH_QUANTUM = 6
    PER_SET = ("E_t", "E_o", "Y", "R", "c0", "xf", "wf", "rounds", "finals", "claim0", "rlc", "c0_batch")

    def __init__(self, cfg, inp: dict, ch: dict, dev=None, keep_z: bool = False, group_o: int = 1):
        super().__init__(cfg, inp, ch, dev, keep_z=keep_z, group_o=group_o)
        if not all(d["fused"] for d in self.mm):
            raise ValueError("overlapped proofs need every map's d_in % 16 == 0")
        dev = self.E_t.device
        T = cfg.T
        self.sets = []
        for b in range(self.SETS):
            st = {"E_t": self.E_t if b == 0 else _f(self.E_t.numel(), dev), "maps": []}
            xf = {}
            for d in self.mm:
                m = d["m"]
                key = (m.x, d["n"])
                if key not in xf:
                    xf[key] = d["xf"] if b == 0 else torch.zeros_like(d["xf"])
                e = {"E_o": d["E_o"] if b == 0 else _f(d["E_o"].numel(), dev), "xf": xf[key],
                     "wf": d["wf"] if b == 0 else torch.zeros_like(d["wf"]),
                     "Y": d["Y"] if b == 0 else torch.empty_like(d["Y"]),
                     "R": d["R"] if b == 0 else torch.empty_like(d["R"]),
                     "Z": (d["Z"] if b == 0 else torch.empty_like(d["Z"])) if d["Z"] is not None else None,
                     "c0": d["c0"] if b == 0 else _f(1, dev)}
                if self.mode == "rlc_out":
                    e.update(rounds=torch.zeros((d["n"], 3), dtype=torch.int64, device=dev),
                             finals=torch.zeros((1, 2), dtype=torch.int64, device=dev),
                             claim0=torch.zeros(1, dtype=torch.int64, device=dev))
                st["maps"].append(e)
            st["x_jobs"] = [(self.tens[x], cp, buf) for (x, n), buf in
                            ((k, xf[k]) for k in xf) for cp in [1 << n]]
            if self.mode == "rlc_out":
                st["rlc"] = _f(1, dev)
            else:
                st["c0_batch"] = _f(1, dev)
                st["rounds"] = torch.zeros((cfg.batched_n, 3), dtype=torch.int64, device=dev)
                st["finals"] = torch.zeros((len(self.mm), 2), dtype=torch.int64, device=dev)
                st["claim0"] = torch.zeros(1, dtype=torch.int64, device=dev)
            self.sets.append(st)
        self.k = 0
        self.step_ws = StepWorkspace()
        # maps in the launch order (longest reduction first), as in the parent's jobs
        self.order = sorted(range(len(self.mm)), key=lambda i: -self.mm[i]["m"].d_in)

    def _set(self, k):
        return self.sets[k % self.SETS]

    def _eq_pairs(self, st):
        return [(self.ch["r_t"], st["E_t"])] + [(self.ch["r_o/" + d["m"].name], e["E_o"])
                                                for d, e in zip(self.mm, st["maps"])]

    def _jobs(self, st):
        return [MatmulJob(self.tens[self.mm[i]["m"].x], self.packed[self.mm[i]["m"].w], st["maps"][i]["Y"],
                          st["maps"][i]["R"], st["maps"][i]["Z"], st["E_t"], st["maps"][i]["E_o"], st["maps"][i]["c0"])
                for i in self.order]

    def _x_folds(self, st):
        return [(M, st["E_t"], cp, out) for (M, cp, out) in st["x_jobs"]]

    def _w_folds(self, st, st2=None):
        """Every map's weight fold of one proof, or of two proofs from one read of the weights."""
        out = []
        for i, d in enumerate(self.mm):
            e = st["maps"][i]
            job = (self.tens[d["m"].w], e["E_o"], 1 << d["n"], e["wf"])
            if st2 is not None:
                job += (st2["maps"][i]["E_o"], st2["maps"][i]["wf"])
            out.append(job)
        return out

    def _step_folds(self, k):
        """Proof k-1's folds of X; on even k the weight folds of proofs k-1 and k (the layer's weights
        read once for both: proof k's fold needs only its eq tables, built in step k-1)."""
        jobs = self._x_folds(self._set(k - 1)) if k >= 1 else []
        if k % 2 == 0:
            jobs += self._w_folds(self._set(k - 1), self._set(k)) if k >= 1 else self._w_folds(self._set(k))
        return jobs

    def _sumchecks(self, st):
        if self.mode == "rlc_out":
            return [SumcheckJob([e["xf"]], [e["wf"]], self.ch["rounds/" + d["m"].name], e["rounds"], e["finals"],
                                e["claim0"]) for d, e in zip(self.mm, st["maps"])]
        return [SumcheckJob([e["xf"] for e in st["maps"]], [e["wf"] for e in st["maps"]], self.ch["rounds"],
                            st["rounds"], st["finals"], st["claim0"], rho=self.rho)]

    def _merge_set(self, st):
        if self.mode == "rlc_out":
            combine_claims([e["rounds"][-1] for e in st["maps"]],
                           [self.ch["rounds/" + d["m"].name][-1:] for d in self.mm], self.rho, out=st["rlc"])
        else:
            linear_combine([e["c0"] for e in st["maps"]], self.rho, out=st["c0_batch"])

    def _step(self, k, tail: bool):
        cur, nxt, old = self._set(k), self._set(k + 1), self._set(k - 2)
        layer_step_multi(self._jobs(cur), self.s, group_o=self.group_o, eq=self._eq_pairs(nxt),
                         folds=self._step_folds(k), sumchecks=self._sumchecks(old) if tail else (), ws=self.step_ws)
        if tail:
            self._merge_set(old)

    def run(self, mark=_nomark):
        mark("step")
        if self.k == 0:
            st = self._set(0)
            eq_table_batched([r for r, _ in self._eq_pairs(st)], [E for _, E in self._eq_pairs(st)])
        self._step(self.k, self.k >= 2)
        mark("end")
        self.k += 1

    def phases(self):
        # the steady state alternates a step with two proofs' weight folds and one without
        wit = "witness" if self.keep_z else "witness(Y,R)"
        n = itertools.count()
        return [(wit + "+claim(acc)+eq+fold(W/2)+sumcheck", lambda: self._step(2 + next(n) % 2, True))]

    def capture(self, steps: int = 1):
        if steps % self.GRAPH_QUANTUM:
            raise ValueError("a captured graph holds a multiple of %d steps" % self.GRAPH_QUANTUM)
        while self.k < 2:
            self.run()
        self.run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                self.run()
        torch.cuda.synchronize()
        self.graph = g
        self.graph_steps = steps
        self.k_graph = self.k
        return g

    def replay(self):
        self.graph.replay()
        self.k = self.k_graph

    def drain(self):
        """The sum-check of the next-to-last proof, then the folds and sum-check of the last one (its
        weight folds were made in its own step when its index is even)."""
        last = self.k - 1
        if last < 0:
            return
        if last >= 1:
            self._finish(self._set(last - 1))
        st = self._set(last)
        fold_claim_batched(self._x_folds(st) + (self._w_folds(st) if last % 2 else []), [])
        self._finish(st)

    def _finish(self, st):
        for j in self._sumchecks(st):
            sumcheck_prove(j.As, j.Bs, j.r, rho=j.rho, rounds=j.rounds, finals=j.finals, claim0=j.claim0)
        self._merge_set(st)

    def output_tensors(self):
        out = []
        for st in self.sets:
            out.append(st["E_t"])
            for e in st["maps"]:
                out += [v for v in e.values() if v is not None]
            out += [st[k] for k in ("rlc", "c0_batch", "rounds", "finals", "claim0") if k in st]
        return out

    def results(self, k: int | None = None) -> dict:
        """Outputs of proof k (default: the last one)."""
        st = self._set(self.k - 1 if k is None else k)
        out = {"E_t": field_numpy(st["E_t"])}
        for d, e in zip(self.mm, st["maps"]):
            r = {"Y": e["Y"].cpu().numpy(), "R": e["R"].cpu().numpy(), "E_o": field_numpy(e["E_o"]),
                 "x_fold": field_numpy(e["xf"]), "w_fold": field_numpy(e["wf"]), "c0": int(field_numpy(e["c0"])[0])}
            if e["Z"] is not None:
                r["Z"] = e["Z"].cpu().numpy()
            if self.mode == "rlc_out":
                r.update(rounds=field_numpy(e["rounds"]), finals=field_numpy(e["finals"]),
                         claim0=int(field_numpy(e["claim0"])[0]))
            out[d["m"].name] = r
        if self.mode == "rlc_out":
            out["rlc"] = int(field_numpy(st["rlc"])[0])
        else:
            out["batch"] = {"rounds": field_numpy(st["rounds"]), "finals": field_numpy(st["finals"]),
                            "claim0": int(field_numpy(st["claim0"])[0]), "c0": int(field_numpy(st["c0_batch"])[0])}
        return out


class MoEBlockProver(_Prover):
    """MoE block: top-1 routed tokens grouped by expert (stable, ascending
    token order), one grouped witness launch per projection, and an
    independent claim + sum-check per expert and projection. A group of T_e
    tokens is logically padded with zero rows to 2^ceil(log2 T_e).

    With d and d_ff multiples of 16 (the full-size block) every expert's
    weights are packed once and the grouped witness reads them
    (fp_witness_grouped_packed), forming each expert's claim from its GEMM's
    accumulators, so Z is neither stored nor read back; the eq tables are
    built before it. Otherwise the row-major grouped witness stores Z and the
    claims come from it in the fold launch. keep_z: also store Z (tests)."""

    OUTPUTS = ("Xg", "Hg", "Zu", "Yu", "Ru", "Zd", "Yd", "Rd", "E_t", "E_ou", "E_od", "Au", "Bu", "Ad", "Bd", "c0",
               "rounds_u", "rounds_d", "finals", "claim0")

    def __init__(self, cfg, inp: dict, ch: dict, dev=None, keep_z: bool = False):
        dev = dev or torch.device("cuda")
        self.cfg = cfg
        s, d, dff = cfg.s, cfg.d_model, cfg.d_ff
        self.s = s
        route = np.asarray(inp["route"], np.int32)
        counts, offsets, perm = moe_plan(route, cfg.n_experts)
        self.counts, self.offsets = counts, offsets
        self.experts = [e for e in range(cfg.n_experts) if counts[e] > 0]
        ne = len(self.experts)
        self.perm = torch.from_numpy(perm.astype(np.int32)).to(dev)
        self.X, self.H = _i8(inp["X"], dev), _i8(inp["H"], dev)
        self.W1 = [_i8(inp["W1_%d" % e], dev) for e in self.experts]
        self.W2 = [_i8(inp["W2_%d" % e], dev) for e in self.experts]
        self.packed = d % 16 == 0 and dff % 16 == 0
        self.keep_z = keep_z or not self.packed
        if self.packed:
            self.W1p = [pack_weights(w) for w in self.W1]
            self.W2p = [pack_weights(w) for w in self.W2]
        T = len(route)
        self.Xg = torch.empty((T, d), dtype=torch.int8, device=dev)
        self.Hg = torch.empty((T, dff), dtype=torch.int8, device=dev)
        self.row_off = [0] + [int(offsets[e + 1]) for e in self.experts]
        self.n_up, self.n_dn = log2ceil(d), log2ceil(dff)   # sum-check rounds over each d_in
        self.Zu = torch.empty((T, dff), dtype=torch.int32, device=dev) if self.keep_z else None
        self.Yu = torch.empty((T, dff), dtype=torch.int8, device=dev)
        self.Ru = torch.empty((T, dff), dtype=torch.int8, device=dev)
        self.Zd = torch.empty((T, d), dtype=torch.int32, device=dev) if self.keep_z else None
        self.Yd = torch.empty((T, d), dtype=torch.int8, device=dev)
        self.Rd = torch.empty((T, d), dtype=torch.int8, device=dev)
        # challenges rearranged per kind (host-side marshalling, once)
        rt = [np.asarray(ch["r_t/%d" % e], np.uint64) for e in self.experts]
        self.nt = [len(v) for v in rt]
        self.ch = _Challenges({"r_t": np.concatenate(rt) if sum(self.nt) else np.zeros(0, np.uint64),
                               "r_o_up": np.concatenate([ch["r_o_up/%d" % e] for e in self.experts]),
                               "r_o_down": np.concatenate([ch["r_o_down/%d" % e] for e in self.experts]),
                               "rounds": np.concatenate([ch["rounds_up/%d" % e] for e in self.experts] +
                                                        [ch["rounds_down/%d" % e] for e in self.experts])}, dev)
        nu, nd = self.n_up, self.n_dn
        self.r_up = self.ch["rounds"][:ne * nu].view(ne, nu)
        self.r_dn = self.ch["rounds"][ne * nu:].view(ne, nd)
        no_up, no_dn = log2ceil(dff), log2ceil(d)
        self.E_t = [_f(1 << k, dev) for k in self.nt]
        self.E_ou = _f(ne << no_up, dev).view(ne, 1 << no_up)
        self.E_od = _f(ne << no_dn, dev).view(ne, 1 << no_dn)
        # x' and w' tables of the up and down claims, one row per expert
        self.Au, self.Bu = _f(ne << nu, dev).view(ne, 1 << nu), _f(ne << nu, dev).view(ne, 1 << nu)
        self.Ad, self.Bd = _f(ne << nd, dev).view(ne, 1 << nd), _f(ne << nd, dev).view(ne, 1 << nd)
        self.c0 = _f(2 * ne, dev)
        self.rounds_u = torch.empty((ne, nu, 3), dtype=torch.int64, device=dev)
        self.rounds_d = torch.empty((ne, nd, 3), dtype=torch.int64, device=dev)
        self.finals = torch.empty((2 * ne, 2), dtype=torch.int64, device=dev)
        self.claim0 = _f(2 * ne, dev)
        self.ws = StepWorkspace()
        # eq descriptor lists
        pos = 0
        self.rt_views = []
        for k in self.nt:
            self.rt_views.append(self.ch["r_t"][pos:pos + k])
            pos += k
        ru = self.ch["r_o_up"].view(ne, no_up)
        rd = self.ch["r_o_down"].view(ne, no_dn)
        self.eq_r = self.rt_views + [ru[i] for i in range(ne)] + [rd[i] for i in range(ne)]
        self.eq_E = self.E_t + [self.E_ou[i] for i in range(ne)] + [self.E_od[i] for i in range(ne)]
        self.fold_jobs = []
        self.claim_jobs = []
        for i in range(ne):
            a, b = self.row_off[i], self.row_off[i + 1]
            # with packed weights the weight folds come from the witness's own pass over the weights
            self.fold_jobs.append((self.Xg[a:b], self.E_t[i], 1 << nu, self.Au[i]))
            if not self.packed:
                self.fold_jobs.append((self.W1[i], self.E_ou[i], 1 << nu, self.Bu[i]))
            self.fold_jobs.append((self.Hg[a:b], self.E_t[i], 1 << nd, self.Ad[i]))
            if not self.packed:
                self.fold_jobs.append((self.W2[i], self.E_od[i], 1 << nd, self.Bd[i]))
            if not self.packed:
                self.claim_jobs.append((self.Zu[a:b], self.E_t[i], self.E_ou[i], self.c0[i:i + 1]))
                self.claim_jobs.append((self.Zd[a:b], self.E_t[i], self.E_od[i], self.c0[ne + i:ne + i + 1]))

    def _group(self):
        gather_rows(self.X, self.perm, self.Xg)
        gather_rows(self.H, self.perm, self.Hg)

    def _witness(self):
        ne = len(self.experts)
        if self.packed:
            witness_grouped_packed(self.Xg, self.W1p, self.row_off, self.s, self.Yu, self.Ru, self.Zu, self.E_t,
                                   self.E_ou, self.c0[:ne], w_fold=self.Bu, ws=self.ws)
            witness_grouped_packed(self.Hg, self.W2p, self.row_off, self.s, self.Yd, self.Rd, self.Zd, self.E_t,
                                   self.E_od, self.c0[ne:], w_fold=self.Bd, ws=self.ws)
        else:
            witness_linear_grouped(self.Xg, self.W1, self.row_off, self.s, self.Zu, self.Yu, self.Ru)
            witness_linear_grouped(self.Hg, self.W2, self.row_off, self.s, self.Zd, self.Yd, self.Rd)

    def _sumcheck(self):
        ne = len(self.experts)
        sumcheck_prove_multi(self.Au, self.Bu, self.r_up, rounds=self.rounds_u, finals=self.finals[:ne],
                             claim0=self.claim0[:ne])
        sumcheck_prove_multi(self.Ad, self.Bd, self.r_dn, rounds=self.rounds_d, finals=self.finals[ne:],
                             claim0=self.claim0[ne:])

    def phases(self):
        eq = ("eq", lambda: eq_table_batched(self.eq_r, self.eq_E))
        if self.packed:
            wname = "witness+claim(acc)+wfold(acc)" if self.keep_z else "witness(Y,R)+claim(acc)+wfold(acc)"
            return [("group", self._group), eq, (wname, self._witness),
                    ("xfold", lambda: fold_claim_batched(self.fold_jobs, [])), ("sumcheck", self._sumcheck)]
        return [("group", self._group), ("witness", self._witness), eq,
                ("fold+claim", lambda: fold_claim_batched(self.fold_jobs, self.claim_jobs)),
                ("sumcheck", self._sumcheck)]

    def results(self) -> dict:
        ne = len(self.experts)
        Au, Bu, Ad, Bd = (field_numpy(t) for t in (self.Au, self.Bu, self.Ad, self.Bd))
        ru, rd, finals = field_numpy(self.rounds_u), field_numpy(self.rounds_d), field_numpy(self.finals)
        c0, cl = field_numpy(self.c0), field_numpy(self.claim0)
        Yu, Ru = self.Yu.cpu().numpy(), self.Ru.cpu().numpy()
        Yd, Rd = self.Yd.cpu().numpy(), self.Rd.cpu().numpy()
        Zu = self.Zu.cpu().numpy() if self.Zu is not None else None
        Zd = self.Zd.cpu().numpy() if self.Zd is not None else None
        out = {}
        for i, e in enumerate(self.experts):
            a, b = self.row_off[i], self.row_off[i + 1]
            toks = self.perm[a:b].cpu().numpy()
            out[e] = {"tokens": toks,
                      "up": {"Y": Yu[a:b], "R": Ru[a:b], "x_fold": Au[i], "w_fold": Bu[i],
                             "c0": int(c0[i]), "rounds": ru[i], "finals": finals[i:i + 1],
                             "claim0": int(cl[i])},
                      "down": {"Y": Yd[a:b], "R": Rd[a:b], "x_fold": Ad[i], "w_fold": Bd[i],
                               "c0": int(c0[ne + i]), "rounds": rd[i], "finals": finals[ne + i:ne + i + 1],
                               "claim0": int(cl[ne + i])}}
            if Zu is not None:
                out[e]["up"]["Z"] = Zu[a:b]
                out[e]["down"]["Z"] = Zd[a:b]
        return out


LAYER_LABEL = b"zkp-layer-committed-rescale-v1"
LAYER_LOG_ROW = 18      # commitment rows of at most 2^18 elements
OPEN_COLUMNS = 64       # columns opened per proof


class FaithfulProver(_Prover):
    """A layer's linear maps proved with the rescale committed and every
    challenge taken from the transcript ("How fast can FlashProve go", §2: the
    prover commits intermediate values, sum-check reduces each matmul to claims
    about them and the weights, openings settle the claims, and every challenge
    hashes all the prover has sent so far; §3.1: g_w and the remainder r are
    committed, never g^, and the claim about g^ reads 2^k g_w + r; §4 footnote
    20: the challenges live in an extension). In order:
      witness    each map's Z, Y, R (Z kept: Q is read from it);
      commit     each map's Q (before the clamp), R and Y as zero-padded
                 [2^n_t, 2^n_o] field tables in whole rows of 2^L elements
                 (L = min(18, min n_t + n_o)), Reed-Solomon encoded, the columns
                 in a salted BLAKE2b Merkle tree;
      transcript the label and the layer's shape, then the root; r_t, each
                 map's r_o and a proximity point r_prox over the rows;
      eq, folds  E_t, E_o over the extension; x'_m, w'_m (two base folds each);
      open rows  the proximity row and, per map, the folded rows of Q and of R
                 at (r_o || r_t) (the verifier reads the claims 2^s Q~ + R~ from
                 them); their Merkle root (zero salts) is absorbed;
      sumcheck   batched layers: rho, then one sum-check of
                 sum_m rho_m x'_m . w'_m; otherwise one sum-check per map, then
                 rho; every round absorbed before its challenge, the finals after;
      columns    64 columns drawn from the transcript, gathered with their
                 salts and Merkle paths.
    The verifier needs no witness: the claims come from the commitment's
    openings and the finals are claims about X and W."""

    def __init__(self, cfg, inp: dict, salts: np.ndarray, dev=None):
        dev = dev or torch.device("cuda")
        self.cfg, self.s = cfg, cfg.s
        self.batched = cfg.kind == "batched"
        T = cfg.T
        self.tens = {}
        for m in cfg.matmuls:
            for nm in (m.x, m.w):
                if nm not in self.tens:
                    self.tens[nm] = _i8(inp[nm], dev)
        self.packed = {m.w: _packed(self.tens[m.w]) for m in cfg.matmuls}
        M = len(cfg.matmuls)
        self.M = M
        self.n_t = log2ceil(T)
        self.n_o = [log2ceil(m.d_out) for m in cfg.matmuls]
        self.L = min(LAYER_LOG_ROW, min(self.n_t + n for n in self.n_o))
        self.base, row = [], 0
        for n in self.n_o:
            k = 1 << (self.n_t + n - self.L)
            self.base.append((row, row + k, row + 2 * k, k))
            row += 3 * k
        self.rows = row
        self.n_prox = log2ceil(row)
        width = 2 << self.L
        assert salts.shape == (width, 16)
        self.salts = _i8(salts.astype(np.uint8), dev)
        self.Z = [torch.empty((T, m.d_out), dtype=torch.int32, device=dev) for m in cfg.matmuls]
        self.Y = [torch.empty((T, m.d_out), dtype=torch.int8, device=dev) for m in cfg.matmuls]
        self.R = [torch.empty((T, m.d_out), dtype=torch.int8, device=dev) for m in cfg.matmuls]
        self.msg = torch.empty((self.rows, 1 << self.L), dtype=torch.int64, device=dev)
        self.code = torch.empty((self.rows, width), dtype=torch.int64, device=dev)
        self.tree = torch.empty((2 * width - 1, 32), dtype=torch.uint8, device=dev)
        self.state = torch.empty(32, dtype=torch.uint8, device=dev)
        words = [T, cfg.s, M, int(self.batched), self.L, OPEN_COLUMNS]
        for m in cfg.matmuls:
            words += [m.d_in, m.d_out]
        self.init_msg = LAYER_LABEL + b"".join(int(v).to_bytes(4, "little") for v in words)
        self.n_ch = self.n_t + sum(self.n_o) + self.n_prox
        self.chal = torch.empty((max(1, self.n_ch), 2), dtype=torch.int64, device=dev)
        self.r_t = self.chal[:self.n_t]
        off = self.n_t
        self.r_o = []
        for n in self.n_o:
            self.r_o.append(self.chal[off:off + n])
            off += n
        self.r_prox = self.chal[off:off + self.n_prox]
        # each claim's row point: the coordinates of (r_o || r_t) from L on
        self.claims = []
        for m, n in enumerate(self.n_o):
            if self.L <= n:
                z1, z2 = self.r_o[m][self.L:], self.r_t
            else:
                z1, z2 = self.r_t[self.L - n:], self.r_t[:0]
            rq, rr, _, _ = self.base[m]
            self.claims += [(rq, z1, z2), (rr, z1, z2)]
        self.Et = [_f(1 << self.n_t, dev), _f(1 << self.n_t, dev)]
        self.Eo = [[_f(1 << n, dev), _f(1 << n, dev)] for n in self.n_o]
        n_all = max(m.n for m in cfg.matmuls)
        self.n_sc = [n_all if self.batched else m.n for m in cfg.matmuls]
        xf = {}
        self.xf, self.wf = [], []
        for m, n in zip(cfg.matmuls, self.n_sc):
            if (m.x, n) not in xf:
                xf[(m.x, n)] = [_f(1 << n, dev), _f(1 << n, dev)]
            self.xf.append(xf[(m.x, n)])
            self.wf.append([_f(1 << n, dev), _f(1 << n, dev)])
        self.x_jobs = [(self.tens[x], n, parts) for (x, n), parts in xf.items()]
        K = 1 + 2 * M
        self.U = torch.empty((K, 2, 1 << self.L), dtype=torch.int64, device=dev)
        self.zero_salts = torch.zeros((1 << self.L, 16), dtype=torch.uint8, device=dev)
        self.tree_u = torch.empty((2 * (1 << self.L) - 1, 32), dtype=torch.uint8, device=dev)
        self.rho = torch.empty((M, 2), dtype=torch.int64, device=dev)
        groups = [list(range(M))] if self.batched else [[m] for m in range(M)]
        self.sc = []
        for g in groups:
            n = self.n_sc[g[0]]
            self.sc.append({"maps": g, "rounds": torch.empty((max(n, 1), 3, 2), dtype=torch.int64, device=dev),
                            "r": torch.empty((max(n, 1), 2), dtype=torch.int64, device=dev),
                            "finals": torch.empty((len(g), 2, 2), dtype=torch.int64, device=dev), "n": n})
        self.chal_cols = torch.empty((OPEN_COLUMNS, 2), dtype=torch.int64, device=dev)
        self.cols = torch.empty((OPEN_COLUMNS, self.rows), dtype=torch.int64, device=dev)
        self.col_salts = torch.empty((OPEN_COLUMNS, 16), dtype=torch.uint8, device=dev)
        self.paths = torch.empty((OPEN_COLUMNS, self.L + 1, 32), dtype=torch.uint8, device=dev)
        self.idx = torch.empty(OPEN_COLUMNS, dtype=torch.int32, device=dev)
        fused = sorted((j for j, m in enumerate(cfg.matmuls) if self.packed[m.w] is not None),
                       key=lambda j: -cfg.matmuls[j].d_in)
        self.jobs = [MatmulJob(self.tens[cfg.matmuls[j].x], self.packed[cfg.matmuls[j].w], self.Y[j], self.R[j],
                               self.Z[j]) for j in fused]
        self.ws = StepWorkspace()

    def _witness(self):
        if self.jobs:
            witness_multi(self.jobs, self.s, ws=self.ws)
        for j, m in enumerate(self.cfg.matmuls):
            if self.packed[m.w] is None:
                witness_linear(self.tens[m.x], self.tens[m.w], self.s, self.Z[j], self.Y[j], self.R[j])

    def _commit(self):
        commit_tables([(self.Z[j], self.n_o[j], *self.base[j][:3]) for j in range(self.M)], self.n_t, self.s,
                      self.msg)
        rs_encode(self.msg, code=self.code)
        merkle_commit(self.code, self.salts, tree=self.tree)

    def _challenges(self):
        fs_init(self.state, self.init_msg)
        fs_absorb(self.state, self.tree[-1].view(torch.int64))
        fs_challenges(self.state, self.n_ch, out=self.chal)

    def _eq(self):
        eq_table_ext(self.r_t, self.Et[0], self.Et[1])
        for j in range(self.M):
            eq_table_ext(self.r_o[j], self.Eo[j][0], self.Eo[j][1])

    def _folds(self):
        jobs = []
        for X, n, parts in self.x_jobs:
            jobs += [(X, self.Et[0], 1 << n, parts[0]), (X, self.Et[1], 1 << n, parts[1])]
        for j, m in enumerate(self.cfg.matmuls):
            W, n = self.tens[m.w], self.n_sc[j]
            jobs += [(W, self.Eo[j][0], 1 << n, self.wf[j][0]), (W, self.Eo[j][1], 1 << n, self.wf[j][1])]
        fold_matrix_batched(jobs)

    def _open_rows(self):
        commit_fold_ext(self.msg, self.r_prox, self.claims, self.U)
        merkle_commit(self.U.view(-1, 1 << self.L), self.zero_salts, tree=self.tree_u)
        fs_absorb(self.state, self.tree_u[-1].view(torch.int64))

    def _sumcheck(self):
        if self.batched:
            fs_challenges(self.state, self.M, out=self.rho)
        for sc in self.sc:
            g = sc["maps"]
            sumcheck_ext_fs_multi([self.xf[j][0] for j in g], [self.xf[j][1] for j in g],
                                  [self.wf[j][0] for j in g], [self.wf[j][1] for j in g], self.state,
                                  rho=self.rho if self.batched else None, rounds=sc["rounds"], r=sc["r"],
                                  finals=sc["finals"])
        if not self.batched:
            fs_challenges(self.state, self.M, out=self.rho)

    def _columns(self):
        # the columns' challenges are read from the final state (nothing absorbed after)
        fs_challenges(self.state, OPEN_COLUMNS, out=self.chal_cols)
        merkle_open(self.code, self.salts, self.tree, self.chal_cols, cols=self.cols, col_salts=self.col_salts,
                    paths=self.paths, idx=self.idx)

    def phases(self):
        return [("witness", self._witness), ("commit", self._commit), ("transcript", self._challenges),
                ("eq", self._eq), ("folds", self._folds), ("open rows", self._open_rows),
                ("sumcheck", self._sumcheck), ("columns", self._columns)]

    def output_tensors(self):
        return ([self.U, self.rho, self.state, self.cols, self.col_salts, self.paths, self.idx, self.tree]
                + [sc[k] for sc in self.sc for k in ("rounds", "r", "finals")])

    def results(self) -> dict:
        e2 = lambda t: [tuple(int(x) for x in row) for row in field_numpy(t.reshape(-1, 2))]
        sumchecks = []
        for sc in self.sc:
            n = sc["n"]
            rounds = [e2(sc["rounds"][i]) for i in range(n)]
            fin = e2(sc["finals"])
            sumchecks.append({"rounds": rounds, "r": e2(sc["r"][:n]),
                              "finals": [(fin[2 * j], fin[2 * j + 1]) for j in range(len(sc["maps"]))]})
        paths = self.paths.cpu().numpy()
        return {"root": bytes(self.tree[-1].cpu().numpy()), "U": field_numpy(self.U),
                "sumchecks": sumchecks, "rho": e2(self.rho), "state": bytes(self.state.cpu().numpy()),
                "idx": [int(v) for v in self.idx.cpu().numpy()], "columns": field_numpy(self.cols),
                "col_salts": self.col_salts.cpu().numpy(),
                "paths": [[bytes(paths[q, d]) for d in range(self.L + 1)] for q in range(OPEN_COLUMNS)],
                "Y": [y.cpu().numpy() for y in self.Y], "R": [r.cpu().numpy() for r in self.R]}


def can_pipeline(cfg) -> bool:
    """Whether proofs of this workload can overlap (one sum-check that fits the
    workgroup inside the witness launch)."""
    return cfg.kind == "single" and (1 << cfg.matmuls[0].n) <= OVERLAP_ENTRIES


def can_overlap(cfg) -> bool:
    """Whether three proofs can be in flight (the packed witness applies to every map, and a single layer's
    sum-check fits the workgroup inside the witness launch)."""
    if cfg.kind in ("rlc_out", "batched"):
        return all(m.d_in % 16 == 0 for m in cfg.matmuls)
    return can_pipeline(cfg) and cfg.matmuls[0].d_in % 16 == 0


def make_prover(cfg, inp: dict, ch: dict, dev=None, pipelined: bool = False, overlapped: bool = False,
                keep_z: bool = False):
    """overlapped: three proofs in flight (OverlappedLayerProver), for single
    layers with packed weights (keep_z: also write Z); pipelined: two
    (SingleLayerProver)."""
    if cfg.kind == "single":
        m = cfg.matmuls[0]
        if overlapped:
            return OverlappedLayerProver(inp[m.x], inp[m.w], cfg.s, ch, dev, keep_z=keep_z)
        return SingleLayerProver(inp[m.x], inp[m.w], cfg.s, ch, dev, pipelined=pipelined)
    if cfg.kind in ("rlc_out", "batched"):
        group_o = 4 if cfg.T >= 2048 else 1
        if overlapped:
            return OverlappedMultiProver(cfg, inp, ch, dev, keep_z=keep_z, group_o=group_o)
        if pipelined:
            raise ValueError("multi-map layers keep one proof in flight or three (overlapped)")
        return MultiMatmulProver(cfg, inp, ch, dev, keep_z=keep_z, group_o=group_o)
    if pipelined:
        raise ValueError("pipelined proofs are implemented for single-matmul layers")
    if cfg.kind == "moe":
        return MoEBlockProver(cfg, inp, ch, dev, keep_z=keep_z)
    raise ValueError(cfg.kind)
