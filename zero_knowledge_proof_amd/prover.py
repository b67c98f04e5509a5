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

import numpy as np
import torch

from . import (StepWorkspace, combine_claims, commit_pack, commit_rows, eq_table_batched, eq_table_ext,
               ext_claim_combine, field_numpy, fold_claim_batched, fs_absorb, fs_challenges, fs_init, gather_rows,
               layer_step, linear_combine, merkle_commit, moe_plan, pack_weights, rs_encode, sumcheck_ext_fs,
               sumcheck_prove, sumcheck_prove_multi, to_field_tensor, witness_linear, witness_linear_grouped,
               witness_linear_packed, witness_linear_packed_with_sumcheck, witness_linear_with_sumcheck)


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
            out.extend(v if isinstance(v, list) else [v])
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
    steps. ``drain()`` finishes the last two proofs; outputs are those of the
    last proof. keep_z: also write Z (which the proof never reads back)."""

    PER_PROOF = ("Z", "Y", "R", "E_t", "E_o", "xf", "wf", "c0")
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
                   rounds=self.rounds, finals=self.finals, claim0=self.claim0, ws=self.ws)

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
            sumcheck_prove([prev["xf"]], [prev["wf"]], self.ch["rounds"], rounds=self.rounds, finals=self.finals,
                           claim0=self.claim0)
        cur = self._buf(last)
        fold_claim_batched(self._folds(cur), [])
        sumcheck_prove([cur["xf"]], [cur["wf"]], self.ch["rounds"], rounds=self.rounds, finals=self.finals,
                       claim0=self.claim0)

    def output_tensors(self):
        return [t for b in self.bufs for t in b.values() if t is not None] + [self.rounds, self.finals, self.claim0]

    def results(self) -> dict:
        b = self._buf(self.k - 1)
        out = {"Y": b["Y"].cpu().numpy(), "R": b["R"].cpu().numpy(),
               "E_t": field_numpy(b["E_t"]), "E_o": field_numpy(b["E_o"]),
               "x_fold": field_numpy(b["xf"]), "w_fold": field_numpy(b["wf"]),
               "c0": int(field_numpy(b["c0"])[0]), "rounds": field_numpy(self.rounds),
               "finals": field_numpy(self.finals), "claim0": int(field_numpy(self.claim0)[0])}
        if b["Z"] is not None:
            out["Z"] = b["Z"].cpu().numpy()
        return out


class MultiMatmulProver(_Prover):
    """Several linear maps of one layer sharing the token axis (one r_t).

    mode "rlc_out": each claim gets its own sum-check; the finished claims are
    merged by a random linear combination (the dense MLP's gate/up/down).
    mode "batched": the claims are merged first (rho-weighted) and proved by
    one batched sum-check over tables padded to 2^batched_n (all seven maps of
    a transformer layer)."""

    def output_tensors(self):
        out = [self.E_t]
        for d in self.mm:
            out += [d[k] for k in ("Z", "Y", "R", "E_o", "xf", "wf", "c0", "rounds", "finals", "claim0") if k in d]
        for k in ("rlc", "c0_batch", "rounds", "finals", "claim0"):
            if hasattr(self, k):
                out.append(getattr(self, k))
        return out

    def __init__(self, cfg, inp: dict, ch: dict, dev=None):
        dev = dev or torch.device("cuda")
        self.cfg = cfg
        self.mode = cfg.kind
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
        for m in cfg.matmuls:
            n = nb if nb is not None else m.n
            key = (m.x, n)
            if key not in xf:
                xf[key] = _f(1 << n, dev)
            d = {"m": m, "n": n, "xf": xf[key], "wf": _f(1 << n, dev), "E_o": _f(1 << m.n_o, dev),
                 "Z": torch.empty((T, m.d_out), dtype=torch.int32, device=dev),
                 "Y": torch.empty((T, m.d_out), dtype=torch.int8, device=dev),
                 "R": torch.empty((T, m.d_out), dtype=torch.int8, device=dev), "c0": _f(1, dev)}
            if self.mode == "rlc_out":
                d.update(rounds=torch.empty((n, 3), dtype=torch.int64, device=dev),
                         finals=torch.empty((1, 2), dtype=torch.int64, device=dev), claim0=_f(1, dev))
            self.mm.append(d)
        self.x_jobs = [(self.tens[x], None, 1 << n, buf) for (x, n), buf in xf.items()]
        self.packed = {m.w: _packed(self.tens[m.w]) for m in cfg.matmuls}
        if self.mode == "rlc_out":
            self.rho = torch.cat([self.ch["rho/" + m.name] for m in cfg.matmuls]).contiguous()
            self.rlc = _f(1, dev)
        else:
            self.rho = torch.cat([self.ch["rho/" + m.name] for m in cfg.matmuls]).contiguous()
            self.c0_batch = _f(1, dev)
            self.rounds = torch.empty((nb, 3), dtype=torch.int64, device=dev)
            self.finals = torch.empty((len(cfg.matmuls), 2), dtype=torch.int64, device=dev)
            self.claim0 = _f(1, dev)

    def _eq_pairs(self):
        return [(self.ch["r_t"], self.E_t)] + [(self.ch["r_o/" + d["m"].name], d["E_o"]) for d in self.mm]

    def _fuse_eq(self) -> bool:
        # the first packed witness launch can build all eq tables (at most 8 per launch)
        return any(v is not None for v in self.packed.values()) and len(self.mm) + 1 <= 8

    def _witness(self, with_eq: bool = False):
        eq = self._eq_pairs() if with_eq else None
        for d in self.mm:
            m = d["m"]
            Wp = self.packed[m.w]
            if Wp is not None:
                witness_linear_packed(self.tens[m.x], Wp, self.s, d["Z"], d["Y"], d["R"], eq=eq)
                eq = None
            else:
                witness_linear(self.tens[m.x], self.tens[m.w], self.s, d["Z"], d["Y"], d["R"])

    def _eq(self):
        eq_table_batched([self.ch["r_t"]] + [self.ch["r_o/" + d["m"].name] for d in self.mm],
                         [self.E_t] + [d["E_o"] for d in self.mm])

    def _fold_claim(self):
        jobs = [(M, self.E_t, cp, out) for (M, _, cp, out) in self.x_jobs]
        jobs += [(self.tens[d["m"].w], d["E_o"], 1 << d["n"], d["wf"]) for d in self.mm]
        fold_claim_batched(jobs, [(d["Z"], self.E_t, d["E_o"], d["c0"]) for d in self.mm])

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
        if self._fuse_eq():
            ph = [("witness+eq", lambda: self._witness(with_eq=True)), ("fold+claim", self._fold_claim),
                  ("sumcheck", self._sumcheck)]
        else:
            ph = [("witness", self._witness), ("eq", self._eq), ("fold+claim", self._fold_claim),
                  ("sumcheck", self._sumcheck)]
        if self.mode == "rlc_out":
            ph.append(("merge", self._merge))
        return ph

    def results(self) -> dict:
        out = {"E_t": field_numpy(self.E_t)}
        for d in self.mm:
            r = {"Z": d["Z"].cpu().numpy(), "Y": d["Y"].cpu().numpy(), "R": d["R"].cpu().numpy(),
                 "E_o": field_numpy(d["E_o"]), "x_fold": field_numpy(d["xf"]), "w_fold": field_numpy(d["wf"]),
                 "c0": int(field_numpy(d["c0"])[0])}
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


class MoEBlockProver(_Prover):
    """MoE block: top-1 routed tokens grouped by expert (stable, ascending
    token order), one grouped witness launch per projection, and an
    independent claim + sum-check per expert and projection. A group of T_e
    tokens is logically padded with zero rows to 2^ceil(log2 T_e)."""

    OUTPUTS = ("Xg", "Hg", "Zu", "Yu", "Ru", "Zd", "Yd", "Rd", "E_t", "E_ou", "E_od", "Au", "Bu", "Ad", "Bd", "c0",
               "rounds_u", "rounds_d", "finals", "claim0")

    def __init__(self, cfg, inp: dict, ch: dict, dev=None):
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
        T = len(route)
        self.Xg = torch.empty((T, d), dtype=torch.int8, device=dev)
        self.Hg = torch.empty((T, dff), dtype=torch.int8, device=dev)
        self.row_off = [0] + [int(offsets[e + 1]) for e in self.experts]
        self.n_up, self.n_dn = log2ceil(d), log2ceil(dff)   # sum-check rounds over each d_in
        self.Zu = torch.empty((T, dff), dtype=torch.int32, device=dev)
        self.Yu = torch.empty((T, dff), dtype=torch.int8, device=dev)
        self.Ru = torch.empty((T, dff), dtype=torch.int8, device=dev)
        self.Zd = torch.empty((T, d), dtype=torch.int32, device=dev)
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
            self.fold_jobs.append((self.Xg[a:b], self.E_t[i], 1 << nu, self.Au[i]))
            self.fold_jobs.append((self.W1[i], self.E_ou[i], 1 << nu, self.Bu[i]))
            self.fold_jobs.append((self.Hg[a:b], self.E_t[i], 1 << nd, self.Ad[i]))
            self.fold_jobs.append((self.W2[i], self.E_od[i], 1 << nd, self.Bd[i]))
            self.claim_jobs.append((self.Zu[a:b], self.E_t[i], self.E_ou[i], self.c0[i:i + 1]))
            self.claim_jobs.append((self.Zd[a:b], self.E_t[i], self.E_od[i], self.c0[ne + i:ne + i + 1]))

    def _group(self):
        gather_rows(self.X, self.perm, self.Xg)
        gather_rows(self.H, self.perm, self.Hg)

    def _witness(self):
        witness_linear_grouped(self.Xg, self.W1, self.row_off, self.s, self.Zu, self.Yu, self.Ru)
        witness_linear_grouped(self.Hg, self.W2, self.row_off, self.s, self.Zd, self.Yd, self.Rd)

    def _sumcheck(self):
        ne = len(self.experts)
        sumcheck_prove_multi(self.Au, self.Bu, self.r_up, rounds=self.rounds_u, finals=self.finals[:ne],
                             claim0=self.claim0[:ne])
        sumcheck_prove_multi(self.Ad, self.Bd, self.r_dn, rounds=self.rounds_d, finals=self.finals[ne:],
                             claim0=self.claim0[ne:])

    def phases(self):
        return [("group", self._group), ("witness", self._witness),
                ("eq", lambda: eq_table_batched(self.eq_r, self.eq_E)),
                ("fold+claim", lambda: fold_claim_batched(self.fold_jobs, self.claim_jobs)),
                ("sumcheck", self._sumcheck)]

    def results(self) -> dict:
        ne = len(self.experts)
        Au, Bu, Ad, Bd = (field_numpy(t) for t in (self.Au, self.Bu, self.Ad, self.Bd))
        ru, rd, finals = field_numpy(self.rounds_u), field_numpy(self.rounds_d), field_numpy(self.finals)
        c0, cl = field_numpy(self.c0), field_numpy(self.claim0)
        Zu, Yu, Ru = self.Zu.cpu().numpy(), self.Yu.cpu().numpy(), self.Ru.cpu().numpy()
        Zd, Yd, Rd = self.Zd.cpu().numpy(), self.Yd.cpu().numpy(), self.Rd.cpu().numpy()
        out = {}
        for i, e in enumerate(self.experts):
            a, b = self.row_off[i], self.row_off[i + 1]
            toks = self.perm[a:b].cpu().numpy()
            out[e] = {"tokens": toks,
                      "up": {"Z": Zu[a:b], "Y": Yu[a:b], "R": Ru[a:b], "x_fold": Au[i], "w_fold": Bu[i],
                             "c0": int(c0[i]), "rounds": ru[i], "finals": finals[i:i + 1],
                             "claim0": int(cl[i])},
                      "down": {"Z": Zd[a:b], "Y": Yd[a:b], "R": Rd[a:b], "x_fold": Ad[i], "w_fold": Bd[i],
                               "c0": int(c0[ne + i]), "rounds": rd[i], "finals": finals[ne + i:ne + i + 1],
                               "claim0": int(cl[ne + i])}}
        return out


FS_LABEL = b"zkp-matmul-sumcheck-fs-v1"


def commit_logn(n_limbs: int) -> int:
    """Row length 2^logn of the commitment of n_limbs limbs: 2^22 elements as on
    the pages, or the smallest power of two holding them all."""
    return min(22, log2ceil(max(1, (n_limbs + 2) // 3)))


class FaithfulLayerProver(_Prover):
    """One linear map proved with soundness-faithful challenges ("How fast can
    FlashProve go", §2: every challenge hashes all the prover has sent so far;
    §4 footnote 20: the challenges live in an extension field). In order:
    the witness; the commitment of Y and R (limbs packed three per element,
    rows Reed-Solomon encoded, salted BLAKE2b Merkle tree); the transcript
    absorbs the layer's shape and the Merkle root and yields r_t, r_o in
    F_p[u]/(u^2 - 7); the eq tables and the folds of X and W (two base folds
    each) and the claim c0 (four base claims combined) follow; c0 is absorbed;
    the sum-check over the extension absorbs each round and draws each r_i
    from the transcript on the device; the finals are absorbed."""

    def __init__(self, X: np.ndarray, W: np.ndarray, s: int, salts: np.ndarray, dev=None):
        dev = dev or torch.device("cuda")
        self.s = s
        self.X, self.W = _i8(X, dev), _i8(W, dev)
        self.Wp = _packed(self.W)
        T, d_in = X.shape
        d_out = W.shape[0]
        self.T, self.d_in, self.d_out = T, d_in, d_out
        self.n_t, self.n_o, self.n = log2ceil(T), log2ceil(d_out), log2ceil(d_in)
        self.Z = torch.empty((T, d_out), dtype=torch.int32, device=dev)
        self.Y = torch.empty((T, d_out), dtype=torch.int8, device=dev)
        self.R = torch.empty((T, d_out), dtype=torch.int8, device=dev)
        self.logn = commit_logn(2 * T * d_out)
        self.rows = commit_rows(T * d_out, T * d_out, self.logn)
        width = 2 << self.logn
        assert salts.shape == (width, 16)
        self.salts = _i8(salts.astype(np.uint8), dev)
        self.msg = torch.empty((self.rows, 1 << self.logn), dtype=torch.int64, device=dev)
        self.code = torch.empty((self.rows, width), dtype=torch.int64, device=dev)
        self.tree = torch.empty((2 * width - 1, 32), dtype=torch.uint8, device=dev)
        self.state = torch.empty(4, dtype=torch.int64, device=dev)
        self.init_msg = FS_LABEL + b"".join(int(v).to_bytes(4, "little") for v in (T, d_in, d_out, s))
        self.chal = torch.empty((max(1, self.n_t + self.n_o), 2), dtype=torch.int64, device=dev)
        self.Et = [_f(1 << self.n_t, dev), _f(1 << self.n_t, dev)]
        self.Eo = [_f(1 << self.n_o, dev), _f(1 << self.n_o, dev)]
        self.xf = [_f(1 << self.n, dev), _f(1 << self.n, dev)]
        self.wf = [_f(1 << self.n, dev), _f(1 << self.n, dev)]
        self.c4 = _f(4, dev)
        self.c0 = _f(2, dev)
        self.rounds = torch.empty((max(1, self.n), 3, 2), dtype=torch.int64, device=dev)
        self.r = torch.empty((max(1, self.n), 2), dtype=torch.int64, device=dev)
        self.finals = torch.empty((2, 2), dtype=torch.int64, device=dev)

    def _commit(self):
        commit_pack(self.Y.reshape(-1), self.R.reshape(-1), self.logn, self.rows, out=self.msg)
        rs_encode(self.msg, code=self.code)
        merkle_commit(self.code, self.salts, tree=self.tree)

    def _challenges(self):
        fs_init(self.state, self.init_msg)
        fs_absorb(self.state, self.tree[-1].view(torch.int64))
        fs_challenges(self.state, self.n_t + self.n_o, out=self.chal)

    def _eq(self):
        eq_table_ext(self.chal[:self.n_t], self.Et[0], self.Et[1])
        eq_table_ext(self.chal[self.n_t:self.n_t + self.n_o], self.Eo[0], self.Eo[1])

    def _fold_claim(self):
        N = 1 << self.n
        Et, Eo, c4 = self.Et, self.Eo, self.c4
        fold_claim_batched([(self.X, Et[0], N, self.xf[0]), (self.X, Et[1], N, self.xf[1]),
                            (self.W, Eo[0], N, self.wf[0]), (self.W, Eo[1], N, self.wf[1])],
                           [(self.Z, Et[0], Eo[0], c4[0:1]), (self.Z, Et[1], Eo[1], c4[1:2]),
                            (self.Z, Et[0], Eo[1], c4[2:3]), (self.Z, Et[1], Eo[0], c4[3:4])])
        ext_claim_combine(self.c4, self.c0)
        fs_absorb(self.state, self.c0)

    def _sumcheck(self):
        sumcheck_ext_fs(self.xf[0], self.xf[1], self.wf[0], self.wf[1], self.state, rounds=self.rounds, r=self.r,
                        finals=self.finals)

    def phases(self):
        return [("witness", lambda: _witness(self.X, self.W, self.Wp, self.s, self.Z, self.Y, self.R)),
                ("commit", self._commit), ("transcript", self._challenges), ("eq", self._eq),
                ("fold+claim", self._fold_claim), ("sumcheck", self._sumcheck)]

    def results(self) -> dict:
        u = lambda t: [tuple(int(x) for x in row) for row in field_numpy(t.reshape(-1, 2))]
        return {"Z": self.Z.cpu().numpy(), "Y": self.Y.cpu().numpy(), "R": self.R.cpu().numpy(),
                "root": bytes(self.tree[-1].cpu().numpy()), "c0": u(self.c0)[0],
                "rounds": [u(self.rounds[i]) for i in range(self.n)], "r": u(self.r[:self.n]),
                "finals": tuple(u(self.finals)), "state": bytes(self.state.cpu().numpy().view(np.uint8)),
                "chal": u(self.chal[:self.n_t + self.n_o])}


def can_pipeline(cfg) -> bool:
    """Whether proofs of this workload can overlap (one sum-check that fits the
    workgroup inside the witness launch)."""
    return cfg.kind == "single" and (1 << cfg.matmuls[0].n) <= OVERLAP_ENTRIES


def can_overlap(cfg) -> bool:
    """Whether three proofs can be in flight (pipelined, and the packed witness applies)."""
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
    if pipelined:
        raise ValueError("pipelined proofs are implemented for single-matmul layers")
    if cfg.kind in ("rlc_out", "batched"):
        return MultiMatmulProver(cfg, inp, ch, dev)
    if cfg.kind == "moe":
        return MoEBlockProver(cfg, inp, ch, dev)
    raise ValueError(cfg.kind)
