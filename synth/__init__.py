"""Seeded synthetic inputs and challenge streams for the matmul sum-check prover.

This package only draws random numbers (SplitMix64, see ``synth.c``); it holds
none of the prover's arithmetic. The CPU oracle and the GPU path both read the
arrays it returns, so inputs are never a parity surface.

Workloads follow the five layer shapes the prover is measured on:
  1  one 256x256 linear layer, T=16 (uniform int8, s=7)
  2  Llama-3.1-8B up-projection, T=512, 4096 -> 14336 (s=8)
  3  Llama-4-Maverick-width dense MLP, T=1024, 5120 <-> 16384 (gate/up/down)
  4  MoE block, 128 experts, top-1 Zipf(1.1) routing of 2048 tokens,
     5120 -> 8192 -> 5120, int4 weights in int8 lanes
  5  a dense Llama-3.1-8B-shaped layer's seven linear maps at T=4096
Tensor j of a workload with seed S is drawn from SplitMix64(S*2^32 + j + 1);
challenges are drawn from SplitMix64(S) reduced mod p, in the order each
workload's ``challenge_plan`` lists.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

P = 0xFFFFFFFF00000001
_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.synth_raw.argtypes = [u64, u64, i64, vp]
        L.synth_challenges.argtypes = [u64, u64, i64, vp]
        for nm in ("synth_uniform127", "synth_int4", "synth_gauss32", "synth_laplace16"):
            getattr(L, nm).argtypes = [u64, i64, vp]
        L.synth_zipf.argtypes = [u64, i64, i32, ctypes.c_double, vp]
        for nm in ("synth_raw", "synth_challenges", "synth_uniform127", "synth_int4",
                   "synth_gauss32", "synth_laplace16", "synth_zipf"):
            getattr(L, nm).restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def raw(seed: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_raw(seed & (2**64 - 1), start, n, _ptr(out))
    return out


def challenges(seed: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_challenges(seed & (2**64 - 1), start, n, _ptr(out))
    return out


_DISTS = {"uniform127": "synth_uniform127", "int4": "synth_int4",
          "gauss32": "synth_gauss32", "laplace16": "synth_laplace16"}


def matrix(seed: int, shape, dist: str, out: np.ndarray | None = None) -> np.ndarray:
    """An int8 matrix of ``shape`` filled from stream ``seed`` with ``dist``."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, dtype=np.int8)
    assert out.dtype == np.int8 and out.size == n
    getattr(lib(), _DISTS[dist])(seed & (2**64 - 1), n, _ptr(out))
    return out


def zipf(seed: int, n: int, n_items: int, a: float) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_zipf(seed & (2**64 - 1), n, n_items, a, _ptr(out))
    return out


def data_seed(cfg_seed: int, j: int) -> int:
    return (cfg_seed << 32) + j + 1


def log2ceil(v: int) -> int:
    return 0 if v <= 1 else (int(v) - 1).bit_length()


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------

@dataclass
class Matmul:
    name: str
    x: str          # activation tensor [T, d_in]
    w: str          # weight tensor [d_out, d_in]
    d_in: int
    d_out: int

    @property
    def n(self) -> int:       # sum-check rounds (over the padded d_in)
        return log2ceil(self.d_in)

    @property
    def n_o(self) -> int:
        return log2ceil(self.d_out)


@dataclass
class Config:
    cid: int
    seed: int
    s: int
    kind: str                     # "single" | "rlc_out" | "moe" | "batched"
    T: int
    tensors: list                 # (name, shape, dist) in data-stream order
    matmuls: list = field(default_factory=list)
    n_experts: int = 0
    zipf_a: float = 0.0
    d_model: int = 0
    d_ff: int = 0
    batched_n: int = 0            # rounds of the batched instance

    @property
    def n_t(self) -> int:
        return log2ceil(self.T)

    def tensor_index(self, name: str) -> int:
        for j, t in enumerate(self.tensors):
            if t[0] == name:
                return j
        raise KeyError(name)


def _cfg1(T=16, d_in=256, d_out=256, seed=1, s=7):
    return Config(1, seed, s, "single", T,
                  [("W", (d_out, d_in), "uniform127"), ("X", (T, d_in), "uniform127")],
                  [Matmul("main", "X", "W", d_in, d_out)])


def _cfg2(T=512, d_in=4096, d_out=14336, seed=2, s=8):
    return Config(2, seed, s, "single", T,
                  [("W", (d_out, d_in), "gauss32"), ("X", (T, d_in), "laplace16")],
                  [Matmul("up", "X", "W", d_in, d_out)])


def _cfg3(T=1024, d=5120, d_ff=16384, seed=3, s=8):
    return Config(3, seed, s, "rlc_out", T,
                  [("W_gate", (d_ff, d), "gauss32"), ("W_up", (d_ff, d), "gauss32"),
                   ("W_down", (d, d_ff), "gauss32"), ("X_mlp", (T, d), "laplace16"),
                   ("H", (T, d_ff), "laplace16")],
                  [Matmul("gate", "X_mlp", "W_gate", d, d_ff), Matmul("up", "X_mlp", "W_up", d, d_ff),
                   Matmul("down", "H", "W_down", d_ff, d)])


def _cfg4(T=2048, d=5120, d_ff=8192, n_experts=128, seed=4, s=8, a=1.1):
    t = [("route", (T,), "zipf")]
    t += [("W1_%d" % e, (d_ff, d), "int4") for e in range(n_experts)]
    t += [("W2_%d" % e, (d, d_ff), "int4") for e in range(n_experts)]
    t += [("X", (T, d), "laplace16"), ("H", (T, d_ff), "laplace16")]
    return Config(4, seed, s, "moe", T, t, [], n_experts=n_experts, zipf_a=a, d_model=d, d_ff=d_ff)


def _cfg5(T=4096, d=4096, d_kv=1024, d_ff=14336, seed=5, s=8):
    W = [("W_q", (d, d)), ("W_k", (d_kv, d)), ("W_v", (d_kv, d)), ("W_o", (d, d)),
         ("W_gate", (d_ff, d)), ("W_up", (d_ff, d)), ("W_down", (d, d_ff))]
    t = [(nm, sh, "gauss32") for nm, sh in W]
    t += [("X_attn", (T, d), "laplace16"), ("A_out", (T, d), "laplace16"),
          ("X_mlp", (T, d), "laplace16"), ("H", (T, d_ff), "laplace16")]
    mm = [Matmul("q", "X_attn", "W_q", d, d), Matmul("k", "X_attn", "W_k", d, d_kv),
          Matmul("v", "X_attn", "W_v", d, d_kv), Matmul("o", "A_out", "W_o", d, d),
          Matmul("gate", "X_mlp", "W_gate", d, d_ff), Matmul("up", "X_mlp", "W_up", d, d_ff),
          Matmul("down", "H", "W_down", d_ff, d)]
    return Config(5, seed, s, "batched", T, t, mm,
                  batched_n=max(m.n for m in mm))


def config(cid: int, **overrides) -> Config:
    """Workload ``cid`` (1..5) at full size, or with shapes overridden
    (``T``, ``d_in``/``d_out``, ``d``/``d_ff``/``d_kv``, ``n_experts``...) for
    reduced parity cases. The distribution and stream rules stay the same."""
    return {1: _cfg1, 2: _cfg2, 3: _cfg3, 4: _cfg4, 5: _cfg5}[cid](**overrides)


def make_inputs(cfg: Config, only=None) -> dict:
    """Generate every tensor of ``cfg`` (or those named in ``only``)."""
    out = {}
    for j, (name, shape, dist) in enumerate(cfg.tensors):
        if only is not None and name not in only:
            continue
        sd = data_seed(cfg.seed, j)
        if dist == "zipf":
            out[name] = zipf(sd, shape[0], cfg.n_experts, cfg.zipf_a)
        else:
            out[name] = matrix(sd, shape, dist)
    return out


def expert_counts(cfg: Config, route: np.ndarray) -> np.ndarray:
    """Tokens routed to each expert (it decides how many challenges to draw)."""
    return np.bincount(route, minlength=cfg.n_experts).astype(np.int64)


def challenge_plan(cfg: Config, route: np.ndarray | None = None) -> list:
    """The ordered (key, length) list in which the challenge stream is consumed."""
    plan = []
    if cfg.kind == "single":
        m = cfg.matmuls[0]
        plan = [("r_t", cfg.n_t), ("r_o", m.n_o), ("rounds", m.n)]
    elif cfg.kind == "rlc_out":
        plan = [("r_t", cfg.n_t)]
        plan += [("r_o/" + m.name, m.n_o) for m in cfg.matmuls]
        plan += [("rounds/" + m.name, m.n) for m in cfg.matmuls]
        plan += [("rho/" + m.name, 1) for m in cfg.matmuls]
    elif cfg.kind == "moe":
        cnt = expert_counts(cfg, route)
        n_up_o, n_dn_o = log2ceil(cfg.d_ff), log2ceil(cfg.d_model)
        n_up, n_dn = log2ceil(cfg.d_model), log2ceil(cfg.d_ff)
        for e in range(cfg.n_experts):
            if cnt[e] == 0:
                continue
            plan += [("r_t/%d" % e, log2ceil(int(cnt[e]))), ("r_o_up/%d" % e, n_up_o),
                     ("r_o_down/%d" % e, n_dn_o), ("rounds_up/%d" % e, n_up),
                     ("rounds_down/%d" % e, n_dn)]
    elif cfg.kind == "batched":
        plan = [("r_t", cfg.n_t)]
        plan += [("r_o/" + m.name, m.n_o) for m in cfg.matmuls]
        plan += [("rho/" + m.name, 1) for m in cfg.matmuls]
        plan += [("rounds", cfg.batched_n)]
    else:
        raise ValueError(cfg.kind)
    return plan


def draw_challenges(cfg: Config, route: np.ndarray | None = None) -> dict:
    plan = challenge_plan(cfg, route)
    total = sum(n for _, n in plan)
    stream = challenges(cfg.seed, total)
    out, pos = {}, 0
    for key, n in plan:
        out[key] = stream[pos:pos + n].copy()
        pos += n
    return out
