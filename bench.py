"""Benchmark: proved tokens/s for the linear maps of one layer on one GPU.

A step is one whole layer proof (witness GEMMs with the rescale epilogue, eq
tables, row folds of X and W, the claims Z~(r_o || r_t), the sum-checks over
d_in, and any random linear combination) over one batch of synthetic tokens
whose inputs and challenges are resident in HBM before timing starts. The
default workload is the seven maps of a T=4096 transformer layer (Q, K, V, O,
gate, up, down; d=4096, GQA 32/8 heads, d_ff=14336, s=8) batched into one
sum-check, with three proofs in flight; ``--config N`` selects another workload
(1..5) and ``secondary`` reports the T=512 up-projection measured the same way.

Prints one JSON line. ``roofline`` describes the dominant kernel, timed with
HIP events on the stream the kernels run on; ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload (rank 0, N=1).
``request_vectors`` measures the batch fold of a weight matrix by 64 requests'
eq vectors (one pass over the weights) beside 64 one-pass folds, with its own
roofline and oracle time; ``commitment`` measures the commitment of Y and R
(limb packing, Reed-Solomon encoding of rows of 2^22 into 2^23 by NTT, a salted
BLAKE2b Merkle tree over the columns); ``lookup`` measures the lookup that
shows the remainders R are small (product tree, multiplicities, a degree-3
sum-check per tree level) and, under ``clamp``, the clamp's lookup of the
pairs (Q, Y); ``faithful`` (the up-projection) and ``faithful_main`` (the
default workload) the layer's proof with its rescale committed (Q, R, Y) and
every challenge over F_p[u]/(u^2 - 7) drawn from the transcript, claims opened
from the commitment.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12        # bytes/s, MI355X HBM3E
MFMA_I8_PEAK = 5.0e15    # ops/s, MI355X dense int8 matrix cores
METRIC = "matmul sum-check proved tokens/s per layer; fold GB/s & int8 MFMA % of peak"
WORKLOADS = {1: "single linear layer T=16 256x256 (uniform int8, s=7)",
             2: "Llama-3.1-8B up-projection T=512 4096->14336 (s=8)",
             3: "Llama-4-Maverick-width dense MLP gate/up/down T=1024 d=5120 d_ff=16384 (s=8), RLC of 3 claims",
             4: "MoE block 128 experts top-1 Zipf(1.1) routing of T=2048, 5120->8192->5120 int4 weights (s=8)",
             5: "dense layer linear maps T=4096 d=4096 GQA 32/8 heads d_ff=14336, 7 claims batched (s=8)"}


def kernel_work(cfg, name: str, prover) -> tuple:
    """(algorithmic bytes, algorithmic int8 ops) of one launch group."""
    if "+" in name:  # a launch that carries several steps
        parts = [kernel_work(cfg, k, prover) for k in name.split("+")]
        return sum(b for b, _ in parts), sum(o for _, o in parts)
    if cfg.kind == "moe":
        T = cfg.T
        d, dff = cfg.d_model, cfg.d_ff
        ne = len(prover.experts)
        wbytes = ne * 2 * d * dff
        if name == "witness":
            return wbytes + T * (d + dff) + 6 * T * (d + dff), 2 * T * d * dff * 2
        if name == "witness(Y,R)":  # Z stays in the accumulators
            return wbytes + T * (d + dff) + 2 * T * (d + dff), 2 * T * d * dff * 2
        if name == "claim(acc)":  # the tile's eq-table entries
            return 8 * (T + ne * (dff + d)), 0
        if name == "wfold(acc)":  # the weight folds from the witness's pass: outputs only (the weights are counted)
            return 8 * ne * ((1 << prover.n_up) + (1 << prover.n_dn)), 0
        if name == "xfold":
            return T * (d + dff) + 8 * ne * ((1 << prover.n_up) + (1 << prover.n_dn)), 0
        if name == "eq":
            return 8 * (sum(1 << k for k in prover.nt) + ne * ((1 << prover.n_up) + (1 << prover.n_dn))), 0
        if name == "group":
            return 2 * T * (d + dff), 0
        if name == "fold":
            return wbytes + T * (d + dff) + 8 * 2 * ne * ((1 << prover.n_up) + (1 << prover.n_dn)), 0
        if name == "claim":
            return 4 * T * (d + dff), 0
        if name == "sumcheck":
            return 16 * ne * ((1 << prover.n_up) + (1 << prover.n_dn)), 0
        return 0, 0
    mms = cfg.matmuls
    T = cfg.T
    if name == "witness":
        b = sum(m.d_in * m.d_out + T * m.d_in + 6 * T * m.d_out for m in mms)
        return b, sum(2 * T * m.d_in * m.d_out for m in mms)
    if name == "witness(Y,R)":  # Z stays in the accumulators
        b = sum(m.d_in * m.d_out + T * m.d_in + 2 * T * m.d_out for m in mms)
        return b, sum(2 * T * m.d_in * m.d_out for m in mms)
    if name == "claim(acc)":  # the claim from the accumulators reads only the eq tables
        return sum(8 * (T + m.d_out) for m in mms), 0
    if name == "fold":
        xs = {(m.x, m.d_in) for m in mms}
        b = sum(m.d_in * m.d_out for m in mms) + sum(T * di for _, di in xs)
        return b, 0
    if name == "fold(W/2)":  # the weights read once for two proofs' folds: half a read per step
        xs = {(m.x, m.d_in) for m in mms}
        b = sum(m.d_in * m.d_out for m in mms) // 2 + sum(T * di for _, di in xs)
        return b, 0
    if name == "claim":
        return sum(4 * T * m.d_out for m in mms), 0
    if name == "sumcheck":
        n = cfg.batched_n if cfg.kind == "batched" else None
        return sum(16 * (1 << (n if n else m.n)) for m in mms), 0
    if name == "eq":  # the tables written (the challenges read are negligible)
        return 8 * ((1 << cfg.n_t) + sum(1 << m.n_o for m in mms)), 0
    return 0, 0


TRAFFIC_FILES = {2: os.path.join(ROOT, "profiles", "layer_T512_step_traffic.txt"),
                 5: os.path.join(ROOT, "profiles", "layer_T4096_7maps_step_traffic.txt"),
                 3: os.path.join(ROOT, "profiles", "mlp_T1024_step_traffic.txt")}


def measured_traffic(cfg, kernel_phase: str):
    """HBM bytes per launch of the dominant launch, from the committed counter
    summary, or None when there is none for this workload and launch or its
    kernel sources changed since the counters were taken."""
    import hashlib
    path = TRAFFIC_FILES.get(cfg.cid)
    if path is None or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        kv[k.strip()] = v.strip()
    if int(kv.get("workload", -1)) != cfg.cid or kv.get("phase") != kernel_phase:
        return None
    h = hashlib.sha256()
    for src in kv["sources"].split():
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest() != kv["sha256"]:
        return None
    return int(round((float(kv["fetch_kib"]) * float(kv["fetch_scale"]) +
                      float(kv["write_kib"]) * float(kv["write_scale"])) * 1024))


def _host_cpu() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_ONE_CORE = """
import sys, time
sys.path.insert(0, %r)
import oracle, synth
cfg = synth.config(%d)
inp = synth.make_inputs(cfg)
ch = synth.draw_challenges(cfg, inp.get("route"))
oracle.lib()
t0 = time.perf_counter()
oracle.prove_config(cfg, inp, ch)
print(time.perf_counter() - t0)
"""


def cpu_baseline(cfg, inp, ch, one_core: bool = True) -> dict:
    """The oracle's whole layer proof of the workload on the host cores (all
    OpenMP threads, and once more on one core in a child process); for the
    large workloads a bounded sample (cpu_baseline_sampled)."""
    import subprocess
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    if cfg.cid not in (1, 2):
        return cpu_baseline_sampled(cfg, inp, ch)
    oracle.lib()
    t0 = time.perf_counter()
    oracle.prove_config(cfg, inp, ch)
    dt = time.perf_counter() - t0
    out = {"value": cfg.T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "the whole layer proof of this workload (all %d tokens), one pass, %.2f s" % (cfg.T, dt),
           "host_cpu": _host_cpu(), "nproc": os.cpu_count()}
    if one_core:
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, "-c", _ONE_CORE % (ROOT, cfg.cid)], env=env, capture_output=True,
                           text=True, timeout=600)
        if r.returncode == 0:
            d1 = float(r.stdout.strip().splitlines()[-1])
            out["value_1core"] = cfg.T / d1
            out["sample_1core"] = "the same proof with OMP_NUM_THREADS=1, %.2f s" % d1
    return out


def cpu_baseline_sampled(cfg, inp, ch, t_sample: int = 2048, max_experts: int = 6) -> dict:
    """The oracle on a bounded sample of a large workload, extrapolated to the
    whole proof: the work that grows with the tokens (every map's witness, the
    claim of each Z, the folds of the activations) is timed on the first
    t_sample tokens (the MoE block: on max_experts experts, the largest among
    them) and scaled; the folds of the weights and the sum-checks, which do not
    grow with the tokens, are timed in full (MoE: per expert, scaled by the
    experts present). Runs on all the host's OpenMP threads."""
    import numpy as np
    import oracle as O
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    O.lib()

    def clock(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    if cfg.kind == "moe":
        groups = O.group_tokens(inp["route"], cfg.n_experts)
        present = [e for e in range(cfg.n_experts) if len(groups[e])]
        by_size = sorted(present, key=lambda e: -len(groups[e]))
        pick = sorted(set(by_size[:max_experts // 2] + by_size[-(max_experts - max_experts // 2):]))
        tok_work = sum(len(groups[e]) for e in pick)
        t_tok = t_fix = 0.0
        for e in pick:
            toks = groups[e]
            for side, Xs, W in (("up", inp["X"], inp["W1_%d" % e]), ("down", inp["H"], inp["W2_%d" % e])):
                Xe = np.ascontiguousarray(Xs[toks])
                r_t = ch["r_t/%d" % e]
                r_o = ch["r_o_%s/%d" % (side, e)]
                rr = ch["rounds_%s/%d" % (side, e)]
                n = len(rr)
                (Z, _, _), dt = clock(lambda: O.witness(Xe, W, cfg.s))
                t_tok += dt
                _, dt = clock(lambda: O.mle_matrix(Z, r_t, r_o))
                t_tok += dt
                xf, dt = clock(lambda: O.fold_rows(Xe, O.eq_table(r_t), 1 << n))
                t_tok += dt
                wf, dt = clock(lambda: O.fold_rows(W, O.eq_table(r_o), 1 << n))
                t_fix += dt
                _, dt = clock(lambda: O.sumcheck([xf], [wf], rr))
                t_fix += dt
        total = t_tok * cfg.T / tok_work + t_fix * len(present) / len(pick)
        sample = ("%d of the %d experts present (the %d largest and the %d smallest, %d tokens): witness, claim and "
                  "activation folds %.2f s scaled by %d / %d tokens; weight folds and sum-checks %.2f s scaled by "
                  "%d / %d experts; whole block extrapolated to %.1f s" %
                  (len(pick), len(present), max_experts // 2, max_experts - max_experts // 2, tok_work, t_tok,
                   cfg.T, tok_work, t_fix, len(present), len(pick), total))
    else:
        Ts = min(t_sample, cfg.T)
        ns = max(0, (Ts - 1).bit_length())
        r_t = ch["r_t"][:ns]
        E_ts = O.eq_table(r_t)
        t_tok = t_fix = 0.0
        xfs, As, Bs, rho = {}, [], [], []
        for m in cfg.matmuls:
            n = cfg.batched_n if cfg.kind == "batched" else m.n
            Xs = np.ascontiguousarray(inp[m.x][:Ts])
            (Z, _, _), dt = clock(lambda: O.witness(Xs, inp[m.w], cfg.s))
            t_tok += dt
            _, dt = clock(lambda: O.mle_matrix(Z, r_t, ch["r_o/" + m.name]))
            t_tok += dt
            if (m.x, n) not in xfs:
                xfs[(m.x, n)], dt = clock(lambda: O.fold_rows(Xs, E_ts, 1 << n))
                t_tok += dt
            wf, dt = clock(lambda: O.fold_rows(inp[m.w], O.eq_table(ch["r_o/" + m.name]), 1 << n))
            t_fix += dt
            if cfg.kind == "batched":
                As.append(xfs[(m.x, n)])
                Bs.append(wf)
                rho.append(int(ch["rho/" + m.name][0]))
            else:
                _, dt = clock(lambda: O.sumcheck([xfs[(m.x, n)]], [wf], ch["rounds/" + m.name]))
                t_fix += dt
        if cfg.kind == "batched":
            _, dt = clock(lambda: O.sumcheck(As, Bs, ch["rounds"], rho=rho))
            t_fix += dt
        total = t_tok * cfg.T / Ts + t_fix
        sample = ("the first %d of %d tokens: every map's witness, its claim and the activation folds %.2f s, scaled "
                  "by %d / %d; the weight folds and the sum-check(s) in full, %.2f s; whole proof extrapolated to "
                  "%.1f s" % (Ts, cfg.T, t_tok, cfg.T, Ts, t_fix, total))
    return {"value": cfg.T / total, "unit": "tokens/s", "cores": threads, "kind": "oracle", "sample": sample,
            "host_cpu": _host_cpu(), "nproc": os.cpu_count()}


def request_vectors_leg(cfg, inp, dev, steps: int, per_graph: int, with_cpu: bool, R: int = 64) -> dict:
    """Request vectors of a batch: the first weight matrix of the workload
    folded by R requests' eq vectors (points drawn like the layer's r_o) in one
    fp_fold_matrix_multi call, against the same R folds done one matrix pass
    each (fp_fold_matrix_batched). Inputs and the prepared transpose are
    resident before timing; each is timed as per_graph calls in one HIP graph."""
    import numpy as np
    import torch

    import synth
    import zero_knowledge_proof_amd as fp
    if not cfg.matmuls:
        return None
    m = cfg.matmuls[0]
    rows, cols = m.d_out, m.d_in
    W = torch.from_numpy(np.ascontiguousarray(inp[m.w])).to(dev)
    n = synth.log2ceil(rows)
    pts = [synth.challenges(synth.data_seed(cfg.seed, 1 << 20 | j), n) for j in range(R)]
    Es = fp.eq_table_batched([fp.to_field_tensor(p) for p in pts])
    E = torch.stack([e[:rows] for e in Es]).contiguous()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    Mt, c = fp.fold_weights_prepare(W)
    t1.record(stream)
    out = torch.empty((R, cols), dtype=torch.int64, device=dev)
    outs1 = [torch.empty(cols, dtype=torch.int64, device=dev) for _ in range(R)]
    jobs = [(W, E[j], cols, outs1[j]) for j in range(R)]

    def timed(fn):
        fn()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, steps // per_graph)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * per_graph) * 1e-3

    t_multi = timed(lambda: fp.fold_matrix_multi(Mt, c, rows, E, cols, out=out))
    t_single = timed(lambda: fp.fold_matrix_batched(jobs))
    same = all(torch.equal(outs1[j], out[j]) for j in range(R))
    ops = 2 * 8 * R * rows * cols
    res = {
        "workload": "%s weights [%d x %d] (int8), %d requests' eq vectors over its %d rows" % (m.name, rows, cols, R,
                                                                                               rows),
        "R": R, "ms": round(t_multi * 1e3, 5), "requests_per_s": round(R / t_multi, 1),
        "one_pass_per_request_ms": round(t_single * 1e3, 5), "speedup": round(t_single / t_multi, 2),
        "outputs_equal_one_pass_per_request": bool(same),
        "prepare_ms_once_per_matrix": round(t0.elapsed_time(t1), 4),
        "roofline": {"bound": "mfma", "achieved": round(ops / t_multi / 1e12, 1), "peak": MFMA_I8_PEAK / 1e12,
                     "unit": "TFLOP/s", "frac": round(ops / t_multi / MFMA_I8_PEAK, 4),
                     "traffic": None, "algorithmic_ops": ops,
                     # the method's own bytes: the weights once, the R eq vectors, the R folded rows
                     "algorithmic_bytes": rows * cols + 8 * R * rows + 8 * R * cols,
                     "hbm_GBps": round((rows * cols + 8 * R * rows + 8 * R * cols) / t_multi / 1e9, 1),
                     "note": "the whole call (digits, limb GEMM, chunk sum) timed; int8 ops of the limb GEMM, whose "
                             "byte digits expand each eq weight into 8 rows; hbm_GBps: the method's own bytes (weights "
                             "once, eq vectors, folded rows) over the call's time"},
    }
    if with_cpu:
        import oracle
        k = 8
        Wn = np.ascontiguousarray(inp[m.w])
        Esn = [fp.field_numpy(E[j]) for j in range(k)]
        oracle.lib()
        c0 = time.perf_counter()
        oracle.request_vectors(Wn, Esn, cols)
        dt = time.perf_counter() - c0
        res["cpu_baseline"] = {"value": round(k / dt, 3), "unit": "requests/s",
                               "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)),
                               "kind": "oracle", "sample": "%d of the %d requests, %.2f s" % (k, R, dt)}
    return res


# gfx950 VALU instructions per BLAKE2b compression at the least: per G, six 64-bit adds (one
# v_lshl_add_u64 each), four 64-bit xors (two v_xor_b32), rotations by 24, 16, 63 (two v_alignbit_b32
# each; by 32 none); 12 rounds of 8 G, then 8 words of h ^= v ^ v' (32 v_xor_b32)
B2_OPS = 12 * 8 * (6 + 8 + 6) + 32
# VALU lane-instructions of one Goldilocks product (4 v_mad_u64_u32 partial products and the reduction with its
# carry and borrow corrections, as compiled for gfx950) and of one field addition or subtraction
GL_MUL_OPS, GL_ADD_OPS = 20, 5
VALU_PEAK = 256 * 4 * 16 * 2.4e9  # 32-bit lane operations/s: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz


def commitment_leg(cfg, inp, dev, steps: int, per_graph: int, with_cpu: bool, logn: int = 22) -> dict:
    """Commitment of the layer's Y and R as the pages commit a table: limbs
    packed three per element into rows of 2^22, each row Reed-Solomon encoded
    into 2^23 by NTT, a salted BLAKE2b-256 Merkle tree over the 2^23 columns.
    Y and R come from the GPU witness of this workload; the salts are seeded
    synthetic bytes. Each step (pack, encode, tree, and all three) is timed as
    per_graph calls in one HIP graph."""
    import numpy as np
    import torch

    import synth
    import zero_knowledge_proof_amd as fp
    if not cfg.matmuls:
        return None
    m = cfg.matmuls[0]
    X = torch.from_numpy(np.ascontiguousarray(inp[m.x])).to(dev)
    W = torch.from_numpy(np.ascontiguousarray(inp[m.w])).to(dev)
    _, Y, R = fp.witness_linear(X, W, cfg.s, with_z=False)
    Y, R = Y.contiguous(), R.contiguous()
    rows = fp.commit_rows(Y.numel(), R.numel(), logn)
    width = 2 << logn
    salts_np = synth.raw(synth.data_seed(cfg.seed, 1 << 21), width * fp.SALT_BYTES // 8).view(np.uint8)
    salts = torch.from_numpy(salts_np.reshape(width, fp.SALT_BYTES)).to(dev)
    msg = torch.empty((rows, 1 << logn), dtype=torch.int64, device=dev)
    code = torch.empty((rows, width), dtype=torch.int64, device=dev)
    tree = torch.empty((2 * width - 1, fp.DIGEST_BYTES), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def pack():
        fp.commit_pack(Y, R, logn, rows, out=msg)

    def encode():
        fp.rs_encode(msg, code=code)

    def merkle():
        fp.merkle_commit(code, salts, tree=tree)

    def chain():
        pack()
        encode()
        merkle()

    def timed(fn):
        fn()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, steps // per_graph)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * per_graph) * 1e-3

    t = {"pack": timed(pack), "encode": timed(encode), "merkle": timed(merkle), "commit": timed(chain)}
    N = width
    enc_bytes = rows * (N // 2 * 8 + N * 8 + 4 * N * 8)  # pass 1 reads half, writes all; passes 2, 3 read + write
    enc_valu = rows * (N // 2) * (logn + 1) * (GL_MUL_OPS + 2 * GL_ADD_OPS)
    leaf_blocks = -(-(fp.SALT_BYTES + 8 * rows) // 128)
    compressions = width * leaf_blocks + (width - 1)
    res = {
        "workload": "Y and R of %s (%d x %d int8 each): %d limbs in %d rows of 2^%d, codewords of 2^%d, "
                    "Merkle tree over %d columns" % (m.name, cfg.T, m.d_out, Y.numel() + R.numel(), rows, logn,
                                                    logn + 1, width),
        "ms": round(t["commit"] * 1e3, 4), "tokens_per_s": round(cfg.T / t["commit"], 1),
        "phases_ms": {k: round(v * 1e3, 4) for k, v in t.items() if k != "commit"},
        "compressions": compressions,
        "roofline": {"bound": "alu", "kernel": "merkle (leaf + tree launches)",
                     "achieved": round(compressions * B2_OPS / t["merkle"] / 1e12, 2),
                     "peak": VALU_PEAK / 1e12, "unit": "T VALU instr/s",
                     "frac": round(compressions * B2_OPS / t["merkle"] / VALU_PEAK, 4), "traffic": None,
                     "G_compressions_per_s": round(compressions / t["merkle"] / 1e9, 2)},
        "encode_roofline": {"bound": "alu", "kernel": "ntt_pass_kernel (3 passes per row)",
                            "achieved": round(enc_valu / t["encode"] / 1e12, 2), "peak": VALU_PEAK / 1e12,
                            "unit": "T VALU instr/s", "frac": round(enc_valu / t["encode"] / VALU_PEAK, 4),
                            "algorithmic_valu_instr": enc_valu, "algorithmic_bytes": enc_bytes,
                            "hbm_GBps": round(enc_bytes / t["encode"] / 1e9, 1),
                            "note": "a radix-2 NTT's work per row of N points: (N/2) log2 N butterflies of one "
                                    "product and two additions (the shift twiddles here are cheaper)"},
    }
    if with_cpu:
        import oracle
        Yn, Rn = Y.cpu().numpy(), R.cpu().numpy()
        oracle.lib()
        c0 = time.perf_counter()
        msg_o = oracle.pack_limbs(Yn, Rn, logn)
        code_o = oracle.rs_encode(msg_o)
        t_enc = time.perf_counter() - c0
        ns = 1 << 15  # leaves of a 2^15-column subtree
        c0 = time.perf_counter()
        oracle.merkle_tree(code_o[:, :ns], salts_np.reshape(width, fp.SALT_BYTES)[:ns])
        t_hash = time.perf_counter() - c0
        total = t_enc + t_hash * compressions / (2 * ns - 1)
        res["cpu_baseline"] = {"value": round(cfg.T / total, 2), "unit": "tokens/s",
                               "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)),
                               "kind": "oracle",
                               "sample": "packing and encoding in full (%.2f s); the hashes of a 2^15-column subtree "
                                         "(%.2f s) scaled to all %d compressions" % (t_enc, t_hash, compressions)}
        res["matches_oracle_code"] = bool(np.array_equal(code.cpu().numpy().view(np.uint64), code_o))
    return res


def lookup_bytes(L: int, n_keys: int, tail: int = 2048, kmax: int = 3) -> int:
    """Algorithmic HBM bytes of the remainder lookup: the tree (keys in, every
    level out once), then per level its eq table written once and, per
    sum-check launch of up to kmax rounds, the three tables read once and
    written folded by all of that launch's challenges, until they fit one
    workgroup (tail entries), whose launch reads them once more."""
    b = n_keys + 8 * ((2 << L) - 1)
    for m in range(L):
        size = 1 << m
        b += 8 * size                # eq table
        while size > tail:
            left = 0
            while (size >> left) > tail:
                left += 1
            b += 24 * size           # E and the level's 2 size entries (then E, A, B) read
            size >>= min(left, kmax)
            b += 24 * size           # folded E, A, B written
        b += 24 * size
    return b


def lookup_leg(cfg, inp, dev, steps: int, per_graph: int, with_cpu: bool) -> dict:
    """The lookup that shows the layer's remainders R are small: the product
    tree of gamma - r over the padded 2^L remainders, the multiplicities of the
    2^s table values, and the level-by-level proof of the tree (a degree-3
    sum-check per level). R comes from the GPU witness of this workload; gamma
    and the challenges are seeded streams. Timed as per_graph runs per graph."""
    import numpy as np
    import torch

    import synth
    import zero_knowledge_proof_amd as fp
    if not cfg.matmuls:
        return None
    m = cfg.matmuls[0]
    X = torch.from_numpy(np.ascontiguousarray(inp[m.x])).to(dev)
    W = torch.from_numpy(np.ascontiguousarray(inp[m.w])).to(dev)
    _, _, R = fp.witness_linear(X, W, cfg.s, with_z=False)
    keys = R.contiguous().reshape(-1)
    n = keys.numel()
    L = max(1, synth.log2ceil(n))
    nch = L * (L + 1) // 2
    gamma_h = synth.challenges(synth.data_seed(cfg.seed, 1 << 22), 1)
    chal_h = synth.challenges(synth.data_seed(cfg.seed, 1 << 22 | 1), nch)
    gamma, chal = fp.to_field_tensor(gamma_h), fp.to_field_tensor(chal_h)
    tree = torch.empty((2 << L) - 1, dtype=torch.int64, device=dev)
    counts = torch.empty((1 << cfg.s) + 1, dtype=torch.int32, device=dev)
    rounds = torch.empty((max(1, L * (L - 1) // 2), 4), dtype=torch.int64, device=dev)
    finals = torch.empty((L, 3), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    def build():
        fp.lookup_tree(keys, L, gamma, tree=tree)

    def count():
        fp.lookup_counts(keys, L, cfg.s, counts=counts)

    def prove():
        fp.lookup_prove(tree, L, chal, rounds=rounds, finals=finals)

    def chain():
        build()
        count()
        prove()

    def timed(fn):
        fn()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, steps // per_graph)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * per_graph) * 1e-3

    t = {"tree": timed(build), "counts": timed(count), "prove": timed(prove), "lookup": timed(chain)}
    nbytes = lookup_bytes(L, n)
    # arithmetic: the tree's 2^L - 1 products (and a subtraction per leaf); level l's sum-check has l rounds
    # over 2^(l-1-i) pairs of entries, each pair 11 products (g at 0..3 of eq * a * b, then three binds) and
    # 12 additions: sum_l (2^l - 1) pairs over l = 1 .. L-1
    pairs = sum((1 << lv) - 1 for lv in range(1, L))
    valu = ((1 << L) - 1) * GL_MUL_OPS + (1 << L) * GL_ADD_OPS + pairs * (11 * GL_MUL_OPS + 12 * GL_ADD_OPS)
    res = {
        "workload": "R of %s (%d x %d int8, s=%d): %d keys padded to 2^%d leaves, table of 2^%d values, "
                    "%d sum-check rounds over %d levels" % (m.name, cfg.T, m.d_out, cfg.s, n, L, cfg.s,
                                                           L * (L - 1) // 2, L),
        "ms": round(t["lookup"] * 1e3, 4), "tokens_per_s": round(cfg.T / t["lookup"], 1),
        "phases_ms": {k: round(v * 1e3, 4) for k, v in t.items() if k != "lookup"},
        "roofline": {"bound": "alu", "achieved": round(valu / t["lookup"] / 1e12, 2), "peak": VALU_PEAK / 1e12,
                     "unit": "T VALU instr/s", "frac": round(valu / t["lookup"] / VALU_PEAK, 4), "traffic": None,
                     "algorithmic_valu_instr": valu, "algorithmic_bytes": nbytes,
                     "hbm_GBps": round(nbytes / t["lookup"] / 1e9, 1),
                     "note": "the whole lookup against the vector ALU (its products are 64-bit Goldilocks "
                             "arithmetic); the challenges are inputs, so its %d levels are proved side by side: "
                             "launches of up to 3 rounds each while a level's tables exceed 2048 entries, then one "
                             "workgroup per level for the last rounds (latency-bound)" % L},
    }
    if with_cpu:
        import oracle
        kn = keys.cpu().numpy()
        oracle.lib()
        c0 = time.perf_counter()
        lev = oracle.product_tree(kn, L, int(gamma_h[0]))
        oracle.lookup_counts(kn, L, cfg.s)
        oracle.grand_product_prove(lev, chal_h)
        dt = time.perf_counter() - c0
        res["cpu_baseline"] = {"value": round(cfg.T / dt, 2), "unit": "tokens/s",
                               "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)),
                               "kind": "oracle", "sample": "the whole lookup of this layer's remainders, %.2f s" % dt}
    res["clamp"] = clamp_leg(cfg, X, W, dev, timed, with_cpu)
    return res


def clamp_leg(cfg, X, W, dev, timed, with_cpu: bool) -> dict:
    """The clamp's lookup over the map's committed Q and Y (zero-padded [2^n_t, 2^n_o] field tables written by
    fp_commit_tables): the tree of gamma - ((Q + 2^15) + 2^16 (Y + 128)), the multiplicities of the 16-bit
    table of (q, clamp(q)), and the level-by-level proof of the tree."""
    import torch

    import synth
    import zero_knowledge_proof_amd as fp
    m = cfg.matmuls[0]
    Z, _, _ = fp.witness_linear(X, W, cfg.s)
    n_t, n_o = synth.log2ceil(cfg.T), synth.log2ceil(m.d_out)
    L = n_t + n_o
    msg = torch.empty((3, 1 << L), dtype=torch.int64, device=dev)
    fp.commit_tables([(Z, n_o, 0, 1, 2)], n_t, cfg.s, msg)
    Q, Y = msg[0], msg[2]
    gamma_h = synth.challenges(synth.data_seed(cfg.seed, 1 << 22 | 2), 1)
    chal_h = synth.challenges(synth.data_seed(cfg.seed, 1 << 22 | 3), L * (L + 1) // 2)
    gamma, chal = fp.to_field_tensor(gamma_h), fp.to_field_tensor(chal_h)
    tree = torch.empty((2 << L) - 1, dtype=torch.int64, device=dev)
    counts = torch.empty((1 << fp.CLAMP_BITS) + 1, dtype=torch.int32, device=dev)
    rounds = torch.empty((max(1, L * (L - 1) // 2), 4), dtype=torch.int64, device=dev)
    finals = torch.empty((L, 3), dtype=torch.int64, device=dev)

    def build():
        fp.lookup_tree_pairs(Q, Y, L, gamma, tree=tree)

    def count():
        fp.lookup_counts_field(Q, counts=counts)

    def prove():
        fp.lookup_prove(tree, L, chal, rounds=rounds, finals=finals)

    def chain():
        build()
        count()
        prove()

    t = {"tree": timed(build), "counts": timed(count), "prove": timed(prove), "lookup": timed(chain)}
    res = {"workload": "(Q, Y) of %s (%d x %d, padded to 2^%d entries): keys (Q + 2^15) + 2^16 (Y + 128) against "
                       "the 2^16 rows (q, clamp(q))" % (m.name, cfg.T, m.d_out, L),
           "ms": round(t["lookup"] * 1e3, 4), "tokens_per_s": round(cfg.T / t["lookup"], 1),
           "phases_ms": {k: round(v * 1e3, 4) for k, v in t.items() if k != "lookup"},
           "outside_16_bits": int(counts[-1].item())}
    if with_cpu:
        import oracle
        Qh, Yh = Q.cpu().numpy().view("uint64"), Y.cpu().numpy().view("uint64")
        c0 = time.perf_counter()
        keys = oracle.clamp_keys(Qh, Yh)
        lev = oracle.product_tree_field(keys, L, int(gamma_h[0]))
        cnt, _ = oracle.clamp_counts(Qh)
        oracle.clamp_table_product(cnt, int(gamma_h[0]))
        oracle.grand_product_prove(lev, chal_h)
        dt = time.perf_counter() - c0
        res["cpu_baseline"] = {"value": round(cfg.T / dt, 2), "unit": "tokens/s",
                               "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)),
                               "kind": "oracle", "sample": "the whole clamp lookup of this map, %.2f s" % dt}
    return res


def faithful_leg(cfg, inp, dev, steps: int, per_graph: int, with_cpu: bool) -> dict:
    """The layer's proof with its rescale committed and every challenge from the transcript: the witness, the
    commitment of each map's Q (before the clamp), R and Y, a BLAKE2b Fiat-Shamir transcript over its root, eq
    tables and folds over F_p[u]/(u^2 - 7), the folded rows that open the claims 2^s Q~ + R~, the extension
    sum-checks hashing each round on the device, and 64 opened columns. Timed as per_graph whole proofs per HIP
    graph, and each phase alone."""
    import numpy as np
    import torch

    import synth
    from zero_knowledge_proof_amd.prover import LAYER_LOG_ROW, FaithfulProver, log2ceil
    if cfg.kind not in ("single", "rlc_out", "batched"):
        return None
    n_t = log2ceil(cfg.T)
    L = min(LAYER_LOG_ROW, min(n_t + log2ceil(m.d_out) for m in cfg.matmuls))
    width = 2 << L
    salts = synth.raw(synth.data_seed(cfg.seed, 1 << 23), width * 2).view(np.uint8).reshape(width, 16)
    pr = FaithfulProver(cfg, inp, salts, dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, steps // per_graph)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * per_graph) * 1e-3

    t_all = timed(pr.run)
    phases = {name: round(timed(fn) * 1e3, 4) for name, fn in pr.phases()}
    maps = ", ".join("%s %d -> %d" % (m.name, m.d_in, m.d_out) for m in cfg.matmuls)
    res = {"workload": "%s (T=%d, s=%d) with each map's Q, R and Y committed (%d rows of 2^%d) and every challenge "
                       "from the transcript, in F_p[u]/(u^2-7); %s" % (
                           maps, cfg.T, cfg.s, pr.rows, L, "one batched sum-check" if pr.batched else
                           "one sum-check per map"),
           "ms": round(t_all * 1e3, 4), "tokens_per_s": round(cfg.T / t_all, 1), "phases_ms": phases}
    del pr
    if with_cpu:
        import oracle
        maps_in = [(inp[m.x], inp[m.w]) for m in cfg.matmuls]
        c0 = time.perf_counter()
        oracle.prove_layer_committed(maps_in, cfg.s, cfg.kind == "batched", salts)
        dt = time.perf_counter() - c0
        res["cpu_baseline"] = {"value": round(cfg.T / dt, 2), "unit": "tokens/s",
                               "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)),
                               "kind": "oracle", "sample": "the whole proof, %.2f s" % dt}
    return res


def layer_bench(cid: int, args, dev, with_cpu: bool, legs: bool):
    """Times K steps of a stream of proofs of workload `cid` (three in flight where it allows) and returns the
    JSON dict of the measurement (with the inputs, for the legs)."""
    import torch

    import synth
    import zero_knowledge_proof_amd as fp
    from zero_knowledge_proof_amd.prover import can_overlap, can_pipeline, make_prover

    cfg = synth.config(cid)
    inp = synth.make_inputs(cfg)
    ch = synth.draw_challenges(cfg, inp.get("route"))
    if cfg.kind in ("rlc_out", "batched"):  # multi-map layers: one proof in flight, or three
        pipelined = False
        overlapped = (not args.no_pipeline) and (not args.no_overlap) and can_overlap(cfg)
    else:
        pipelined = (not args.no_pipeline) and can_pipeline(cfg)
        overlapped = pipelined and (not args.no_overlap) and can_overlap(cfg)
    prover = make_prover(cfg, inp, ch, dev, pipelined=pipelined, overlapped=overlapped)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        prover.run()
    torch.cuda.synchronize()

    # several steps per HIP graph spread the graph-launch cost (K must be a multiple; with three
    # proofs in flight a multiple of three steps per graph; steps beyond whole graphs run eagerly
    # after the replays, inside the timed region, and so does the drain of the last proofs)
    quantum = getattr(prover, "GRAPH_QUANTUM", 1)
    per_graph = next((d for d in (30, 12, 10, 6, 5, 4, 3, 2, 1) if d % quantum == 0 and args.steps % d == 0), quantum)
    per_graph = min(per_graph, max(quantum, args.steps - args.steps % quantum))
    n_graphs = args.steps // per_graph
    prover.capture(per_graph)
    for _ in range(max(1, args.warmup // per_graph)):
        prover.replay()
    # the drain path's one-time set-up (its workspace) outside the timed region
    prover.drain()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(n_graphs + 1)]
    start.record(stream)
    marks[0].record(stream)
    for i in range(n_graphs):
        prover.replay()
        marks[i + 1].record(stream)
    for _ in range(args.steps - n_graphs * per_graph):
        prover.run()
    prover.drain()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) / per_graph for i in range(len(marks) - 1))
    value = cfg.T / (ms * 1e-3)

    # per-phase launch durations: each phase captured alone, per_graph times in one graph (so the
    # graph-launch cost is spread as in the step graph), K launches back to back between two events
    # on the stream the kernels run on
    phase_ms = {}
    for name, fn in prover.phases():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(max(1, n_graphs)):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        phase_ms[name] = e0.elapsed_time(e1) / (max(1, n_graphs) * per_graph)
    # one-time weight preparation (outside the timed step): the packed layout the witness reads
    packed = None
    if getattr(prover, "Wp", None) is not None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fp.pack_weights(prover.W, out=prover.Wp)
        e0.record(stream)
        fp.pack_weights(prover.W, out=prover.Wp)
        e1.record(stream)
        torch.cuda.synchronize()
        packed = {"ms": round(e0.elapsed_time(e1), 4), "bytes": prover.Wp.data.numel(),
                  "note": "the layer's weights packed once for the matrix cores (fp_witness_pack_weights); "
                          "a fixed layer is packed when it is loaded, so this is not part of a step"}
    dom = max(phase_ms, key=lambda k: phase_ms[k])
    b, ops = kernel_work(cfg, dom, prover)
    t = phase_ms[dom] * 1e-3
    t_hbm, t_mfma = b / HBM_PEAK, ops / MFMA_I8_PEAK
    if ops and t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": ops / t / 1e12, "peak": MFMA_I8_PEAK / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": b / t / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(cfg, dom)  # HBM bytes per launch (counters), None if stale
    roof["algorithmic_bytes"] = b
    roof["algorithmic_int8_ops"] = ops
    roof["kernel"] = dom
    roof["launch_ms"] = round(phase_ms[dom], 5)
    extras = {}
    for k, v in phase_ms.items():
        bb, oo = kernel_work(cfg, k, prover)
        extras[k] = {"ms": round(v, 5), "GB/s": round(bb / (v * 1e-3) / 1e9, 1) if bb else None,
                     "TOPS": round(oo / (v * 1e-3) / 1e12, 1) if oo else None}
    wb, wops = kernel_work(cfg, "witness", prover)
    wkey = next(k for k in phase_ms if k.startswith("witness"))
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "ms_per_step_replays": {"median": round(per_step[len(per_step) // 2], 5), "min": round(per_step[0], 5),
                                "max": round(per_step[-1], 5), "replays": len(per_step)}, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8->int32 witness; u64 Goldilocks field",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[cfg.cid], "T": cfg.T, "seed": cfg.seed, "s": cfg.s,
                   "matmuls": [[m.name, m.d_in, m.d_out] for m in cfg.matmuls] if cfg.matmuls else None,
                   "pipelined": pipelined or overlapped, "proofs_in_flight": 3 if overlapped else (2 if pipelined else 1),
                   "steps_per_graph": per_graph},
        "roofline": roof,
        "fold_claim_GBps": extras.get("fold+claim", {}).get("GB/s"),
        "witness_int8_TOPS": extras.get(wkey, {}).get("TOPS"),
        "witness_mfma_frac": round(wops / (phase_ms[wkey] * 1e-3) / MFMA_I8_PEAK, 4),
        "phases": extras,
        "weights_packed": packed,
        "wall_s": round(wall, 3),
    }
    del prover
    torch.cuda.empty_cache()
    out["cpu_baseline"] = cpu_baseline(cfg, inp, ch) if with_cpu else None
    return out, (cfg, inp)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=90)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--config", type=int, default=5,
                    help="the workload timed (default 5: the seven maps of a T=4096 transformer layer, the largest "
                         "that fits one GPU)")
    ap.add_argument("--secondary-config", type=int, default=2,
                    help="a second workload timed the same way and reported under 'secondary' (0: none)")
    ap.add_argument("--legs-config", type=int, default=2,
                    help="the workload whose first matrix the faithful, lookup, commitment and request-vector legs "
                         "use")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="prove steps one after another instead of overlapping consecutive proofs")
    ap.add_argument("--no-overlap", action="store_true",
                    help="single layers: two proofs in flight instead of three; multi-map layers: one")
    ap.add_argument("--no-faithful", action="store_true",
                    help="skip the soundness-faithful proof (commitment, Fiat-Shamir, extension-field challenges)")
    ap.add_argument("--no-lookup", action="store_true",
                    help="skip the remainder lookup measurement (product tree, multiplicities, proof of the tree)")
    ap.add_argument("--no-commitment", action="store_true",
                    help="skip the commitment measurement (Y and R packed, Reed-Solomon encoded, Merkle hashed)")
    ap.add_argument("--no-request-vectors", action="store_true",
                    help="skip the batch request-vector measurement (64 eq vectors folded against the first weight "
                         "matrix in one pass)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one device-to-device copy of MIB MiB (a reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this prover runs on one GPU; --gpus %d is not supported (each box has one GPU)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import zero_knowledge_proof_amd as fp

    fp.require_gpu()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    out, _ = layer_bench(args.config, args, dev, not args.no_cpu_baseline, True)
    if args.secondary_config and args.secondary_config != args.config:
        sec, _ = layer_bench(args.secondary_config, args, dev, False, False)
        out["secondary"] = {k: sec[k] for k in ("value", "unit", "ms_per_step", "ms_per_step_replays", "config",
                                                  "roofline", "witness_mfma_frac", "phases")}
    legs = synth.config(args.legs_config)
    need_legs = not (args.no_faithful and args.no_lookup and args.no_commitment and args.no_request_vectors)
    linp = synth.make_inputs(legs) if need_legs else None
    quantum_graph = 10
    with_cpu = not args.no_cpu_baseline
    if not args.no_faithful:
        out["faithful"] = faithful_leg(legs, linp, dev, args.steps, quantum_graph, with_cpu)
        if args.config != args.legs_config:
            main_cfg = synth.config(args.config)
            out["faithful_main"] = faithful_leg(main_cfg, synth.make_inputs(main_cfg), dev, max(args.steps // 3, 2),
                                                2, False)
    if not args.no_lookup:
        out["lookup"] = lookup_leg(legs, linp, dev, args.steps, quantum_graph, with_cpu)
    if not args.no_commitment:
        out["commitment"] = commitment_leg(legs, linp, dev, args.steps, quantum_graph, with_cpu)
    if not args.no_request_vectors:
        out["request_vectors"] = request_vectors_leg(legs, linp, dev, args.steps, quantum_graph, with_cpu)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
