"""Benchmark of the LiftQuant layer on one MI355X.

A step is one pass of the layer's hot path over one batch: for the 70B-class
LQ-19/8 MLP pair at batch 1 (up 28672 x 8192, then down 8192 x 28672) each
projection runs the activation lift (T^-1 blocks, then M^T per group) and the
packed-sign GEMV with its diag(s) epilogue.  Inputs are resident in HBM and
rotate over enough copies (> 2x the 256 MB Infinity Cache) that every step
reads its weights from HBM.

Printed: one JSON line with the whole-step algorithmic GB/s (`value`), the
dominant kernel's roofline (the one-token GEMV: algorithmic bytes per call /
the call's average duration from HIP events on its stream; the call is the
weight-streaming kernel plus the small kernel that adds the per-slice partial
sums, so the figure is conservative for the streaming kernel alone), the
batch-512 MFMA GEMM in TFLOP/s, per-workload GEMV figures, and the float64
oracle timed on the host cores over a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}   # dense
PEAK_FP32_FLOPS = 157.3e12     # float32 matrix (and vector) peak, FLOP/s
MALL_BYTES = 256 << 20
METRIC = ("LQ GEMV achieved HBM GB/s (% of peak) at batch 1; "
          "MFMA TFLOP/s at batch 512")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--gemm-dtype", default="f16", choices=["f16", "bf16"])
    p.add_argument("--no-cases", action="store_true", help="skip the per-workload sweep")
    p.add_argument("--tokens", type=int, default=0,
                   help="cases: only the workload cases with this many tokens")
    p.add_argument("--layer-path", default="split", choices=["fused", "split"],
                   help="one-token step: the lift inside the GEMV (lq_layer_b1) or the lift "
                        "and the GEMV as two calls")
    p.add_argument("--only", default="all",
                   choices=["all", "layer", "gemm", "cases", "kron", "encode", "learn"],
                   help="layer: only the timed 70B steps; gemm: only the batch-512 GEMM; "
                        "cases: only the per-workload GEMV and lift sweep; kron: only the "
                        "Kronecker-whitened lift")
    return p.parse_args()


# ----------------------------------------------------------------- byte counts
def gemv_bytes(m, K, B):
    """Algorithmic bytes of one GEMV launch: weights, scales, lifted activations, output."""
    return m * K // 8 + 4 * m + 4 * K * B + 4 * m * B


def lift_bytes(n, d, D, B, act_bytes=2, out_bytes=4):
    K = n // d * D
    return act_bytes * n * B + 2 * n * 128 + 4 * d * D + out_bytes * K * B


def layer_bytes(m, n, d, D, B):
    """Whole layer: a, T^-1 (16-bit), M, W_q, s, o; the a_hat round trip excluded."""
    K = n // d * D
    return 2 * n * B + 2 * n * 128 + 4 * d * D + m * K // 8 + 4 * m + 4 * m * B


def src_sha(names):
    """First 16 hex digits of sha256 over the named csrc files, in order."""
    h = hashlib.sha256()
    for name in ([names] if isinstance(names, str) else names):
        h.update(open(os.path.join(ROOT, "bit_lifted_gemv_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


GEMV_SRC = ["f4_parts.h", "k_gemv_f4r.hip", "k_gemv_f4.hip"]


def load_traffic(kernel_src, key):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source (a file or a list of files; else None)."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data.get(key)
        if ent and ent.get("source_sha") == src_sha(kernel_src):
            return ent.get("hbm_bytes_per_launch")
    except (ValueError, OSError):
        return None
    return None


# ----------------------------------------------------------------- GPU side
class Rotation:
    """R device copies of a layer so that R * footprint > 2 x MALL."""

    def __init__(self, L, torch, lq, dev, min_bytes=2 * MALL_BYTES):
        base = lq.DeviceLayer.from_synth(L, device=dev)
        foot = base.w.numel() * 4 + base.t_inv.numel() * 2 + base.s.numel() * 4
        self.R = max(2, int(np.ceil(min_bytes / foot)))
        self.copies = [base]
        for _ in range(self.R - 1):
            c = lq.DeviceLayer.__new__(lq.DeviceLayer)
            c.__dict__.update(base.__dict__)
            c.w = base.w.clone()
            c.t_inv = base.t_inv.clone()
            c.s = base.s.clone()
            c.M = base.M.clone()
            self.copies.append(c)
        self.a = lq.to_torch_16(L.a, L.dtype).to(dev)
        self.L = L

    def __getitem__(self, i):
        return self.copies[i % self.R]


def run_gpu(args):
    import torch

    from bit_lifted_gemv_amd import lq, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lq.load_library()
    if args.only == "gemm":
        return dict(gemm=run_gemm(args, torch, lq, synth, dev))
    if args.only == "cases":
        return dict(cases=run_cases(torch, lq, synth, dev, args.tokens))
    if args.only == "kron":
        return dict(kron=run_kron(torch, lq, synth, dev))
    if args.only == "encode":
        return dict(encode=run_encode(torch, lq, synth, dev))
    if args.only == "learn":
        return dict(learn=run_learn(torch, lq, synth, dev))
    cfg = synth.CONFIGS[3]                     # LQ-19/8 70B-class MLP
    layers = [synth.make_case(cfg, si, 1) for si in range(len(cfg.shapes))]
    rots = [Rotation(L, torch, lq, dev) for L in layers]
    st = torch.cuda.current_stream()
    # lifted activations and outputs, allocated once
    al = [torch.empty((1, L.K), dtype=torch.float32, device=dev) for L in layers]
    outs = [torch.empty((1, L.m), dtype=torch.float32, device=dev) for L in layers]

    def step_fused(i):
        for j, (rot, L) in enumerate(zip(rots, layers)):
            c = rot[i]
            lq.layer_b1(rot.a, c.t_inv, c.M, L.d, L.D, c.w, c.s, out=outs[j])

    def step_split(i):
        for j, (rot, L) in enumerate(zip(rots, layers)):
            c = rot[i]
            lq.lift(rot.a, c.t_inv, c.M, L.d, L.D, out=al[j])
            lq.gemv(c.w, c.s, al[j], L.K, out=outs[j])

    R = rots[0].R

    def time_step(step, steps):
        """Warm up, capture one HIP graph per weight copy (each one whole
        step, so that the timed loop measures the GPU, not the host's launch
        rate), check every replay bit for bit against the eager step on the
        same copy, then time `steps` replays between synchronisations."""
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        graphs = capture_graphs(torch, [lambda k=k: step(k) for k in range(R)])
        for k in range(R):
            step(k)
            torch.cuda.synchronize()
            want = [o.clone() for o in outs]
            for o in outs:
                o.fill_(float("nan"))
            graphs[k].replay()
            torch.cuda.synchronize()
            for o, w in zip(outs, want):
                if not torch.equal(o, w):
                    raise RuntimeError(f"graph replay {k} differs from the eager step")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[(args.warmup + i) % R].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / steps

    fused = args.layer_path == "fused"
    ms_step = time_step(step_fused if fused else step_split, args.steps)
    ms_other = time_step(step_split if fused else step_fused, max(3, min(args.steps, 20)))
    step_bytes = sum(layer_bytes(L.m, L.n, L.d, L.D, 1) for L in layers)
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # dominant kernel: the one-token layer call (fused: lq_layer_b1, its
    # stream kernel with the lift in the table prologue plus the slice
    # reduction; split: the lq_gemv call); per-call duration from HIP events
    # around replays of a graph of back-to-back calls over the copies
    per = {}
    for j, (rot, L) in enumerate(zip(rots, layers)):
        if fused:
            calls = lambda: [lq.layer_b1(rot.a, rot[k].t_inv, rot[k].M, L.d, L.D, rot[k].w,
                                         rot[k].s, out=outs[j]) for k in range(R)]
        else:
            calls = lambda: [lq.gemv(rot[k].w, rot[k].s, al[j], L.K, out=outs[j])
                             for k in range(R)]
        g = capture_graphs(torch, [calls])[0]
        replay_warm(torch, g)
        n_rep = max(3, min(args.steps, 20))
        per[j] = time_launches(torch, lambda i: g.replay(), n_rep, st) / R
    # the plain-read reference: every byte of each rotating weight copy of
    # both shapes read once by lq_stream_read, same graph timing
    sink = torch.zeros(4 * torch.cuda.get_device_properties(dev).multi_processor_count + 64,
                       dtype=torch.int32, device=dev)
    read_rates = {}
    for j, (rot, L) in enumerate(zip(rots, layers)):
        nbytes = rot[0].w.numel() * 4
        t_read = graph_time(torch, lambda k: lq.stream_read(rot[k].w, sink), R,
                            max(3, min(args.steps, 20)), st)
        read_rates[f"{L.m}x{L.n}"] = {"bytes": nbytes, "us": round(t_read * 1e3, 3),
                                      "GBs": round(nbytes / (t_read * 1e-3) / 1e9, 1)}
    ceiling_gbs = sum(v["GBs"] for v in read_rates.values()) / len(read_rates)
    g_bytes = [layer_bytes(L.m, L.n, L.d, L.D, 1) if fused else gemv_bytes(L.m, L.K, 1)
               for L in layers]
    gemv_ms = sum(per.values()) / len(per)
    gemv_bytes_avg = sum(g_bytes) / len(g_bytes)
    achieved = gemv_bytes_avg / (gemv_ms * 1e-3) / 1e9
    traffic = load_traffic("k_gemv1.hip" if fused else GEMV_SRC,
                           "layer_b1_lq19_8_70b" if fused else "gemv_lq19_8_70b_b1")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": ("lq_layer_b1 (gemv1_kernel with the lift in its table prologue + "
                           "gemv1_reduce_kernel)" if fused else
                           "lq_gemv B=1: gemv_f4r_kernel (one launch) on 28672x8192, "
                           "gemv_f4_kernel + gemv_f4_reduce_kernel on 8192x28672"),
                "bytes_per_launch": int(gemv_bytes_avg),
                "avg_launch_us": round(gemv_ms * 1e3, 3),
                "per_shape_us": {f"{L.m}x{L.n}": round(per[j] * 1e3, 3)
                                 for j, L in enumerate(layers)},
                "read_ceiling": {"kernel": "lq_stream_read (plain read of each weight copy, "
                                           "row padding included)",
                                 "GBs": round(ceiling_gbs, 1),
                                 "frac_of_peak": round(ceiling_gbs / HBM_PEAK_GBS, 4),
                                 "per_shape": read_rates},
                "frac_of_read_ceiling": round(achieved / ceiling_gbs, 4)}
    (step_fused if fused else step_split)(0)
    torch.cuda.synchronize()
    outs_host = [o.cpu().numpy().copy() for o in outs]
    rot_info = {"copies": rots[0].R, "bytes_per_copy": int(layers[0].packed.nbytes),
                "timing": "HIP graph per step, replayed; checked bit for bit against eager",
                "path": args.layer_path,
                "other_path_ms_per_step": round(ms_other, 5)}

    gemm = None if args.only == "layer" else run_gemm(args, torch, lq, synth, dev)
    cases = None if (args.no_cases or args.only != "all") else run_cases(torch, lq, synth, dev)
    kron = None if args.only != "all" else run_kron(torch, lq, synth, dev)
    enc = None if args.only != "all" else run_encode(torch, lq, synth, dev)
    learn = None if args.only != "all" else run_learn(torch, lq, synth, dev)
    return dict(value=value, ms_step=ms_step, roofline=roofline, gemm=gemm, cases=cases, kron=kron,
                encode=enc, learn=learn,
                layers=layers, outs=outs_host, rot=rot_info, step_bytes=step_bytes)


def capture_graphs(torch, fns):
    """One HIP graph per callable (captured on a side stream, as torch asks);
    the callables must allocate nothing."""
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in fns:
            fn()                                   # eager run on the capture stream
        torch.cuda.synchronize()
        for fn in fns:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                fn()
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return graphs


def graph_time(torch, fn, R, n_rep, st):
    """Average duration of one fn(k) launch: a HIP graph of fn(0) .. fn(R - 1)
    back to back, replayed n_rep times between HIP events on st, so the host's
    launch rate does not enter."""
    g = capture_graphs(torch, [lambda: [fn(k) for k in range(R)]])[0]
    replay_warm(torch, g)
    return time_launches(torch, lambda i: g.replay(), n_rep, st) / R


def replay_warm(torch, g, n=2):
    """Untimed replays of a new graph: its first replay carries one-time
    set-up costs that would otherwise be charged to the timed ones."""
    for _ in range(n):
        g.replay()
    torch.cuda.synchronize()


def time_launches(torch, fn, n, st):
    """Average duration of fn() over n back-to-back calls, HIP events on st."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(n):
        fn(i)
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / n


def run_gemm(args, torch, lq, synth, dev):
    """Batch-512 LQ-40/16 GEMM: lift to 16-bit, then the MFMA contraction."""
    cfg = synth.CONFIGS[4]
    L = synth.make_case(cfg, 0, cfg.batches[0])
    rot = Rotation(L, torch, lq, dev)
    odt = torch.float16 if args.gemm_dtype == "f16" else torch.bfloat16
    als = [torch.empty((L.B, L.K), dtype=odt, device=dev) for _ in range(2)]
    out = torch.empty((L.B, L.m), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream()
    for i in range(3):
        c = rot[i]
        lq.lift(rot.a, c.t_inv, c.M, L.d, L.D, out=als[i % 2])
        lq.gemm(c.w, c.s, als[i % 2], L.K, out=out)
    torch.cuda.synchronize()
    n = max(3, min(args.steps, 20))
    lift_ms = graph_time(torch, lambda k: lq.lift(rot.a, rot[k].t_inv, rot[k].M, L.d, L.D,
                                                  out=als[k % 2]), rot.R, n, st)
    gemm_ms = graph_time(torch, lambda k: lq.gemm(rot[k].w, rot[k].s, als[k % 2], L.K, out=out),
                         rot.R, n, st)
    flops = 2.0 * L.m * L.K * L.B
    tf = flops / (gemm_ms * 1e-3) / 1e12
    decoded = run_decoded(torch, lq, L, rot, st, lift_ms + gemm_ms, n)
    return {"workload": f"LQ-40/16 {L.m}x{L.n} batch {L.B}, lifted K={L.K}",
            "decoded": decoded,
            "operand_dtype": args.gemm_dtype, "gemm_us": round(gemm_ms * 1e3, 2),
            "lift_us": round(lift_ms * 1e3, 2), "tflops": round(tf, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                         "peak": MFMA_PEAK_TFLOPS[args.gemm_dtype], "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_PEAK_TFLOPS[args.gemm_dtype], 4),
                         "traffic": load_traffic("k_gemm.hip", "gemm_lq40_16_b512"),
                         "flops_per_launch": flops}}


def run_decoded(torch, lq, L, rot, st, lifted_ms, n_rep):
    """The same batch on the decode-weights path: u = T^-1 a (lift with
    M = I_4, float16), then one kernel that decodes s-free weights M y on the
    matrix cores and contracts them over n.  Own flop count: 2 m n B for the
    product plus 2 m n D for the decoding.  Graph timing like the other legs."""
    eye = torch.eye(4, dtype=torch.float32, device=rot.a.device)
    u = torch.empty((L.B, L.n), dtype=torch.float16, device=rot.a.device)
    out = torch.empty((L.B, L.m), dtype=torch.float32, device=rot.a.device)
    for i in range(3):
        lq.lift(rot.a, rot[i].t_inv, eye, 4, 4, out=u)
        lq.gemm_decoded(rot[i].w, rot[i].s, rot[i].M, L.d, L.D, u, out=out)
    torch.cuda.synchronize()
    lift_ms = graph_time(torch, lambda k: lq.lift(rot.a, rot[k].t_inv, eye, 4, 4, out=u),
                         rot.R, n_rep, st)
    prod_ms = graph_time(torch, lambda k: lq.gemm_decoded(rot[k].w, rot[k].s, rot[k].M, L.d,
                                                          L.D, u, out=out), rot.R, n_rep, st)
    flops = 2.0 * L.m * L.n * L.B + 2.0 * L.m * L.n * L.D
    tf = flops / (prod_ms * 1e-3) / 1e12
    return {"kernel": "gemm_dec_kernel (decode on the matrix cores + product, one launch)",
            "lift_u_us": round(lift_ms * 1e3, 2), "decode_and_product_us": round(prod_ms * 1e3, 2),
            "total_us": round((lift_ms + prod_ms) * 1e3, 2),
            "lifted_path_total_us": round(lifted_ms * 1e3, 2),
            "speedup_over_lifted": round(lifted_ms / (lift_ms + prod_ms), 3),
            "flops_per_call": flops, "tflops": round(tf, 1),
            "fp16_mfma_frac": round(tf / MFMA_PEAK_TFLOPS["f16"], 4),
            "timing": "HIP graph of back-to-back calls on rotating copies, replayed"}


def kron_lift_bytes(n, n1, d, D, B, act_bytes=2, out_bytes=4):
    """Algorithmic bytes of one Kronecker-whitened lift: a, s1, P1^-1, P2^-1,
    s2, M and a_hat (the n1 x n2 intermediate's round trip excluded)."""
    n2 = n // n1
    return (B * n * act_bytes + 4 * n + 4 * n1 * n1 + 4 * n2 * n2 + 4 * (n // d) + 4 * d * D
            + B * (n // d) * D * out_bytes)


# LiftQuant notes, table "Llama-2-7B Wikitext-2 PPL (标准 Gaussian 源)": code, D,
# d, MSE (learned M) and search time per 1M parameters (s; "<<0.1" for
# LQ-16/8), on the authors' hardware.
ENCODE_TABLE = (("LQ-32/20", 32, 20, 0.146, 0.3), ("LQ-16/8", 16, 8, 0.089, "<<0.1"),
                ("LQ-32/16", 32, 16, 0.082, 4.0), ("LQ-30/14", 30, 14, 0.070, 4.0),
                ("LQ-24/10", 24, 10, 0.053, 1.0))
# vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-operations per second
# (one wave64 instruction every 4 cycles per SIMD; packed float32 is not used)
ALU_PEAK_OPS = 256 * 4 * 16 * 2.4e9


def run_encode(torch, lq, synth, dev):
    """Lattice encoder over 1M unit-Gaussian weights per code of the table:
    the auxiliary-vector search with M the first d rows of a Haar orthogonal
    D x D matrix and A its other rows (the orthogonal initialisation; the
    table's M is learned), plus the exhaustive search for LQ-16/8."""
    res = []
    n_params = 1_000_000
    st = torch.cuda.current_stream()
    runs = [(c, D, d, mse, ts, True) for c, D, d, mse, ts in ENCODE_TABLE]
    runs.append(("LQ-16/8", 16, 8, 0.089, None, False))
    for code, D, d, mse_tab, t_tab, search in runs:
        G = -(-n_params // d)
        Q = synth.haar_orthogonal(np.random.default_rng(1000 * D + d), D)   # same M per code
        M = torch.from_numpy(Q[:d].astype(np.float32)).to(dev)
        A = torch.from_numpy(Q[d:].astype(np.float32)).to(dev) if search else None
        gen = torch.Generator(device=dev)
        gen.manual_seed(100 * D + d)
        W = torch.randn((G, d), generator=gen, device=dev, dtype=torch.float32)
        codes = torch.empty((G, D), dtype=torch.int8, device=dev)
        err = torch.empty((G,), dtype=torch.float32, device=dev)
        lq.encode(W, M, A, codes, err)
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            lq.encode(W, M, A, codes, err)
        e1.record(st)
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / reps * 1e-3
        kb = D - d if search else D
        cands = G * (1 << kb)
        ops = 2 * D + d * D + d if search else 2 * d      # per candidate, algorithmic
        mse = float(err.double().sum().item()) / (G * d)
        res.append({
            "code": code, "mode": "search" if search else "exhaustive",
            "candidates_per_group": 1 << kb, "groups": G,
            "seconds_per_1M_weights": round(sec * n_params / (G * d), 5),
            "candidates_per_s": float(f"{cands / sec:.4g}"),
            "alu": ({"bound": "alu", "achieved": float(f"{cands * ops / sec:.4g}"),
                     "peak": ALU_PEAK_OPS, "unit": "lane-op/s",
                     "frac": round(cands * ops / sec / ALU_PEAK_OPS, 4),
                     "ops_per_candidate": ops,
                     "ops_counted": "executed (residual update d + error d)"}
                    if not search else
                    {"bound": "alu", "frac": None,
                     "definition_ops_per_candidate": ops,
                     "definition_rate": float(f"{cands * ops / sec:.4g}"),
                     "note": ("no fraction: the search moves the residual only along the "
                              "columns whose sign flipped (about 4 of D per step, data "
                              "dependent), so the executed count is not the definition's")}),
            "mse_per_weight": round(mse, 5), "info_bits": round(float(-0.5 * np.log2(mse)), 3),
            "pages": {"mse_learned_M": mse_tab, "search_s_per_1M": t_tab,
                      "note": "the authors' hardware and learned M: context, not a target"}})
    return res


def run_learn(torch, lq, synth, dev):
    """Learning M (soft-argmin objective at T = 10, Adam, lr 0.01) from the
    orthogonal start on fresh unit-Gaussian batches: time per step, pair
    throughput (samples x codes per second) and the hard nearest-point MSE
    per weight of the start and the learned M (exhaustive encoder over 200k
    fresh weights) beside the table's."""
    res = []
    st = torch.cuda.current_stream()
    for code, d, D, N, steps, mse_tab in (("LQ-16/8", 8, 16, 4096, 400, 0.089),
                                          ("LQ-20/8", 8, 20, 2048, 200, None)):
        Q = synth.haar_orthogonal(np.random.default_rng(1000 * D + d), D)
        M0 = torch.from_numpy(Q[:d].astype(np.float32)).to(dev)

        def hard_mse(M, n=200_000):
            g = torch.Generator(device=dev)
            g.manual_seed(99)
            W = torch.randn((n // d, d), generator=g, device=dev)
            _, err = lq.encode(W, M)
            return float(err.double().sum().item()) / n

        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        batches = [torch.randn((N, d), generator=gen, device=dev) for _ in range(steps)]
        M = M0.clone()
        m1, m2, grad = torch.zeros_like(M), torch.zeros_like(M), torch.empty_like(M)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        last = None
        for i, W in enumerate(batches, start=1):
            last, _ = lq.softmin_grad(W, M, 10.0, grad=grad)
            lq.adam_update(M, grad, m1, m2, i, 0.01)
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        pairs = N * (1 << D)
        # vector operations per (sample, code) pair, forward + backward: as
        # the definition states them (distance, exponential, the D-term sums
        # over y_t), and as the kernels execute them (the D-term sums reduced
        # to the low 6 / 8 code bits, the rest formed once per chunk or per
        # staged sample)
        ops_def = 3 * d + D + 8 + 3 * d + D + 4
        ops_run = 3 * d + 4 + min(D, 6) + 3 * d + min(D, 8) + 6
        res.append({"code": code, "samples_per_step": N, "codes": 1 << D, "steps": steps,
                    "ms_per_step": round(ms, 3),
                    "pairs_per_s": float(f"{pairs / (ms * 1e-3):.4g}"),
                    "ops_per_pair": {"definition": ops_def, "executed": ops_run},
                    "alu_frac": round(pairs * ops_run / (ms * 1e-3) / ALU_PEAK_OPS, 4),
                    "final_soft_loss": round(float(last.cpu()[0]), 5),
                    "mse_orthogonal_start": round(hard_mse(M0), 5),
                    "mse_learned": round(hard_mse(M), 5),
                    "pages_mse_learned_M": mse_tab})
    return res


def kron_lift_flops(n, n1, D, B):
    """Algorithmic flops of one Kronecker-whitened lift: per token the two
    factor products, 2 n (n1 + n2), and the per-group M^T step, 2 n D."""
    n2 = n // n1
    return B * (2 * n * (n1 + n2) + 2 * n * D)


def run_kron(torch, lq, synth, dev):
    """Lift with the Kronecker-factored whitening against the block-diagonal
    lift on the same activations: the 70B-class shapes at batch 1 (float32
    a_hat, as the GEMV takes) and LQ-40/16 at batch 512 (float16 a_hat)."""
    res = []
    st = torch.cuda.current_stream()
    for cfg_i, si, B, odt in ((3, 0, 1, torch.float32), (3, 1, 1, torch.float32),
                              (4, 0, 512, torch.float16)):
        cfg = synth.CONFIGS[cfg_i]
        L = synth.make_case(cfg, si, B, m=128)
        f = synth.make_kron_factors(L.n, L.d, 1000 + si)
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        s1, p1, p2, s2 = t(f.s1), t(f.p1_inv), t(f.p2_inv), t(f.s2)
        M = t(L.M)
        a = lq.to_torch_16(L.a, L.dtype).to(dev)
        tinv = lq.to_torch_16(L.t_inv, L.dtype).to(dev)
        out = torch.empty((B, L.K), dtype=odt, device=dev)
        fn_k = lambda k: lq.lift_kron(a, s1, p1, p2, s2, M, L.d, L.D, out=out)
        fn_b = lambda k: lq.lift(a, tinv, M, L.d, L.D, out=out)
        fn_k(0)
        fn_b(0)
        torch.cuda.synchronize()
        tk = graph_time(torch, fn_k, 20, 10, st)
        tb = graph_time(torch, fn_b, 20, 10, st)
        ob = 4 if odt == torch.float32 else 2
        kb = kron_lift_bytes(L.n, f.n1, L.d, L.D, B, out_bytes=ob)
        kf = kron_lift_flops(L.n, f.n1, L.D, B)
        res.append({"case": f"{cfg.name} n={L.n} (n1 x n2 = {f.n1} x {f.n2}) B={B}",
                    "kron_lift_us": round(tk * 1e3, 2), "kron_lift_GBs": round(kb / (tk * 1e-3) / 1e9, 1),
                    "kron_lift_TFLOPs": round(kf / (tk * 1e-3) / 1e12, 2),
                    "kron_lift_fp32_mfma_frac": round(kf / (tk * 1e-3) / PEAK_FP32_FLOPS, 4),
                    "blockdiag_lift_us": round(tb * 1e3, 2),
                    "whitening_bytes": {"kron": 4 * (L.n + f.n1 ** 2 + f.n2 ** 2 + L.n // L.d),
                                        "blockdiag": 256 * L.n}})
    return res


def run_cases(torch, lq, synth, dev, tokens=0):
    """GEMV (B <= 16) per workload case: graphs of back-to-back launches on
    rotating copies (only the cases with `tokens` tokens when it is set)."""
    res = []
    st = torch.cuda.current_stream()
    for cfg, si, (m, n), B in synth.all_cases():
        if B > 16 or (tokens and B != tokens):
            continue
        L = synth.make_case(cfg, si, B)
        rot = Rotation(L, torch, lq, dev)
        al = torch.empty((B, L.K), dtype=torch.float32, device=dev)
        out = torch.empty((B, m), dtype=torch.float32, device=dev)
        lq.lift(rot.a, rot[0].t_inv, rot[0].M, L.d, L.D, out=al)
        for i in range(3):
            lq.gemv(rot[i].w, rot[i].s, al, L.K, out=out)
        torch.cuda.synchronize()
        g = graph_time(torch, lambda k: lq.gemv(rot[k].w, rot[k].s, al, L.K, out=out), rot.R, 10, st)
        lt = graph_time(torch, lambda k: lq.lift(rot.a, rot[k].t_inv, rot[k].M, L.d, L.D, out=al),
                        rot.R, 10, st)
        gb = gemv_bytes(m, L.K, B) / (g * 1e-3) / 1e9
        rec = {"case": f"{cfg.name} {m}x{n} B={B}", "gemv_us": round(g * 1e3, 2),
               "gemv_GBs": round(gb, 1), "gemv_frac": round(gb / HBM_PEAK_GBS, 3),
               "lift_us": round(lt * 1e3, 2)}
        if B >= 6:
            # the layer's default for 6 - 16 tokens: the lift writes the
            # GEMV's float8-part operand image, the GEMV reads it
            img = torch.empty(lq.lift_parts_size(L.K), dtype=torch.uint8, device=dev)
            lq.lift_parts(rot.a, rot[0].t_inv, rot[0].M, L.d, L.D, out=img)
            for i in range(3):
                lq.gemv_parts(rot[i].w, rot[i].s, img, L.K, B, out=out)
            torch.cuda.synchronize()
            gp = graph_time(torch, lambda k: lq.gemv_parts(rot[k].w, rot[k].s, img, L.K, B, out=out),
                            rot.R, 10, st)
            lp = graph_time(torch, lambda k: lq.lift_parts(rot.a, rot[k].t_inv, rot[k].M, L.d, L.D,
                                                           out=img), rot.R, 10, st)
            gpb = gemv_bytes(m, L.K, B) / (gp * 1e-3) / 1e9
            rec["parts_path"] = {"gemv_us": round(gp * 1e3, 2), "gemv_GBs": round(gpb, 1),
                                 "gemv_frac": round(gpb / HBM_PEAK_GBS, 3),
                                 "lift_us": round(lp * 1e3, 2),
                                 "lift_plus_gemv_us": round((gp + lp) * 1e3, 2),
                                 "float32_path_lift_plus_gemv_us": round((g + lt) * 1e3, 2)}
        res.append(rec)
        del rot
        torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------- CPU baseline
def cpu_baseline(layers, outs, seconds):
    """The float64 oracle (as it stands) on a bounded sample of the same
    workload: whole rows of the up and down projections, chunk by chunk (each
    chunk pays its own unpack, reconstruction, T^-1 product and dgemm), passes
    over the layers repeated until about `seconds` of work; reported in the
    same unit as `value`.  Each chunk's result is also checked against the
    GPU output of the timed steps."""
    from oracle import lq_oracle as O
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(threads)
    except Exception:   # noqa: BLE001
        pass
    total_t = 0.0
    total_bytes = 0
    rows_done = [0, 0]
    passes = 0
    max_err = 0.0
    chunk = 1024
    j = 0
    while total_t < seconds:
        L = layers[j % len(layers)]
        r0 = rows_done[j % len(layers)] % L.m
        rows = np.arange(r0, min(r0 + chunk, L.m))
        t0 = time.perf_counter()
        ref = O.forward(L.packed, L.K, L.M, L.t_inv, L.s, L.a, L.d, L.D, L.dtype, rows=rows)
        dt = time.perf_counter() - t0
        total_t += dt
        total_bytes += rows.size * (L.K // 8 + 4 + 4 * L.B)
        if r0 == 0:
            total_bytes += 2 * L.n * L.B + 2 * L.n * 128 + 4 * L.d * L.D
        got = outs[j % len(layers)][:, rows]
        max_err = max(max_err, O.rel_err_colmax(got, ref))
        rows_done[j % len(layers)] += rows.size
        j += 1
    passes = min(r // L.m for r, L in zip(rows_done, layers))
    gbs = total_bytes / total_t / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle (unpack, W_hat = M y, T^-1 a, dgemm) in 1024-row "
                      f"chunks: {rows_done[0]} rows of the up projection (28672 x 8192) and "
                      f"{rows_done[1]} of the down (8192 x 28672), {passes} full passes, "
                      f"{total_t:.1f} s of CPU time",
            "seconds": round(total_t, 2), "gpu_vs_oracle_max_rel_err": float(f"{max_err:.3e}")}


def machine_info():
    """GPU, clocks, ROCm version, host CPU model and usable cores."""
    info = {}
    try:
        import torch
        p = torch.cuda.get_device_properties(0)
        info["gpu"] = p.name
        info["arch"] = getattr(p, "gcnArchName", None)
        info["compute_units"] = p.multi_processor_count
        for attr in ("clock_rate", "memory_clock_rate"):
            v = getattr(p, attr, None)
            if v:
                info[attr + "_khz"] = int(v)
    except Exception as e:  # noqa: BLE001
        info["gpu_error"] = str(e)
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                info["cpu"] = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    info["host_cores"] = len(os.sched_getaffinity(0))
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                             timeout=20).stdout
        info["clocks"] = [ln.strip() for ln in out.splitlines()
                          if "sclk" in ln or "mclk" in ln or "fclk" in ln][:6]
    except Exception:  # noqa: BLE001
        pass
    return info


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the path runs on one GPU; sharding over several is not built)", file=sys.stderr)
        sys.exit(2)
    r = run_gpu(args)
    if args.only in ("gemm", "cases", "kron", "encode", "learn"):
        print(json.dumps({args.only: r[args.only]}), flush=True)
        return
    cpu = None if args.no_cpu else cpu_baseline(r["layers"], r["outs"], args.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": round(r["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f8x3-parts+f32",
        "precision": ("1-5 tokens: three float8 (E4M3) parts per lifted activation "
                      "(12 significant bits, power-of-two scale per 1024-position slice) x "
                      "float4 0/1 sign nibbles on the matrix cores, float32 accumulation, "
                      "2R - sum(a) per slice in float32; 6-16 tokens: the same parts "
                      "(scale per 128-position step) as column blocks x float4 +-1 signs; "
                      "batch 512: 16-bit operands, float32 accumulation"),
        "data": "synthetic (seeded; shapes of the 70B-class LQ-19/8 MLP)",
        "config": {"workload": "LQ-19/8 70B-class MLP at batch 1: up 28672x8192 then down "
                               "8192x28672, lift + GEMV each, inputs bf16, weights 2.375 bit",
                   "batch": 1, "step_bytes": r["step_bytes"], "rotation": r["rot"]},
        "frac_of_hbm_peak": round(r["value"] / HBM_PEAK_GBS, 4),
        "machine": machine_info(),
        "roofline": r["roofline"],
        "cpu_baseline": cpu,
        "gemm": r["gemm"],
        "cases": r["cases"],
        "kron_lift": r["kron"],
        "encode": r["encode"],
        "learn_m": r["learn"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
