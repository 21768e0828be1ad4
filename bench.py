"""Benchmark of the block-quantized product path on one MI355X.

One step is one pass over every stage of the hot path on its synthetic
workload:
  dequant   Q4_K 2048x2048 -> fp32                         (2048x2048, seed 101)
  qmv_c1    Q4_K 2048x2048 GEMV, fp32 x/y                  (seed 101)
  qmv_c2    Q4_K 14336x4096 and 4096x14336 GEMV, fp16 x at batch 1/4/8, fp16 y  (seed 102)
  qmm_c3    Q4_K and Q8_0 4096x4096 and 14336x4096, bf16 x at M=512/2048, bf16 y (seed 103)
  moe_c4    128 experts, Q4_K gate/up 2048x7168, down 7168x2048, top-8;
            fp16 x, fp32 h and output; 1 token (decode) and 256 tokens (seed 104)
  tq1_c5    TQ1_G128 17408x5120 and 5120x17408, fp16 x at batch 1 and M=512 (seed 105)
  ggml_mv   Q8_0 and the further GGUF blocks (Q4_0, Q5_0, Q5_1, Q6_K, Q2_K, Q3_K, Q5_K)
            in the C2 GEMV shapes 14336x4096 and 4096x14336, fp16 x at batch 1 (and batch 8 as
            extra rows), fp16 y, and the
            further blocks' prefill GEMM in the C3 shape 14336x4096 at M=2048, bf16 x (seed 106)
  ggml_moe  one-token and 256-token MoE layers (gate/up + SwiGLU, down + weighted sum) with
            those blocks at the C4 matrix shapes: 32 experts, top-8, fp16 x, fp32 h (seed 107)

The headline value is the Q4_K decode GEMV (the six qmv_c2 calls): weight
bytes streamed per second.  Every call reads weights from HBM: weight-bound
stages rotate over >= 1 GiB of distinct weight copies (the 256 MB Infinity
Cache would otherwise serve them), and MoE decode rotates over tokens, whose
expert choices differ.  Each stage's calls run back to back between one pair
of HIP events on the stream the kernels are launched on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--stages a,b] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_K GEMV weight-GB/s (% of HBM peak); prefill qmm TFLOP/s; MoE tokens/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFS = 2500.0
GIB = 1 << 30
# (workgroups, loads in flight per lane) of the streaming-read ceiling
READ_SHAPES = ((1024, 4), (2048, 4), (4096, 2), (4096, 4), (1024, 8), (2048, 8), (4096, 8))
STAGES = ("dequant", "qmv_c1", "qmv_c2", "qmm_c3", "moe_c4", "tq1_c5", "ggml_mv", "ggml_moe")
GGML_KINDS = ("q8_0", "q4_0", "q5_0", "q5_1", "q6_k", "q2_k", "q3_k", "q5_k")
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--stages", default=",".join(STAGES))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a 256 MiB device copy (counter calibration)")
    return p.parse_args()


class Stage:
    """A list of calls timed as one group; `work` gives the algorithmic
    bytes and flops of one pass over `calls`."""

    def __init__(self, name, calls, bytes_, flops, tokens=0, note=""):
        self.name, self.calls, self.bytes, self.flops = name, calls, bytes_, flops
        self.tokens, self.note = tokens, note
        self.ms = []

    def run(self):
        for c in self.calls:
            c()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                          f"--gpus {args.gpus} is not supported"}))
        sys.exit(2)

    import torch

    from block_quantized_weight_q4_amd import _build, kq
    import synth
    from synth import workloads

    _build.build_if_missing()
    kq.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": 256 << 20}))
        return

    wanted = [s for s in args.stages.split(",") if s]

    def d8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def d16(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dt).to(dev)

    def copies(t, nbytes_each, min_total=GIB):
        n = max(1, -(-min_total // nbytes_each))
        return [t] + [t.clone() for _ in range(n - 1)]

    stages = []
    rot = {"i": 0}

    def nxt(lst):
        rot["i"] += 1
        return lst[rot["i"] % len(lst)]

    if "dequant" in wanted or "qmv_c1" in wanted:
        c = workloads.c1()
        w = d8(c["w"])
        ws = copies(w, w.numel())
        if "dequant" in wanted:
            outs = [torch.empty((2048, 2048), dtype=torch.float32, device=dev) for _ in range(8)]
            calls = [lambda ws=ws, outs=outs: kq.kq_dequantize("q4_k", nxt(ws), 2048, 2048,
                                                                nxt(outs)) for _ in range(20)]
            stages.append(Stage("dequant", calls, 20 * (w.numel() + 2048 * 2048 * 4), 0,
                                note="Q4_K 2048x2048 -> fp32"))
        if "qmv_c1" in wanted:
            x = torch.from_numpy(c["x"]).to(dev)
            y = torch.empty((1, 2048), dtype=torch.float32, device=dev)
            calls = [lambda ws=ws, x=x, y=y: kq.kq_qmv("q4_k", nxt(ws), 2048, 2048, x, 1, y)
                     for _ in range(40)]
            stages.append(Stage("qmv_c1", calls, 40 * (w.numel() + 2 * 2048 * 4),
                                40 * 2 * 2048 * 2048, note="Q4_K 2048x2048 GEMV fp32"))

    c2_parts = []
    if "qmv_c2" in wanted:
        calls, nbytes, flops = [], 0, 0
        c2_ws = {}
        for case in workloads.c2():
            n, k = case["n"], case["k"]
            w = d8(case["w"])
            ws = copies(w, w.numel())
            c2_ws[(n, k)] = ws
            x = d16(case["x"], torch.float16)
            for b in (1, 4, 8):
                y = torch.empty((b, n), dtype=torch.float16, device=dev)
                reps = len(ws)
                part = [(lambda n=n, k=k, x=x, b=b, y=y, ws=ws:
                         kq.kq_qmv("q4_k", nxt(ws), n, k, x, b, y)) for _ in range(reps)]
                pbytes = reps * (w.numel() + b * (k + n) * 2)
                c2_parts.append(Stage(f"qmv_c2_{n}x{k}_b{b}", part, pbytes, reps * 2 * b * n * k))
                calls += part
                nbytes += pbytes
                flops += reps * 2 * b * n * k
        stages.append(Stage("qmv_c2", calls, nbytes, flops,
                            note="Q4_K 14336x4096 + 4096x14336, batch 1/4/8, fp16"))
        # dependency chain at batch 1: each call's output row is the next
        # call's activation row (14336x4096 then 4096x14336, alternating)
        wa, wb = c2_ws[(14336, 4096)], c2_ws[(4096, 14336)]
        va = d16(workloads.c2()[0]["x"][:1], torch.float16)
        vb = torch.empty((1, 14336), dtype=torch.float16, device=dev)
        chain = []
        for _ in range(len(wa)):
            chain.append(lambda: kq.kq_qmv("q4_k", nxt(wa), 14336, 4096, va, 1, vb))
            chain.append(lambda: kq.kq_qmv("q4_k", nxt(wb), 4096, 14336, vb, 1, va))
        cbytes = len(chain) * (wa[0].numel() + (4096 + 14336) * 2)
        stages.append(Stage("qmv_c2_chain_b1", chain, cbytes, len(chain) * 2 * 4096 * 14336,
                            note="batch 1, each output feeds the next call (values may overflow "
                                 "fp16; the work is the same)"))

    def scratch(kind, n, k, m, dt):
        nb = kq.kq_qmm_workspace_bytes(kind, n, k, m, dt)
        return torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)

    c3_parts, extra_parts = [], []
    if "qmm_c3" in wanted:
        cases, xh = workloads.c3()
        x = d16(xh, torch.bfloat16)
        for case in cases:
            kind, n, k = case["kind"], case["n"], case["k"]
            w = d8(case["w"])
            ws = copies(w, w.numel())  # >= 1 GiB of distinct weight copies
            for m in (512, 2048):
                y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                xm = x[:m]
                sc = scratch(kind, n, k, m, torch.bfloat16)
                part = [(lambda kind=kind, n=n, k=k, m=m, y=y, ws=ws, xm=xm, sc=sc:
                         kq.kq_qmm_ws(kind, nxt(ws), n, k, xm, m, y, sc)) for _ in range(len(ws))]
                c3_parts.append(Stage(f"qmm_c3_{kind}_{n}x{k}_m{m}", part,
                                      len(part) * (w.numel() + m * (k + n) * 2),
                                      len(part) * 2 * m * n * k, note="kq_qmm_ws"))
                # the same product without a workspace (bf16 rows scaled per tile column)
                part = [(lambda kind=kind, n=n, k=k, m=m, y=y, ws=ws, xm=xm:
                         kq.kq_qmm(kind, nxt(ws), n, k, xm, m, y)) for _ in range(8)]
                extra_parts.append(Stage(f"qmm_c3_noworkspace_{kind}_{n}x{k}_m{m}", part,
                                         len(part) * (w.numel() + m * (k + n) * 2),
                                         len(part) * 2 * m * n * k, note="kq_qmm"))

    if "tq1_c5" in wanted:
        calls_v, calls_m, bv, bm, fv, fm = [], [], 0, 0, 0, 0
        calls_q, bq = [], 0
        for case in workloads.c5():
            n, k = case["n"], case["k"]
            w = d8(case["w"])
            ws = copies(w, w.numel())
            x = d16(case["x"], torch.float16)
            y1 = torch.empty((1, n), dtype=torch.float16, device=dev)
            ym = torch.empty((512, n), dtype=torch.float16, device=dev)
            # batch 1 through the workspace form: K split for the 5120-row
            # shape; also the no-workspace GEMV (kq_qmv) beside it
            s1 = scratch("tq1_g128", n, k, 1, torch.float16)
            part, pb = [], 0
            for _ in range(len(ws)):
                part.append(lambda n=n, k=k, ws=ws, x=x, y1=y1, s1=s1:
                            kq.kq_qmm_ws("tq1_g128", nxt(ws), n, k, x[:1], 1, y1, s1))
                pb += w.numel() + (k + n) * 2
                calls_q.append(lambda n=n, k=k, ws=ws, x=x, y1=y1:
                               kq.kq_qmv("tq1_g128", nxt(ws), n, k, x[:1], 1, y1))
                fv += 2 * n * k
            calls_v += part
            bv += pb
            bq += pb
            extra_parts.append(Stage(f"tq1_c5_b1_{n}x{k}", part, pb, len(part) * 2 * n * k,
                                     note="TQ1 GEMV batch 1, fp16 (kq_qmm_ws)"))
            sc = scratch("tq1_g128", n, k, 512, torch.float16)
            for _ in range(len(ws)):
                calls_m.append(lambda n=n, k=k, ws=ws, x=x, ym=ym, sc=sc:
                               kq.kq_qmm_ws("tq1_g128", nxt(ws), n, k, x, 512, ym, sc))
                bm += w.numel() + 512 * (k + n) * 2
                fm += 2 * 512 * n * k
        stages.append(Stage("tq1_c5_b1", calls_v, bv, fv,
                            note="TQ1 GEMV batch 1, fp16 (kq_qmm_ws: K split on the 5120-row shape)"))
        extra_parts.append(Stage("tq1_c5_b1_noworkspace", calls_q, bq, fv,
                                 note="TQ1 GEMV batch 1, fp16 (kq_qmv, no workspace)"))
        stages.append(Stage("tq1_c5_m512", calls_m, bm, fm, note="TQ1 qmm M=512, fp16 (kq_qmm_ws)"))

    if "ggml_mv" in wanted:
        rng = synth.rng_for(106)
        for kind in GGML_KINDS:
            calls, nbytes = [], 0
            for n, k in ((14336, 4096), (4096, 14336)):
                w = d8(synth.weight_blocks(kind, rng, n, k))
                ws = copies(w, w.numel())
                x = d16(synth.activations(rng, (1, k), "f16"), torch.float16)
                y = torch.empty((1, n), dtype=torch.float16, device=dev)
                part = [(lambda kind=kind, n=n, k=k, x=x, y=y, ws=ws:
                         kq.kq_qmv(kind, nxt(ws), n, k, x, 1, y)) for _ in range(len(ws))]
                pb = len(part) * (w.numel() + (k + n) * 2)
                extra_parts.append(Stage(f"ggml_mv_{kind}_{n}x{k}_b1", part, pb,
                                         len(part) * 2 * n * k, note=f"{kind} GEMV batch 1, fp16"))
                calls += part
                nbytes += pb
                # batch 8 (the matrix-core decode kernel)
                x8 = d16(synth.activations(rng, (8, k), "f16"), torch.float16)
                y8 = torch.empty((8, n), dtype=torch.float16, device=dev)
                part8 = [(lambda kind=kind, n=n, k=k, x8=x8, y8=y8, ws=ws:
                          kq.kq_qmv(kind, nxt(ws), n, k, x8, 8, y8)) for _ in range(len(ws))]
                extra_parts.append(Stage(f"ggml_mv_{kind}_{n}x{k}_b8", part8,
                                         len(part8) * (w.numel() + 8 * (k + n) * 2),
                                         len(part8) * 2 * 8 * n * k, note=f"{kind} GEMV batch 8, fp16"))
            stages.append(Stage(f"ggml_mv_{kind}", calls, nbytes, 0,
                                note=f"{kind} GEMV batch 1, fp16, both C2 shapes"))
            if kind == "q8_0":
                continue  # (its prefill GEMM is timed by qmm_c3)
            # the prefill GEMM in the largest C3 shape (bf16 x, kq_qmm_ws)
            n, k, mm = 14336, 4096, 2048
            w = d8(synth.weight_blocks(kind, rng, n, k))
            ws = copies(w, w.numel())
            xm = d16(synth.activations(rng, (mm, k), "bf16"), torch.bfloat16)
            y = torch.empty((mm, n), dtype=torch.bfloat16, device=dev)
            sc = scratch(kind, n, k, mm, torch.bfloat16)
            part = [(lambda kind=kind, n=n, k=k, mm=mm, ws=ws, xm=xm, y=y, sc=sc:
                     kq.kq_qmm_ws(kind, nxt(ws), n, k, xm, mm, y, sc)) for _ in range(8)]
            extra_parts.append(Stage(f"ggml_mm_{kind}_{n}x{k}_m{mm}", part,
                                     len(part) * (w.numel() + mm * (k + n) * 2),
                                     len(part) * 2 * mm * n * k, note=f"{kind} prefill GEMM, bf16 x (kq_qmm_ws)"))

    if "ggml_moe" in wanted:
        # one-token MoE layers (gate/up + SwiGLU, down + weighted sum) with
        # Q8_0 and the further GGUF codecs at the C4 matrix shapes: 32 experts
        # (their 0.5-1.5 GB exceed the 256 MB Infinity Cache), top-8, fp16 x,
        # fp32 h, 64 tokens of distinct routings
        rng = synth.rng_for(107)
        E, H, F, top_k, T = 32, 7168, 2048, 8, 64
        xg = d16(synth.activations(rng, (T, H), "f16"), torch.float16)
        idg = torch.from_numpy(np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)])
                               .astype(np.int32)).to(dev)
        scg = torch.from_numpy(rng.uniform(0.05, 1.0, size=(T, top_k)).astype(np.float32)).to(dev)
        TP = 256
        xp = d16(synth.activations(rng, (TP, H), "f16"), torch.float16)
        idp = torch.from_numpy(np.stack([rng.choice(E, top_k, replace=False) for _ in range(TP)])
                               .astype(np.int32)).to(dev)
        scp = torch.from_numpy(rng.uniform(0.05, 1.0, size=(TP, top_k)).astype(np.float32)).to(dev)
        for kind in GGML_KINDS:
            gs, ds = F * synth.row_bytes(kind, H), H * synth.row_bytes(kind, F)
            g_w = d8(synth.weight_blocks(kind, rng, E * F, H))
            u_w = d8(synth.weight_blocks(kind, rng, E * F, H))
            dn_w = d8(synth.weight_blocks(kind, rng, E * H, F))
            mws_g = torch.empty(kq.kq_moe_workspace_bytes(E, 1, top_k, H), dtype=torch.uint8, device=dev)
            h_g = torch.empty((1, top_k, F), dtype=torch.float32, device=dev)
            o_g = torch.empty((1, H), dtype=torch.float32, device=dev)

            def layer1(t, kind=kind, g_w=g_w, u_w=u_w, dn_w=dn_w, gs=gs, ds=ds, mws_g=mws_g, h_g=h_g, o_g=o_g,
                       E=E, H=H, F=F, top_k=top_k, xg=xg, idg=idg, scg=scg):
                kq.kq_moe_glu(kind, g_w, u_w, E, F, H, gs, xg[t:t + 1], idg[t:t + 1], 1, top_k, h_g, mws_g)
                kq.kq_qmm_id(kind, dn_w, E, H, F, ds, h_g, kq.LAYOUT_SLOTTED, idg[t:t + 1], 1, top_k,
                             scg[t:t + 1], o_g, mws_g)

            calls = [lambda t=t, layer1=layer1: layer1(t) for t in range(T)]
            extra_parts.append(Stage(f"ggml_moe_{kind}_decode", calls, T * top_k * (2 * gs + ds),
                                     T * top_k * 2 * 3 * F * H,
                                     note=f"{kind} one-token MoE layer at the C4 shapes, 32 experts, top-8"))
            # the 256-token layer over the schedule (the down projection reuses it)
            mws_p = torch.empty(kq.kq_moe_workspace_bytes(E, TP, top_k, H), dtype=torch.uint8, device=dev)
            h_p = torch.empty((TP, top_k, F), dtype=torch.float32, device=dev)
            o_p = torch.empty((TP, H), dtype=torch.float32, device=dev)

            def layerp(kind=kind, g_w=g_w, u_w=u_w, dn_w=dn_w, gs=gs, ds=ds, mws_p=mws_p, h_p=h_p, o_p=o_p,
                       E=E, H=H, F=F, top_k=top_k, TP=TP, xp=xp, idp=idp, scp=scp):
                kq.kq_moe_glu(kind, g_w, u_w, E, F, H, gs, xp, idp, TP, top_k, h_p, mws_p)
                kq.kq_qmm_id(kind, dn_w, E, H, F, ds, h_p, kq.LAYOUT_SLOTTED | kq.REUSE_SCHEDULE, idp, TP, top_k,
                             scp, o_p, mws_p)

            extra_parts.append(Stage(f"ggml_moe_{kind}_prefill", [layerp] * 2, 2 * E * (2 * gs + ds),
                                     2 * TP * top_k * 2 * 3 * F * H,
                                     note=f"{kind} 256-token MoE layer at the C4 shapes, 32 experts, top-8"))

    # Streaming-read ceiling: a plain 16-byte-load read of the same number of
    # bytes as one C2 / C5 weight matrix (libkq_hbmread.so), rotated over
    # >= 1 GiB of copies like the GEMVs, in a few launch shapes; the best
    # shape is the ceiling reported beside the 8 TB/s figure
    ceil_parts = []
    if "qmv_c2" in wanted or "tq1_c5" in wanted:
        rd = ctypes.CDLL(_build.READ_LIB)
        rd.kq_hbm_read.restype = ctypes.c_int
        rd.kq_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
        sink = torch.zeros(1, dtype=torch.int32, device=dev)

        def hbm_read(buf, nbytes, grid, unroll):
            rc = rd.kq_hbm_read(buf.data_ptr(), nbytes, grid, unroll, 0x9E3779B9, sink.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"kq_hbm_read failed ({rc})")

        for nbytes, tag in ((33030144, "33MB"), (19496960, "19.5MB")):
            base = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
            bufs = copies(base, nbytes)
            for grid, unroll in READ_SHAPES:
                part = [(lambda bufs=bufs, nb=nbytes, g=grid, u=unroll: hbm_read(nxt(bufs), nb, g, u))
                        for _ in range(len(bufs))]
                ceil_parts.append(Stage(f"hbm_read_ceiling_{tag}_g{grid}_u{unroll}", part,
                                        len(part) * nbytes, 0,
                                        note=f"plain streaming read: {grid} workgroups of 256 "
                                             f"threads, {unroll} 16-byte loads in flight per lane"))

    if "moe_c4" in wanted:
        c = workloads.c4()
        E, H, F, T, top_k = c["n_experts"], c["hidden"], c["ffn"], c["T"], c["top_k"]
        gate, up, down = d8(c["gate"]), d8(c["up"]), d8(c["down"])
        xall = d16(c["x"], torch.float16)
        ids = torch.from_numpy(c["ids"].view(np.int32)).to(dev)
        scores = torch.from_numpy(c["scores"]).to(dev)
        mws = torch.empty(kq.kq_moe_workspace_bytes(E, T, top_k, H), dtype=torch.uint8, device=dev)
        h = torch.empty((T, top_k, F), dtype=torch.float32, device=dev)
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
        per_expert = 3 * F * synth.row_bytes("q4_k", H)

        def layer(t0, nt):
            kq.kq_moe_glu("q4_k", gate, up, E, F, H, c["gate_stride"], xall[t0:t0 + nt],
                          ids[t0:t0 + nt], nt, top_k, h[:nt], mws)
            # the down projection keeps the schedule the gate/up call built
            kq.kq_qmm_id("q4_k", down, E, H, F, c["down_stride"], h[:nt],
                         kq.LAYOUT_SLOTTED | kq.REUSE_SCHEDULE, ids[t0:t0 + nt], nt, top_k,
                         scores[t0:t0 + nt], out[:nt], mws)

        dec_calls = [lambda t=t, layer=layer: layer(t, 1) for t in range(0, 64)]
        # every decode token reads its 8 experts' three matrices
        stages.append(Stage("moe_c4_decode", dec_calls, len(dec_calls) * 8 * per_expert,
                            len(dec_calls) * 8 * 3 * 2 * F * H, tokens=len(dec_calls),
                            note="1 token, top-8 of 128"))
        # decode as a dependency chain: each token's mixed output (fp16) is the
        # next token's activation row, so no layer overlaps the one before it
        cx = [d16(c["x"][:1], torch.float16), torch.empty((1, H), dtype=torch.float16, device=dev)]

        def chain_layer(t):
            src, dst = cx[t % 2], cx[(t + 1) % 2]
            kq.kq_moe_glu("q4_k", gate, up, E, F, H, c["gate_stride"], src, ids[t:t + 1], 1, top_k,
                          h[:1], mws)
            kq.kq_qmm_id("q4_k", down, E, H, F, c["down_stride"], h[:1],
                         kq.LAYOUT_SLOTTED | kq.REUSE_SCHEDULE, ids[t:t + 1], 1, top_k,
                         scores[t:t + 1], dst, mws)

        chain_calls = [lambda t=t: chain_layer(t) for t in range(0, 64)]
        stages.append(Stage("moe_c4_decode_chain", chain_calls, len(chain_calls) * 8 * per_expert,
                            len(chain_calls) * 8 * 3 * 2 * F * H, tokens=len(chain_calls),
                            note="1 token, top-8 of 128, each token's fp16 output feeds the next "
                                 "(values may overflow fp16; the work is the same)"))
        pre_calls = [lambda layer=layer, T=T: layer(0, T) for _ in range(2)]
        used = len(np.unique(c["ids"]))
        stages.append(Stage("moe_c4_prefill", pre_calls, 2 * used * per_expert,
                            2 * T * top_k * 3 * 2 * F * H, tokens=2 * T,
                            note=f"256 tokens, {used} experts hit"))

    # ---------------------------------------------------------------- timing
    # Each stage's calls are captured once into a HIP graph and replayed, so
    # the kernels run back to back instead of waiting on Python launches.
    timed = ([s for s in stages if s.name not in ("qmv_c2",)] + c2_parts + c3_parts + extra_parts
             + ceil_parts)
    graphs = {}
    for s in timed:
        s.run()  # eager pass: lazy initialisation outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s.run()
        graphs[s.name] = g
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        for s in timed:
            graphs[s.name].replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = {s.name: [] for s in timed}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for s in timed:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            graphs[s.name].replay()
            b.record(stream)
            ev[s.name].append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for s in timed:
        s.ms = [a.elapsed_time(b) for a, b in ev[s.name]]

    rows = {}
    for s in timed:
        ms = float(np.median(s.ms))
        r = {"ms": round(ms, 4), "calls": len(s.calls), "us_per_call": round(1000 * ms / len(s.calls), 3),
             "us_per_call_min": round(1000 * min(s.ms) / len(s.calls), 3),
             "us_per_call_max": round(1000 * max(s.ms) / len(s.calls), 3)}
        if s.bytes:
            r["GB/s"] = round(s.bytes / (ms * 1e-3) / 1e9, 1)
            r["frac_hbm"] = round(r["GB/s"] / HBM_PEAK_GBS, 4)
        if s.flops:
            r["TFLOP/s"] = round(s.flops / (ms * 1e-3) / 1e12, 2)
        if s.tokens:
            r["tokens/s"] = round(s.tokens / (ms * 1e-3), 1)
        if s.note:
            r["note"] = s.note
        rows[s.name] = r
    ceil = {}
    for p in ceil_parts:
        tag = "hbm_read_ceiling_" + p.name.split("_")[3]
        ceil[tag] = max(ceil.get(tag, 0.0), rows[p.name]["GB/s"])
    for tag, v in ceil.items():
        rows[tag] = {"GB/s": v, "frac_hbm": round(v / HBM_PEAK_GBS, 4),
                     "note": "best launch shape of the plain streaming read"}
    for name, r in rows.items():
        c = ceil.get("hbm_read_ceiling_33MB") if name.startswith("qmv_c2") else (
            ceil.get("hbm_read_ceiling_19.5MB") if name.startswith("tq1_c5_b1") else None)
        if c and "GB/s" in r:
            r["frac_read_ceiling"] = round(r["GB/s"] / c, 4)
    if c2_parts:
        ms = sum(float(np.median(p.ms)) for p in c2_parts)
        nbytes = sum(p.bytes for p in c2_parts)
        launches = sum(len(p.calls) for p in c2_parts)
        rows["qmv_c2"] = {"ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                          "bytes_per_launch": round(nbytes / launches),
                          "us_per_launch": round(1000 * ms / launches, 3),
                          "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if ceil.get("hbm_read_ceiling_33MB"):
            rows["qmv_c2"]["read_ceiling_GB/s"] = ceil["hbm_read_ceiling_33MB"]
            rows["qmv_c2"]["frac_read_ceiling"] = round(rows["qmv_c2"]["GB/s"] /
                                                        ceil["hbm_read_ceiling_33MB"], 4)
    if c3_parts:
        ms = sum(float(np.median(p.ms)) for p in c3_parts)
        fl = sum(p.flops for p in c3_parts)
        rows["qmm_c3"] = {"ms": round(ms, 4), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2),
                          "frac_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFS, 4)}
        for p in c3_parts:
            rows[p.name]["frac_bf16_peak"] = round(rows[p.name]["TFLOP/s"] / BF16_PEAK_TFS, 4)

    result = {
        "metric": METRIC,
        "value": rows.get("qmv_c2", {}).get("GB/s"),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1000 * wall / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "Q4_K decode GEMV 14336x4096 and 4096x14336, fp16 activations at "
                               "batch 1/4/8, fp16 output, weights rotated over >=1 GiB of copies",
                   "stages": wanted},
        "roofline": roofline(rows),
        "rows": rows,
    }
    if not args.no_cpu_baseline and "qmv_c2" in wanted:
        result["cpu_baseline"] = cpu_baseline()
        result["cpu_baseline_rows"] = cpu_baseline_rows()
    print(json.dumps(result))


# sources that define the decode GEMV kernels and their dispatch; the
# committed counter figures hold only while these are unchanged
GEMV_SOURCES = ("mmv2.hip", "mmv3.hip", "skinny.hip", "lds_dma.h", "q4k_mfma.h", "kq_device.h",
                "kq_internal.h")


def _kernel_sha():
    h = hashlib.sha256()
    src = os.path.join(ROOT, "block_quantized_weight_q4_amd", "csrc")
    for f in GEMV_SOURCES:
        h.update(open(os.path.join(src, f), "rb").read())
    return h.hexdigest()[:16]


def _traffic():
    """HBM bytes per dispatch of the GEMV (FETCH_SIZE + WRITE_SIZE, each scaled
    by its plain-copy calibration factor, averaged over the six launches) from
    the committed counter summary, when it was taken on the current kernel
    sources; else None."""
    path = os.path.join(PROFILE_DIR, "q4k_decode_gemv_counters.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("kernel_sha") != _kernel_sha():
        return None
    return d.get("hbm_bytes_per_dispatch")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline_rows():
    """The fp64 CPU oracle on a bounded sample of every other workload: whole
    calls where they take a few seconds at most, else a contiguous slice of
    the output rows (weight rows, or tokens for the MoE layer) timed and
    scaled linearly to the whole call."""
    import oracle
    from synth import workloads

    oracle.lib()
    threads, cpu = oracle.num_threads(), _cpu_model()
    out = {}

    def timed(fn, budget=1.5):
        if budget >= 1.0:
            fn()  # untimed run (the slices of the largest calls are timed once, cold)
        t0, n = time.perf_counter(), 0
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 >= budget:
                return (time.perf_counter() - t0) / n

    c = workloads.c1()
    t = timed(lambda: oracle.qmm("q4_k", c["w"], 2048, 2048, c["x"], "f32", 1))
    out["qmv_c1"] = {"us_per_call": round(t * 1e6, 1), "GB/s": round(c["w"].nbytes / t / 1e9, 3),
                     "sample": "whole Q4_K 2048x2048 GEMV, fp32 x"}
    t = timed(lambda: oracle.dequant_as("q4_k", c["w"], 2048, 2048, "f32"))
    out["dequant"] = {"us_per_call": round(t * 1e6, 1),
                      "GB/s": round((c["w"].nbytes + 2048 * 2048 * 4) / t / 1e9, 3),
                      "sample": "whole Q4_K 2048x2048 -> fp32"}

    cases, x = workloads.c3(("q4_k", 14336))
    w, n, k, m = cases[0]["w"], 14336, 4096, 2048
    ns = 717  # 5 % of the weight rows
    t = timed(lambda: oracle.qmm("q4_k", w[:ns], ns, k, x[:m], "bf16", m), budget=0.1)
    full = t * n / ns
    out["qmm_c3_q4_k_14336x4096_m2048"] = {
        "us_per_call": round(full * 1e6, 1), "TFLOP/s": round(2 * m * n * k / full / 1e12, 5),
        "sample": f"first {ns} of {n} weight rows (5 %), M=2048, timed once and scaled x{n / ns:.1f}"}

    c4 = workloads.c4()
    E, H, F, top_k = c4["n_experts"], c4["hidden"], c4["ffn"], c4["top_k"]

    def layer(t0, nt):
        return oracle.moe_layer("q4_k", c4["gate"], c4["up"], c4["down"], E, H, F,
                                c4["gate_stride"], c4["down_stride"], c4["x"][t0:t0 + nt], "f16",
                                c4["ids"][t0:t0 + nt], nt, top_k, c4["scores"][t0:t0 + nt])

    t = timed(lambda: layer(0, 1), budget=0.1)
    out["moe_c4_decode"] = {"us_per_call": round(t * 1e6, 1), "tokens/s": round(1 / t, 2),
                            "sample": "one token, whole layer (8 experts x 3 matrices)"}
    nt = 13  # 5 % of the 256 tokens
    t = timed(lambda: layer(0, nt), budget=0.1)
    full = t * 256 / nt
    out["moe_c4_prefill"] = {"us_per_call": round(full * 1e6, 1), "tokens/s": round(256 / full, 2),
                             "sample": f"first {nt} of 256 tokens (5 %), timed once and scaled "
                                       f"x{256 / nt:.1f}"}

    c5 = workloads.c5()[0]
    t = timed(lambda: oracle.qmm("tq1_g128", c5["w"], c5["n"], c5["k"], c5["x"][:1], "f16", 1))
    out["tq1_c5_b1"] = {"us_per_call": round(t * 1e6, 1), "GB/s": round(c5["w"].nbytes / t / 1e9, 3),
                        "sample": "whole TQ1 17408x5120 GEMV, fp16 x"}
    ns = 871  # 5 % of 17408
    rb = c5["w"].shape[1]
    t = timed(lambda: oracle.qmm("tq1_g128", c5["w"][:ns], ns, c5["k"], c5["x"], "f16", 512),
              budget=0.1)
    full = t * c5["n"] / ns
    out["tq1_c5_m512"] = {"us_per_call": round(full * 1e6, 1),
                          "TFLOP/s": round(2 * 512 * c5["n"] * c5["k"] / full / 1e12, 5),
                          "sample": f"first {ns} of {c5['n']} weight rows (5 %), M=512, scaled "
                                    f"x{c5['n'] / ns:.1f} (row bytes {rb})"}
    for r in out.values():
        r["cores"] = threads
        r["kind"] = "oracle"
        r["cpu"] = cpu
    return out


def roofline(rows):
    r = rows.get("qmv_c2")
    if not r:
        return None
    return {"bound": "hbm", "achieved": r["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(r["GB/s"] / HBM_PEAK_GBS, 4), "traffic": _traffic(),
            "read_ceiling": r.get("read_ceiling_GB/s"), "frac_read_ceiling": r.get("frac_read_ceiling"),
            "kernel": "kq_qmv Q4_K decode GEMV: mmv3_q4k_f16_kernel (batch 1), mmv3m_q4k_f16_kernel "
                      "(batch 4), mmv2_q4k_f16_kernel (batch 8)",
            "bytes_per_launch": r.get("bytes_per_launch"), "us_per_launch": r.get("us_per_launch")}


def cpu_baseline():
    """The fp64 CPU oracle on a bounded sample of the headline workload."""
    import oracle
    from synth import workloads

    oracle.lib()
    cases = workloads.c2()
    threads = oracle.num_threads()
    t_total, nbytes, calls, passes = 0.0, 0, 0, 0
    # whole passes over the six calls until about 10 s of CPU work
    while t_total < 10.0 and passes < 50:
        for case in cases:
            for b in (1, 4, 8):
                t0 = time.perf_counter()
                oracle.qmm("q4_k", case["w"], case["n"], case["k"], case["x"][:b], "f16", b)
                t_total += time.perf_counter() - t0
                nbytes += case["w"].nbytes
                calls += 1
        passes += 1
    cpu = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(nbytes / t_total / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{passes} passes over the 6 Q4_K GEMV calls (14336x4096 and 4096x14336 "
                      f"at batch 1/4/8), {calls} calls, fp64 accumulation, {t_total:.1f} s, "
                      f"{threads} threads on {cpu}"}


if __name__ == "__main__":
    main()
