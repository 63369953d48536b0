#!/usr/bin/env python3
"""Benchmark of the NVFP4 quantize -> GEMM hot path on one MI355X.

One step is one training pass of a 12B-style MLP up-projection linear layer
(tokens M = 8192, in K = 5120, out N = 20480) through the whole path, as the
recipe on the pages prescribes ("Pretraining Large Language Models with
NVFP4", Technische Zusammenfassung 2.B.2-2.B.4):

  quantise X   (M x K, 1x16, RNE)          quantise W (N x K, 16x16, RNE, + W^T copy)
  fprop  Y  = X^ W^T          (bf16 out)
  quantise dY  (M x N, 1x16, SR)
  dgrad  dX = dY^ W^          (bf16 out)
  RHT-quantise dY^T (SR), X^T (RNE)        one random sign vector for both
  wgrad  dW = RHT(dY)^T^ RHT(X)^T^ T       (fp32 out)

Inputs are synthetic and seeded (quantize_precision_gemm_amd.workloads):
X Student-t(4) at unit variance, W ~ N(0, 0.02), dY with log-normal row
magnitudes.  They are resident in HBM before timing starts.

value = 3 * 2*M*N*K / (wall time of one step), in TFLOP/s, quantisation
included; dgrad and wgrad run concurrently on two streams.  Per-operation
times come from separate serialised passes with HIP events on the stream
the library launches on.  The roofline entry is for the dominant kernel, the
bf16-output GEMM (fprop and dgrad launches).  The CPU baseline is the
oracle run on a token slice of the same step.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, K, N = 8192, 5120, 20480
SEED = 0
PEAK_F16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E


def gemm_source_hash():
    h = hashlib.sha256()
    for f in ["gemm.hip", "nvfp4_device.hpp"]:
        with open(os.path.join(ROOT, "quantize_precision_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(avg_launch_ms):
    """HBM bytes per launch of the bf16 GEMM from the committed rocprofv3 PMC
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "gemm_nt_bf16_12b_layer_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source hash: (\w+)", text)
    t = re.search(r"scaled HBM bytes per launch: ([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != gemm_source_hash():
        return None
    return float(t.group(1))


def make_inputs(dev):
    import numpy as np
    import torch
    from quantize_precision_gemm_amd import workloads as wl

    t0 = time.time()
    data = wl.layer_inputs(wl.LAYER_12B, seed=SEED)
    to_dev = lambda u: torch.from_numpy(u.view(np.int16)).to(dev).view(torch.bfloat16)
    out = {k: to_dev(v) for k, v in data.items()}
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    return data, out


class Step:
    """Buffers and launch sequence of one step (no allocation inside run()).

    dgrad and wgrad only depend on the quantised dY, W and X, so wgrad's
    operands are quantised and its GEMM runs on a second stream, concurrently
    with dgrad: each GEMM's last, partial wave of workgroups is filled by the
    other's (dgrad is 2.5 and wgrad 6.25 waves of 256 tiles on 256 CUs).
    """

    def __init__(self, q, torch, dev, x, w, dy):
        self.q, self.torch = q, torch
        self.x, self.w, self.dy = x, w, dy
        self.gx = q.alloc_nvfp4(M, K, q.BLOCK_1X16)
        self.gw = q.alloc_nvfp4(N, K, q.BLOCK_16X16, with_transpose=True)
        self.gdy = q.alloc_nvfp4(M, N, q.BLOCK_1X16)
        self.gdyt = q.alloc_nvfp4(N, M, q.BLOCK_1X16)
        self.gxt = q.alloc_nvfp4(K, M, q.BLOCK_1X16)
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        self.dw = torch.empty((N, K), dtype=torch.float32, device=dev)
        self.mask = q.nvfp4_rht_sign_mask(SEED + 1000)
        f32 = lambda: torch.empty(1, dtype=torch.float32, device=dev)
        self.ax, self.ax_rht, self.ady, self.ady_rht = f32(), f32(), f32(), f32()
        self.side = torch.cuda.Stream(device=dev)  # default priority
        self.ops = ["amax_X", "quant_X", "quant_W", "fprop", "amax_dY", "quant_dY", "dgrad",
                    "rht_dY", "rht_X", "wgrad"]

    def calls(self):
        q = self.q
        # X and dY are each quantised twice (1x16, and through the RHT for
        # wgrad): one fused pass computes both tensor maxima of each.
        return [
            lambda: q.nvfp4_amax(self.x, self.mask, self.ax, self.ax_rht),
            lambda: q.nvfp4_quantize(self.x, q.BLOCK_1X16, q.RNE, amax_in=self.ax, out=self.gx),
            lambda: q.nvfp4_quantize(self.w, q.BLOCK_16X16, q.RNE, out=self.gw),
            lambda: q.nvfp4_gemm(q.FPROP, self.gx, self.gw, out=self.y),
            lambda: q.nvfp4_amax(self.dy, self.mask, self.ady, self.ady_rht),
            lambda: q.nvfp4_quantize(self.dy, q.BLOCK_1X16, q.SR, SEED + 100, amax_in=self.ady,
                                     out=self.gdy),
            lambda: q.nvfp4_gemm(q.DGRAD, self.gdy, self.gw, out=self.dx),
            lambda: q.nvfp4_rht_quantize(self.dy, self.mask, q.SR, SEED + 101,
                                         amax_in=self.ady_rht, out=self.gdyt),
            lambda: q.nvfp4_rht_quantize(self.x, self.mask, q.RNE, amax_in=self.ax_rht,
                                         out=self.gxt),
            lambda: q.nvfp4_gemm(q.WGRAD, self.gdyt, self.gxt, out=self.dw),
        ]

    def run(self):
        """One step: wgrad's branch on the side stream, joined at the end."""
        torch = self.torch
        c = self.calls()
        main = torch.cuda.current_stream()
        for f in c[:6]:          # quantise X, W; fprop; amax and 1x16 SR of dY
            f()
        self.side.wait_stream(main)
        c[6]()                   # dgrad on the main stream
        with torch.cuda.stream(self.side):
            c[7](); c[8](); c[9]()   # RHT operands and wgrad on the side stream
        main.wait_stream(self.side)

    def run_timed_ops(self):
        """One step, serialised on one stream, with an event around every
        operation (for per-operation times; events add small gaps)."""
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(self.ops) + 1)]
        ev[0].record()
        for i, f in enumerate(self.calls()):
            f()
            ev[i + 1].record()
        return ev


def quant_bytes():
    """Algorithmic HBM bytes of each quantisation operation: the fused amax
    passes read their tensor once; the encode passes read it and write codes
    and scales; W is quantised with its own amax pass and a transposed copy."""
    e_x, e_w, e_dy = M * K, N * K, M * N
    enc = lambda e: 2 * e + e // 2 + e // 16                  # read bf16, write codes, scales
    return {"amax_X": 2 * e_x, "quant_X": enc(e_x),
            "quant_W": 2 * e_w + 2 * e_w + 2 * (e_w // 2 + e_w // 256),
            "amax_dY": 2 * e_dy, "quant_dY": enc(e_dy), "rht_dY": enc(e_dy), "rht_X": enc(e_x)}


def cpu_baseline(data, tokens=M):
    """The oracle on a token slice of the step; W's quantisation, which does not
    scale with tokens, is timed in full and counted at tokens/M of its time."""
    import numpy as np
    import oracle

    x, w, dy = data["X"][:tokens], data["W"], data["dY"][:tokens]
    mask = oracle.rht_sign_mask(SEED + 1000)
    t0 = time.perf_counter()
    qw = oracle.quantize(w, oracle.BLOCK_16X16, oracle.RNE)
    t_w = time.perf_counter() - t0
    t0 = time.perf_counter()
    qx = oracle.quantize(x, oracle.BLOCK_1X16, oracle.RNE)
    oracle.gemm(oracle.FPROP, qx, qw)
    qdy = oracle.quantize(dy, oracle.BLOCK_1X16, oracle.SR, SEED + 100)
    oracle.gemm(oracle.DGRAD, qdy, qw)
    qdyt = oracle.rht_quantize(dy, mask, oracle.SR, SEED + 101)
    qxt = oracle.rht_quantize(x, mask, oracle.RNE)
    oracle.gemm(oracle.WGRAD, qdyt, qxt)
    t_tok = time.perf_counter() - t0
    t = t_tok + t_w * tokens / M
    flops = 3 * 2.0 * tokens * N * K
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{tokens} of {M} tokens through the whole step (all quantisations and "
                      f"the three GEMMs, fp64 numpy GEMM over dequantised operands); W "
                      f"quantised in full ({t_w:.2f} s) and counted at {tokens}/{M}; "
                      f"measured {t_tok + t_w:.2f} s",
            "seconds": t}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the layer shards by tokens; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import quantize_precision_gemm_amd as q

    q.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    data, t = make_inputs(dev)
    step = Step(q, torch, dev, t["X"], t["W"], t["dY"])

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # timed steps: nothing but the step itself between the two synchronisations
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-operation times: separate, serialised passes with events
    per_op = {k: [] for k in step.ops}
    evs = [step.run_timed_ops() for _ in range(max(5, args.steps // 2))]
    torch.cuda.synchronize()
    for ev in evs:
        for i, k in enumerate(step.ops):
            per_op[k].append(ev[i].elapsed_time(ev[i + 1]))

    ms_step = wall * 1e3 / args.steps
    gemm_flop = 2.0 * M * N * K
    avg = {k: sum(v) / len(v) for k, v in per_op.items()}
    qb = quant_bytes()
    bf16_launches = per_op["fprop"] + per_op["dgrad"]
    gemm_bf16_ms = sum(bf16_launches) / len(bf16_launches)
    achieved = gemm_flop / (gemm_bf16_ms * 1e-3) / 1e12

    result = {
        "metric": "NVFP4 GEMM TFLOP/s (fprop/dgrad/wgrad) + quantize GB/s, 12B-layer shapes",
        "value": round(3 * gemm_flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "12B-style MLP up-projection linear layer, one training step "
                               "(fprop + dgrad + wgrad, all NVFP4 quantisations included)",
                   "tokens_M": M, "in_K": K, "out_N": N, "operand_format": "nvfp4",
                   "mfma": "f16 32x32x16, fp32 accumulate", "parallelism": "none (1 GPU)"},
        "gemm_tflops": {p: round(gemm_flop / (avg[p] * 1e-3) / 1e12, 1)
                        for p in ("fprop", "dgrad", "wgrad")},
        "quantize_gbps": {k: round(qb[k] / (avg[k] * 1e-3) / 1e9, 1) for k in qb},
        "quantize_frac_of_hbm_peak": {k: round(qb[k] / (avg[k] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 3)
                                      for k in qb},
        "ms_per_op": {k: round(v, 4) for k, v in avg.items()},
        "roofline": {"kernel": "k_gemm_nt<bf16 out> (fprop, dgrad launches)", "bound": "mfma",
                     "achieved": round(achieved, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                     "avg_launch_ms": round(gemm_bf16_ms, 4),
                     "traffic": counter_traffic(gemm_bf16_ms)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a token slice", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(data)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
