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
included; W's quantisation and the wgrad operands' run on a second stream
beside the other work, dgrad and wgrad one after the other with their last
partial wave of tiles split along K (nvfp4_gemm_split).  Per-operation
times come from separate serialised passes with HIP events on the stream
the library launches on.  The roofline entry is for the dominant kernel, the
NVFP4 GEMM k_gemm_nv (its fprop launches), beside the throughput the matrix
instruction alone sustains.  The CPU baseline is the oracle run on a token
slice of the same step.

--workload mlp times the 4-block MLP training step instead (tokens 16384,
hidden 5120, FFN 20480; 8 linear layers, the last block's two in bf16; all
fprops, then the backward pass in reverse layer order), value = its 24
GEMMs' FLOPs / step time.  It is a separate line, not the default.
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
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense fp4/fp6 MFMA


def gemm_source_hash():
    """Hash of the GEMM kernels' code (comments and blank lines removed, so
    that a comment edit does not invalidate the committed counter summary)."""
    h = hashlib.sha256()
    for f in ["gemm.hip", "nvfp4_device.hpp"]:
        with open(os.path.join(ROOT, "quantize_precision_gemm_amd", "csrc", f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per fprop launch of the bf16-output GEMM from the committed
    rocprofv3 PMC summary, if it was taken on the current kernel source;
    else None."""
    path = os.path.join(ROOT, "profiles", "gemm_nv_bf16_12b_layer_pmc.md")
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


def quant_bytes():
    """Algorithmic HBM bytes of each quantisation operation: the fused amax
    passes read their tensor once; the encode passes read it and write codes
    and scales (the dual passes both operands' codes and scales); W is
    quantised with its own amax pass and a transposed copy."""
    e_x, e_w, e_dy = M * K, N * K, M * N
    enc = lambda e: 2 * e + e // 2 + e // 16                  # read bf16, write codes, scales
    enc2 = lambda e: 2 * e + 2 * (e // 2 + e // 16)          # one read, both operands written
    return {"amax_X": 2 * e_x, "quant_X": enc(e_x),
            "quant_W": 2 * e_w + 2 * e_w + 2 * (e_w // 2 + e_w // 256),
            "amax_dY": 2 * e_dy, "quant_dY": enc(e_dy), "rht_dY": enc(e_dy), "rht_X": enc(e_x),
            "dual_dY": enc2(e_dy), "dual_X": enc2(e_x)}


def mx_comparison(q, torch, layer, reps=5):
    """The layer's three GEMMs in the comparison format MXFP4 (32-element
    blocks, UE8M0 scales) on the native block-scaled FP4 MFMA, on the same
    bf16 tensors: each operand quantised in the layout its pass contracts
    over, then every GEMM and quantiser timed serialised with events."""
    m = layer.mask
    # name: (tensor, layout, sign mask, rounding, seed)
    quants = {
        "X rows (fprop)": (layer.x, q.MX_ROWS, 0, q.RNE, 0),
        "W rows (fprop)": (layer.w, q.MX_ROWS, 0, q.RNE, 0),
        "W cols (dgrad)": (layer.w, q.MX_COLS, 0, q.RNE, 0),
        "dY rows SR (dgrad)": (layer.dy, q.MX_ROWS, 0, q.SR, 100),
        "dY cols RHT SR (wgrad)": (layer.dy, q.MX_COLS_RHT, m, q.SR, 101),
        "X cols RHT (wgrad)": (layer.x, q.MX_COLS_RHT, m, q.RNE, 0),
    }
    ops = {k: q.nvfp4_mx_quantize(*a) for k, a in quants.items()}
    gemms = {
        "fprop": (ops["X rows (fprop)"], ops["W rows (fprop)"], torch.bfloat16),
        "dgrad": (ops["dY rows SR (dgrad)"], ops["W cols (dgrad)"], torch.bfloat16),
        "wgrad": (ops["dY cols RHT SR (wgrad)"], ops["X cols RHT (wgrad)"], torch.float32),
    }
    outs = {k: q.nvfp4_mx_gemm(a, b, dt) for k, (a, b, dt) in gemms.items()}
    torch.cuda.synchronize()

    def timed(f):
        f()
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record()
        for _ in range(reps):
            f()
        e_.record()
        torch.cuda.synchronize()
        return s_.elapsed_time(e_) / reps

    flop = 2.0 * layer.M * layer.N * layer.K
    gemm_ms = {k: timed(lambda a=a, b=b, o=outs[k]: q.nvfp4_mx_gemm(a, b, out=o))
               for k, (a, b, _) in gemms.items()}
    quant_ms = {k: timed(lambda a=a, o=ops[k]: q.nvfp4_mx_quantize(*a, out=o))
                for k, a in quants.items()}
    tf = {k: flop / (v * 1e-3) / 1e12 for k, v in gemm_ms.items()}
    return {"gemm_tflops": {k: round(v, 1) for k, v in tf.items()},
            "gemm_ms": {k: round(v, 4) for k, v in gemm_ms.items()},
            "frac_of_fp4_peak": {k: round(v / PEAK_FP4_TFLOPS, 4) for k, v in tf.items()},
            "quantize_ms": {k: round(v, 4) for k, v in quant_ms.items()},
            "kernel": "k_gemm_mx (v_mfma_scale_f32_32x32x64_f8f6f4, fp4 operands)",
            "peak_tflops": PEAK_FP4_TFLOPS}


def epilogue_amax_comparison(q, torch, layer, reps=5, rounds=5):
    """Quantise-in-epilogue: the fprop output Y (the next layer's X) and the
    dgrad output dX (the previous layer's dY) are quantised into both of
    their operands by the dual quantiser.  Separate: GEMM, then the dual
    quantiser with its own read for the two maxima.  Fused: the GEMM
    epilogue emits the maxima (nvfp4_gemm_amax) and the dual quantiser takes
    them.  Each op and each pair is timed serialised with events on the
    layer's operands (reps launches per timing, the variants alternating,
    median of `rounds`); both schedules must give identical operands."""
    dev = layer.y.device
    f32 = lambda: torch.empty(1, dtype=torch.float32, device=dev)

    def timed(f):
        f()
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record()
        for _ in range(reps):
            f()
        e_.record()
        torch.cuda.synchronize()
        return s_.elapsed_time(e_) / reps

    out, same = {}, True
    for name, P, a, out_t, rnd in (("fprop (Y, next X: RNE)", q.FPROP, layer.gx, layer.y, q.RNE),
                                   ("dgrad (dX, previous dY: SR)", q.DGRAD, layer.gdy, layer.dx, q.SR)):
        rows, cols = out_t.shape
        ops = [q.alloc_nvfp4(rows, cols, q.BLOCK_1X16, device=dev, layout=layer.layout)
               for _ in range(2)]
        opsr = [q.alloc_nvfp4(cols, rows, q.BLOCK_1X16, device=dev, layout=layer.layout)
                for _ in range(2)]
        am, ar = f32(), f32()
        gemm = lambda: q.nvfp4_gemm(P, a, layer.gw, out=out_t)
        gemm_amax = lambda: q.nvfp4_gemm_amax(P, a, layer.gw, layer.mask, out=out_t, amax=am,
                                              amax_rht=ar)
        dual = lambda: q.nvfp4_quantize_dual(out_t, layer.mask, rnd, 11, 12, out=ops[0],
                                             out_rht=opsr[0])
        dual_in = lambda: q.nvfp4_quantize_dual(out_t, layer.mask, rnd, 11, 12, amax_in=am,
                                                amax_rht_in=ar, out=ops[1], out_rht=opsr[1])
        fns = {"gemm_ms": gemm, "gemm_amax_ms": gemm_amax, "dual_quant_own_amax_ms": dual,
               "dual_quant_given_amax_ms": dual_in,
               "separate_pair_ms": lambda: (gemm(), dual()),
               "fused_pair_ms": lambda: (gemm_amax(), dual_in())}
        runs = {k: [] for k in fns}
        for _ in range(rounds):  # alternate the variants; median of the rounds
            for k, f in fns.items():
                runs[k].append(timed(f))
        t = {k: sorted(v)[len(v) // 2] for k, v in runs.items()}
        t["saving_ms"] = t["separate_pair_ms"] - t["fused_pair_ms"]
        gemm(), dual(), gemm_amax(), dual_in()
        torch.cuda.synchronize()
        for u, v in ((ops[0], ops[1]), (opsr[0], opsr[1])):
            same = same and torch.equal(u.codes, v.codes) and torch.equal(u.scales, v.scales) \
                and u.s_enc.item() == v.s_enc.item()
        out[name] = {k: round(v, 4) for k, v in t.items()}
    out["identical_operands"] = bool(same)
    out["kernel"] = "k_gemm_nv<bf16 out, epilogue maxima> + k_dual_quant (amax given)"
    return out


def rht_size_study(q, torch, dev, reps=3, rows=40):
    """RHT ablations (Technische Zusammenfassung 2.B.2: 16 x 16 was the best
    size, and the transform brought no significant benefit on fprop and
    dgrad): for transforms of 1 (none), 4, 16 and 64 tokens, the 12B-layer
    wgrad dW = dY^T X with both operands quantised through the transform (dY
    SR, X RNE, one sign vector), its relative Frobenius error on sampled
    output rows against the exact product of the bf16 inputs and the
    quantiser times; then fprop and dgrad with and without the transform
    along their contraction dimension."""
    import numpy as np
    from quantize_precision_gemm_amd import workloads as wl

    out = {}
    settings = {
        "layer inputs (dY log-normal rows, X Student-t(4))": None,
        "outliers (dY and X normal with 0.1 % of entries x 50)": "outliers",
    }
    for name, kind in settings.items():
        if kind is None:
            data = wl.layer_inputs(wl.LAYER_12B, seed=SEED, with_w=False)
        else:
            rng = np.random.default_rng(SEED + 7)
            data = {"X": wl.normal_with_outliers(rng, (M, K)),
                    "dY": wl.normal_with_outliers(rng, (M, N))}
        to_dev = lambda u: torch.from_numpy(u.view(np.int16)).to(dev).view(torch.bfloat16)
        x, dy = to_dev(data["X"]), to_dev(data["dY"])
        pick = np.sort(np.random.default_rng(SEED + 3).choice(N, rows, replace=False))
        xf = wl.bf16_bits_to_f32(data["X"]).astype(np.float64)
        exact = wl.bf16_bits_to_f32(np.ascontiguousarray(data["dY"][:, pick])).astype(np.float64).T @ xf
        signs = q.nvfp4_rht_signs64(SEED + 1000)
        res = {}
        for size in (1, 4, 16, 64):
            gdyt = q.nvfp4_rht_quantize_sized(dy, size, signs, q.SR, SEED + 101)
            gxt = q.nvfp4_rht_quantize_sized(x, size, signs, q.RNE)
            dw = q.nvfp4_gemm(q.WGRAD, gdyt, gxt, out_dtype=torch.float32)
            torch.cuda.synchronize()
            got = dw[torch.from_numpy(pick).to(dev)].double().cpu().numpy()
            err = float(np.linalg.norm(got - exact) / np.linalg.norm(exact))

            def timed(f):
                f()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(reps):
                    f()
                b.record()
                torch.cuda.synchronize()
                return a.elapsed_time(b) / reps
            t_dy = timed(lambda: q.nvfp4_rht_quantize_sized(dy, size, signs, q.SR, SEED + 101, out=gdyt))
            t_x = timed(lambda: q.nvfp4_rht_quantize_sized(x, size, signs, q.RNE, out=gxt))
            res[str(size)] = {"wgrad_rel_fro_err": err, "quant_dY_ms": round(t_dy, 4),
                              "quant_X_ms": round(t_x, 4)}
        out[name] = res
        del x, dy
    # RHT on fprop and dgrad: the 16-point transform along the contraction
    # dimension of both operands (X, W along K; dY, W^T along N) against
    # the recipe's untransformed operands, on the layer inputs
    data = wl.layer_inputs(wl.LAYER_12B, seed=SEED)
    to_dev = lambda u: torch.from_numpy(u.view(np.int16)).to(dev).view(torch.bfloat16)
    x, w, dy = to_dev(data["X"]), to_dev(data["W"]), to_dev(data["dY"])
    wt = w.t().contiguous()          # W^T (K x N): its rows run along N
    pick = np.sort(np.random.default_rng(SEED + 5).choice(M, rows, replace=False))
    pt = torch.from_numpy(pick).to(dev)
    xf = wl.bf16_bits_to_f32(data["X"][pick]).astype(np.float64)
    wf = wl.bf16_bits_to_f32(data["W"]).astype(np.float64)
    dyf = wl.bf16_bits_to_f32(data["dY"][pick]).astype(np.float64)
    exact_y, exact_dx = xf @ wf.T, dyf @ wf
    mask = q.nvfp4_rht_sign_mask(SEED + 1000)
    err = lambda got, ref: float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    gx = q.nvfp4_quantize(x, q.BLOCK_1X16, q.RNE)
    gw = q.nvfp4_quantize(w, q.BLOCK_16X16, q.RNE, with_transpose=True)
    gdy = q.nvfp4_quantize(dy, q.BLOCK_1X16, q.SR, SEED + 100)
    y0 = q.nvfp4_gemm(q.FPROP, gx, gw, out_dtype=torch.float32)[pt].double().cpu().numpy()
    dx0 = q.nvfp4_gemm(q.DGRAD, gdy, gw, out_dtype=torch.float32)[pt].double().cpu().numpy()
    hx = q.nvfp4_quantize_rht_rows(x, mask, q.BLOCK_1X16, q.RNE)
    hw = q.nvfp4_quantize_rht_rows(w, mask, q.BLOCK_16X16, q.RNE)
    hdy = q.nvfp4_quantize_rht_rows(dy, mask, q.BLOCK_1X16, q.SR, SEED + 100)
    hwt = q.nvfp4_quantize_rht_rows(wt, mask, q.BLOCK_16X16, q.RNE)
    y1 = q.nvfp4_gemm(q.FPROP, hx, hw, out_dtype=torch.float32)[pt].double().cpu().numpy()
    dx1 = q.nvfp4_gemm(q.FPROP, hdy, hwt, out_dtype=torch.float32)[pt].double().cpu().numpy()
    torch.cuda.synchronize()
    fd = {"fprop": {"no transform (recipe)": err(y0, exact_y), "RHT along K": err(y1, exact_y)},
          "dgrad": {"no transform (recipe)": err(dx0, exact_dx), "RHT along N": err(dx1, exact_dx)}}
    return {"study": "wgrad RHT size (1 = no transform); RHT on fprop / dgrad",
            "workload": f"12B layer: M={M}, N={N}, K={K}; relative Frobenius error on {rows} "
                        f"sampled output rows against the exact product of the bf16 inputs",
            "results": out, "fprop_dgrad_rht": fd}


def quantize_cold(q, torch, layer, reps=20):
    """Each quantisation pass of the layer timed cold: before every rep a
    1 GiB buffer is written (more than the 256 MB Infinity Cache and the L2s
    hold), so the pass reads its tensor from HBM.  Events bracket the single
    launch sequence of the pass on the current stream; median over `reps`.

    kernel_gbps: algorithmic bytes of the pass / its time.
    op_gbps: the whole quantisation (its amax pass plus its encode pass, both
    cold) -- 2 B/element for the amax read plus the encode pass's bytes --
    over the sum of the two times; the headline against the 70 % target.
    W is reported with the transposed copy the dgrad GEMM reads (the bytes
    this library moves) and on the plain 16x16 quantisation's bytes (one
    read for the amax, one read, codes and scales written once)."""
    dev = layer.x.device
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    aw = torch.empty(1, dtype=torch.float32, device=dev)
    e_x, e_w, e_dy = layer.M * layer.K, layer.N * layer.K, layer.M * layer.N
    dy_rne = q.alloc_nvfp4(layer.M, layer.N, q.BLOCK_1X16, device=dev, layout=layer.layout)
    enc = lambda e: 2 * e + e // 2 + e // 16
    passes = {
        "amax_X (plain + RHT maxima)": (lambda: q.nvfp4_amax(layer.x, layer.mask, layer.ax, layer.ax_rht), 2 * e_x),
        "quant_X (1x16 RNE)": (lambda: q.nvfp4_quantize(layer.x, q.BLOCK_1X16, q.RNE, amax_in=layer.ax,
                                                        out=layer.gx), enc(e_x)),
        "rht_X (RHT 1x16 RNE)": (lambda: q.nvfp4_rht_quantize(layer.x, layer.mask, q.RNE,
                                                             amax_in=layer.ax_rht, out=layer.gxt), enc(e_x)),
        "amax_W": (lambda: q.nvfp4_amax(layer.w, None, aw), 2 * e_w),
        "quant_W (16x16 RNE + transposed copy)": (
            lambda: q.nvfp4_quantize(layer.w, q.BLOCK_16X16, q.RNE, amax_in=aw, out=layer.gw),
            2 * e_w + 2 * (e_w // 2 + e_w // 256)),
        "amax_dY (plain + RHT maxima)": (lambda: q.nvfp4_amax(layer.dy, layer.mask, layer.ady, layer.ady_rht), 2 * e_dy),
        "quant_dY (1x16 SR)": (lambda: q.nvfp4_quantize(layer.dy, q.BLOCK_1X16, q.SR, layer.seed + 100,
                                                        amax_in=layer.ady, out=layer.gdy), enc(e_dy)),
        "rht_dY (RHT 1x16 SR)": (lambda: q.nvfp4_rht_quantize(layer.dy, layer.mask, q.SR, layer.seed + 101,
                                                             amax_in=layer.ady_rht, out=layer.gdyt), enc(e_dy)),
        # not a pass of the step: the 1x16 RNE encoder on the largest tensor
        # (336 MB), where its launch and drain weigh less than on X (84 MB)
        "quant_dY_rne (1x16 RNE on dY, encoder characterisation)": (
            lambda: q.nvfp4_quantize(layer.dy, q.BLOCK_1X16, q.RNE, amax_in=layer.ady, out=dy_rne), enc(e_dy)),
    }
    times = {k: [] for k in passes}
    for _ in range(reps):
        for k, (f, _) in passes.items():
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            times[k].append((a, b))
    torch.cuda.synchronize()
    med = {k: sorted(x.elapsed_time(y) for x, y in v)[len(v) // 2] for k, v in times.items()}
    del flush
    kern = {k: {"ms": round(med[k], 4), "gbps": round(passes[k][1] / (med[k] * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(passes[k][1] / (med[k] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 3)}
            for k in passes}
    ops = {  # op: (amax pass, encode pass, bytes of the whole op)
        "X 1x16 RNE": ("amax_X (plain + RHT maxima)", "quant_X (1x16 RNE)", 2 * e_x + enc(e_x)),
        "X RHT 1x16 RNE (wgrad)": ("amax_X (plain + RHT maxima)", "rht_X (RHT 1x16 RNE)", 2 * e_x + enc(e_x)),
        "W 16x16 RNE + transposed copy": ("amax_W", "quant_W (16x16 RNE + transposed copy)",
                                          2 * e_w + passes["quant_W (16x16 RNE + transposed copy)"][1]),
        "W 16x16 RNE (bytes without the copy)": ("amax_W", "quant_W (16x16 RNE + transposed copy)",
                                                 2 * e_w + 2 * e_w + e_w // 2 + e_w // 256),
        "dY 1x16 SR": ("amax_dY (plain + RHT maxima)", "quant_dY (1x16 SR)", 2 * e_dy + enc(e_dy)),
        "dY RHT 1x16 SR (wgrad)": ("amax_dY (plain + RHT maxima)", "rht_dY (RHT 1x16 SR)", 2 * e_dy + enc(e_dy)),
    }
    op = {}
    for k, (pa, pe, nbytes) in ops.items():
        t = med[pa] + med[pe]
        gbps = nbytes / (t * 1e-3) / 1e9
        op[k] = {"ms": round(t, 4), "gbps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 3)}
    return {"method": f"cold: 1 GiB written before every rep; median of {reps} reps; events around "
                      "each pass's launches", "kernel": kern, "op": op}


def small_fprop_latency(q, torch, dev, reps=50):
    """The 256 x 256 x 256 fprop (X N(0,1) with 0.1 % outliers x 50, W N(0,
    0.02), seed 0): latency of each call and of the whole path (quantise X,
    quantise W with its transposed copy, GEMM), median over `reps`.  Too small
    for a roofline (33.5 MFLOP)."""
    import numpy as np
    from quantize_precision_gemm_amd import workloads as wl
    X, W = wl.small_fprop(seed=0)
    to_dev = lambda u: torch.from_numpy(u.view(np.int16)).to(dev).view(torch.bfloat16)
    x, w = to_dev(X), to_dev(W)
    gx = q.alloc_nvfp4(256, 256, q.BLOCK_1X16, device=dev, layout=q.LAYOUT_INTERLEAVED)
    gw = q.alloc_nvfp4(256, 256, q.BLOCK_16X16, with_transpose=True, device=dev,
                       layout=q.LAYOUT_INTERLEAVED)
    y = torch.empty((256, 256), dtype=torch.bfloat16, device=dev)
    steps = {"quant_X": lambda: q.nvfp4_quantize(x, q.BLOCK_1X16, q.RNE, out=gx),
             "quant_W": lambda: q.nvfp4_quantize(w, q.BLOCK_16X16, q.RNE, out=gw),
             "fprop": lambda: q.nvfp4_gemm(q.FPROP, gx, gw, out=y)}
    steps["whole path"] = lambda: [f() for f in list(steps.values())[:3]]
    for f in steps.values():
        f()
    torch.cuda.synchronize()
    out = {}
    for k, f in steps.items():
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        out[k] = round(sorted(a.elapsed_time(b) for a, b in ts)[reps // 2] * 1e3, 1)
    return {"workload": "fprop 256 x 256 x 256 (X 1x16 RNE, W 16x16 RNE, bf16 out), seed 0",
            "latency_us": out, "note": "median of %d event-timed calls each" % reps}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def mfma_sustained(q, torch, dev, blocks=1024, iters=16000, reps=3):
    """Matrix throughput the GPU sustains on register-resident operands
    (nvfp4_mfma_sustain: a GEMM's matrix instruction with nothing else in the
    loop): the fp16 instruction of nvfp4_gemm on decoded-NVFP4-like and on
    random fp16 operands, and the block-scaled FP4 instruction of
    nvfp4_mx_gemm.  Launches of ~0.15 s, one untimed first, so the clock has
    settled where the power limit holds it: the ceiling the published peak
    does not show."""
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    res = {}
    for name, ops, it in (("decoded_nvfp4_operands", q.MFMA_SUSTAIN_DECODED, iters),
                          ("random_fp16_operands", q.MFMA_SUSTAIN_RANDOM, iters),
                          ("fp4_block_scaled_e2m1", q.MFMA_SUSTAIN_FP4, iters)):
        _, flops = q.nvfp4_mfma_sustain(blocks, it, ops, out=out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            q.nvfp4_mfma_sustain(blocks, it, ops, out=out)
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(flops / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12, 1)
    return res


def copy_gbps(torch, dev, reps=5):
    """Device copy of 1 GiB of bf16 (read + write bytes / time), the measured
    stream rate the quantisers are also reported against."""
    n = 1 << 29
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_.record()
    for _ in range(reps):
        dst.copy_(src)
    e_.record()
    torch.cuda.synchronize()
    ms = s_.elapsed_time(e_) / reps
    del src, dst
    return 2.0 * 2 * n / (ms * 1e-3) / 1e9


def device_info(torch, dev):
    """Name, architecture, compute units and the current shader-clock DPM
    level (from sysfs, if readable) of the GPU the bench ran on."""
    p = torch.cuda.get_device_properties(dev)
    sclk = None
    try:
        import glob
        for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            lines = [l.strip() for l in open(f) if "*" in l]
            if lines:
                sclk = lines[0]
                break
    except OSError:
        sclk = None
    return {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
            "sclk_dpm_level": sclk}


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
            "cpu_model": cpu_model(),
            "sample": f"{tokens} of {M} tokens through the whole step (all quantisations and "
                      f"the three GEMMs, fp64 numpy GEMM over dequantised operands); W "
                      f"quantised in full ({t_w:.2f} s) and counted at {tokens}/{M}; "
                      f"measured {t_tok + t_w:.2f} s",
            "seconds": t}


# Backward schedule of each workload's headline step: (split_tail,
# serial_gemms).  Both run dgrad and then wgrad on the main stream through
# nvfp4_gemm_split (each GEMM fills its own last, partial wave of tiles),
# with only the wgrad operands' quantisation on the second stream beside
# dgrad.  On the layer step that measured 2 % faster than dgrad and the
# wgrad branch concurrently through nvfp4_gemm (4.327 against 4.414 ms, one
# run); on the 8-layer MLP step 2-3 % faster.  Every bench line times the
# other schedules beside it.
HEADLINE_SCHEDULE = {"layer": (True, True), "mlp": (True, True)}


def schedule_name(fused_quant, split_tail, serial_gemms, rht_x_forward=False, row_major=False):
    return ("dual quantisers (nvfp4_quantize_dual)" if fused_quant else "separate quantisers") + \
        (", RHT(X) encoded before fprop" if rht_x_forward and not fused_quant else "") + \
        (", dgrad then wgrad on one stream" if serial_gemms else ", dgrad || wgrad branch") + \
        (", tail split (nvfp4_gemm_split)" if split_tail else "") + \
        (", row-major codes" if row_major else "")


def build_layer_step(q, torch, dev, fused_quant=False, split_tail=False, serial_gemms=False):
    """The 12B-layer step: one NVFP4 linear layer, numpy-drawn inputs."""
    from quantize_precision_gemm_amd.step import NVFP4Linear, TrainingStep
    data, t = make_inputs(dev)
    layer = NVFP4Linear(q, torch, t["X"], t["W"], t["dY"], SEED, fused_quant, split_tail)
    return data, TrainingStep(torch, [layer], dev, serial_gemms)


def as_mxfp4(q, torch, dev, step):
    """The same step over the same tensors with every NVFP4 layer in MXFP4."""
    from quantize_precision_gemm_amd.step import MXFP4Linear, NVFP4Linear, TrainingStep
    layers = [MXFP4Linear(q, torch, l.x, l.w, l.dy, l.seed) if isinstance(l, NVFP4Linear) else l
              for l in step.layers]
    return TrainingStep(torch, layers, dev)


def with_schedule(q, torch, dev, step, fused_quant, split_tail=False, serial_gemms=False,
                  rht_x_forward=False, layout=None):
    """The same step over the same tensors, with the NVFP4 layers' quantisers
    fused (nvfp4_quantize_dual) or separate, dgrad / wgrad through
    nvfp4_gemm_split (split_tail) or nvfp4_gemm, the two backward GEMMs
    concurrent on two streams or one after the other (serial_gemms), X's
    RHT operand encoded in the forward part or in the wgrad branch, and the
    codes in the given layout (default: the layers' own, interleaved)."""
    from quantize_precision_gemm_amd.step import NVFP4Linear, TrainingStep
    layers = [NVFP4Linear(q, torch, l.x, l.w, l.dy, l.seed, fused_quant, split_tail, rht_x_forward,
                          layout)
              if isinstance(l, NVFP4Linear) else l for l in step.layers]
    return TrainingStep(torch, layers, dev, serial_gemms)


def build_mlp_step(q, torch, dev, fused_quant=False, split_tail=True, serial_gemms=True):
    """The 4-block MLP step: 8 linear layers (3 NVFP4 blocks, the last block
    in bf16), each with its own inputs drawn on the GPU."""
    from quantize_precision_gemm_amd import workloads as wl
    from quantize_precision_gemm_amd.step import BF16Linear, NVFP4Linear, TrainingStep
    t0 = time.time()
    shapes = wl.mlp_layers()
    layers = []
    for i, sh in enumerate(shapes):
        seed = wl.layer_seed(wl.MLP_SEED, i)
        d = wl.layer_inputs_device(torch, dev, sh, seed)
        cls = BF16Linear if i >= len(shapes) - 2 else NVFP4Linear
        layers.append(NVFP4Linear(q, torch, d["X"], d["W"], d["dY"], seed, fused_quant, split_tail)
                      if cls is NVFP4Linear else cls(q, torch, d["X"], d["W"], d["dY"], seed))
    torch.cuda.synchronize()
    print(f"# MLP inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    return TrainingStep(torch, layers, dev, serial_gemms)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20 for the layer, 5 for the MLP step)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 10 for the layer, 2 for the MLP step)")
    ap.add_argument("--workload", choices=["layer", "mlp"], default="layer",
                    help="layer: one 12B-style linear layer (the default bench line); "
                         "mlp: the 4-block MLP training step at 16384 tokens")
    ap.add_argument("--fused-quant", action="store_true",
                    help="time the step with the dual quantisers (one encode pass per tensor "
                         "for both operands) instead of separate ones; the other schedule is "
                         "timed beside it either way")
    ap.add_argument("--rht-study", action="store_true",
                    help="only run the wgrad RHT size ablation (sizes 1, 4, 16, 64) and print its "
                         "JSON line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain elementwise copy of 1 GiB (bf16 negation, 3 launches): "
                         "the reference that scales hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the layer would shard by tokens, with an all-reduce of dW and of the "
              "tensor maxima). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    mlp = args.workload == "mlp"
    steps = args.steps if args.steps is not None else (5 if mlp else 20)
    # the first steps after the inputs are made run ~0.4 % slower than later
    # ones (clock and power settling): 10 untimed steps before the layer's
    # timed ones
    warmup = args.warmup if args.warmup is not None else (2 if mlp else 10)

    import torch
    import quantize_precision_gemm_amd as q

    q.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = 1 << 29                      # bf16 elements: 1 GiB read, 1 GiB written
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "torch.neg bf16", "bytes_read_per_launch": 2 * n,
                          "bytes_written_per_launch": 2 * n, "launches": 3}), flush=True)
        return
    if args.rht_study:
        print(json.dumps(rht_size_study(q, torch, dev)), flush=True)
        return
    head_split, head_serial = HEADLINE_SCHEDULE[args.workload]
    if mlp:
        data, step = None, build_mlp_step(q, torch, dev, args.fused_quant, head_split, head_serial)
    else:
        data, step = build_layer_step(q, torch, dev, args.fused_quant, head_split, head_serial)

    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()

    # timed steps: the step itself, with timing events around the fprop
    # launches only (the roofline's kernel; nothing else runs on the GPU
    # meanwhile).  A timing event is a barrier in the stream: the kernel
    # after fprop cannot start during fprop's last wave, which costs the step
    # a little; schedules_ms_per_step times every schedule without events
    marks = {"fprop": []}
    t0 = time.perf_counter()
    for _ in range(steps):
        step.run(marks)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    live = [s.elapsed_time(e) for s, e in marks["fprop"]]

    # every schedule over the same tensors, timed the same way (no events):
    # the headline's, the other quantiser form, and the backward GEMMs
    # concurrent or one after the other, with or without the tail split
    def timed_steps(st):
        for _ in range(warmup):
            st.run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            st.run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    head_name = schedule_name(args.fused_quant, head_split, head_serial)
    sched_ms = {head_name: timed_steps(step)}
    alt = with_schedule(q, torch, dev, step, not args.fused_quant, head_split, head_serial)
    sched_ms[schedule_name(not args.fused_quant, head_split, head_serial)] = timed_steps(alt)
    for sp, se in ((False, False), (True, False), (True, True)):
        if (sp, se) == (head_split, head_serial):
            continue
        other = with_schedule(q, torch, dev, step, args.fused_quant, sp, se)
        sched_ms[schedule_name(args.fused_quant, sp, se)] = timed_steps(other)
        del other
    if not args.fused_quant:  # X's RHT operand encoded before fprop instead
        other = with_schedule(q, torch, dev, step, False, head_split, head_serial, True)
        sched_ms[schedule_name(False, head_split, head_serial, True)] = timed_steps(other)
        del other
    # the headline schedule with every NVFP4 tensor's codes row-major (the
    # GEMMs then touch a quarter of a cache line per row and K step)
    other = with_schedule(q, torch, dev, step, args.fused_quant, head_split, head_serial,
                          layout=q.LAYOUT_ROW_MAJOR)
    sched_ms[schedule_name(args.fused_quant, head_split, head_serial, row_major=True)] = \
        timed_steps(other)
    del other
    # the GEMMs of the tail-split step serialised, events around each
    spl = with_schedule(q, torch, dev, step, args.fused_quant, True, False)
    split_ops = {}
    for _ in range(max(3, steps // 2)):
        ops, ev = spl.run_timed_ops()
        torch.cuda.synchronize()
        for j, (i, name, _) in enumerate(ops):
            if name in ("dgrad", "wgrad"):
                split_ops.setdefault(name, []).append(ev[j].elapsed_time(ev[j + 1]))
    del spl

    # the same step in the comparison format MXFP4, timed the same way
    mxs = as_mxfp4(q, torch, dev, step)
    for _ in range(warmup):
        mxs.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        mxs.run()
    torch.cuda.synchronize()
    mx_ms = (time.perf_counter() - t0) * 1e3 / steps
    del mxs

    # per-operation times: separate, serialised passes with events; for the
    # layer through nvfp4_gemm (the kernel the roofline describes; the split
    # calls are timed above)
    opstep = step if mlp or not head_split else with_schedule(q, torch, dev, step, args.fused_quant)
    times = {}
    for _ in range(max(3, steps // 2)):
        ops, ev = opstep.run_timed_ops()
        torch.cuda.synchronize()
        for j, (i, name, _) in enumerate(ops):
            times.setdefault((i, name), []).append(ev[j].elapsed_time(ev[j + 1]))
        if not mlp:  # the other schedule's quantisers, for their bandwidth
            ops, ev = alt.run_timed_ops()
            torch.cuda.synchronize()
            for j, (i, name, _) in enumerate(ops):
                if name.startswith(("dual_", "quant_X", "quant_dY", "rht_")):
                    times.setdefault((i, name), []).append(ev[j].elapsed_time(ev[j + 1]))
    avg_op = {k: sum(v) / len(v) for k, v in times.items()}
    by_name = {}
    for (i, name), v in avg_op.items():
        by_name.setdefault(name, []).append(v)

    # the second NVFP4 GEMM datapath (FP8 MFMA per 16-element block),
    # serialised, on the same quantised operands: measured beside the first
    datapaths = None
    if not mlp:
        L = step.layers[0]
        runs = [("fprop", q.FPROP, L.gx, L.gw, L.y), ("dgrad", q.DGRAD, L.gdy, L.gw, L.dx),
                ("wgrad", q.WGRAD, L.gdyt, L.gxt, L.dw)]
        fp8 = {}
        for name, p_, a_, b_, o_ in runs:
            q.nvfp4_gemm(p_, a_, b_, out=o_, fp8_blocks=True)
            s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record()
            for _ in range(3):
                q.nvfp4_gemm(p_, a_, b_, out=o_, fp8_blocks=True)
            e_.record()
            torch.cuda.synchronize()
            fp8[name] = 2.0 * L.M * L.N * L.K / (s_.elapsed_time(e_) / 3 * 1e-3) / 1e12
        datapaths = fp8

    mx = None if mlp else mx_comparison(q, torch, step.layers[0])
    epi = None if mlp else epilogue_amax_comparison(q, torch, step.layers[0])

    ms_step = wall * 1e3 / steps
    layer0 = step.layers[0]
    gemm_flop = 2.0 * layer0.M * layer0.N * layer0.K   # equal for every layer here
    mean = lambda v: sum(v) / len(v)
    gemm_bf16_ms = mean(live)
    achieved = gemm_flop / (gemm_bf16_ms * 1e-3) / 1e12

    result = {
        "metric": "NVFP4 GEMM TFLOP/s (fprop/dgrad/wgrad) + quantize GB/s, 12B-layer shapes",
        "value": round(step.flops() / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "device": device_info(torch, dev),
    }
    result["schedule"] = head_name
    result["schedules_ms_per_step"] = {k: round(v, 4) for k, v in sched_ms.items()}
    gemm_names = [n for n in ("fprop", "dgrad", "wgrad", "bf16_fprop", "bf16_dgrad", "bf16_wgrad")
                  if n in by_name]
    result["gemm_tflops"] = {n: round(gemm_flop / (mean(by_name[n]) * 1e-3) / 1e12, 1)
                             for n in gemm_names}
    result["gemm_split_tflops"] = {
        n: round(gemm_flop / (mean(v) * 1e-3) / 1e12, 1) for n, v in split_ops.items()}
    if datapaths is not None:
        result["gemm_datapaths_tflops"] = {
            "fp16_decode (nvfp4_gemm)": {n: result["gemm_tflops"][n] for n in datapaths},
            "fp8_blocks (nvfp4_gemm_fp8blk)": {n: round(v, 1) for n, v in datapaths.items()}}
    if mlp:
        result["config"] = {
            "workload": "4-block MLP training step (per block an up- and a down-projection "
                        "linear layer; fprop + dgrad + wgrad of all 8; blocks 1-3 NVFP4 with "
                        "all quantisations, block 4 bf16)",
            "tokens_M": wl_mlp("MLP_TOKENS"), "hidden": wl_mlp("MLP_HIDDEN"),
            "ffn": wl_mlp("MLP_FFN"), "blocks": wl_mlp("MLP_BLOCKS"),
            "activations": "Student-t(3), unit variance", "seed": wl_mlp("MLP_SEED"),
            "operand_format": "nvfp4 (6 layers), bf16 (2 layers)",
            "mfma": "f16 (nvfp4 decoded) and bf16 32x32x16, fp32 accumulate",
            "parallelism": "none (1 GPU)"}
        result["dtype"] = "f16+bf16"
        result["ms_per_op_total"] = {n: round(sum(v), 4) for n, v in by_name.items()}
    else:
        result["config"] = {
            "workload": "12B-style MLP up-projection linear layer, one training step "
                        "(fprop + dgrad + wgrad, all NVFP4 quantisations included)",
            "tokens_M": M, "in_K": K, "out_N": N, "operand_format": "nvfp4",
            "mfma": "f16 32x32x16, fp32 accumulate", "parallelism": "none (1 GPU)"}
        qb = quant_bytes()
        avg = {n: mean(v) for n, v in by_name.items()}
        result["quantize_gbps"] = {k: round(qb[k] / (avg[k] * 1e-3) / 1e9, 1) for k in qb}
        result["quantize_frac_of_hbm_peak"] = {
            k: round(qb[k] / (avg[k] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 3) for k in qb}
        cgb = copy_gbps(torch, dev)
        result["copy_gbps"] = round(cgb, 1)
        result["quantize_frac_of_copy"] = {
            k: round(qb[k] / (avg[k] * 1e-3) / 1e9 / cgb, 3) for k in qb}
        result["ms_per_op"] = {k: round(v, 4) for k, v in avg.items()}
        result["quantize_cold"] = quantize_cold(q, torch, step.layers[0])
        result["config_256_fprop"] = small_fprop_latency(q, torch, dev)
    sus = mfma_sustained(q, torch, dev)
    if mx is not None:
        mx["frac_of_sustained_fp4"] = {k: round(v / sus["fp4_block_scaled_e2m1"], 3)
                                       for k, v in mx["gemm_tflops"].items()}
        mx["speedup_vs_nvfp4"] = {k: round(v / result["gemm_tflops"][k], 2)
                                  for k, v in mx["gemm_tflops"].items()}
        result["mxfp4_comparison"] = mx
    if epi is not None:
        result["quantize_in_epilogue"] = epi
    result["mxfp4_step"] = {
        "ms_per_step": round(mx_ms, 4),
        "tflops": round(step.flops() / (mx_ms * 1e-3) / 1e12, 2),
        "note": "the same step with every NVFP4 layer in MXFP4 (MXFP4Linear: no amax passes, "
                "W quantised along K and along N), timed the same way"}
    result["roofline"] = {
        "kernel": "k_gemm_nv<bf16 out> (fprop launches)", "bound": "mfma",
        "achieved": round(achieved, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_F16_TFLOPS, 4), "avg_launch_ms": round(gemm_bf16_ms, 4),
        "launches": len(live),
        "timing": "HIP events around each fprop launch in the timed steps, on its stream",

        "traffic": None if mlp else counter_traffic()}
    result["roofline"]["sustained_mfma_tflops"] = sus
    result["roofline"]["frac_of_sustained"] = round(achieved / sus["decoded_nvfp4_operands"], 4)
    # every pass of the kernel, each launch serialised (events after every op)
    result["roofline"]["per_pass_serialised"] = {
        n: {"ms": round(mean(by_name[n]), 4),
            "achieved": round(gemm_flop / (mean(by_name[n]) * 1e-3) / 1e12, 1),
            "frac": round(gemm_flop / (mean(by_name[n]) * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)}
        for n in ("fprop", "dgrad", "wgrad") if n in by_name}
    # the calls the headline step makes for dgrad and wgrad (k_gemm_nv with
    # the last partial wave split along K, then k_splitk_reduce)
    for n, v in split_ops.items():
        result["roofline"]["per_pass_serialised"][n + " (nvfp4_gemm_split)"] = {
            "ms": round(mean(v), 4),
            "achieved": round(gemm_flop / (mean(v) * 1e-3) / 1e12, 1),
            "frac": round(gemm_flop / (mean(v) * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)}
    result["cpu_baseline"] = None
    if not args.no_cpu_baseline and not mlp:
        print("# timing the CPU oracle on a token slice", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(data)
    print(json.dumps(result), flush=True)


def wl_mlp(name):
    from quantize_precision_gemm_amd import workloads as wl
    return getattr(wl, name)


if __name__ == "__main__":
    main()
