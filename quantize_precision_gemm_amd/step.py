"""Training step of linear layers through the library: buffers and launch order.

A linear layer y = x W^T (tokens M, inputs K, outputs N) runs three GEMMs per
training step ("Pretraining Large Language Models with NVFP4", gist.science
summary, Technische Zusammenfassung 2.B.2): fprop Y = X W^T, dgrad
dX = dY W and wgrad dW = dY^T X.  In an NVFP4 layer every GEMM input is
quantised first, by role (2.A, 2.B.2-2.B.4):

  X   1x16 blocks, round-to-nearest-even       (fprop)
  W   16x16 blocks, RNE, plus the transposed copy dgrad reads
  dY  1x16 blocks, stochastic rounding         (dgrad)
  dY, X  16-point random Hadamard transform along tokens, transposed, 1x16;
         SR for dY, RNE for X, one sign vector for both   (wgrad)

A layer kept in BF16 (2.B.1) runs the same three GEMMs on the bf16 tensors.

Every operation is a library call; this module only allocates buffers (once,
in the constructors) and orders the launches.  Nothing here computes.
"""

SR_SEED_DY = 100       # seed offsets of a layer's stochastic-rounding calls
SR_SEED_DY_RHT = 101
RHT_SEED = 1000        # offset of the seed the layer's RHT sign vector is drawn from


class NVFP4Linear:
    """One linear layer's training step in NVFP4.

    x (M x K), w (N x K), dy (M x N): bf16 device tensors, row-major.
    Outputs: y (M x N, bf16), dx (M x K, bf16), dw (N x K, fp32).
    """

    def __init__(self, q, torch, x, w, dy, seed, fused_quant=False, split_tail=False,
                 rht_x_forward=False, layout=None):
        self.q, self.torch = q, torch
        self.fused_quant = fused_quant
        self.split_tail = split_tail
        # rht_x_forward: X's RHT-transposed wgrad operand is encoded in the
        # forward part, right after X's 1x16 operand, instead of at the start
        # of the wgrad branch beside dgrad (measured on the 12B layer: 2 %
        # slower, so off by default; there the encode fills dgrad's partial
        # last wave of workgroups)
        self.rht_x_forward = rht_x_forward
        self.x, self.w, self.dy = x, w, dy
        M, K = x.shape
        N = w.shape[0]
        assert w.shape == (N, K) and dy.shape == (M, N)
        self.M, self.K, self.N = M, K, N
        dev = x.device
        self.seed = seed
        # codes 4-row interleaved unless asked otherwise: the GEMMs then read
        # each 64-element K step of 4 rows as one whole cache line
        lay = q.LAYOUT_INTERLEAVED if layout is None else layout
        self.layout = lay
        self.gx = q.alloc_nvfp4(M, K, q.BLOCK_1X16, device=dev, layout=lay)
        self.gw = q.alloc_nvfp4(N, K, q.BLOCK_16X16, with_transpose=True, device=dev, layout=lay)
        self.gdy = q.alloc_nvfp4(M, N, q.BLOCK_1X16, device=dev, layout=lay)
        self.gdyt = q.alloc_nvfp4(N, M, q.BLOCK_1X16, device=dev, layout=lay)
        self.gxt = q.alloc_nvfp4(K, M, q.BLOCK_1X16, device=dev, layout=lay)
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        self.dw = torch.empty((N, K), dtype=torch.float32, device=dev)
        self.mask = q.nvfp4_rht_sign_mask(seed + RHT_SEED)
        f32 = lambda: torch.empty(1, dtype=torch.float32, device=dev)
        self.ax, self.ax_rht, self.ady, self.ady_rht = f32(), f32(), f32(), f32()
        # with split_tail, dgrad and wgrad run nvfp4_gemm_split (the last,
        # partial wave of tiles split along K); they run concurrently, so
        # each has its own workspace
        self.ws_dgrad = self.ws_wgrad = None
        if split_tail:
            ws = lambda n: torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
            self.ws_dgrad = ws(q.nvfp4_gemm_split_workspace(q.DGRAD, self.gdy, self.gw))
            self.ws_wgrad = ws(q.nvfp4_gemm_split_workspace(q.WGRAD, self.gdyt, self.gxt))

    def flops(self):
        return 3 * 2.0 * self.M * self.N * self.K

    # X and dY are each quantised twice (1x16, and through the RHT for
    # wgrad): one fused pass computes both tensor maxima of each.  With
    # fused_quant one encode pass also emits both operands of each tensor
    # (nvfp4_quantize_dual), so X and dY are read twice per step instead of
    # three times; the RHT encodes then run before fprop and dgrad instead of
    # beside them on the second stream.
    def weight_ops(self):
        q = self.q
        return [("quant_W", lambda: q.nvfp4_quantize(self.w, q.BLOCK_16X16, q.RNE, out=self.gw))]

    def forward_ops(self):
        q = self.q
        if self.fused_quant:
            quant = ("dual_X", lambda: q.nvfp4_quantize_dual(
                self.x, self.mask, q.RNE, amax_in=self.ax, amax_rht_in=self.ax_rht,
                out=self.gx, out_rht=self.gxt))
        else:
            quant = ("quant_X", lambda: q.nvfp4_quantize(self.x, q.BLOCK_1X16, q.RNE,
                                                         amax_in=self.ax, out=self.gx))
        ops = [("amax_X", lambda: q.nvfp4_amax(self.x, self.mask, self.ax, self.ax_rht)), quant]
        if self.rht_x_forward and not self.fused_quant:
            ops.append(self._rht_x())
        return ops + [("fprop", lambda: q.nvfp4_gemm(q.FPROP, self.gx, self.gw, out=self.y))]

    def _rht_x(self):
        q = self.q
        return ("rht_X", lambda: q.nvfp4_rht_quantize(self.x, self.mask, q.RNE,
                                                      amax_in=self.ax_rht, out=self.gxt))

    def backward_shared_ops(self):
        """The backward work both branches (dgrad, wgrad) wait for."""
        q = self.q
        ops = [("amax_dY", lambda: q.nvfp4_amax(self.dy, self.mask, self.ady, self.ady_rht))]
        if self.fused_quant:
            ops.append(("dual_dY", lambda: q.nvfp4_quantize_dual(
                self.dy, self.mask, q.SR, self.seed + SR_SEED_DY, self.seed + SR_SEED_DY_RHT,
                amax_in=self.ady, amax_rht_in=self.ady_rht, out=self.gdy, out_rht=self.gdyt)))
        return ops

    def backward_quant_ops(self):
        q = self.q
        if self.fused_quant:
            return []
        return [("quant_dY", lambda: q.nvfp4_quantize(self.dy, q.BLOCK_1X16, q.SR,
                                                      self.seed + SR_SEED_DY, amax_in=self.ady,
                                                      out=self.gdy))]

    def dgrad_ops(self):
        q = self.q
        if self.split_tail:
            return [("dgrad", lambda: q.nvfp4_gemm_split(q.DGRAD, self.gdy, self.gw, self.ws_dgrad,
                                                         out=self.dx))]
        return [("dgrad", lambda: q.nvfp4_gemm(q.DGRAD, self.gdy, self.gw, out=self.dx))]

    def wgrad_ops(self):
        q = self.q
        if self.split_tail:
            wgrad = ("wgrad", lambda: q.nvfp4_gemm_split(q.WGRAD, self.gdyt, self.gxt, self.ws_wgrad,
                                                         out=self.dw))
        else:
            wgrad = ("wgrad", lambda: q.nvfp4_gemm(q.WGRAD, self.gdyt, self.gxt, out=self.dw))
        if self.fused_quant:
            return [wgrad]
        rht_dy = ("rht_dY", lambda: q.nvfp4_rht_quantize(self.dy, self.mask, q.SR,
                                                         self.seed + SR_SEED_DY_RHT,
                                                         amax_in=self.ady_rht, out=self.gdyt))
        if self.rht_x_forward:
            return [rht_dy, wgrad]
        return [rht_dy, self._rht_x(), wgrad]


class MXFP4Linear:
    """One linear layer's training step in MXFP4, the format the pages set
    NVFP4 against (Technische Zusammenfassung 2.A): E2M1 with one UE8M0
    scale per 32 elements, no tensor scale, so no amax passes.  The roles
    follow the NVFP4 recipe: X and W RNE, dY SR, the wgrad operands through
    the 16-point RHT along tokens.  MXFP4 has no 2D blocks, so W is
    quantised twice: along K for fprop and along N for dgrad.
    Outputs as NVFP4Linear's."""

    def __init__(self, q, torch, x, w, dy, seed):
        self.q, self.torch = q, torch
        self.x, self.w, self.dy = x, w, dy
        M, K = x.shape
        N = w.shape[0]
        assert w.shape == (N, K) and dy.shape == (M, N)
        self.M, self.K, self.N = M, K, N
        dev = x.device
        self.seed = seed
        mx = lambda r, c: q.alloc_nvfp4(r, c, q.BLOCK_MX32, device=dev)
        self.gx, self.gw, self.gwt = mx(M, K), mx(N, K), mx(K, N)
        self.gdy, self.gdyt, self.gxt = mx(M, N), mx(N, M), mx(K, M)
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        self.dw = torch.empty((N, K), dtype=torch.float32, device=dev)
        self.mask = q.nvfp4_rht_sign_mask(seed + RHT_SEED)

    def flops(self):
        return 3 * 2.0 * self.M * self.N * self.K

    def weight_ops(self):
        q = self.q
        return [("mx_quant_W", lambda: q.nvfp4_mx_quantize(self.w, q.MX_ROWS, out=self.gw)),
                ("mx_quant_Wt", lambda: q.nvfp4_mx_quantize(self.w, q.MX_COLS, out=self.gwt))]

    def forward_ops(self):
        q = self.q
        return [("mx_quant_X", lambda: q.nvfp4_mx_quantize(self.x, q.MX_ROWS, out=self.gx)),
                ("mx_fprop", lambda: q.nvfp4_mx_gemm(self.gx, self.gw, out=self.y))]

    def backward_shared_ops(self):
        return []

    def backward_quant_ops(self):
        q = self.q
        return [("mx_quant_dY", lambda: q.nvfp4_mx_quantize(self.dy, q.MX_ROWS, 0, q.SR,
                                                            self.seed + SR_SEED_DY, out=self.gdy))]

    def dgrad_ops(self):
        q = self.q
        return [("mx_dgrad", lambda: q.nvfp4_mx_gemm(self.gdy, self.gwt, out=self.dx))]

    def wgrad_ops(self):
        q = self.q
        return [
            ("mx_rht_dY", lambda: q.nvfp4_mx_quantize(self.dy, q.MX_COLS_RHT, self.mask, q.SR,
                                                      self.seed + SR_SEED_DY_RHT, out=self.gdyt)),
            ("mx_rht_X", lambda: q.nvfp4_mx_quantize(self.x, q.MX_COLS_RHT, self.mask, q.RNE,
                                                     out=self.gxt)),
            ("mx_wgrad", lambda: q.nvfp4_mx_gemm(self.gdyt, self.gxt, out=self.dw)),
        ]


class BF16Linear:
    """One linear layer's training step kept in bf16: the three GEMMs on the
    layer's own tensors, fp32 accumulation; outputs as NVFP4Linear's."""

    def __init__(self, q, torch, x, w, dy, seed=None):
        self.q, self.torch = q, torch
        self.x, self.w, self.dy = x, w, dy
        M, K = x.shape
        N = w.shape[0]
        assert w.shape == (N, K) and dy.shape == (M, N)
        self.M, self.K, self.N = M, K, N
        dev = x.device
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        self.dw = torch.empty((N, K), dtype=torch.float32, device=dev)

    def flops(self):
        return 3 * 2.0 * self.M * self.N * self.K

    def weight_ops(self):
        return []

    def forward_ops(self):
        q = self.q
        return [("bf16_fprop", lambda: q.nvfp4_bf16_gemm(q.FPROP, self.x, self.w, out=self.y))]

    def backward_shared_ops(self):
        return []

    def backward_quant_ops(self):
        return []

    def dgrad_ops(self):
        q = self.q
        return [("bf16_dgrad", lambda: q.nvfp4_bf16_gemm(q.DGRAD, self.dy, self.w, out=self.dx))]

    def wgrad_ops(self):
        q = self.q
        return [("bf16_wgrad", lambda: q.nvfp4_bf16_gemm(q.WGRAD, self.dy, self.x, out=self.dw))]


class TrainingStep:
    """Fprop of every layer in order, then the backward pass in reverse order.

    The weights do not depend on anything else in the step: the first
    layer's weight is quantised on the main stream while its activation's
    amax and quantisation run on a second stream, and every later layer's
    weight follows on the second stream; each fprop waits for both of its
    operands.  Per layer in the backward pass, the
    main stream first runs the amax pass over dY and dY's dgrad operand (the
    SR encode, or the dual encode when the layer fuses its quantisers); then
    it runs dgrad while the wgrad branch (RHT operands, unless already
    encoded, and the wgrad GEMM) runs on the second stream.  Wgrad feeds
    nothing later in the step, so it overlaps with dgrad
    and with the next layer's backward work: each GEMM's last, partial wave
    of workgroups is filled by the other's.  The step ends with the main
    stream waiting for the second one (with serial_gemms it already has, at
    each wgrad).
    """

    def __init__(self, torch, layers, device, serial_gemms=False):
        self.torch = torch
        self.layers = list(layers)
        self.side = torch.cuda.Stream(device=device)  # default priority
        # serial_gemms: dgrad then wgrad on the main stream (each filling its
        # own partial last wave, e.g. with nvfp4_gemm_split), only the wgrad
        # operands' quantisation on the second stream beside dgrad
        self.serial_gemms = serial_gemms

    def flops(self):
        return sum(l.flops() for l in self.layers)

    def run(self, marks=None):
        """One step.  marks: optional {op name: list}; every launch of a named
        operation is bracketed by two timing events on the stream it is
        launched on, appended to the list as (start, end)."""
        torch = self.torch
        main = torch.cuda.current_stream()

        def call(name, f):
            if marks is None or name not in marks:
                f()
                return
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            f()
            e.record()
            marks[name].append((s, e))

        # Before the first fprop both its operands are quantised concurrently;
        # the longer of the two (the weight: amax, then the 16x16 encode with
        # the transposed copy) runs on the main stream, so the fprop launch
        # does not wait on the other stream for it (that wait cost ~17 us on
        # the 12B layer).  The other layers' weights follow on the second
        # stream, each ready long before its fprop.
        self.side.wait_stream(main)
        first = self.layers[0]
        ops0 = first.forward_ops()
        ready = [None]
        with torch.cuda.stream(self.side):
            for n, f in ops0[:-1]:
                call(n, f)
            x0 = torch.cuda.Event()
            x0.record()
            for layer in self.layers[1:]:
                for n, f in layer.weight_ops():
                    call(n, f)
                ev = torch.cuda.Event()
                ev.record()
                ready.append(ev)
        for n, f in first.weight_ops():
            call(n, f)
        main.wait_event(x0)
        call(*ops0[-1])  # the first layer's fprop
        for layer, ev in zip(self.layers[1:], ready[1:]):
            ops = layer.forward_ops()
            for n, f in ops[:-1]:
                call(n, f)
            main.wait_event(ev)
            call(*ops[-1])  # the layer's fprop
        for layer in reversed(self.layers):
            # dY's amax and its dgrad operand first, alone on the main stream
            # (the SR encode is on the path to dgrad; started beside it, the
            # wgrad branch's encodes slowed it); then the wgrad branch on the
            # second stream beside dgrad
            for n, f in layer.backward_shared_ops() + layer.backward_quant_ops():
                call(n, f)
            self.side.wait_stream(main)
            wg = layer.wgrad_ops()
            for n, f in layer.dgrad_ops():
                call(n, f)
            with torch.cuda.stream(self.side):
                for n, f in (wg[:-1] if self.serial_gemms else wg):
                    call(n, f)
            if self.serial_gemms:
                main.wait_stream(self.side)
                call(*wg[-1])
        if not self.serial_gemms:  # (serial: every launch on the second stream is waited for already)
            main.wait_stream(self.side)

    def serial_ops(self):
        """(layer index, name, call) of the whole step in one serial order."""
        ops = []
        for i, layer in enumerate(self.layers):
            fw = layer.forward_ops()
            ops += [(i, n, f) for n, f in fw[:-1] + layer.weight_ops() + fw[-1:]]
        for i in reversed(range(len(self.layers))):
            layer = self.layers[i]
            for part in (layer.backward_shared_ops(), layer.backward_quant_ops(), layer.dgrad_ops(),
                         layer.wgrad_ops()):
                ops += [(i, n, f) for n, f in part]
        return ops

    def run_timed_ops(self):
        """One step serialised on the current stream with an event after every
        operation; returns (ops, events), events[0] before the first op."""
        torch = self.torch
        ops = self.serial_ops()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)]
        ev[0].record()
        for j, (_, _, f) in enumerate(ops):
            f()
            ev[j + 1].record()
        return ops, ev
