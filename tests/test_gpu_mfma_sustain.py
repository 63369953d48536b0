"""The matrix-throughput measurement aid (nvfp4_mfma_sustain) computes the
products it is timed for: per thread, the sum of its accumulators after
`iters` rounds of 64 matrix instructions, against a float64 model of the
same fragments and of the instructions' lane layout.  fp16 32x32x16: lane l
supplies row (A) or column (B) l % 32 and k 8 (l // 32) .. +7; block-scaled
FP4 32x32x64 (unit scales): lane l supplies k 32 (l // 32) .. +31 as 16
bytes of E2M1 codes, low nibble first; both: accumulator element e of lane
l is row 8 (e // 4) + 4 (l // 32) + e % 4, column l % 32.  Not a pass of the
method; it backs the sustained-throughput figures beside the roofline."""
import numpy as np
import pytest

from tests.gpu_util import ensure_built

pytestmark = pytest.mark.gpu

MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


U = np.uint64
M32 = U(0xFFFFFFFF)


def _mix32(x):
    x = x & M32
    x ^= x >> U(16)
    x = (x * U(0x7FEB352D)) & M32
    x ^= x >> U(15)
    x = (x * U(0x846CA68B)) & M32
    x ^= x >> U(16)
    return x


def _fragments(tids, operands):
    """fa, fb: [thread, pool entry p, element e] as float64 (exact fp16 values)."""
    p = np.arange(8, dtype=U).reshape(1, 8, 1)
    e = np.arange(8, dtype=U).reshape(1, 1, 8)
    t = tids.astype(U).reshape(-1, 1, 1)
    h1 = _mix32(t * U(131) + U(17) * p + e)
    h2 = _mix32(h1 + U(0x9E3779B9))
    out = []
    for h in (h1, h2):
        if operands == 0:
            s = (1.0 + (h >> U(29)).astype(np.float64) * 0.125) * 2.0 ** ((h >> U(20)) & U(3)).astype(np.float64) / 64.0
            v = MAG[(h & U(7)).astype(np.int64)] * s
            v = np.where((h & U(8)) != 0, -v, v)
        else:
            v = (h & U(0xFFFF)).astype(np.float64) / 32768.0 - 1.0
        out.append(v.astype(np.float16).astype(np.float64))
    return out


def _fp4_fragments(tids):
    """[thread, p, 32 k] E2M1 values of the first four dwords (h1 / h2)."""
    p = np.arange(8, dtype=U).reshape(1, 8, 1)
    e = np.arange(4, dtype=U).reshape(1, 1, 4)
    t = tids.astype(U).reshape(-1, 1, 1)
    h1 = _mix32(t * U(131) + U(17) * p + e)
    h2 = _mix32(h1 + U(0x9E3779B9))
    out = []
    for h in (h1, h2):
        nib = np.stack([(h >> U(4 * i)) & U(15) for i in range(8)], axis=-1)  # [t, p, dword, nibble]
        c = nib.reshape(h.shape[0], 8, 32).astype(np.int64)
        out.append(np.where(c & 8, -MAG[c & 7], MAG[c & 7]))
    return out


def _model(blocks, iters, operands):
    tids = np.arange(blocks * 512)
    fa, fb = _fp4_fragments(tids) if operands == 2 else _fragments(tids, operands)
    res = np.zeros(blocks * 512)
    lanes = np.arange(64)
    for w in range(blocks * 8):
        a, b = fa[64 * w:64 * w + 64], fb[64 * w:64 * w + 64]
        # A_p[r, k] = a[r + 32 (k // kh), p, k % kh]; B_q likewise (kh = 8 or 32)
        A = np.concatenate([a[:32], a[32:]], axis=2)          # [32 rows, p, K k]
        B = np.concatenate([b[:32], b[32:]], axis=2)          # [32 cols, q, K k]
        C = np.zeros((8, 32, 32))
        for j in range(64):
            C[j & 7] += A[:, j & 7, :] @ B[:, ((j >> 3) + j) & 7, :].T
        C *= iters
        rows = (8 * (np.arange(16) // 4))[None, :] + 4 * (lanes // 32)[:, None] + (np.arange(16) % 4)[None, :]
        res[64 * w:64 * w + 64] = C[:, rows, (lanes % 32)[:, None]].sum(axis=(0, 2))
    return res


@pytest.mark.parametrize("operands", [0, 1, 2])
def test_mfma_sustain_products(operands):
    import torch
    ensure_built()
    import quantize_precision_gemm_amd as q
    dev = torch.device("cuda:0")
    blocks, iters = 2, 3
    print(f"mfma_sustain operands={operands}", flush=True)
    out, flops = q.nvfp4_mfma_sustain(blocks, iters, operands, device=dev)
    out2, _ = q.nvfp4_mfma_sustain(blocks, iters, operands, device=dev)
    torch.cuda.synchronize()
    assert flops == 2.0 * 32 * 32 * (64 if operands == 2 else 16) * 64 * 8 * iters * blocks
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, out2.cpu().numpy()), "not deterministic"
    want = _model(blocks, iters, operands)
    err = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert err < 1e-6, f"relative error {err:.3e}"
