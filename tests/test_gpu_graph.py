"""Every entry point captured in a HIP graph and replayed.

The library enqueues only kernels on the caller's stream (no allocation, no
memset, no host synchronisation), so a captured sequence must replay to the
same bits as the eager calls. Each graph is replayed several times with
other eager work and synchronisations in between, and every replay is
compared with the eager result.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

qm = pytest.importorskip("quantized_matmul_amd")

DEV = "cuda:0"


def _weight(shape, wid, mode, g, bits, transpose=True):
    w, _ = synth.normal(shape, 0.02, wid, synth.WEIGHT, "bf16")
    return qm.quantize(w.to(DEV), g, bits, mode, transpose=transpose)


def _check_graph(calls, outs):
    """calls: zero-argument functions writing into the tensors of outs."""
    for f in calls:
        f()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for o in outs:
        o.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in calls:
            f()
    noise = torch.randn(1 << 20, device=DEV)
    for rep in range(3):
        for o in outs:
            o.zero_()
        (noise * 2.0).sum()                 # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e), rep


def test_graph_matmul_paths():
    """Decode, many-row, [in, out] and dense forms in one graph."""
    qd = _weight((1024, 2048), 61, "affine", 64, 4)
    qn = _weight((2048, 1024), 62, "affine", 64, 4, transpose=False)
    qx = _weight((512, 1024), 63, "mxfp4", 32, 4)
    x1, _ = synth.normal((1, 2048), 1.0, 61, synth.ACT, "bf16")
    x4, _ = synth.normal((4, 2048), 1.0, 62, synth.ACT, "bf16")
    xp, _ = synth.normal((300, 1024), 1.0, 63, synth.ACT, "bf16")
    x1, x4, xp = x1.to(DEV), x4.to(DEV), xp.to(DEV)
    b, _ = synth.normal((1024,), 1.0, 61, synth.BIAS, "bf16")
    b = b.to(DEV)
    y1 = torch.empty((1, 1024), dtype=torch.bfloat16, device=DEV)
    y4 = torch.empty((4, 1024), dtype=torch.bfloat16, device=DEV)
    yp = torch.empty((300, 512), dtype=torch.bfloat16, device=DEV)
    yd = torch.empty((4, 1024), dtype=torch.bfloat16, device=DEV)
    yn1 = torch.empty((1, 1024), dtype=torch.bfloat16, device=DEV)
    # the [in, out] calls take the K-split form with a workspace from torch's
    # allocator (allocated while capturing, from the graph's pool)
    assert qm.quantized_matmul_workspace_bytes(4, 2048, 1024, False, 64, 4) > 0
    calls = [lambda: qm.quantized_matmul(x1, qd, out=y1),
             lambda: qm.quantized_matmul(x4, qn, out=y4),
             lambda: qm.quantized_matmul(x1, qn, out=yn1),
             lambda: qm.quantized_matmul(xp, qx, out=yp),
             lambda: qm.quantized_dense(x4, qd, b, out=yd)]
    _check_graph(calls, [y1, y4, yn1, yp, yd])


def test_graph_gather_and_qqmm():
    """Bucketed and direct gathers (their bucketing kernel inside the graph)
    and qqmm with its activation step."""
    E, N, K = 16, 256, 512
    qe = _weight((E, N, K), 64, "affine", 64, 4)
    x, _ = synth.normal((64, 1, K), 1.0, 64, synth.ACT, "bf16")
    x = x.to(DEV)
    rhs = torch.from_numpy(synth.topk_distinct(64, E, 4, 64).astype(np.int32)).reshape(-1).to(DEV)
    lhs = torch.arange(64, dtype=torch.int32, device=DEV).repeat_interleave(4)
    R = rhs.numel()
    ws = torch.empty(qm.gather_qmm_workspace_bytes(R, E), dtype=torch.uint8, device=DEV)
    yg = torch.empty((R, 1, N), dtype=torch.bfloat16, device=DEV)
    rs, ls = rhs[:4].contiguous(), lhs[:4].contiguous()   # few rows: direct decode form
    ys = torch.empty((4, 1, N), dtype=torch.bfloat16, device=DEV)
    wss = torch.empty(qm.gather_qmm_workspace_bytes(4, E), dtype=torch.uint8, device=DEV)
    qq = _weight((N, K), 65, "mxfp8", 32, 8)
    xq, _ = synth.normal((7, K), 1.0, 65, synth.ACT, "bf16")
    xq = xq.to(DEV)
    wq = torch.empty(qm.qqmm_workspace_bytes(7, K), dtype=torch.uint8, device=DEV)
    yq = torch.empty((7, N), dtype=torch.bfloat16, device=DEV)
    calls = [lambda: qm.gather_qmm(x, qe, rhs, lhs, workspace=ws, out=yg),
             lambda: qm.gather_qmm(x, qe, rs, ls, workspace=wss, out=ys),
             lambda: qm.qqmm(xq, qq, workspace=wq, out=yq)]
    _check_graph(calls, [yg, ys, yq])
