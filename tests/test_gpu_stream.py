"""Weight streaming (the offloading setting the compression was made for):
packed weights copied from pinned host memory on a second stream into two
alternating device buffers while the previous step's GEMM runs.  Every step's
result must equal, bit for bit, the same GEMM on resident weights (same
kernels, same inputs), whatever the interleaving of copies and compute; the
resident GEMM is anchored to the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

try:
    import torch
    _HAS_GPU = torch.cuda.is_available()
except ImportError:   # pragma: no cover
    _HAS_GPU = False

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not _HAS_GPU, reason="needs an MI355X GPU")]


def test_streamed_weights_double_buffered_match_resident():
    gu.torch_cuda()
    K, N, g, m = 2048, 3072, 8, 4
    sets = []
    for tag in range(3):                          # three different weight matrices, cycled
        Wt = synth.to_f16(synth.normal(synth.stream_key(85, tag, K, N), K * N, 0.02)).reshape(K, N)
        codes, meta = gu.quantize(Wt)
        pc, pm = gu.pack(gu.to_dev(codes), gu.to_dev(meta), K, N)
        sets.append((pc, pm, codes, meta))
    X = [gu.to_dev(synth.to_f16(synth.normal(synth.stream_key(86, i, K), g * m * K)).reshape(g * m, K))
         for i in range(6)]
    wsb = gu.fgq.fgq_dequant_gemm_ws_bytes(g * m, K, N)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")

    def gemm(x, pc, pm, y, s):
        gu.fgq.fgq_dequant_gemm_packed(x, g, m, K, N, pc, pm, y, gu.fgq.FGQ_DTYPE_F32, ws, wsb, s)

    main = torch.cuda.current_stream()
    resident = []
    for i in range(6):
        y = torch.empty((g * m, N), dtype=torch.float32, device="cuda")
        gemm(X[i], sets[i % 3][0], sets[i % 3][1], y, main.cuda_stream)
        resident.append(y)
    torch.cuda.synchronize()
    exp = oracle.dequant_gemm(gu.to_host(X[0]), g, m, sets[0][2], sets[0][3])
    gu.assert_close(gu.to_host(resident[0]), exp, "resident GEMM vs oracle")

    host = [(pc.cpu().pin_memory(), pm.cpu().pin_memory()) for pc, pm, _, _ in sets]
    bufs = [(torch.empty_like(sets[0][0]), torch.empty_like(sets[0][1])) for _ in range(2)]
    copy_stream = torch.cuda.Stream()
    copied = [torch.cuda.Event() for _ in range(2)]
    freed = [torch.cuda.Event() for _ in range(2)]
    for e in freed:
        e.record(main)
    outs = [torch.full((g * m, N), float("nan"), dtype=torch.float32, device="cuda") for _ in range(6)]
    torch.cuda.synchronize()
    gu.note("streamed weights: 6 steps over 2 buffers")

    def copy(i):
        b = i % 2
        with torch.cuda.stream(copy_stream):
            copy_stream.wait_event(freed[b])
            bufs[b][0].copy_(host[i % 3][0], non_blocking=True)
            bufs[b][1].copy_(host[i % 3][1], non_blocking=True)
            copied[b].record(copy_stream)

    copy(0)
    for i in range(6):
        if i + 1 < 6:
            copy(i + 1)
        main.wait_event(copied[i % 2])
        gemm(X[i], bufs[i % 2][0], bufs[i % 2][1], outs[i], main.cuda_stream)
        freed[i % 2].record(main)
    torch.cuda.synchronize()
    for i in range(6):
        assert np.array_equal(gu.to_host(outs[i]), gu.to_host(resident[i])), i
