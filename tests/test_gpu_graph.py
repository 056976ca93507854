"""A decode layer step (append -> attention -> the layer's weight GEMMs)
captured into HIP graphs through the C ABI and replayed: every replay, with
eager work and synchronisations in between, must reproduce the eager step's
outputs and cache bytes exactly (the kernels are deterministic and the
library enqueues nothing but kernel launches), and the eager step itself is
anchored to the oracle."""
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

G, MB, H, D, PROMPT, STEPS = 4, 4, 8, 128, 1000, 3
B = G * MB
HID = H * D
# (name, K, N): fused Q|K|V, output projection, the two FFN matrices
GEMMS = [("qkv", HID, 3 * HID), ("out", HID, HID), ("ffn1", HID, 4 * HID), ("ffn2", 4 * HID, HID)]


def _f16(tag, n, sigma=1.0):
    return synth.to_f16(synth.normal(synth.stream_key(70, tag, n), n, sigma))


class _Step:
    """Static device buffers of one layer step (what a graph binds to)."""

    def __init__(self, t, weights, canonical=False):
        self.t = t
        self.canonical = canonical
        self.k = gu.to_dev(_f16(10 + t, B * HID).reshape(B, 1, HID))
        self.v = gu.to_dev(_f16(20 + t, B * HID).reshape(B, 1, HID))
        self.q = gu.to_dev(_f16(30 + t, B * HID).reshape(B, HID))
        self.x = [gu.to_dev(_f16(40 + 8 * t + i, B * K).reshape(B, K)) for i, (_, K, _) in enumerate(GEMMS)]
        self.attn = torch.empty((B, HID), dtype=torch.float32, device="cuda")
        self.y = [torch.empty((B, N), dtype=torch.float32, device="cuda") for _, _, N in GEMMS]
        self.weights = weights

    def enqueue(self, kv, attn_ws, gemm_ws):
        s = torch.cuda.current_stream().cuda_stream
        L = PROMPT + self.t
        gu.fgq.fgq_kv_append(kv.struct, self.k, self.v, L - 1, 1, s)
        gu.fgq.fgq_decode_attn_q4kv(kv.struct, self.q, L, 0.0, self.attn, gu.fgq.FGQ_DTYPE_F32, attn_ws,
                                    attn_ws.numel(), s)
        for i, (_, K, N) in enumerate(GEMMS):
            wc, wm = self.weights[i]
            gemm = gu.fgq.fgq_dequant_gemm if self.canonical else gu.fgq.fgq_dequant_gemm_packed
            gemm(self.x[i], G, MB, K, N, wc, wm, self.y[i], gu.fgq.FGQ_DTYPE_F32, gemm_ws, gemm_ws.numel(), s)

    def outputs(self):
        return [gu.to_host(self.attn)] + [gu.to_host(y) for y in self.y]


def _kv_with_prompt(pk, pv):
    kv = gu.DevKV(B, H, D, PROMPT + STEPS)
    kv.append(pk, pv, 0)
    return kv


@pytest.mark.parametrize("canonical", [False, True])
def test_graph_layer_step_replays_match_eager(canonical):
    gu.torch_cuda()
    gu.note("graph layer step (canonical GEMM layout: %s): setup" % canonical)
    weights, host_w = [], []
    for i, (_, K, N) in enumerate(GEMMS):
        Wt = _f16(60 + i, K * N, 0.02).reshape(K, N)
        codes, meta = gu.quantize(Wt)
        cd, md = gu.to_dev(codes), gu.to_dev(meta)
        weights.append((cd, md) if canonical else gu.pack(cd, md, K, N))
        host_w.append((codes, meta))
    pk = _f16(1, B * PROMPT * HID).reshape(B, PROMPT, HID)
    pv = _f16(2, B * PROMPT * HID).reshape(B, PROMPT, HID)
    eager_kv, graph_kv = _kv_with_prompt(pk, pv), _kv_with_prompt(pk, pv)
    attn_wsb = max(gu.fgq.fgq_decode_attn_ws_bytes(B, H, D, PROMPT + t) for t in range(1, STEPS + 1))
    gemm_wsb = max(gu.fgq.fgq_dequant_gemm_ws_bytes(B, K, N) for _, K, N in GEMMS)
    # the graph holds the attention split merge and at least one split-K reduction
    assert attn_wsb > 0 and gemm_wsb > 0
    attn_ws = torch.empty(attn_wsb, dtype=torch.uint8, device="cuda")
    gemm_ws = torch.empty(gemm_wsb, dtype=torch.uint8, device="cuda")
    steps = [_Step(t, weights, canonical) for t in range(1, STEPS + 1)]
    other = _Step(1, weights, canonical)     # eager work between replays, on buffers of its own

    gu.note("graph layer step: eager pass")
    eager = []
    for st in steps:
        st.enqueue(eager_kv, attn_ws, gemm_ws)
        torch.cuda.synchronize()
        eager.append(st.outputs())
    eager_cache = eager_kv.host()

    # anchor the eager step to the oracle: attention of two sequences at the
    # last step, and the split-K GEMM of the last step
    ref = oracle.KVCache(2, H, D, PROMPT + STEPS)
    sel = [0, B - 1]
    oracle.kv_append(ref, pk[sel], pv[sel], 0)
    for st in steps:
        oracle.kv_append(ref, gu.to_host(st.k)[sel], gu.to_host(st.v)[sel], PROMPT + st.t - 1)
    for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
        assert np.array_equal(eager_cache[a][sel], getattr(ref, a)), a
    exp = oracle.decode_attn(ref, gu.to_host(steps[-1].q)[sel], PROMPT + STEPS)
    gu.assert_close(eager[-1][0][sel], exp, "eager attention vs oracle")
    rc, rm = oracle.quantize_g64(_f16(63, 4 * HID * HID, 0.02).reshape(4 * HID, HID))
    assert np.array_equal(rc, host_w[3][0]) and np.array_equal(rm, host_w[3][1])
    exp = oracle.dequant_gemm(gu.to_host(steps[-1].x[3]), G, MB, rc, rm)
    gu.assert_close(eager[-1][4], exp, "eager ffn2 GEMM vs oracle")

    gu.note("graph layer step: capture %d graphs" % STEPS)
    graphs = []
    for st in steps:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st.enqueue(graph_kv, attn_ws, gemm_ws)
        graphs.append(g)
    torch.cuda.synchronize()

    for rep in range(3):
        gu.note("graph layer step: replay round %d" % rep)
        for i, (g, st) in enumerate(zip(graphs, steps)):
            for y in [st.attn] + st.y:
                y.fill_(float("nan"))        # a replay must rewrite every output
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = st.outputs()
            for j, (a, b) in enumerate(zip(got, eager[i])):
                assert np.array_equal(a, b), ("replay", rep, "step", st.t, "output", j)
            # eager work on the same stream between replays
            other.enqueue(eager_kv, attn_ws, gemm_ws)
            torch.cuda.synchronize()
        h = graph_kv.host()
        for a in h:
            assert np.array_equal(h[a], eager_cache[a]), ("cache", a, rep)


@pytest.mark.parametrize("B2,Hkv,R,L", [(2, 2, 8, 3000), (64, 32, 2, 300)])
def test_graph_gqa_step_replays_match_eager(B2, Hkv, R, L):
    """A grouped-query decode step (append + attention; with splits the graph
    also holds the split merge) captured and replayed three times with eager
    work in between: every replay equals the eager step bit for bit."""
    gu.torch_cuda()
    Hq, D = Hkv * R, 128
    gu.note("graph gqa step B=%d Hkv=%d R=%d L=%d" % (B2, Hkv, R, L))
    pk = _f16(80, B2 * L * Hkv * D).reshape(B2, L, Hkv * D)
    pv = _f16(81, B2 * L * Hkv * D).reshape(B2, L, Hkv * D)
    kv_e, kv_g = gu.DevKV(B2, Hkv, D, L + 1), gu.DevKV(B2, Hkv, D, L + 1)
    kv_e.append(pk, pv, 0)
    kv_g.append(pk, pv, 0)
    k1 = gu.to_dev(_f16(82, B2 * Hkv * D).reshape(B2, 1, Hkv * D))
    v1 = gu.to_dev(_f16(83, B2 * Hkv * D).reshape(B2, 1, Hkv * D))
    q = gu.to_dev(_f16(84, B2 * Hq * D).reshape(B2, Hq * D))
    q_other = gu.to_dev(_f16(85, B2 * Hq * D).reshape(B2, Hq * D))
    wsb = gu.fgq.fgq_decode_attn_gqa_ws_bytes(B2, Hq, Hkv, D, L + 1)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((B2, Hq * D), dtype=torch.float32, device="cuda")
    out_other = torch.empty_like(out)

    def enqueue(kv, qq, o):
        s = torch.cuda.current_stream().cuda_stream
        gu.fgq.fgq_kv_append(kv.struct, k1, v1, L, 1, s)
        gu.fgq.fgq_decode_attn_gqa_q4kv(kv.struct, qq, Hq, L + 1, 0.0, o, gu.fgq.FGQ_DTYPE_F32, ws, ws.numel(), s)

    enqueue(kv_e, q, out)
    torch.cuda.synchronize()
    eager = gu.to_host(out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enqueue(kv_g, q, out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gu.to_host(out), eager), ("replay", rep)
        enqueue(kv_e, q_other, out_other)     # eager work on the same stream and workspace
        torch.cuda.synchronize()
    h_e, h_g = kv_e.host(), kv_g.host()
    for a in h_e:
        assert np.array_equal(h_e[a], h_g[a]), a


def test_graph_chained_step_replays_match_eager():
    """The chained layer step (the one the bench replays): the Q|K|V product
    feeds the append (K and V read at a row stride) and the attention (q at
    a row stride), attention feeds Wout, Wout feeds W1 and W1 feeds W2, every
    hand-off in fp16.  Each decode step is captured as one graph and replayed
    three times with eager work in between: every replay equals the eager
    step bit for bit, so no launch of the graph runs ahead of one it reads."""
    gu.torch_cuda()
    gu.note("graph chained step: setup")
    weights = []
    for i, (_, K, N) in enumerate(GEMMS):
        codes, meta = gu.quantize(_f16(160 + i, K * N, 0.02).reshape(K, N))
        weights.append(gu.pack(gu.to_dev(codes), gu.to_dev(meta), K, N))
    pk = _f16(101, B * PROMPT * HID).reshape(B, PROMPT, HID)
    pv = _f16(102, B * PROMPT * HID).reshape(B, PROMPT, HID)
    eager_kv, graph_kv = _kv_with_prompt(pk, pv), _kv_with_prompt(pk, pv)
    f16 = gu.fgq.FGQ_DTYPE_F16
    x0 = [gu.to_dev(_f16(120 + t, B * HID).reshape(B, HID)) for t in range(1, STEPS + 1)]
    qkv = torch.empty((B, 3 * HID), dtype=torch.float16, device="cuda")
    attn = torch.empty((B, HID), dtype=torch.float16, device="cuda")
    ys = [torch.empty((B, N), dtype=torch.float16, device="cuda") for _, _, N in GEMMS[1:]]
    attn_wsb = max(gu.fgq.fgq_decode_attn_ws_bytes(B, H, D, PROMPT + t) for t in range(1, STEPS + 1))
    gemm_wsb = max(gu.fgq.fgq_dequant_gemm_ws_bytes(B, K, N) for _, K, N in GEMMS)
    assert attn_wsb > 0 and gemm_wsb > 0     # the split merge and a split-K reduction are in the graph
    attn_ws = torch.empty(attn_wsb, dtype=torch.uint8, device="cuda")
    gemm_ws = torch.empty(gemm_wsb, dtype=torch.uint8, device="cuda")

    def enqueue(kv, t):
        s = torch.cuda.current_stream().cuda_stream
        gemm = gu.fgq.fgq_dequant_gemm_packed

        def mm(i, x, y):
            _, K, N = GEMMS[i]
            gemm(x, G, MB, K, N, weights[i][0], weights[i][1], y, f16, gemm_ws, gemm_ws.numel(), s)

        mm(0, x0[t - 1], qkv)
        gu.fgq.fgq_kv_append_ld(kv.struct, qkv[:, HID:2 * HID], qkv[:, 2 * HID:], 3 * HID, PROMPT + t - 1, 1, s)
        gu.fgq.fgq_decode_attn_q4kv_ld(kv.struct, qkv[:, :HID], 3 * HID, PROMPT + t, 0.0, attn, f16, attn_ws,
                                       attn_ws.numel(), s)
        mm(1, attn, ys[0])
        mm(2, ys[0], ys[1])
        mm(3, ys[1], ys[2])

    def outputs():
        return [gu.to_host(a) for a in [qkv, attn] + ys]

    gu.note("graph chained step: eager pass")
    eager = []
    for t in range(1, STEPS + 1):
        enqueue(eager_kv, t)
        torch.cuda.synchronize()
        eager.append(outputs())
    eager_cache = eager_kv.host()
    assert all(np.all(np.isfinite(a.astype(np.float32))) for a in eager[-1])

    gu.note("graph chained step: capture %d graphs" % STEPS)
    graphs = []
    for t in range(1, STEPS + 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            enqueue(graph_kv, t)
        graphs.append(g)
    torch.cuda.synchronize()

    for rep in range(3):
        gu.note("graph chained step: replay round %d" % rep)
        for i, g in enumerate(graphs):
            for a in [qkv, attn] + ys:
                a.fill_(float("nan"))        # a replay must rewrite every output
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for j, (a, b) in enumerate(zip(outputs(), eager[i])):
                assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), ("replay", rep, "step", i + 1, "output", j)
            enqueue(eager_kv, 1)             # eager work on the same stream between replays
            torch.cuda.synchronize()
        h = graph_kv.host()
        for a in h:
            assert np.array_equal(h[a], eager_cache[a]), ("cache", a, rep)
