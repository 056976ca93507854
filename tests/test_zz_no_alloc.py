"""fgq_decode_attn_q4kv_noalloc (the allocation-free entry: split states in a
fixed scratch array inside the library) against fgq_decode_attn_q4kv with a
caller workspace, on calls in a row, each with a smaller input than the one
before (the first with four waves per item): outputs equal bit for bit (same
kernels, same plan), and each within the attention bar of the oracle.  Runs
last: a failure here hides nothing."""
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


def _case(nb, L, tag):
    """A cache of nb sequences (OPT-175B heads) holding L positions of the
    long-context recipe, its oracle twin, and a query."""
    w = synth.WORKLOADS["long-t3"]
    dev = gu.DevKV(nb, w.heads, w.head_dim, L)
    ref = oracle.KVCache(nb, w.heads, w.head_dim, L)
    k = synth.prompt_kv(w, "k", b0=tag, nb=nb, nt=L)
    v = synth.prompt_kv(w, "v", b0=tag, nb=nb, nt=L)
    dev.append(k, v, 0)
    oracle.kv_append(ref, k, v, 0)
    q = synth.step_q(w, 1 + tag)[:nb]
    return dev, ref, q


def _noalloc(dev, q, L):
    torch = gu.torch_cuda()
    out = torch.full((dev.batch, dev.heads * dev.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    gu.fgq.fgq_decode_attn_q4kv_noalloc(dev.struct, gu.to_dev(q), L, 0.0, out, gu.fgq.FGQ_DTYPE_F32)
    torch.cuda.synchronize()
    return gu.to_host(out)


def test_noalloc_attention_two_calls_second_smaller():
    # each call smaller than the one before; the first (>= 1024 positions, few
    # pairs) gives each (pair, split) item the four waves of a workgroup, the
    # others one wave per item
    cases = [(3, 2600, 7), (3, 1000, 0), (1, 600, 5)]
    for nb, L, tag in cases:
        gu.note("noalloc attention nb=%d L=%d" % (nb, L))
        dev, ref, q = _case(nb, L, tag)
        # every plan splits the sequence, so the scratch really holds split states
        assert gu.fgq.fgq_decode_attn_ws_bytes(nb, dev.heads, dev.head_dim, L) > 0
        got = _noalloc(dev, q, L)
        exp_ws = dev.attend(q, L)
        assert np.array_equal(got, exp_ws), "noalloc differs from the workspace entry point"
        gu.assert_close(got, oracle.decode_attn(ref, q, L), "noalloc attention nb=%d L=%d" % (nb, L))
