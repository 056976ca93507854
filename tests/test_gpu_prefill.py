"""GPU parity of prefill attention over fp16 (through the C ABI) against the
oracle on the same seeded inputs: ragged prompt lengths that span several
query blocks (256 rows below 1024 tokens, 384 from there) and 64-key blocks,
both head sizes, fp16 output, the
scale argument, a workload-shaped launch (OPT-175B heads, prompt 512) on
sampled rows, and bitwise repeatability.  Bar: max-abs 1e-2 and rel-L2 1e-3.
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


def _qkv(B, s, H, D, tag):
    n = B * s * H * D
    return [synth.to_f16(synth.normal(synth.stream_key(80, tag + i, B, s), n)).reshape(B, s, H * D)
            for i in range(3)]


def _gpu(q, k, v, H, scale=0.0, out_f16=False):
    torch = gu.torch_cuda()
    B, s, h = q.shape
    qd, kd, vd = gu.to_dev(q), gu.to_dev(k), gu.to_dev(v)
    out = torch.full((B, s, h), float("nan"), dtype=torch.float16 if out_f16 else torch.float32, device="cuda")
    gu.fgq.fgq_prefill_attn_f16(qd, kd, vd, B, s, H, h // H, scale, out,
                                gu.fgq.FGQ_DTYPE_F16 if out_f16 else gu.fgq.FGQ_DTYPE_F32)
    torch.cuda.synchronize()
    return gu.to_host(out).astype(np.float32)


@pytest.mark.parametrize("B,s,H,D", [(1, 1, 1, 64), (2, 37, 3, 64), (2, 64, 2, 128), (1, 65, 2, 128),
                                     (2, 200, 3, 128), (1, 513, 2, 128), (3, 130, 4, 64),
                                     (1, 1024, 1, 64), (1, 1100, 2, 128),
                                     # several sequences, heads and row blocks in one launch: the
                                     # flattened longest-rows-first workgroup order, both launches
                                     (2, 600, 3, 128), (2, 1100, 3, 64),
                                     # 4-wave launch (prompts <= 640 whose last 256-row block is full
                                     # or at most half full): ragged, the longest, head_dim 64;
                                     # 8-wave launch past 640 and with a more than half full block
                                     (2, 300, 3, 64), (1, 640, 2, 128), (1, 250, 2, 64), (2, 700, 2, 128)])
def test_prefill_against_oracle(B, s, H, D):
    q, k, v = _qkv(B, s, H, D, 0)
    gu.note("prefill B=%d s=%d H=%d D=%d" % (B, s, H, D))
    got = _gpu(q, k, v, H)
    gu.assert_close(got, oracle.prefill_attn(q, k, v, H), "prefill %dx%dx%dx%d" % (B, s, H, D))


@pytest.mark.parametrize("s", [150, 100])   # the 8-wave and the 4-wave launch
def test_prefill_fp16_output_and_scale(s):
    B, H, D = 2, 2, 128
    q, k, v = _qkv(B, s, H, D, 10)
    gu.note("prefill fp16 out / scale, s=%d" % s)
    gu.assert_close(_gpu(q, k, v, H, out_f16=True), oracle.prefill_attn(q, k, v, H), "prefill fp16 out")
    gu.assert_close(_gpu(q, k, v, H, scale=0.3), oracle.prefill_attn(q, k, v, H, scale=0.3), "prefill scale 0.3")


def test_prefill_long_launch_fp16_output_and_scale():
    """The 12-wave launch (prompts of 1024+ tokens, Q staged in LDS) with
    fp16 output and an explicit softmax scale."""
    B, s, H, D = 1, 1030, 2, 128
    q, k, v = _qkv(B, s, H, D, 40)
    gu.note("prefill 12-wave fp16 out / scale 0.07")
    exp = oracle.prefill_attn(q, k, v, H, scale=0.07)
    gu.assert_close(_gpu(q, k, v, H, scale=0.07, out_f16=True), exp, "prefill 12-wave fp16 out scale 0.07")


def test_prefill_workload_shape_sampled_rows():
    """OPT-175B attention shape (96 heads of 128, prompt 512) for 8 sequences
    of the prompt's synthetic K and V: the first and last rows of every
    sequence, every head, against the oracle."""
    w = synth.WORKLOADS["opt-175b"]
    B, s, H, D = 8, w.prompt, w.heads, w.head_dim
    k = synth.prompt_kv(w, "k", nb=B)
    v = synth.prompt_kv(w, "v", nb=B)
    q = synth.prompt_q(w, nb=B)
    gu.note("prefill opt-175b shape B=%d s=%d" % (B, s))
    got = _gpu(q, k, v, H)
    assert np.all(np.isfinite(got))
    for r0, r1 in ((0, 3), (255, 257), (s - 3, s)):
        exp = oracle.prefill_attn(q, k, v, H, rows=(r0, r1))
        gu.assert_close(got[:, r0:r1], exp[:, r0:r1], "opt-175b rows %d..%d" % (r0, r1 - 1))


def test_prefill_long_prompt_sampled_rows():
    """OPT-175B heads at a 2048-token prompt (the 12-wave launch): the first,
    middle and last rows of each sequence, every head, against the oracle."""
    w = synth.WORKLOADS["opt-175b"]
    B, s, H = 1, 2048, w.heads
    q, k, v = _qkv(B, s, H, w.head_dim, 30)
    gu.note("prefill long prompt B=%d s=%d" % (B, s))
    got = _gpu(q, k, v, H)
    assert np.all(np.isfinite(got))
    for r0, r1 in ((0, 2), (383, 386), (1151, 1153), (s - 2, s)):
        exp = oracle.prefill_attn(q, k, v, H, rows=(r0, r1))
        gu.assert_close(got[:, r0:r1], exp[:, r0:r1], "long prompt rows %d..%d" % (r0, r1 - 1))


def test_prefill_repeatable_bitwise():
    q, k, v = _qkv(1, 300, 2, 128, 20)
    gu.note("prefill repeatability")
    assert np.array_equal(_gpu(q, k, v, 2), _gpu(q, k, v, 2))
