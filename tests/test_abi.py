"""C-ABI checks that need no GPU: the library loads, exports every function
include/fgq.h declares, and rejects bad arguments on the host before any
HIP call (so nothing is enqueued and outputs stay untouched)."""
import ctypes
import os
import subprocess

import pytest

import int4_group_quantized_fgq_amd as fgq

BAD = 0x1001            # a non-null, misaligned address (never dereferenced)
GOOD = 0x7f0000000000   # a non-null, 16-byte aligned address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fgq.LIB_PATH):
        pytest.skip("libfgq.so not built")
    return fgq.load()


def test_every_declared_symbol_is_exported(lib):
    names = fgq.declared_symbols()
    assert {"fgq_quantize_g64", "fgq_kv_append", "fgq_decode_attn_q4kv", "fgq_dequant_gemm",
            "fgq_dequant_gemm_packed", "fgq_kv_append_ld", "fgq_decode_attn_q4kv_ld",
            "fgq_decode_attn_q4kv_noalloc"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fgq.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported


def test_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "fgq.h"\nint main(void){ fgq_kv_cache kv; (void)kv; return fgq_abi_version() != 3; }\n')
    inc = os.path.join(os.path.dirname(fgq.HEADER_PATH))
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-c", str(src), "-I", inc, "-o",
                           str(tmp_path / "t.o")])


def test_version_and_status_strings(lib):
    assert fgq.fgq_abi_version() == 3
    assert fgq.status_string(fgq.FGQ_OK) == "ok"
    codes = [fgq.FGQ_ERR_INVALID_ARG, fgq.FGQ_ERR_SHAPE, fgq.FGQ_ERR_ALIGN, fgq.FGQ_ERR_CAPACITY,
             fgq.FGQ_ERR_WORKSPACE, fgq.FGQ_ERR_DTYPE, fgq.FGQ_ERR_DEVICE, fgq.FGQ_ERR_UNSUPPORTED]
    texts = {fgq.status_string(c) for c in codes}
    assert len(texts) == len(codes)
    assert fgq.status_string(12345) == "unknown status"


def _status(call):
    try:
        call()
    except fgq.FgqError as e:
        return e.status
    return fgq.FGQ_OK


def test_quantize_validation(lib):
    q = fgq.fgq_quantize_g64
    assert _status(lambda: q(GOOD, 4, 96, 96, GOOD, GOOD, 0)) == fgq.FGQ_ERR_SHAPE
    assert "multiple of 64" in fgq.last_error()
    assert _status(lambda: q(GOOD, -1, 64, 64, GOOD, GOOD, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: q(GOOD, 4, 128, 64, GOOD, GOOD, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: q(0, 4, 64, 64, GOOD, GOOD, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: q(BAD, 4, 64, 64, GOOD, GOOD, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: q(GOOD, 4, 64, 68, GOOD, GOOD, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: q(0, 0, 64, 64, 0, 0, 0)) == fgq.FGQ_OK          # empty: no-op


def _kv(batch=2, heads=2, head_dim=128, cap=16, ptr=GOOD):
    return fgq.fgq_kv_cache(ptr, ptr, ptr, ptr, batch, heads, head_dim, cap)


def test_kv_append_validation(lib):
    a = fgq.fgq_kv_append
    assert _status(lambda: a(_kv(), GOOD, GOOD, 10, 7, 0)) == fgq.FGQ_ERR_CAPACITY
    assert _status(lambda: a(_kv(), GOOD, GOOD, -1, 1, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: a(_kv(head_dim=96), GOOD, GOOD, 0, 1, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: a(_kv(head_dim=256), GOOD, GOOD, 0, 1, 0)) == fgq.FGQ_ERR_UNSUPPORTED
    assert _status(lambda: a(_kv(ptr=BAD), GOOD, GOOD, 0, 1, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: a(_kv(ptr=0), GOOD, GOOD, 0, 1, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: a(_kv(), BAD, GOOD, 0, 1, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: a(_kv(), GOOD, GOOD, 16, 0, 0)) == fgq.FGQ_OK      # n_new = 0 at the end: no-op
    assert _status(lambda: a(_kv(batch=0), 0, 0, 0, 4, 0)) == fgq.FGQ_OK
    null_kv = ctypes.cast(None, ctypes.POINTER(fgq.fgq_kv_cache))
    assert lib.fgq_kv_append(null_kv, GOOD, GOOD, 0, 1, None) == fgq.FGQ_ERR_INVALID_ARG


def test_attention_validation_and_workspace(lib):
    d = fgq.fgq_decode_attn_q4kv
    assert _status(lambda: d(_kv(), GOOD, 0, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: d(_kv(), GOOD, 17, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_CAPACITY
    assert _status(lambda: d(_kv(), GOOD, 4, 0.0, GOOD, 7, 0, 0, 0)) == fgq.FGQ_ERR_DTYPE
    assert _status(lambda: d(_kv(), GOOD, 4, float("nan"), GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: d(_kv(), BAD, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_ALIGN
    # a shape that needs a workspace (few sequences, long context)
    B, H, D, L = 1, 2, 128, 4096
    need = fgq.fgq_decode_attn_ws_bytes(B, H, D, L)
    assert need > 0 and need % 16 == 0
    kv = _kv(B, H, D, L)
    assert _status(lambda: d(kv, GOOD, L, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_WORKSPACE
    assert _status(lambda: d(kv, GOOD, L, 0.0, GOOD, 0, GOOD, need - 16, 0)) == fgq.FGQ_ERR_WORKSPACE
    assert _status(lambda: d(kv, GOOD, L, 0.0, GOOD, 0, BAD, need, 0)) == fgq.FGQ_ERR_ALIGN
    # many sequences: one split, no workspace
    assert fgq.fgq_decode_attn_ws_bytes(144, 96, 128, 544) == 0
    assert fgq.fgq_decode_attn_ws_bytes(0, 96, 128, 544) == 0
    # the split rule: once the waves cover every wave slot (2048 on 256 CUs at
    # two waves per SIMD), a sequence is split only into parts of >= 768
    # tokens per wave; with fewer waves, >= 256 tokens per wave.  From 1024
    # positions, fewer than 8192 pairs take four waves per pair (one
    # workgroup), which counts four times towards the 8192-wave target.
    ws = lambda B, H, L, n: B * H * n * (128 + 4) * 4
    assert fgq.fgq_decode_attn_ws_bytes(64, 32, 128, 530) == 0               # 2048 pairs: none
    assert fgq.fgq_decode_attn_ws_bytes(60, 32, 128, 530) == ws(60, 32, 530, 2)
    assert fgq.fgq_decode_attn_ws_bytes(8, 32, 128, 1023) == ws(8, 32, 1023, 3)  # one wave per item
    assert fgq.fgq_decode_attn_ws_bytes(8, 32, 128, 1024) == 0               # 256 pairs x 4 waves, one split
    assert fgq.fgq_decode_attn_ws_bytes(32, 96, 128, 2047) == 0              # 3072 pairs x 4 waves
    assert fgq.fgq_decode_attn_ws_bytes(32, 96, 128, 4128) == 0
    assert fgq.fgq_decode_attn_ws_bytes(16, 32, 128, 16416) == ws(16, 32, 16416, 4)  # 512 x 4 waves x 4
    assert fgq.fgq_decode_attn_ws_bytes(96, 56, 128, 1040) == 0              # 5376 pairs, 1040 tokens


def test_gqa_attention_validation_and_workspace(lib):
    a = fgq.fgq_decode_attn_gqa_q4kv
    kv = _kv(batch=2, heads=2, head_dim=128, cap=16)
    assert _status(lambda: a(kv, GOOD, 3, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE      # 3 % 2 != 0
    assert _status(lambda: a(kv, GOOD, 1, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE      # fewer than kv heads
    assert _status(lambda: a(kv, GOOD, -2, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: a(kv, GOOD, 66, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_UNSUPPORTED  # R = 33
    assert _status(lambda: a(_kv(heads=0), GOOD, 4, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: a(kv, GOOD, 8, 0, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: a(kv, GOOD, 8, 17, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_CAPACITY
    assert _status(lambda: a(kv, GOOD, 8, 4, 0.0, GOOD, 3, 0, 0, 0)) == fgq.FGQ_ERR_DTYPE
    assert _status(lambda: a(kv, GOOD, 8, 4, float("nan"), GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: a(kv, BAD, 8, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: a(kv, GOOD, 8, 4, 0.0, 0, 0, 0, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: a(_kv(head_dim=96), GOOD, 8, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: a(_kv(batch=0), 0, 8, 4, 0.0, 0, 0, 0, 0, 0)) == fgq.FGQ_OK
    huge = _kv(batch=1, heads=1, head_dim=128, cap=2 ** 27)     # 2^27 positions x 64 code bytes = 2^33
    assert _status(lambda: a(huge, GOOD, 8, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_UNSUPPORTED
    # few sequences and K/V heads over a long context need split states
    B, Hq, Hkv, D, L = 2, 32, 8, 128, 16384
    need = fgq.fgq_decode_attn_gqa_ws_bytes(B, Hq, Hkv, D, L)
    assert need > 0 and need % 16 == 0
    big = _kv(B, Hkv, D, L)
    assert _status(lambda: a(big, GOOD, Hq, L, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_WORKSPACE
    assert _status(lambda: a(big, GOOD, Hq, L, 0.0, GOOD, 0, GOOD, need - 16, 0)) == fgq.FGQ_ERR_WORKSPACE
    assert _status(lambda: a(big, GOOD, Hq, L, 0.0, GOOD, 0, BAD, need, 0)) == fgq.FGQ_ERR_ALIGN
    # one query head per K/V head is the multi-head call, with its workspace
    assert fgq.fgq_decode_attn_gqa_ws_bytes(1, 2, 2, 128, 4096) == fgq.fgq_decode_attn_ws_bytes(1, 2, 128, 4096)
    assert fgq.fgq_decode_attn_gqa_ws_bytes(2, 30, 8, 128, 64) == 0        # not a multiple
    assert fgq.fgq_decode_attn_gqa_ws_bytes(2, 8 * 33, 8, 128, 64) == 0    # group of 33


def test_topk_attention_validation(lib):
    t = fgq.fgq_decode_attn_topk_q4kv
    assert _status(lambda: t(_kv(), GOOD, 0, 1, 0.0, GOOD, 0, None, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: t(_kv(), GOOD, 17, 1, 0.0, GOOD, 0, None, 0)) == fgq.FGQ_ERR_CAPACITY
    assert _status(lambda: t(_kv(), GOOD, 4, 0, 0.0, GOOD, 0, None, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: t(_kv(), GOOD, 4, -3, 0.0, GOOD, 0, None, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: t(_kv(), GOOD, 4, 2, 0.0, GOOD, 7, None, 0)) == fgq.FGQ_ERR_DTYPE
    assert _status(lambda: t(_kv(), GOOD, 4, 2, float("inf"), GOOD, 0, None, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: t(_kv(), BAD, 4, 2, 0.0, GOOD, 0, None, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: t(_kv(), GOOD, 4, 2, 0.0, GOOD, 0, BAD, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: t(_kv(), 0, 4, 2, 0.0, GOOD, 0, None, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: t(_kv(head_dim=96), GOOD, 4, 2, 0.0, GOOD, 0, None, 0)) == fgq.FGQ_ERR_SHAPE
    # the selection state of one (sequence, head) must fit on chip: kv_len <= 65536
    assert fgq.FGQ_TOPK_MAX_POSITIONS == 65536
    cap = 70000
    assert _status(lambda: t(_kv(cap=cap), GOOD, 65537, 1, 0.0, GOOD, 0, None, 0)) == fgq.FGQ_ERR_UNSUPPORTED
    assert _status(lambda: t(_kv(cap=cap), GOOD, 70000, 7000, 0.0, GOOD, 0, None, 0)) == fgq.FGQ_ERR_UNSUPPORTED
    # empty batch: nothing to do, no pointer is touched
    assert _status(lambda: t(_kv(batch=0), 0, 4, 2, 0.0, 0, 0, None, 0)) == fgq.FGQ_OK


def test_prefill_attention_validation(lib):
    p = fgq.fgq_prefill_attn_f16
    assert _status(lambda: p(GOOD, GOOD, GOOD, 2, 16, 2, 96, 0.0, GOOD, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: p(GOOD, GOOD, GOOD, 2, 16, 2, 256, 0.0, GOOD, 0, 0)) == fgq.FGQ_ERR_UNSUPPORTED
    assert _status(lambda: p(GOOD, GOOD, GOOD, -1, 16, 2, 128, 0.0, GOOD, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: p(GOOD, GOOD, GOOD, 2, 16, 2, 128, 0.0, GOOD, 5, 0)) == fgq.FGQ_ERR_DTYPE
    assert _status(lambda: p(GOOD, GOOD, GOOD, 2, 16, 2, 128, float("nan"), GOOD, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: p(GOOD, GOOD, GOOD, 70000, 16, 2, 128, 0.0, GOOD, 0, 0)) == fgq.FGQ_ERR_SHAPE
    # within 2^40 elements, but 65535 x 65535 workgroups of one row block overflow the 32-bit numbering
    assert _status(lambda: p(GOOD, GOOD, GOOD, 65535, 1, 65535, 64, 0.0, GOOD, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: p(GOOD, BAD, GOOD, 2, 16, 2, 128, 0.0, GOOD, 0, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: p(GOOD, GOOD, 0, 2, 16, 2, 128, 0.0, GOOD, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: p(0, 0, 0, 2, 0, 2, 128, 0.0, 0, 0, 0)) == fgq.FGQ_OK     # empty prompt


def test_canonical_gemm_signature_takes_the_quantiser_layout(lib):
    """fgq_dequant_gemm takes the quantiser's own layout: uint8 codes
    [K][N/2] and the metadata words [K][N/64], as const pointers."""
    import re
    text = open(fgq.HEADER_PATH).read()
    m = re.search(r"fgq_status fgq_dequant_gemm\((.*?)\);", text, re.S)
    params = [p.strip() for p in " ".join(m.group(1).split()).split(",")]
    assert params == ["const void *x_f16", "int32_t g", "int32_t m", "int64_t K", "int64_t N",
                      "const uint8_t *w_codes", "const void *w_meta", "void *y", "int32_t y_dtype", "void *ws",
                      "size_t ws_bytes", "void *stream"]


def test_canonical_gemm_validation(lib):
    gm = fgq.fgq_dequant_gemm
    # the canonical layout takes K in multiples of 64 (the packed one: 32)
    assert _status(lambda: gm(GOOD, 4, 1, 96, 64, GOOD, GOOD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: gm(GOOD, 4, 1, 64, 96, GOOD, GOOD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: gm(GOOD, 4, 1, 64, 2 ** 28, GOOD, GOOD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: gm(GOOD, 4, 1, 64, 64, GOOD, GOOD, GOOD, 5, 0, 0, 0)) == fgq.FGQ_ERR_DTYPE
    assert _status(lambda: gm(GOOD, 4, -1, 64, 64, GOOD, GOOD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: gm(GOOD, 4, 1, 64, 64, GOOD, BAD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: gm(GOOD, 4, 1, 64, 64, GOOD, 0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: gm(0, 4, 0, 64, 64, 0, 0, 0, 0, 0, 0, 0)) == fgq.FGQ_OK   # empty block
    need = fgq.fgq_dequant_gemm_ws_bytes(144, 12288, 12288)
    assert _status(lambda: gm(GOOD, 36, 4, 12288, 12288, GOOD, GOOD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_WORKSPACE
    assert _status(lambda: gm(GOOD, 36, 4, 12288, 12288, GOOD, GOOD, GOOD, 0, BAD, need, 0)) == fgq.FGQ_ERR_ALIGN


def test_strided_append_and_attention_validation(lib):
    a = fgq.fgq_kv_append_ld
    h = 2 * 128
    assert _status(lambda: a(_kv(), GOOD, GOOD, h - 8, 0, 1, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: a(_kv(), GOOD, GOOD, 3 * h + 4, 0, 1, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: a(_kv(), GOOD, GOOD, 3 * h, 10, 7, 0)) == fgq.FGQ_ERR_CAPACITY
    assert _status(lambda: a(_kv(), BAD, GOOD, 3 * h, 0, 1, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: a(_kv(), GOOD, GOOD, 3 * h, 0, 0, 0)) == fgq.FGQ_OK          # nothing to append
    d = fgq.fgq_decode_attn_q4kv_ld
    assert _status(lambda: d(_kv(), GOOD, h - 8, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: d(_kv(), GOOD, 3 * h + 4, 4, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: d(_kv(), GOOD, 3 * h, 17, 0.0, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_CAPACITY
    assert _status(lambda: d(_kv(), GOOD, 3 * h, 4, 0.0, GOOD, 3, 0, 0, 0)) == fgq.FGQ_ERR_DTYPE


def test_noalloc_attention_validation_and_scratch_bound(lib):
    """The allocation-free entry validates like the workspace one, and the
    split states of every plan fit its fixed scratch: the plan only splits
    when batch * heads < 8192, into at most ceil(8192 / (batch * heads))
    parts, so batch * heads * splits * (head_dim + 4) * 4 < 2 * 8192 * 132 * 4."""
    n = fgq.fgq_decode_attn_q4kv_noalloc
    assert _status(lambda: n(_kv(), GOOD, 0, 0.0, GOOD, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: n(_kv(), GOOD, 17, 0.0, GOOD, 0, 0)) == fgq.FGQ_ERR_CAPACITY
    assert _status(lambda: n(_kv(), GOOD, 4, 0.0, GOOD, 9, 0)) == fgq.FGQ_ERR_DTYPE
    assert _status(lambda: n(_kv(), BAD, 4, 0.0, GOOD, 0, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: n(_kv(), GOOD, 4, float("nan"), GOOD, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: n(_kv(batch=0), 0, 4, 0.0, 0, 0, 0)) == fgq.FGQ_OK
    worst = 0
    for bh in list(range(1, 300)) + [511, 512, 1000, 2047, 2048, 4095, 4096, 6000, 8191, 8192, 20000]:
        for D in (64, 128):
            for L in (1, 255, 256, 700, 4100, 16416, 100000):
                worst = max(worst, fgq.fgq_decode_attn_ws_bytes(bh, 1, D, L))
    assert 0 < worst <= 16383 * 132 * 4 <= fgq.FGQ_NOALLOC_SCRATCH_BYTES


def test_attention_rejects_more_than_2_31_work_items(lib):
    """batch * heads beyond the kernel's 32-bit item index is a shape error
    on the host, not a wrapped grid."""
    d = fgq.fgq_decode_attn_q4kv
    big = _kv(batch=2 ** 20, heads=2 ** 12, cap=16)
    assert _status(lambda: d(big, GOOD, 4, 0.0, GOOD, 0, GOOD, 2 ** 40, 0)) == fgq.FGQ_ERR_SHAPE


def test_gemm_validation_and_workspace(lib):
    gm = fgq.fgq_dequant_gemm_packed
    assert _status(lambda: gm(GOOD, 4, 1, 48, 64, GOOD, GOOD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: gm(GOOD, 4, 1, 64, 96, GOOD, GOOD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: gm(GOOD, 4, 1, 64, 64, GOOD, GOOD, GOOD, 5, 0, 0, 0)) == fgq.FGQ_ERR_DTYPE
    assert _status(lambda: gm(GOOD, -4, 1, 64, 64, GOOD, GOOD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: gm(BAD, 4, 1, 64, 64, GOOD, GOOD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: gm(GOOD, 4, 1, 64, 64, 0, GOOD, GOOD, 0, 0, 0, 0)) == fgq.FGQ_ERR_INVALID_ARG
    assert _status(lambda: gm(0, 0, 4, 64, 64, 0, 0, 0, 0, 0, 0, 0)) == fgq.FGQ_OK   # empty block
    need = fgq.fgq_dequant_gemm_ws_bytes(144, 12288, 12288)
    assert need > 0 and need % 16 == 0
    assert _status(lambda: gm(GOOD, 36, 4, 12288, 12288, GOOD, GOOD, GOOD, 0, GOOD, need - 4, 0)) == \
        fgq.FGQ_ERR_WORKSPACE
    pk = fgq.fgq_pack_weight_g64
    assert _status(lambda: pk(GOOD, GOOD, 48, 64, GOOD, GOOD, 0)) == fgq.FGQ_ERR_SHAPE
    assert _status(lambda: pk(GOOD, GOOD, 64, 64, BAD, GOOD, 0)) == fgq.FGQ_ERR_ALIGN
    assert _status(lambda: pk(0, 0, 0, 64, 0, 0, 0)) == fgq.FGQ_OK


def test_gemm_workspace_covers_every_workload():
    import synth
    for w in synth.WORKLOADS.values():
        for K, N in w.weights:
            need = fgq.fgq_dequant_gemm_ws_bytes(w.batch, K, N)
            assert need % 16 == 0
            assert need <= 64 * w.batch * N * 4        # at most 64 split-K partial tiles


def test_binding_constants_match_the_header():
    import re
    text = open(fgq.HEADER_PATH).read()
    defs = dict(re.findall(r"^#define (FGQ_[A-Z0-9_]+) +\(?(-?[0-9]+)\)? *(?:/\*.*)?$", text, re.M))
    names = ["FGQ_OK", "FGQ_ERR_INVALID_ARG", "FGQ_ERR_SHAPE", "FGQ_ERR_ALIGN", "FGQ_ERR_CAPACITY",
             "FGQ_ERR_WORKSPACE", "FGQ_ERR_DTYPE", "FGQ_ERR_DEVICE", "FGQ_ERR_UNSUPPORTED", "FGQ_DTYPE_F32",
             "FGQ_DTYPE_F16", "FGQ_GQA_MAX_GROUP", "FGQ_TOPK_MAX_POSITIONS"]
    for n in names:
        assert n in defs, n
        assert getattr(fgq, n) == int(defs[n]), n
    assert "FGQ_NOALLOC_SCRATCH_BYTES ((size_t)9 << 20)" in text and fgq.FGQ_NOALLOC_SCRATCH_BYTES == 9 << 20
