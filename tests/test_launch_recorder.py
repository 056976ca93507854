"""Launch plans and argument marshalling of every entry point, on the CPU.

The library's sources are compiled host-only (no device code) and linked
against tests/launch_recorder/recorder.cpp instead of the HIP runtime: every
kernel launch is recorded (kernel, grid, block, dynamic LDS, stream and, for
kernels whose parameter types are declared here, the argument values) instead
of run.  Device pointers are made-up aligned addresses; nothing is
dereferenced and no kernel body executes.  This checks what the host side
decides and passes: which kernel instantiation a shape takes, its grid, the
split-K and split-softmax merge launches and their workspace, the default
softmax scale, the caller's stream, and the device address of the
allocation-free entry's scratch array.
"""
import concurrent.futures
import ctypes
import math
import os
import subprocess

import pytest

import int4_group_quantized_fgq_amd as fgq
from int4_group_quantized_fgq_amd import build as hip_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
LOG2E = 1.4426950408889634
STREAM = 0x5A5A00
# made-up device addresses, 256-byte aligned and distinct
Q, K, V, OUT, WS, X, Y, WC, WM, SEL = (0x100000000 * (i + 1) for i in range(10))


def _run(cmd, timeout=600):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=timeout)
    return res.returncode, res.stdout


@pytest.fixture(scope="module")
def rec(tmp_path_factory):
    tmp = tmp_path_factory.mktemp("recorder")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(hip_build.HERE, "csrc")]
    jobs = []
    for src in hip_build.sources():
        obj = str(tmp / (os.path.basename(src) + ".o"))
        jobs.append(([HIPCC] + hip_build.HIPCC_FLAGS + hip_build.EXTRA_FLAGS.get(os.path.basename(src), []) +
                     ["--cuda-host-only", "-fPIC"] + inc + ["-c", src, "-o", obj], obj))
    rec_obj = str(tmp / "recorder.o")
    jobs.append(([CLANGXX, "-std=c++17", "-O1", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                  "-c", os.path.join(HERE, "launch_recorder", "recorder.cpp"), "-o", rec_obj], rec_obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: _run(j[0]), jobs))
    for (rc, out), (cmd, _) in zip(results, jobs):
        assert rc == 0, " ".join(cmd) + "\n" + out
    objs = [o for _, o in jobs]
    # each translation unit's constructor names its (absent) device code
    # object; point those symbols at a dummy
    rc, out = _run(["nm", "-u"] + objs)
    assert rc == 0, out
    fatbins = sorted({ln.split()[-1] for ln in out.splitlines() if "__hip_fatbin" in ln})
    assert fatbins
    lib = str(tmp / "libfgq_recorded.so")
    rc, out = _run([CLANGXX, "-shared", "-fPIC", "-Wl,--no-undefined", "-o", lib] + objs +
                   ["-Wl,--defsym,%s=rec_count" % f for f in fatbins] + ["-lpthread"])
    assert rc == 0, out
    r = fgq.declare(ctypes.CDLL(lib))
    r.rec_get.argtypes = [ctypes.c_int, ctypes.c_char_p, ctypes.c_int, ctypes.POINTER(ctypes.c_uint),
                          ctypes.POINTER(ctypes.c_uint), ctypes.POINTER(ctypes.c_size_t),
                          ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_uint64), ctypes.c_int]
    r.rec_decode.argtypes = [ctypes.c_char_p, ctypes.c_char_p]
    for f in ("rec_device_address", "rec_host_stand_in"):
        getattr(r, f).argtypes = [ctypes.c_char_p]
        getattr(r, f).restype = ctypes.c_uint64
    assert r.rec_modules() == len(fatbins)
    return r


def _demangle(names):
    rc, out = _run(["c++filt"] + names) if names else (0, "")
    assert rc == 0
    return out.splitlines()


def _launches(r):
    """Run nothing; return the launches recorded since the last reset."""
    n = r.rec_count()
    raw = []
    for i in range(n):
        name = ctypes.create_string_buffer(512)
        g, b = (ctypes.c_uint * 3)(), (ctypes.c_uint * 3)()
        lds, st = ctypes.c_size_t(), ctypes.c_void_p()
        args = (ctypes.c_uint64 * 32)()
        na = r.rec_get(i, name, 512, g, b, ctypes.byref(lds), ctypes.byref(st), args, 32)
        raw.append((name.value.decode(), tuple(g), tuple(b), lds.value, st.value or 0, list(args[:na])))
    names = _demangle([x[0] for x in raw])
    return [dict(kernel=nm, grid=x[1], block=x[2], lds=x[3], stream=x[4], args=x[5]) for nm, x in zip(names, raw)]


def _call(r, decoders, fn, *args):
    r.rec_reset()
    for frag, types in decoders:
        r.rec_decode(frag.encode(), types.encode())
    st = fn(*args)
    assert st == fgq.FGQ_OK, (st, r.fgq_last_error())
    return _launches(r)


def _f32(bits):
    return ctypes.c_float.from_buffer(ctypes.c_uint32(bits)).value


def _kv(batch, heads, head_dim, capacity):
    return fgq.fgq_kv_cache(K, V, K + 0x80000000, V + 0x80000000, batch, heads, head_dim, capacity)


# attn_split_kernel(k_codes, k_meta, v_codes, v_meta, q, ld_q, heads, capacity, kv_len, n_split,
#                   tok_per_split, total, sl2, ws, out, f16)
ATTN_ARGS = ("attn_split_kernel", "pppppliiiiiifppi")


@pytest.mark.parametrize("B,H,D,L,chunk,wpi", [(144, 96, 128, 530, 6, 1), (144, 96, 128, 255, 4, 1),
                                               (8, 32, 128, 1024, 6, 4), (32, 96, 128, 4100, 6, 4),
                                               (3, 5, 64, 77, 4, 1)])
def test_decode_attention_plan_and_arguments(rec, B, H, D, L, chunk, wpi):
    kv = _kv(B, H, D, L + 40)
    ws_bytes = rec.fgq_decode_attn_ws_bytes(B, H, D, L)
    got = _call(rec, [ATTN_ARGS], rec.fgq_decode_attn_q4kv, ctypes.byref(kv), Q, L, 0.0, OUT,
                fgq.FGQ_DTYPE_F16, WS if ws_bytes else 0, ws_bytes, STREAM)
    main = got[0]
    assert "attn_split_kernel<%d, %d, %d>" % (D, chunk, wpi) in main["kernel"], main["kernel"]
    a = main["args"]
    assert a[:5] == [K, K + 0x80000000, V, V + 0x80000000, Q]
    assert a[5] == H * D and a[6] == H and a[7] == L + 40 and a[8] == L   # ld_q, heads, capacity, kv_len
    n_split, per, total = a[9], a[10], a[11]
    assert total == B * H * n_split and (n_split - 1) * per < L <= n_split * per
    assert ws_bytes == (0 if n_split == 1 else B * H * n_split * (D + 4) * 4)
    assert _f32(a[12]) == pytest.approx(LOG2E / math.sqrt(D), rel=1e-6)
    assert a[13] == (WS if n_split > 1 else 0) and a[14] == OUT and a[15] == 1
    assert main["grid"] == ((total if wpi > 1 else (total + 3) // 4), 1, 1) and main["block"] == (256, 1, 1)
    assert all(x["stream"] == STREAM for x in got)
    if n_split > 1:
        assert len(got) == 2 and "attn_merge_kernel" in got[1]["kernel"] and got[1]["grid"][0] == B * H
    else:
        assert len(got) == 1


def test_allocation_free_attention_passes_the_scratch_device_address(rec):
    B, H, D, L = 3, 2, 128, 2600            # splits, so the partial states go to the scratch array
    kv = _kv(B, H, D, L)
    q0 = rec.rec_symbol_queries()
    for _ in range(2):
        got = _call(rec, [ATTN_ARGS], rec.fgq_decode_attn_q4kv_noalloc, ctypes.byref(kv), Q, L, 0.25, OUT,
                    fgq.FGQ_DTYPE_F32, STREAM)
        dev = rec.rec_device_address(b"scratch")
        assert dev and got[0]["args"][13] == dev != rec.rec_host_stand_in(b"scratch")
        assert got[0]["args"][9] > 1 and "attn_merge_kernel" in got[1]["kernel"]
        assert _f32(got[0]["args"][12]) == pytest.approx(0.25 * LOG2E, rel=1e-6)
    assert rec.rec_symbol_queries() - q0 <= 1    # looked up once per device, then kept


# prefill_attn_kernel(q, k, v, S, H, sl2, out, out_f16)
PREFILL_ARGS = ("prefill_attn_kernel", "pppiifpi")


@pytest.mark.parametrize("B,S,H,D,nw", [(8, 512, 96, 128, 4), (2, 600, 3, 128, 4), (32, 200, 96, 128, 8),
                                        (2, 700, 2, 64, 8), (1, 1030, 2, 128, 12), (1, 1, 1, 64, 4)])
def test_prefill_launch_by_prompt_length(rec, B, S, H, D, nw):
    got = _call(rec, [PREFILL_ARGS], rec.fgq_prefill_attn_f16, Q, K, V, B, S, H, D, 0.0, OUT,
                fgq.FGQ_DTYPE_F32, STREAM)
    assert len(got) == 1
    g = got[0]
    assert "prefill_attn_kernel<%d, %d>" % (D, nw) in g["kernel"], g["kernel"]
    rows = 32 * nw
    assert g["grid"] == ((S + rows - 1) // rows, H, B) and g["block"] == (64 * nw, 1, 1)
    a = g["args"]
    assert a[:3] == [Q, K, V] and a[3] == S and a[4] == H and a[6] == OUT and a[7] == 0
    assert _f32(a[5]) == pytest.approx(LOG2E / math.sqrt(D), rel=1e-6)
    assert g["stream"] == STREAM


@pytest.mark.parametrize("M,Kd,N", [(144, 12288, 36864), (144, 12288, 12288), (64, 4096, 4096), (4, 128, 256)])
def test_gemm_launches_and_split_k_workspace(rec, M, Kd, N):
    for entry in (rec.fgq_dequant_gemm_packed, rec.fgq_dequant_gemm):
        ws_bytes = rec.fgq_dequant_gemm_ws_bytes(M, Kd, N)
        got = _call(rec, [], entry, X, M, 1, Kd, N, WC, WM, Y, fgq.FGQ_DTYPE_F16, WS if ws_bytes else 0,
                    ws_bytes, STREAM)
        kernels = [x["kernel"] for x in got]
        assert "dq_gemm_kernel" in kernels[0], kernels
        assert all(x["stream"] == STREAM for x in got)
        # a split-K plan writes partial tiles and reduces them in a second launch
        assert any("splitk_reduce_kernel" in k for k in kernels) == (ws_bytes > 0), (kernels, ws_bytes)
        assert len(got) == 1 + (ws_bytes > 0)
        assert got[0]["block"] == (512, 1, 1)


def test_gqa_and_top_k_launches(rec):
    B, R, KVH, D, L = 2, 4, 8, 128, 16400
    kv = _kv(B, KVH, D, L)
    ws_bytes = rec.fgq_decode_attn_gqa_ws_bytes(B, R * KVH, KVH, D, L)
    got = _call(rec, [], rec.fgq_decode_attn_gqa_q4kv, ctypes.byref(kv), Q, R * KVH, L, 0.0, OUT,
                fgq.FGQ_DTYPE_F32, WS if ws_bytes else 0, ws_bytes, STREAM)
    assert "attn_gqa_kernel" in got[0]["kernel"]
    assert (len(got) == 2 and "attn_gqa_merge_kernel" in got[1]["kernel"]) == (ws_bytes > 0)
    # top-K: the wave kernel up to 2048 positions, the workgroup kernel below
    # the LDS limit, the 16-bit-key long kernel beyond; each sizes its LDS at
    # launch, within the 160 KB of a workgroup
    for L, kern in ((530, "attn_topk_wave_kernel"), (16416, "attn_topk_kernel<"), (40000, "attn_topk_long_kernel")):
        kv = _kv(4, 8, 128, L)
        got = _call(rec, [], rec.fgq_decode_attn_topk_q4kv, ctypes.byref(kv), Q, L, (L + 9) // 10, 0.0, OUT,
                    fgq.FGQ_DTYPE_F32, SEL, STREAM)
        assert len(got) == 1 and kern in got[0]["kernel"], (L, got[0]["kernel"])
        assert 0 < got[0]["lds"] <= 160 * 1024 and got[0]["stream"] == STREAM


def test_quantiser_append_and_pack_launches(rec):
    got = _call(rec, [], rec.fgq_quantize_g64, X, 100, 192, 200, WC, WM, STREAM)
    assert len(got) == 1 and "quantize_g64_kernel" in got[0]["kernel"]
    assert got[0]["grid"] == ((100 * 192 // 64 + 31) // 32, 1, 1) and got[0]["stream"] == STREAM
    kv = _kv(2, 3, 128, 600)
    for n_new in (1, 512):
        got = _call(rec, [], rec.fgq_kv_append, ctypes.byref(kv), X, Y, 7, n_new, STREAM)
        assert len(got) == 1 and "kv_append_kernel" in got[0]["kernel"] and got[0]["stream"] == STREAM
    got = _call(rec, [], rec.fgq_pack_weight_g64, WC, WM, 256, 512, X, Y, STREAM)
    assert [k for k in ("pack_codes_kernel", "pack_exponent_kernel", "pack_meta_kernel")
            if any(k in x["kernel"] for x in got)] == ["pack_codes_kernel", "pack_exponent_kernel",
                                                        "pack_meta_kernel"]


def test_rejected_calls_launch_nothing(rec):
    kv = _kv(2, 2, 96, 64)                         # head_dim 96: rejected before any launch
    rec.rec_reset()
    st = rec.fgq_decode_attn_q4kv(ctypes.byref(kv), Q, 10, 0.0, OUT, fgq.FGQ_DTYPE_F32, 0, 0, STREAM)
    assert st != fgq.FGQ_OK and rec.rec_count() == 0
    st = rec.fgq_prefill_attn_f16(Q, K, V, 65535, 1, 65535, 64, 0.0, OUT, 0, STREAM)
    assert st == fgq.FGQ_ERR_SHAPE and rec.rec_count() == 0
    ws_bytes = rec.fgq_dequant_gemm_ws_bytes(144, 12288, 12288)
    if ws_bytes:
        st = rec.fgq_dequant_gemm_packed(X, 144, 1, 12288, 12288, WC, WM, Y, 1, WS, ws_bytes - 1, STREAM)
        assert st != fgq.FGQ_OK and rec.rec_count() == 0
