"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status before
touching any device memory (all pointers here are null or fake)."""
import ctypes
import math
import os
import re

import pytest

from attention_pass_cascaded_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rf_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rf_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("librfattn.so is not built; run python -m attention_pass_cascaded_amd.build")
    return B.load_library()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(4):
        assert lib.rf_status_string(code)
    assert lib.rf_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    assert lib.rf_splitkv_workspace_bytes(16, 32, 1, 128, 64) == 16 * 32 * 64 * 129 * 4
    assert lib.rf_splitkv_workspace_bytes(1, 1, 1, 64, 0) == 0
    assert lib.rf_splitkv_workspace_bytes(-1, 1, 1, 64, 1) == 0


FAKE = ctypes.c_void_p(4096)   # aligned, never dereferenced: validation fails first


def fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=2, Hkv=2, Nq=8, Nk=8, D=64,
             scale=0.125, mask=0, window=0, rope=0.0, dtype=1)
    a.update(kw)
    return lib.rf_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                           a["Nq"], a["Nk"], a["D"], a["scale"], a["mask"], a["window"], a["rope"],
                           a["dtype"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(Hq=3, Hkv=2), B.RF_ERR_INVALID_ARG, "multiple"),
    (dict(Hkv=0), B.RF_ERR_INVALID_ARG, ">= 1"),
    (dict(B=-1), B.RF_ERR_INVALID_ARG, "negative"),
    (dict(Nk=-5), B.RF_ERR_INVALID_ARG, "negative"),
    (dict(dtype=7), B.RF_ERR_INVALID_ARG, "dtype"),
    (dict(mask=3), B.RF_ERR_INVALID_ARG, "mask"),
    (dict(mask=2, window=0), B.RF_ERR_INVALID_ARG, "window"),
    (dict(scale=-1.0), B.RF_ERR_INVALID_ARG, "scale"),
    (dict(scale=math.inf), B.RF_ERR_INVALID_ARG, "scale"),
    (dict(rope=math.nan), B.RF_ERR_INVALID_ARG, "rope"),
    (dict(D=96), B.RF_ERR_UNSUPPORTED, "96"),
    (dict(D=256), B.RF_ERR_UNSUPPORTED, "256"),
    (dict(q=None), B.RF_ERR_INVALID_ARG, "null"),
    (dict(k=None), B.RF_ERR_INVALID_ARG, "null"),
    (dict(q=ctypes.c_void_p(4098)), B.RF_ERR_INVALID_ARG, "aligned"),
    (dict(o=None), B.RF_ERR_INVALID_ARG, "required"),
    (dict(lse=None), B.RF_ERR_INVALID_ARG, "required"),
    # one KV head of 2^31 bytes (bf16, D = 128) is one key row too many
    (dict(D=128, Nk=(1 << 31) // 256, dtype=2), B.RF_ERR_UNSUPPORTED, "2 GiB"),
    (dict(D=64, Nk=(1 << 31) // 256, dtype=0), B.RF_ERR_UNSUPPORTED, "2 GiB"),
])
def test_fwd_rejects_bad_arguments(lib, kw, status, needle):
    assert fwd(lib, **kw) == status
    assert needle in lib.rf_last_error().decode()


def test_empty_problem_is_ok_without_touching_memory(lib):
    assert fwd(lib, q=None, o=None, lse=None, Nq=0) == B.RF_OK
    assert fwd(lib, q=None, k=None, v=None, o=None, lse=None, B=0) == B.RF_OK


def test_splitkv_and_merge_reject_bad_arguments(lib):
    st = lib.rf_attn_splitkv_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 1, 100, 128, 0.1, 0, 0, 0.0,
                                 0, 2, None)
    assert st == B.RF_ERR_INVALID_ARG and b"num_splits" in lib.rf_last_error()
    st = lib.rf_attn_splitkv_fwd(FAKE, FAKE, FAKE, None, FAKE, 1, 4, 1, 1, 100, 128, 0.1, 0, 0, 0.0,
                                 4, 2, None)
    assert st == B.RF_ERR_INVALID_ARG and b"required" in lib.rf_last_error()
    assert lib.rf_lse_merge(FAKE, FAKE, FAKE, FAKE, 4, 0, 128, 2, None) == B.RF_ERR_INVALID_ARG
    assert lib.rf_lse_merge(FAKE, FAKE, FAKE, FAKE, 4, 8, 80, 2, None) == B.RF_ERR_UNSUPPORTED
    assert lib.rf_lse_merge(None, FAKE, FAKE, FAKE, 4, 8, 128, 2, None) == B.RF_ERR_INVALID_ARG
    assert lib.rf_lse_merge(None, None, None, None, 0, 8, 128, 2, None) == B.RF_OK


def test_last_error_is_thread_local(lib):
    import threading
    assert fwd(lib, D=96) == B.RF_ERR_UNSUPPORTED
    seen = {}

    def other():
        fwd(lib, Hq=3, Hkv=2)
        seen["msg"] = lib.rf_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert "multiple" in seen["msg"]
    assert "96" in lib.rf_last_error().decode()


def test_oracle_not_reachable_from_product_package():
    pkg = os.path.join(ROOT, "attention_pass_cascaded_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_rope_rotate_rejects_bad_arguments(lib):
    assert lib.rf_rope_rotate(FAKE, FAKE, 1, 4, 64, 0.0, 0, 1, None) == B.RF_ERR_INVALID_ARG   # base <= 0
    assert lib.rf_rope_rotate(FAKE, FAKE, 1, 4, 96, 1e4, 0, 1, None) == B.RF_ERR_UNSUPPORTED   # D
    assert lib.rf_rope_rotate(None, FAKE, 1, 4, 64, 1e4, 0, 1, None) == B.RF_ERR_INVALID_ARG
    assert lib.rf_rope_rotate(FAKE, FAKE, 1, 4, 64, 1e4, -1, 1, None) == B.RF_ERR_INVALID_ARG   # offset
    assert lib.rf_rope_rotate(None, None, 0, 4, 64, 1e4, 0, 1, None) == B.RF_OK                 # empty


def test_bwd_rejects_bad_arguments(lib):
    args = [FAKE] * 10
    # float32 inputs have no backward instance
    st = lib.rf_attn_bwd(*args, 1, 2, 2, 8, 8, 64, 0.125, 1, 0, 0.0, None, 0, None)  # dtype 0: float32
    assert st == B.RF_ERR_UNSUPPORTED and b"float16 and bfloat16" in lib.rf_last_error()
    # missing dk
    a = list(args)
    a[7] = None
    st = lib.rf_attn_bwd(*a, 1, 2, 2, 8, 8, 64, 0.125, 1, 0, 0.0, None, 1, None)
    assert st == B.RF_ERR_INVALID_ARG and b"dk and dv" in lib.rf_last_error()
    # missing workspace
    a = list(args)
    a[9] = None
    st = lib.rf_attn_bwd(*a, 1, 2, 2, 8, 8, 64, 0.125, 1, 0, 0.0, None, 1, None)
    assert st == B.RF_ERR_INVALID_ARG and b"workspace" in lib.rf_last_error()
    assert lib.rf_attn_bwd_workspace_bytes(2, 3, 5) == 2 * 3 * 5 * 4
    assert lib.rf_attn_bwd_workspace_bytes(-1, 3, 5) == 0


def test_layernorm_rejects_bad_arguments(lib):
    assert lib.rf_layernorm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 12, 1e-5, 2, None) == B.RF_ERR_UNSUPPORTED
    assert b"multiple of 8" in lib.rf_last_error()
    assert lib.rf_layernorm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32768, 1e-5, 2, None) == B.RF_ERR_UNSUPPORTED
    assert lib.rf_layernorm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, -1.0, 2, None) == B.RF_ERR_INVALID_ARG
    assert lib.rf_layernorm_fwd(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 64, 1e-5, 2, None) == B.RF_ERR_INVALID_ARG
    assert lib.rf_layernorm_fwd(None, None, None, None, None, None, 0, 64, 1e-5, 2, None) == B.RF_OK


def test_softmax_topk_rejects_bad_arguments(lib):
    assert lib.rf_softmax_topk(FAKE, FAKE, FAKE, 4, 16, 17, 2, None) == B.RF_ERR_INVALID_ARG    # k > E
    assert lib.rf_softmax_topk(FAKE, FAKE, FAKE, 4, 256, 65, 2, None) == B.RF_ERR_INVALID_ARG   # k > 64
    assert lib.rf_softmax_topk(FAKE, FAKE, FAKE, 4, 2048, 8, 2, None) == B.RF_ERR_UNSUPPORTED   # E
    assert lib.rf_softmax_topk(FAKE, None, FAKE, 4, 256, 8, 2, None) == B.RF_ERR_INVALID_ARG
    assert lib.rf_softmax_topk(None, None, None, 0, 256, 8, 2, None) == B.RF_OK


# ---------------------------------------------------------------------------
# The binding checks every caller-provided output buffer before a pointer
# reaches the C ABI (a buffer of the wrong shape or dtype would otherwise be
# written past its end by the kernels).
# ---------------------------------------------------------------------------
import torch


def test_out_buffer_allocated_when_absent():
    t = B._out("out", None, (2, 3), torch.float32, "cpu")
    assert t.shape == (2, 3) and t.dtype == torch.float32 and t.is_contiguous()


def test_out_buffer_accepted_when_exact():
    t = torch.empty(4, 5, dtype=torch.float16)
    assert B._out("out", t, (4, 5), torch.float16, "cpu") is t


@pytest.mark.parametrize("t,needle", [
    (torch.empty(4, 5, dtype=torch.float32), "float16"),      # wrong dtype
    (torch.empty(4, 4, dtype=torch.float16), "shape"),        # too small
    (torch.empty(4, 6, dtype=torch.float16), "shape"),        # too large is refused as well
    (torch.empty(5, 4, dtype=torch.float16).t(), "contiguous"),
    (torch.empty(20, dtype=torch.float16), "shape"),          # right size, wrong shape
    ("not a tensor", "tensor"),
])
def test_out_buffer_rejected(t, needle):
    with pytest.raises(ValueError, match=needle):
        B._out("out", t, (4, 5), torch.float16, "cpu")


def test_out_buffer_on_another_device_rejected():
    with pytest.raises(ValueError, match="must be on"):
        B._out("out", torch.empty(4, 5, dtype=torch.float16, device="meta"), (4, 5), torch.float16, "cpu")


@pytest.mark.parametrize("B,Hkv,Nk,cu,want", [
    (16, 8, 32768, 256, 4),      # ceil(2*256 / 128) = 4 chunks of 8192
    (1, 8, 32768, 256, 64),      # ceil(512 / 8) = 64 chunks of 512 keys
    (1, 8, 4096, 256, 32),       # 64 wanted, capped at ceil(4096 / 128) = 32
    (1, 8, 4097, 256, 33),       # the cap rounds up
    (16, 8, 16384, 256, 4),
    (64, 8, 4096, 256, 1),       # 512 (batch, KV head) groups fill the GPU unsplit
    (1, 1, 10, 256, 1),          # fewer keys than one chunk's minimum
    (3, 1, 0, 256, 1),           # no keys: one (empty) chunk
    (1, 1, 1 << 30, 100000, 4096),  # clamped to the ABI's maximum
    (0, 8, 4096, 256, 0),        # invalid sizes
    (1, 0, 4096, 256, 0),
    (1, 8, -1, 256, 0),
])
def test_num_splits_rule(lib, B, Hkv, Nk, cu, want):
    assert lib.rf_splitkv_num_splits(B, Hkv, Nk, cu) == want


def bwd_noalloc(lib, **kw):
    a = dict(B=1, Hq=2, Hkv=2, Nq=8, Nk=8, D=64, scale=0.125, mask=1, window=0, rope=0.0, dtype=1)
    a.update(kw)
    return lib.rf_attn_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], a["Hq"], a["Hkv"],
                                   a["Nq"], a["Nk"], a["D"], a["scale"], a["mask"], a["window"], a["rope"], None,
                                   a["dtype"], None)


@pytest.mark.parametrize("kw,status,needle", [
    # one row past the static row-term array (2^22 rows): refused before any launch
    (dict(B=1, Hq=64, Hkv=64, Nq=(1 << 16) + 1, Nk=8), B.RF_ERR_UNSUPPORTED, "static row-term array"),
    (dict(B=2, Hq=32, Hkv=8, Nq=65537, Nk=8), B.RF_ERR_UNSUPPORTED, "static row-term array"),
    (dict(dtype=0), B.RF_ERR_UNSUPPORTED, "float16 and bfloat16"),
    (dict(Hq=3, Hkv=2), B.RF_ERR_INVALID_ARG, "multiple"),
    (dict(D=96), B.RF_ERR_UNSUPPORTED, "96"),
])
def test_bwd_noalloc_rejects_before_launch(lib, kw, status, needle):
    assert bwd_noalloc(lib, **kw) == status
    assert needle in lib.rf_last_error().decode()
