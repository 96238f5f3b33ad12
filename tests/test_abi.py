"""CPU checks of the C ABI: the library loads, exports what include/ep.h
declares, sizes buffers as documented and rejects bad arguments before it
touches the GPU (every case here returns before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

import combine_ep_layout_02_amd as ep
from combine_ep_layout_02_amd import ep as epmod
from combine_ep_layout_02_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(epmod.library_path()):
        from combine_ep_layout_02_amd.build import build_library
        build_library()
    return ep.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_api():
    names = declared_functions()
    assert {"ep_layout", "ep_dispatch", "ep_combine", "ep_recv_rows", "ep_layout_workspace_bytes"} <= set(names)
    assert set(names) == set(epmod.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", epmod.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)
    # nothing but the C API leaks out of the library
    assert {n for n in exported if not n.startswith("_")} == set(declared_functions())


def test_abi_version_and_status_strings(L):
    header = open(HEADER).read()
    assert ep.ep_abi_version() == int(re.search(r"#define EP_ABI_VERSION (\d+)", header).group(1)) == 6
    for code in range(6):
        s = ep.ep_status_string(code)
        assert s.startswith("EP_"), s
    assert "unknown" in ep.ep_status_string(42)
    assert "#define EP_MAX_EXPERTS %d" % epmod.EP_MAX_EXPERTS in header
    assert "#define EP_MAX_TOPK %d" % epmod.EP_MAX_TOPK in header


def shape_c(**kw):
    base = dict(num_tokens=16, hidden=256, num_topk=2, num_experts=8, num_ranks=2, expert_alignment=1,
                capacity=0, num_cus=0)
    base.update(kw)
    return epmod._Shape(*[base[n] for n, _ in epmod._Shape._fields_])


def rows_status(L, **kw):
    out = ctypes.c_int64(-1)
    return L.ep_recv_rows(ctypes.byref(shape_c(**kw)), ctypes.byref(out)), out.value


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_recv_rows_matches_workloads(L, name):
    w = wl.WORKLOADS[name]
    s = ep.EpShape(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, w.expert_alignment,
                   w.capacity)
    assert ep.ep_recv_rows(s) == w.recv_rows
    assert ep.ep_layout_workspace_bytes(s) > 0


def test_shape_struct_matches_header():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct ep_shape_t \{(.*?)\} ep_shape_t;", src, re.S).group(1)
    fields = re.findall(r"int32_t (\w+);", body)
    assert fields == [n for n, _ in epmod._Shape._fields_]
    assert "#define EP_MAX_NUM_CUS %d" % epmod.EP_MAX_NUM_CUS in open(HEADER).read()


def test_num_cus_accepted_in_range(L):
    assert rows_status(L, num_cus=1)[0] == OK
    assert rows_status(L, num_cus=65535)[0] == OK


def test_recv_rows_formula(L):
    assert rows_status(L, num_tokens=10, num_topk=3, num_experts=6, num_ranks=3, expert_alignment=4) == (OK, 30 + 18)
    assert rows_status(L, num_tokens=10, num_topk=3, num_experts=6, num_ranks=3, capacity=7) == (OK, 42)
    assert rows_status(L, num_tokens=0) == (OK, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(num_tokens=-1), INVALID), (dict(hidden=0), INVALID), (dict(num_topk=0), INVALID),
    (dict(num_experts=0), INVALID), (dict(num_ranks=0), INVALID), (dict(num_ranks=3), INVALID),
    (dict(num_topk=9), INVALID), (dict(expert_alignment=0), INVALID), (dict(capacity=-1), INVALID),
    (dict(expert_alignment=2, capacity=4), INVALID),
    (dict(hidden=100), UNSUPPORTED), (dict(num_experts=4096, num_ranks=8), UNSUPPORTED),
    (dict(num_experts=128, num_topk=65), UNSUPPORTED),
    (dict(num_tokens=1 << 30, num_topk=4), UNSUPPORTED),
    (dict(num_experts=2048, num_ranks=8, capacity=1 << 21), UNSUPPORTED),
    (dict(num_cus=-1), INVALID), (dict(num_cus=65536), UNSUPPORTED),
    (dict(num_tokens=1 << 20, hidden=1 << 20, num_topk=1), UNSUPPORTED),   # 2^31 (token, chunk) items
])
def test_bad_shapes_rejected(L, kw, code):
    st, _ = rows_status(L, **kw)
    assert st == code
    ws = ctypes.c_size_t()
    assert L.ep_layout_workspace_bytes(ctypes.byref(shape_c(**kw)), ctypes.byref(ws)) == code
    assert L.ep_layout(ctypes.byref(shape_c(**kw)), *([None] * 9), 0, None) == code
    assert L.ep_dispatch(ctypes.byref(shape_c(**kw)), None, None, 0, None, None, None) == code
    assert L.ep_dispatch_prequantized(ctypes.byref(shape_c(**kw)), *([None] * 5), None) == code
    assert L.ep_layout_dispatch(ctypes.byref(shape_c(**kw)), *([None] * 9), 0, None, 0, None, None, None) == code
    assert L.ep_combine(ctypes.byref(shape_c(**kw)), None, None, None, None, None) == code
    assert L.ep_dispatch_backward(ctypes.byref(shape_c(**kw)), None, None, None, None) == code
    assert L.ep_combine_backward(ctypes.byref(shape_c(**kw)), *([None] * 6), None) == code


def test_null_shape_and_outputs(L):
    out = ctypes.c_int64()
    assert L.ep_recv_rows(None, ctypes.byref(out)) == INVALID
    assert L.ep_recv_rows(ctypes.byref(shape_c()), None) == INVALID
    assert L.ep_layout_workspace_bytes(ctypes.byref(shape_c()), None) == INVALID


FAKE = 0x10000  # a non-null, 64 KiB-aligned address; never dereferenced on these paths


def test_layout_argument_checks(L):
    s = ctypes.byref(shape_c())
    p = [FAKE] * 8
    ws_need = ctypes.c_size_t()
    assert L.ep_layout_workspace_bytes(s, ctypes.byref(ws_need)) == OK
    # missing required outputs
    for i in (1, 2, 3, 4):
        q = list(p)
        q[i] = None
        assert L.ep_layout(s, *q, FAKE, ws_need.value, None) == INVALID
    q = list(p)
    q[0] = None  # topk_idx needed when T > 0
    assert L.ep_layout(s, *q, FAKE, ws_need.value, None) == INVALID
    # misaligned int32 pointer
    q = list(p)
    q[5] = FAKE + 2
    assert L.ep_layout(s, *q, FAKE, ws_need.value, None) == MISALIGNED
    # workspace missing / too small / misaligned
    assert L.ep_layout(s, *p, None, ws_need.value, None) == WORKSPACE
    assert L.ep_layout(s, *p, FAKE, ws_need.value - 1, None) == WORKSPACE
    assert L.ep_layout(s, *p, FAKE + 4, ws_need.value, None) == MISALIGNED


def test_dispatch_argument_checks(L):
    s = ctypes.byref(shape_c())
    assert L.ep_dispatch(s, FAKE, FAKE, 7, FAKE, FAKE, None) == INVALID              # dtype
    assert L.ep_dispatch(s, None, FAKE, 0, FAKE, None, None) == INVALID              # x
    assert L.ep_dispatch(s, FAKE, None, 0, FAKE, None, None) == INVALID              # slot
    assert L.ep_dispatch(s, FAKE, FAKE, 1, FAKE, None, None) == INVALID              # fp8 needs scales
    assert L.ep_dispatch(s, FAKE + 8, FAKE, 0, FAKE, None, None) == MISALIGNED       # x 16-byte
    assert L.ep_dispatch(s, FAKE, FAKE, 0, FAKE + 4, None, None) == MISALIGNED       # recv_x 16-byte
    s2 = ctypes.byref(shape_c(hidden=136))
    assert L.ep_dispatch(s2, FAKE, FAKE, 1, FAKE, FAKE, None) == UNSUPPORTED         # fp8 needs H % 128
    # T = 0 is a no-op that needs no buffers
    assert L.ep_dispatch(ctypes.byref(shape_c(num_tokens=0)), None, None, 1, None, None, None) == OK


def test_mx_dispatch_argument_checks(L):
    s = ctypes.byref(shape_c())
    for dt in (2, 3):
        assert L.ep_dispatch(s, FAKE, FAKE, dt, FAKE, None, None) == INVALID          # MX needs scales
        assert L.ep_dispatch(s, FAKE, FAKE, dt, FAKE, FAKE + 2, None) == MISALIGNED    # scales 4-byte
        assert L.ep_dispatch(ctypes.byref(shape_c(hidden=48)), FAKE, FAKE, dt, FAKE, FAKE, None) == UNSUPPORTED
        assert L.ep_dispatch(ctypes.byref(shape_c(num_tokens=0)), None, None, dt, None, None, None) == OK
    assert L.ep_dispatch(s, FAKE, FAKE, 4, FAKE, FAKE, None) == INVALID               # no dtype 4
    assert L.ep_dispatch(ctypes.byref(shape_c(hidden=160)), FAKE, FAKE, 1, FAKE, FAKE, None) == UNSUPPORTED


def test_layout_dispatch_argument_checks(L):
    s = ctypes.byref(shape_c())
    ws = ctypes.c_size_t()
    assert L.ep_layout_workspace_bytes(s, ctypes.byref(ws)) == OK
    lay = [FAKE] * 8
    # layout side: missing output, workspace too small
    q = list(lay)
    q[1] = None
    assert L.ep_layout_dispatch(s, *q, FAKE, ws.value, FAKE, 1, FAKE, FAKE, None) == INVALID
    assert L.ep_layout_dispatch(s, *lay, FAKE, ws.value - 1, FAKE, 1, FAKE, FAKE, None) == WORKSPACE
    # dispatch side: x missing, bad dtype, FP8 without scales, misaligned recv_x
    assert L.ep_layout_dispatch(s, *lay, FAKE, ws.value, None, 1, FAKE, FAKE, None) == INVALID
    assert L.ep_layout_dispatch(s, *lay, FAKE, ws.value, FAKE, 9, FAKE, FAKE, None) == INVALID
    assert L.ep_layout_dispatch(s, *lay, FAKE, ws.value, FAKE, 1, FAKE, None, None) == INVALID
    assert L.ep_layout_dispatch(s, *lay, FAKE, ws.value, FAKE, 0, FAKE + 4, None, None) == MISALIGNED


def test_prequantized_dispatch_argument_checks(L):
    s = ctypes.byref(shape_c())
    for i in range(5):
        q = [FAKE] * 5
        q[i] = None
        assert L.ep_dispatch_prequantized(s, *q, None) == INVALID, i
    for i, off in ((0, 8), (1, 2), (2, 2), (3, 8), (4, 2)):
        q = [FAKE] * 5
        q[i] += off
        assert L.ep_dispatch_prequantized(s, *q, None) == MISALIGNED, i
    assert L.ep_dispatch_prequantized(ctypes.byref(shape_c(hidden=160)), *([FAKE] * 5), None) == UNSUPPORTED
    assert L.ep_dispatch_prequantized(ctypes.byref(shape_c(num_tokens=0)), *([None] * 5), None) == OK


def test_combine_argument_checks(L):
    s = ctypes.byref(shape_c())
    for i in range(4):
        q = [FAKE] * 4
        q[i] = None
        assert L.ep_combine(s, *q, None) == INVALID
    assert L.ep_combine(s, FAKE + 8, FAKE, FAKE, FAKE, None) == MISALIGNED
    assert L.ep_combine(s, FAKE, FAKE, FAKE, FAKE + 8, None) == MISALIGNED
    assert L.ep_combine(s, FAKE, FAKE + 1, FAKE, FAKE, None) == MISALIGNED
    assert L.ep_combine(ctypes.byref(shape_c(num_tokens=0)), None, None, None, None, None) == OK


def test_dispatch_backward_argument_checks(L):
    s = ctypes.byref(shape_c())
    for i in range(3):
        q = [FAKE] * 3
        q[i] = None
        assert L.ep_dispatch_backward(s, *q, None) == INVALID
    assert L.ep_dispatch_backward(s, FAKE + 8, FAKE, FAKE, None) == MISALIGNED     # grad_recv_x 16-byte
    assert L.ep_dispatch_backward(s, FAKE, FAKE + 2, FAKE, None) == MISALIGNED     # slot 4-byte
    assert L.ep_dispatch_backward(s, FAKE, FAKE, FAKE + 8, None) == MISALIGNED     # grad_x 16-byte
    assert L.ep_dispatch_backward(ctypes.byref(shape_c(num_tokens=0)), None, None, None, None) == OK


def test_combine_backward_argument_checks(L):
    s = ctypes.byref(shape_c())
    # grad_out, y, slot, topk_weights, grad_y, grad_weights
    for i in (0, 2, 3, 4):
        q = [FAKE] * 6
        q[i] = None
        assert L.ep_combine_backward(s, *q, None) == INVALID
    q = [FAKE] * 6
    q[1] = None   # y is needed for grad_weights ...
    assert L.ep_combine_backward(s, *q, None) == INVALID
    q[5] = None   # ... and not without them (nothing is launched for T = 0 below)
    assert L.ep_combine_backward(ctypes.byref(shape_c(num_tokens=0)), *q, None) == OK
    for i, off in ((0, 8), (1, 8), (2, 2), (3, 2), (4, 8), (5, 2)):
        q = [FAKE] * 6
        q[i] += off
        assert L.ep_combine_backward(s, *q, None) == MISALIGNED, i
    assert L.ep_combine_backward(ctypes.byref(shape_c(num_tokens=0)), *([None] * 6), None) == OK


def test_check_helpers_argument_checks(L):
    assert L.ep_check_cvt_e4m3(None, None, -1, None) == INVALID
    assert L.ep_check_cvt_e4m3(None, FAKE, 4, None) == INVALID
    assert L.ep_check_cvt_e4m3(FAKE + 1, FAKE, 4, None) == MISALIGNED
    assert L.ep_check_cvt_bf16(FAKE, FAKE + 1, 4, None) == MISALIGNED
    assert L.ep_check_cvt_e4m3(None, None, 0, None) == OK
    assert L.ep_check_cvt_e2m1(None, None, -1, None) == INVALID
    assert L.ep_check_cvt_e2m1(FAKE + 1, FAKE, 4, None) == MISALIGNED
    assert L.ep_check_cvt_e2m1(None, None, 0, None) == OK
    assert L.ep_check_quant_e4m3(None, FAKE, FAKE, 4, None) == INVALID
    assert L.ep_check_quant_e4m3(FAKE + 1, FAKE, FAKE, 4, None) == MISALIGNED
    assert L.ep_check_quant_e4m3(FAKE, FAKE + 2, FAKE, 4, None) == MISALIGNED
    assert L.ep_check_quant_e4m3(None, None, None, 0, None) == OK
    assert L.ep_probe_stream(FAKE, FAKE, -1, 1, 1, 0, None) == INVALID
    assert L.ep_probe_stream(FAKE, FAKE, 4, 3, 1, 0, None) == INVALID
    assert L.ep_probe_stream(FAKE, FAKE, 4, 1, 0, 0, None) == INVALID
    assert L.ep_probe_stream(FAKE, FAKE, 4, 1, 65, 0, None) == INVALID
    assert L.ep_probe_stream(FAKE, FAKE, 4, 1, 1, 8, None) == INVALID
    assert L.ep_probe_stream(FAKE, FAKE, 4, 1, 1, -1, None) == INVALID
    assert L.ep_probe_stream(None, FAKE, 4, 1, 1, 0, None) == INVALID
    assert L.ep_probe_stream(FAKE + 8, FAKE, 4, 1, 1, 0, None) == MISALIGNED
    assert L.ep_probe_stream(FAKE, FAKE + 4, 4, 1, 1, 0, None) == MISALIGNED
    assert L.ep_probe_stream(None, None, 0, 16, 64, 7, None) == OK


def test_binding_rejects_host_tensors():
    import torch
    s = ep.EpShape(4, 256, 2, 8, 2)
    with pytest.raises(ValueError):
        ep.ep_combine(s, torch.zeros((8, 256), dtype=torch.bfloat16), torch.zeros((4, 2), dtype=torch.int32),
                      torch.zeros((4, 2)), torch.zeros((4, 256), dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        ep.ep_combine(s, torch.zeros((8, 256)), torch.zeros((4, 2), dtype=torch.int32),
                      torch.zeros((4, 2)), torch.zeros((4, 256), dtype=torch.bfloat16))
