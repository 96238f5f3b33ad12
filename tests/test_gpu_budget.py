"""GPU parity of the CU-budget launches (ep_shape_t.num_cus > 0) against the CPU oracle.

A budget launch runs num_cus persistent workgroups that loop over the work;
the results must be the same bits as the oracle's (and so as the whole-GPU
launch's) for every budget, including budgets of one workgroup and budgets
larger than the work.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import combine_ep_layout_02_amd as ep
from combine_ep_layout_02_amd import workloads as wl
from test_gpu_parity import (DEV, _idx, dev_bf16, dev_f32, dev_i32, host_u16, inputs, log, setup_module,  # noqa: F401
                             shape_of)

pytestmark = pytest.mark.gpu

SENTINEL = 0x7BAD
BUDGETS = [1, 3, 64, 256, 5000]


def budget(shape, n):
    return dataclasses.replace(shape, num_cus=n)


def dispatch(shape, x_bits, slot, dtype):
    rows = shape.recv_rows
    if dtype == ep.EP_BF16:
        rx = torch.full((rows, shape.hidden), SENTINEL, dtype=torch.int16, device=DEV)
        ep.ep_dispatch(shape, dev_bf16(x_bits), dev_i32(slot), dtype, rx)
        torch.cuda.synchronize()
        return host_u16(rx), None
    rq = torch.full((rows, shape.hidden), 0x5A, dtype=torch.uint8, device=DEV)
    rs = torch.full((rows, shape.hidden // 128), -1.0, dtype=torch.float32, device=DEV)
    ep.ep_dispatch(shape, dev_bf16(x_bits), dev_i32(slot), dtype, rq, rs)
    torch.cuda.synchronize()
    return rq.cpu().numpy(), rs.cpu().numpy()


@pytest.mark.parametrize("n", BUDGETS)
@pytest.mark.parametrize("name,dtype", [("tiny", ep.EP_FP8_E4M3), ("mid", ep.EP_BF16), ("decode", ep.EP_FP8_E4M3)])
def test_dispatch_under_budget(name, dtype, n):
    w, inp, lay = inputs(name)
    log(f"[budget-dispatch] {name} num_cus={n}")
    got, got_s = dispatch(budget(shape_of(w), n), inp.x, lay.slot, dtype)
    held = lay.src_pair >= 0
    if dtype == ep.EP_BF16:
        want = oracle.dispatch_bf16(inp.x, lay.slot, w.recv_rows)
        assert np.array_equal(got[held], want[held]) and (got[~held] == SENTINEL).all()
    else:
        wq, ws = oracle.dispatch_fp8(inp.x, lay.slot, w.recv_rows)
        assert np.array_equal(got[held], wq[held]) and np.array_equal(got_s[held], ws[held])
        assert (got[~held] == 0x5A).all() and (got_s[~held] == -1.0).all()


@pytest.mark.parametrize("n", BUDGETS)
@pytest.mark.parametrize("name", ["tiny", "mid", "decode"])
def test_combine_and_backward_under_budget(name, n):
    w, inp, lay = inputs(name, with_y=True)
    log(f"[budget-combine] {name} num_cus={n}")
    shape = budget(shape_of(w), n)
    y, slot, wts = dev_bf16(inp.y), dev_i32(lay.slot), dev_f32(inp.topk_weights)
    out = torch.empty((w.num_tokens, w.hidden), dtype=torch.bfloat16, device=DEV)
    ep.ep_combine(shape, y, slot, wts, out)
    gx = torch.empty_like(out)
    ep.ep_dispatch_backward(shape, y, slot, gx)
    g = wl.normal_bf16(w.seed, 5, w.num_tokens, w.hidden)
    gy = torch.full((w.recv_rows, w.hidden), SENTINEL, dtype=torch.int16, device=DEV)
    gw = torch.empty_like(wts)
    ep.ep_combine_backward(shape, dev_bf16(g), y, slot, wts, gy, gw)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(out), oracle.combine(inp.y, lay.slot, inp.topk_weights))
    assert np.array_equal(host_u16(gx), oracle.dispatch_backward(inp.y, lay.slot))
    want_gy, want_gw = oracle.combine_backward(g, inp.y, lay.slot, inp.topk_weights)
    held = lay.src_pair >= 0
    assert np.array_equal(host_u16(gy)[held], want_gy[held])
    # grad_w: same tree as the whole-GPU launch, so the same bits
    gw_full = torch.empty_like(wts)
    ep.ep_combine_backward(shape_of(w), dev_bf16(g), y, slot, wts, gy, gw_full)
    torch.cuda.synchronize()
    assert torch.equal(gw.view(torch.int32), gw_full.view(torch.int32))
    assert np.allclose(gw.cpu().numpy(), want_gw, rtol=1e-4, atol=1e-3)


@pytest.mark.parametrize("n", [1, 24, 128])
def test_full_size_budget_matches_whole_gpu(n):
    """The 8192-token FP8 dispatch and combine under a budget give the whole-GPU
    launch's bits, which the parity tests pin to the oracle; sampled tokens are
    checked against the oracle directly as well."""
    w, inp, lay = inputs("v3", with_y=True)
    log(f"[budget-v3] num_cus={n}")
    shape = shape_of(w)
    q0, s0 = dispatch(shape, inp.x, lay.slot, ep.EP_FP8_E4M3)
    q1, s1 = dispatch(budget(shape, n), inp.x, lay.slot, ep.EP_FP8_E4M3)
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)
    y, slot, wts = dev_bf16(inp.y), dev_i32(lay.slot), dev_f32(inp.topk_weights)
    o0 = torch.empty((w.num_tokens, w.hidden), dtype=torch.bfloat16, device=DEV)
    o1 = torch.empty_like(o0)
    ep.ep_combine(shape, y, slot, wts, o0)
    ep.ep_combine(budget(shape, n), y, slot, wts, o1)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    tok = np.sort(np.random.default_rng(n).choice(w.num_tokens, 64, replace=False))
    assert np.array_equal(host_u16(o1)[tok], oracle.combine(inp.y, lay.slot[tok], inp.topk_weights[tok]))
    wq, ws = oracle.dispatch_fp8(inp.x[tok], lay.slot[tok], w.recv_rows)
    rows = lay.slot[tok].ravel()
    rows = rows[rows >= 0]
    assert np.array_equal(q1[rows], wq[rows]) and np.array_equal(s1[rows], ws[rows])


@pytest.mark.parametrize("case", [("k3_masked_h640", 300, 640, 3, 16, 4, 0.1), ("k64_h256", 32, 256, 64, 64, 8, 0.0),
                                  ("h16384", 24, 16384, 8, 64, 8, 0.0)], ids=lambda c: c[0])
def test_generic_shapes_under_budget(case):
    name, T, H, k, E, R, mask = case
    log(f"[budget-edge] {name}")
    w = wl.custom(name, T, H, E, R, k, seed=95)
    rng = np.random.default_rng(95)
    lay = oracle.layout(_idx(rng, T, k, E, mask), E, R)
    x = wl.normal_bf16(95, 0, T, H)
    y = wl.normal_bf16(95, 2, w.recv_rows, H)
    wts = rng.standard_normal((T, k)).astype(np.float32)
    shape = budget(shape_of(w), 2)
    got, _ = dispatch(shape, x, lay.slot, ep.EP_BF16)
    held = lay.src_pair >= 0
    assert np.array_equal(got[held], oracle.dispatch_bf16(x, lay.slot, w.recv_rows)[held])
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ep.ep_combine(shape, dev_bf16(y), dev_i32(lay.slot), dev_f32(wts), out)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(out), oracle.combine(y, lay.slot, wts))
