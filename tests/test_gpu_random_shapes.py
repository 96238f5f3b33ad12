"""Seeded random shapes through every entry point, against the CPU oracle.

The fixed edge cases elsewhere pin one corner each; here 200 seeded draws mix them: token counts from 0 to
500, hidden sizes of 128 to 2048 columns, 1 to 2048 experts in any dividing number of ranks, top-k up to 12
with repeated experts, masked and invalid ids, flat layouts with alignment 1 to 16 and padded layouts whose
capacity may drop pairs.  Each draw runs ep_layout, ep_layout_dispatch, BF16 / FP8 / MXFP8 / MXFP4 and
pre-quantised dispatch, combine and the backward pair through the C ABI and compares every output with the
oracle (bit for bit; grad_weights within its stated bound); every fourth draw repeats dispatch, combine
and the backward pair under a CU budget (persistent workgroups), which must give the same bytes.  Inputs
come from the seeded generators only.  Eight more draws sit above the 64 MiB streaming threshold (up to 3300
tokens, 5120 to 8192 columns, k = 3 to 8, flat and padded layouts), where the large-batch code paths run: layout,
every dispatch format, combine and the backward pair, each compared in full.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import combine_ep_layout_02_amd as ep
from combine_ep_layout_02_amd import workloads as wl
from test_gpu_parity import (DEV, assert_layout_equal, bf16_ulp_distance, dev_bf16, dev_f32, dev_i32,  # noqa: F401
                             host_u16, log, setup_module)
from test_gpu_backward import SENTINEL, gw_bound

pytestmark = pytest.mark.gpu

NCASES = 200
EXPERTS = [1, 2, 3, 8, 16, 48, 64, 100, 256, 512, 2048]


def draw(seed):
    """One random shape and its routing ids (numpy PCG64, seeded)."""
    rng = np.random.default_rng([seed, 777])
    E = int(rng.choice(EXPERTS))
    R = int(rng.choice([d for d in range(1, E + 1) if E % d == 0]))
    k = int(rng.integers(1, min(E, 12) + 1))
    T = 0 if seed % 17 == 5 else int(rng.integers(1, 501))
    H = 128 * int(rng.integers(1, 17))
    if rng.random() < 0.3:
        A, C = 1, int(rng.integers(1, max(2, 2 * T * k // E) + 1))
    else:
        A, C = int(rng.choice([1, 1, 1, 2, 4, 16])), 0
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    u = rng.random(idx.shape)
    mask, bad = float(rng.choice([0.0, 0.05, 0.3])), float(rng.choice([0.0, 0.02]))
    idx[u < mask] = -1
    b = (u >= mask) & (u < mask + bad)
    idx[b] = rng.choice([-5, E, E + 7], size=int(b.sum()))
    weights = rng.standard_normal((T, k)).astype(np.float32)
    return dict(T=T, H=H, k=k, E=E, R=R, A=A, C=C, idx=idx, weights=weights)


def fill_u8(t, v):
    t.view(torch.uint8).fill_(v)
    return t


@pytest.mark.parametrize("seed", range(NCASES))
def test_random_shape(seed):
    d = draw(seed)
    T, H, k, E, R, A, C = (d[n] for n in ("T", "H", "k", "E", "R", "A", "C"))
    log(f"[random {seed}] T={T} H={H} k={k} E={E} R={R} A={A} C={C}")
    shape = ep.EpShape(T, H, k, E, R, A, C)
    rows = ep.ep_recv_rows(shape)
    lay = oracle.layout(d["idx"], E, R, A, C)
    held = lay.src_pair >= 0
    x = wl.normal_bf16(seed, 0, T, H)
    y = wl.normal_bf16(seed, 2, rows, H)

    # layout
    bufs = ep.LayoutBuffers.allocate(shape, DEV)
    bufs.src_pair.fill_(-7)
    bufs.run(dev_i32(d["idx"]))
    torch.cuda.synchronize()
    assert_layout_equal(bufs, lay)
    if T == 0:
        return
    slot = bufs.slot

    # layout + FP8 dispatch as one call, into fresh buffers
    fused = ep.LayoutBuffers.allocate(shape, DEV)
    fused.src_pair.fill_(-7)
    fq, fs = ep.alloc_recv(shape, ep.EP_FP8_E4M3, DEV)
    fill_u8(fq, 0x5A)
    fused.run_dispatch(dev_i32(d["idx"]), dev_bf16(x), ep.EP_FP8_E4M3, fq, fs)
    torch.cuda.synchronize()
    assert_layout_equal(fused, lay)
    wq, ws = oracle.dispatch_fp8(x, lay.slot, rows)
    got_q = fq.view(torch.uint8).cpu().numpy()
    assert np.array_equal(got_q[held], wq[held]) and np.array_equal(fs.cpu().numpy()[held], ws[held])
    assert (got_q[~held] == 0x5A).all()

    # BF16 and FP8 dispatch
    rb, _ = ep.alloc_recv(shape, ep.EP_BF16, DEV)
    fill_u8(rb, 0x5A)
    ep.ep_dispatch(shape, dev_bf16(x), slot, ep.EP_BF16, rb)
    rq, rs = ep.alloc_recv(shape, ep.EP_FP8_E4M3, DEV)
    ep.ep_dispatch(shape, dev_bf16(x), slot, ep.EP_FP8_E4M3, rq, rs)
    torch.cuda.synchronize()
    got_b = rb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_b[held], oracle.dispatch_bf16(x, lay.slot, rows)[held])
    assert (got_b[~held] == 0x5A5A).all()
    assert np.array_equal(rq.view(torch.uint8).cpu().numpy()[held], wq[held])
    assert np.array_equal(rs.cpu().numpy()[held], ws[held])

    # MX dispatch
    for dtype, bits in ((ep.EP_MXFP8_E4M3, 8), (ep.EP_MXFP4_E2M1, 4)):
        mq, ms = ep.alloc_recv(shape, dtype, DEV)
        ep.ep_dispatch(shape, dev_bf16(x), slot, dtype, mq, ms)
        torch.cuda.synchronize()
        want_q, want_s = oracle.dispatch_mx(x, lay.slot, rows, bits)
        assert np.array_equal(mq.view(torch.uint8).cpu().numpy()[held], want_q[held]), f"MX{bits} codes"
        assert np.array_equal(ms.view(torch.uint8).cpu().numpy()[held], want_s[held]), f"MX{bits} scales"

    # caller-quantised codes and scales, passed through
    prng = np.random.default_rng([seed, 779])
    xq = prng.integers(0, 256, (T, H), dtype=np.uint8)
    xs = prng.standard_normal((T, H // 128)).astype(np.float32)
    pq = torch.full((rows, H), 0x5A, dtype=torch.uint8, device=DEV)
    ps = torch.full((rows, H // 128), -1.0, dtype=torch.float32, device=DEV)
    ep.ep_dispatch_prequantized(shape, torch.from_numpy(xq).to(DEV), dev_f32(xs), slot, pq, ps)
    torch.cuda.synchronize()
    want_pq, want_ps = oracle.dispatch_prequantized(xq, xs, lay.slot, rows)
    assert np.array_equal(pq.cpu().numpy()[held], want_pq[held]) and np.array_equal(ps.cpu().numpy()[held], want_ps[held])
    assert (pq.cpu().numpy()[~held] == 0x5A).all()

    # combine (the fixed FMA chain: bit for bit)
    out = torch.full((T, H), SENTINEL, dtype=torch.int16, device=DEV)
    ep.ep_combine(shape, dev_bf16(y), slot, dev_f32(d["weights"]), out)
    torch.cuda.synchronize()
    want = oracle.combine(y, lay.slot, d["weights"])
    assert bf16_ulp_distance(host_u16(out), want).max() == 0

    # backward pair
    gx = torch.full((T, H), SENTINEL, dtype=torch.int16, device=DEV)
    ep.ep_dispatch_backward(shape, dev_bf16(y), slot, gx)
    gy = torch.full((rows, H), SENTINEL, dtype=torch.int16, device=DEV)
    gw = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    ep.ep_combine_backward(shape, dev_bf16(x), dev_bf16(y), slot, dev_f32(d["weights"]), gy, gw)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(gx), oracle.dispatch_backward(y, lay.slot))
    want_gy, want_gw = oracle.combine_backward(x, y, lay.slot, d["weights"], np.full((rows, H), SENTINEL, np.uint16))
    got_gy = host_u16(gy)
    assert np.array_equal(got_gy[held], want_gy[held]) and (got_gy[~held] == SENTINEL).all()
    err = np.abs(gw.cpu().numpy().astype(np.float64) - want_gw)
    assert (err <= gw_bound(x, y, lay.slot, H)).all()

    if seed % 4 == 1:
        # the same calls under a CU budget: persistent workgroups looping over the work, same bytes
        budget = dataclasses.replace(shape, num_cus=int(np.random.default_rng([seed, 778]).choice([1, 3, 17, 100])))
        log(f"  budget {budget.num_cus}")
        bq, bs = ep.alloc_recv(shape, ep.EP_FP8_E4M3, DEV)
        ep.ep_dispatch(budget, dev_bf16(x), slot, ep.EP_FP8_E4M3, bq, bs)
        bout = torch.full((T, H), SENTINEL, dtype=torch.int16, device=DEV)
        ep.ep_combine(budget, dev_bf16(y), slot, dev_f32(d["weights"]), bout)
        bgx = torch.full((T, H), SENTINEL, dtype=torch.int16, device=DEV)
        ep.ep_dispatch_backward(budget, dev_bf16(y), slot, bgx)
        bgy = torch.full((rows, H), SENTINEL, dtype=torch.int16, device=DEV)
        bgw = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
        ep.ep_combine_backward(budget, dev_bf16(x), dev_bf16(y), slot, dev_f32(d["weights"]), bgy, bgw)
        torch.cuda.synchronize()
        assert np.array_equal(bq.view(torch.uint8).cpu().numpy()[held], wq[held])
        assert np.array_equal(bs.cpu().numpy()[held], ws[held])
        assert torch.equal(bout, out) and torch.equal(bgx, gx) and torch.equal(bgy, gy) and torch.equal(bgw, gw)


NLARGE = 8


def draw_large(seed):
    """A random shape above the 64 MiB streaming threshold (the large-batch code paths: non-temporal row
    traffic, XCD-contiguous dispatch order, two-group combine items)."""
    rng = np.random.default_rng([seed, 779])
    E = int(rng.choice([64, 128, 256]))
    R = int(rng.choice([d for d in (1, 2, 4, 8) if E % d == 0]))
    k = int(rng.choice([3, 4, 6, 8]))
    H = 128 * int(rng.integers(40, 65))           # 5120 .. 8192 columns, not always a multiple of 1024
    T = int(np.ceil((64 << 20) / (k * H))) + int(rng.integers(0, 1500))
    C = int(rng.integers(T * k // E, 2 * T * k // E)) if rng.random() < 0.25 else 0
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.05] = -1
    weights = rng.standard_normal((T, k)).astype(np.float32)
    return dict(T=T, H=H, k=k, E=E, R=R, C=C, idx=idx, weights=weights)


@pytest.mark.parametrize("seed", range(NLARGE))
def test_random_streaming_shape(seed):
    d = draw_large(seed)
    T, H, k, E, R, C = (d[n] for n in ("T", "H", "k", "E", "R", "C"))
    log(f"[random-large {seed}] T={T} H={H} k={k} E={E} R={R} C={C}")
    shape = ep.EpShape(T, H, k, E, R, 1, C)
    rows = ep.ep_recv_rows(shape)
    lay = oracle.layout(d["idx"], E, R, 1, C)
    held = lay.src_pair >= 0
    x = wl.normal_bf16(seed, 0, T, H)
    y = wl.normal_bf16(seed, 2, rows, H)
    bufs = ep.LayoutBuffers.allocate(shape, DEV)
    bufs.run(dev_i32(d["idx"]))
    torch.cuda.synchronize()
    assert_layout_equal(bufs, lay)
    slot = bufs.slot

    rq, rs = ep.alloc_recv(shape, ep.EP_FP8_E4M3, DEV)
    fill_u8(rq, 0x5A)
    ep.ep_dispatch(shape, dev_bf16(x), slot, ep.EP_FP8_E4M3, rq, rs)
    torch.cuda.synchronize()
    wq, ws = oracle.dispatch_fp8(x, lay.slot, rows)
    got_q = rq.view(torch.uint8).cpu().numpy()
    assert np.array_equal(got_q[held], wq[held]) and np.array_equal(rs.cpu().numpy()[held], ws[held])
    assert (got_q[~held] == 0x5A).all()
    del rq, rs, got_q, wq, ws

    rb, _ = ep.alloc_recv(shape, ep.EP_BF16, DEV)
    ep.ep_dispatch(shape, dev_bf16(x), slot, ep.EP_BF16, rb)
    torch.cuda.synchronize()
    assert np.array_equal(rb.view(torch.int16).cpu().numpy().view(np.uint16)[held],
                          oracle.dispatch_bf16(x, lay.slot, rows)[held])
    del rb

    out = torch.full((T, H), SENTINEL, dtype=torch.int16, device=DEV)
    ep.ep_combine(shape, dev_bf16(y), slot, dev_f32(d["weights"]), out)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(out), oracle.combine(y, lay.slot, d["weights"]))
    del out

    # the MX formats and the pre-quantised passthrough
    for dtype, bits in ((ep.EP_MXFP8_E4M3, 8), (ep.EP_MXFP4_E2M1, 4)):
        mq, ms = ep.alloc_recv(shape, dtype, DEV)
        ep.ep_dispatch(shape, dev_bf16(x), slot, dtype, mq, ms)
        torch.cuda.synchronize()
        want_q, want_s = oracle.dispatch_mx(x, lay.slot, rows, bits)
        assert np.array_equal(mq.view(torch.uint8).cpu().numpy()[held], want_q[held]), f"MX{bits} codes"
        assert np.array_equal(ms.view(torch.uint8).cpu().numpy()[held], want_s[held]), f"MX{bits} scales"
        del mq, ms, want_q, want_s
    prng = np.random.default_rng([seed, 780])
    xq = prng.integers(0, 256, (T, H), dtype=np.uint8)
    xs = prng.standard_normal((T, H // 128)).astype(np.float32)
    pq = torch.full((rows, H), 0x5A, dtype=torch.uint8, device=DEV)
    ps = torch.full((rows, H // 128), -1.0, dtype=torch.float32, device=DEV)
    ep.ep_dispatch_prequantized(shape, torch.from_numpy(xq).to(DEV), dev_f32(xs), slot, pq, ps)
    torch.cuda.synchronize()
    want_pq, want_ps = oracle.dispatch_prequantized(xq, xs, lay.slot, rows)
    assert np.array_equal(pq.cpu().numpy()[held], want_pq[held]) and np.array_equal(ps.cpu().numpy()[held], want_ps[held])
    del pq, ps, want_pq, want_ps

    # the backward pair
    gx = torch.full((T, H), SENTINEL, dtype=torch.int16, device=DEV)
    ep.ep_dispatch_backward(shape, dev_bf16(y), slot, gx)
    gy = torch.full((rows, H), SENTINEL, dtype=torch.int16, device=DEV)
    gw = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    ep.ep_combine_backward(shape, dev_bf16(x), dev_bf16(y), slot, dev_f32(d["weights"]), gy, gw)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(gx), oracle.dispatch_backward(y, lay.slot))
    want_gy, want_gw = oracle.combine_backward(x, y, lay.slot, d["weights"], np.full((rows, H), SENTINEL, np.uint16))
    got_gy = host_u16(gy)
    assert np.array_equal(got_gy[held], want_gy[held]) and (got_gy[~held] == SENTINEL).all()
    assert (np.abs(gw.cpu().numpy().astype(np.float64) - want_gw) <= gw_bound(x, y, lay.slot, H)).all()
