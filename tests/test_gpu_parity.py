"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Layout, slots, src_pair, BF16 copies, FP8 codes and scales must match bit for
bit; combine must be within 1 BF16 ulp (the fixed FMA order makes it
bit-exact, which the strict test checks too).  Inputs come from the seeded
generators only; no expected value comes from the GPU.
"""
import os
import sys
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import combine_ep_layout_02_amd as ep
from combine_ep_layout_02_amd import ep as epmod
from combine_ep_layout_02_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def setup_module(module):
    if not os.path.exists(epmod.library_path()):
        from combine_ep_layout_02_amd.build import build_library
        build_library()
    assert torch.cuda.is_available(), "these tests need the GPU"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def shape_of(w):
    return ep.EpShape(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, w.expert_alignment,
                      w.capacity)


_CACHE = {}
_Y = {}


def inputs(name, with_y=False):
    """Seeded inputs and the oracle layout; x/routing cached for all workloads,
    the (large) expert outputs y only for the most recent one."""
    if name not in _CACHE:
        log(f"[gen] {name}")
        w = wl.WORKLOADS[name]
        inp = wl.make_inputs(w, with_y=False)
        lay = oracle.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment, w.capacity)
        _CACHE[name] = (w, inp, lay)
    w, inp, lay = _CACHE[name]
    if with_y and inp.y is None:
        for other in list(_Y):
            _CACHE[other][1].y = None
            del _Y[other]
        log(f"[gen-y] {name}")
        inp.y = wl.normal_bf16(w.seed, wl.STREAM_Y, w.recv_rows, w.hidden)
        _Y[name] = True
    return w, inp, lay


def gpu_layout(shape, idx_np):
    bufs = ep.LayoutBuffers.allocate(shape, DEV)
    bufs.run(dev_i32(idx_np.reshape(shape.num_tokens, shape.num_topk)))
    torch.cuda.synchronize()
    return bufs


def assert_layout_equal(bufs, lay):
    assert np.array_equal(bufs.expert_count.cpu().numpy(), lay.expert_count)
    assert np.array_equal(bufs.expert_offset.cpu().numpy(), lay.expert_offset)
    assert np.array_equal(bufs.rank_count.cpu().numpy(), lay.rank_count)
    assert np.array_equal(bufs.rank_offset.cpu().numpy(), lay.rank_offset)
    assert np.array_equal(bufs.slot.cpu().numpy().reshape(lay.slot.shape), lay.slot)
    assert np.array_equal(bufs.src_pair.cpu().numpy(), lay.src_pair)
    assert np.array_equal(bufs.diag.cpu().numpy(), lay.diag)


def bf16_ulp_distance(a, b):
    def ordered(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u & 0x7FFF)
    return np.abs(ordered(a) - ordered(b))


# --------------------------------------------------------------------------
# layout
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_layout_matches_oracle(name):
    w, inp, lay = inputs(name)
    log(f"[layout] {name} T={w.num_tokens} k={w.num_topk} E={w.num_experts} C={w.capacity}")
    bufs = gpu_layout(shape_of(w), inp.topk_idx)
    assert_layout_equal(bufs, lay)
    # the same call again gives the same bits (and the workspace was left reusable)
    bufs.run(dev_i32(inp.topk_idx))
    torch.cuda.synchronize()
    assert_layout_equal(bufs, lay)


def _idx(rng, T, k, E, mask=0.0, bad=0.0, hot=None):
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else np.zeros((0, k), np.int32)
    if hot is not None and T:
        idx[:, 0] = hot
        for t in range(T):  # keep the token's experts distinct
            row = idx[t]
            dup = np.flatnonzero(row[1:] == hot) + 1
            for d in dup:
                row[d] = next(e for e in range(E) if e not in row)
    if mask:
        idx[rng.random(idx.shape) < mask] = -1
    if bad:
        b = rng.random(idx.shape) < bad
        idx[b] = rng.choice([-5, -2, E, E + 11], size=int(b.sum()))
    return idx


LAYOUT_EDGE = [
    # name, T, k, E, R, A, C, mask, bad, hot
    ("empty_flat", 0, 2, 8, 2, 3, 0, 0, 0, None),
    ("empty_padded", 0, 2, 8, 2, 1, 5, 0, 0, None),
    ("one_token", 1, 1, 1, 1, 1, 0, 0, 0, None),
    ("masked_invalid_multitile", 3000, 4, 64, 8, 1, 0, 0.1, 0.05, None),
    ("aligned16", 1000, 6, 64, 8, 16, 0, 0.0, 0.0, None),
    ("padded_overflow", 500, 4, 16, 4, 1, 50, 0.05, 0.0, None),
    ("padded_overflow_one_tile", 100, 4, 16, 4, 1, 10, 0.0, 0.01, None),
    ("experts_2048", 700, 8, 2048, 16, 1, 0, 0.0, 0.0, None),
    ("odd_k3", 5000, 3, 12, 3, 2, 0, 0.02, 0.0, None),
    ("k64", 100, 64, 128, 4, 1, 0, 0.0, 0.0, None),
    ("hot_expert", 20000, 2, 8, 4, 1, 0, 0.0, 0.0, 0),
    ("many_tiles", 65536, 8, 256, 8, 1, 0, 0.0, 0.0, None),
    # more tiles than can be resident at once: the two-kernel path
    ("too_many_tiles_for_one_launch", 70000, 8, 256, 8, 1, 0, 0.01, 0.0, None),
    ("padded_multitile", 3000, 8, 64, 8, 1, 200, 0.0, 0.0, None),
    # divisors of 1 (k, E / R, R, E): the multiply-high division's special case
    ("k1_one_tile", 300, 1, 8, 2, 1, 0, 0.0, 0.0, None),
    ("k1_multitile", 5000, 1, 16, 4, 1, 0, 0.05, 0.0, None),
    ("one_rank_multitile", 3000, 4, 16, 1, 1, 0, 0.0, 0.0, None),
    ("one_expert_per_rank", 2000, 2, 8, 8, 1, 0, 0.0, 0.0, None),
    ("one_expert_multitile", 3000, 1, 1, 1, 1, 0, 0.0, 0.0, None),
    ("one_expert_per_rank_r128", 900, 4, 128, 128, 1, 0, 0.0, 0.0, None),
    # no valid pair at all: empty segments, every slot -1
    ("all_masked_one_tile", 100, 4, 16, 4, 1, 0, 1.0, 0.0, None),
    ("all_masked_multitile_aligned", 3000, 4, 64, 8, 2, 0, 1.0, 0.0, None),
    ("all_invalid_padded_multitile", 3000, 4, 64, 8, 1, 20, 0.0, 1.0, None),
]


@pytest.mark.parametrize("case", LAYOUT_EDGE, ids=lambda c: c[0])
def test_layout_edge_cases(case):
    name, T, k, E, R, A, C, mask, bad, hot = case
    log(f"[layout-edge] {name}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    idx = _idx(rng, T, k, E, mask, bad, hot)
    lay = oracle.layout(idx, E, R, A, C)
    bufs = gpu_layout(ep.EpShape(T, 256, k, E, R, A, C), idx)
    assert_layout_equal(bufs, lay)


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------

SENTINEL = 0x5A


def run_dispatch(w, inp, lay, dtype):
    shape = shape_of(w)
    rows = shape_rows = ep.ep_recv_rows(shape)
    x = dev_bf16(inp.x)
    slot = dev_i32(lay.slot)
    if dtype == ep.EP_BF16:
        rx = torch.full((rows, w.hidden), SENTINEL, dtype=torch.int16, device=DEV)
        ep.ep_dispatch(shape, x, slot, dtype, rx)
        torch.cuda.synchronize()
        return host_u16(rx), None
    rx = torch.full((shape_rows, w.hidden), SENTINEL, dtype=torch.uint8, device=DEV)
    rs = torch.full((shape_rows, w.hidden // 128), -7.0, dtype=torch.float32, device=DEV)
    ep.ep_dispatch(shape, x, slot, dtype, rx, rs)
    torch.cuda.synchronize()
    return rx.cpu().numpy(), rs.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_dispatch_bf16_matches_oracle(name):
    w, inp, lay = inputs(name)
    log(f"[dispatch-bf16] {name}")
    got, _ = run_dispatch(w, inp, lay, ep.EP_BF16)
    want = oracle.dispatch_bf16(inp.x, lay.slot, w.recv_rows)
    held = lay.src_pair >= 0
    assert np.array_equal(got[held], want[held])
    assert (got[~held] == SENTINEL).all()  # rows nobody maps to are untouched


@pytest.mark.parametrize("name", ["tiny", "v3", "decode", "skew"])
def test_dispatch_fp8_matches_oracle(name):
    w, inp, lay = inputs(name)
    log(f"[dispatch-fp8] {name}")
    q, s = run_dispatch(w, inp, lay, ep.EP_FP8_E4M3)
    wq, ws = oracle.dispatch_fp8(inp.x, lay.slot, w.recv_rows)
    held = lay.src_pair >= 0
    bad_rows = np.flatnonzero(held & (q != wq).any(axis=1))
    assert len(bad_rows) == 0, f"{len(bad_rows)} rows differ, first {bad_rows[:5]}"
    assert np.array_equal(s[held].view(np.uint32), ws[held].view(np.uint32))
    assert (q[~held] == SENTINEL).all() and (s[~held] == -7.0).all()


DISPATCH_EDGE = [
    # name, T, H, k, E, R, A, C, mask
    ("h384_fp8", 300, 384, 4, 16, 4, 1, 0, 0.05),
    ("h136_bf16", 300, 136, 3, 12, 3, 2, 0, 0.05),
    ("h2176_padded", 200, 2176, 6, 32, 8, 1, 30, 0.0),
    ("k1", 257, 1024, 1, 4, 2, 1, 0, 0.0),
    ("k16_generic", 64, 512, 16, 64, 8, 1, 0, 0.1),
    ("h3584_odd_chunks", 100, 3584, 8, 32, 8, 1, 0, 0.0),
    ("h640_partial_chunk", 200, 640, 2, 8, 2, 1, 0, 0.0),
    ("h9216_two_slices", 40, 9216, 4, 16, 4, 1, 0, 0.05),
    ("h16384_two_slices", 24, 16384, 3, 12, 3, 1, 0, 0.0),
    ("all_masked", 300, 1024, 4, 16, 4, 1, 0, 1.0),
]


@pytest.mark.parametrize("case", DISPATCH_EDGE, ids=lambda c: c[0])
def test_dispatch_edge_cases(case):
    name, T, H, k, E, R, A, C, mask = case
    log(f"[dispatch-edge] {name}")
    w = wl.custom(name, T, H, E, R, k, seed=77, capacity=C, expert_alignment=A)
    rng = np.random.default_rng(5)
    x = wl.normal_bf16(77, 0, T, H)
    x[0, :] = 0                     # an all-zero token: scale floor
    x[1 % T, : min(H, 128)] = 0x8000  # negative zeros
    idx = _idx(rng, T, k, E, mask)
    lay = oracle.layout(idx, E, R, A, C)
    inp = wl.Inputs(w, x, idx, np.ones((T, k), np.float32))
    held = lay.src_pair >= 0
    got, _ = run_dispatch(w, inp, lay, ep.EP_BF16)
    want = oracle.dispatch_bf16(x, lay.slot, w.recv_rows)
    assert np.array_equal(got[held], want[held]) and (got[~held] == SENTINEL).all()
    if H % 128 == 0:
        q, s = run_dispatch(w, inp, lay, ep.EP_FP8_E4M3)
        wq, ws = oracle.dispatch_fp8(x, lay.slot, w.recv_rows)
        assert np.array_equal(q[held], wq[held])
        assert np.array_equal(s[held].view(np.uint32), ws[held].view(np.uint32))
        assert (q[~held] == SENTINEL).all()


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

def run_combine(w, y_bits, slot, weights):
    shape = shape_of(w)
    out = torch.full((w.num_tokens, w.hidden), 0x7BAD, dtype=torch.int16, device=DEV)
    ep.ep_combine(shape, dev_bf16(y_bits), dev_i32(slot), dev_f32(weights), out)
    torch.cuda.synchronize()
    return host_u16(out)


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_combine_within_one_ulp(name):
    w, inp, lay = inputs(name, with_y=True)
    log(f"[combine] {name}")
    got = run_combine(w, inp.y, lay.slot, inp.topk_weights)
    want = oracle.combine(inp.y, lay.slot, inp.topk_weights)
    d = bf16_ulp_distance(got, want)
    log(f"  max ulp {d.max()}, elements off by >0 ulp: {(d > 0).sum()} of {d.size}")
    assert d.max() <= 1
    # the chain order is fixed, so the result is in fact bit-exact
    assert (d == 0).all()


COMBINE_EDGE = [
    # name, T, H, k, E, R, A, C, mask
    ("k3_generic_masked", 400, 640, 3, 16, 4, 1, 0, 0.1),
    ("k16_generic", 128, 1024, 16, 64, 8, 1, 0, 0.05),
    ("k64_generic", 32, 256, 64, 64, 8, 1, 0, 0.0),
    ("padded_drops", 300, 1024, 4, 16, 4, 1, 40, 0.0),
    ("h136", 100, 136, 2, 8, 2, 4, 0, 0.0),
    ("all_masked", 300, 1024, 4, 16, 4, 1, 0, 1.0),       # every output is +0
    ("all_masked_padded", 200, 512, 4, 16, 4, 1, 20, 1.0),
]


@pytest.mark.parametrize("case", COMBINE_EDGE, ids=lambda c: c[0])
def test_combine_edge_cases(case):
    name, T, H, k, E, R, A, C, mask = case
    log(f"[combine-edge] {name}")
    w = wl.custom(name, T, H, E, R, k, seed=91, capacity=C, expert_alignment=A)
    rng = np.random.default_rng(9)
    idx = _idx(rng, T, k, E, mask)
    lay = oracle.layout(idx, E, R, A, C)
    y = wl.normal_bf16(91, 2, w.recv_rows, H)
    wts = rng.standard_normal((T, k)).astype(np.float32)  # signed: cancellation on purpose
    got = run_combine(w, y, lay.slot, wts)
    want = oracle.combine(y, lay.slot, wts)
    assert (bf16_ulp_distance(got, want) == 0).all()
    assert np.array_equal(got, want)  # bit for bit, signs of zero included


def test_combine_k1_unit_weight_is_gather():
    T, H = 333, 2048
    w = wl.custom("gather", T, H, 4, 2, 1, seed=3)
    rng = np.random.default_rng(3)
    slot = rng.permutation(T)[:, None].astype(np.int32)
    y = wl.normal_bf16(3, 2, T, H)
    got = run_combine(w, y, slot, np.ones((T, 1), np.float32))
    assert np.array_equal(got, y[slot[:, 0]])


@pytest.mark.parametrize("name", ["tiny", "mid", "decode"])
def test_identity_round_trip(name):
    """BF16 dispatch, identity experts, weights summing to 1: combine gives x back."""
    w, inp, lay = inputs(name)
    log(f"[round-trip] {name}")
    shape = ep.EpShape(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, 1, w.capacity)
    bufs = ep.LayoutBuffers.allocate(shape, DEV).run(dev_i32(inp.topk_idx))
    rx, _ = ep.alloc_recv(shape, ep.EP_BF16, DEV)
    x = dev_bf16(inp.x)
    ep.ep_dispatch(shape, x, bufs.slot, ep.EP_BF16, rx)
    out = torch.empty_like(x)
    ep.ep_combine(shape, rx, bufs.slot, dev_f32(inp.topk_weights), out)
    torch.cuda.synchronize()
    # equal as numbers: acc starts at +0, so a -0 input comes back as +0
    assert torch.equal(out.float(), x.float())
    assert bf16_ulp_distance(host_u16(out), inp.x).max() == 0


def test_cached_handle_reuse():
    """One layout, two dispatch/combine rounds with new tensors (the cached-handle path)."""
    w, inp, lay = inputs("tiny", with_y=True)
    shape = shape_of(w)
    bufs = ep.LayoutBuffers.allocate(shape, DEV).run(dev_i32(inp.topk_idx))
    for seed in (21, 22):
        x = wl.normal_bf16(seed, 0, w.num_tokens, w.hidden)
        y = wl.normal_bf16(seed, 2, w.recv_rows, w.hidden)
        rq, rs = ep.alloc_recv(shape, ep.EP_FP8_E4M3, DEV)
        ep.ep_dispatch(shape, dev_bf16(x), bufs.slot, ep.EP_FP8_E4M3, rq, rs)
        out = torch.empty((w.num_tokens, w.hidden), dtype=torch.bfloat16, device=DEV)
        ep.ep_combine(shape, dev_bf16(y), bufs.slot, dev_f32(inp.topk_weights), out)
        torch.cuda.synchronize()
        wq, ws = oracle.dispatch_fp8(x, lay.slot, w.recv_rows)
        held = lay.src_pair >= 0
        assert np.array_equal(rq.cpu().numpy()[held], wq[held])
        assert np.array_equal(host_u16(out), oracle.combine(y, lay.slot, inp.topk_weights))


# --------------------------------------------------------------------------
# the conversion instructions, swept
# --------------------------------------------------------------------------

def test_e4m3_conversion_exhaustive():
    """Every float32 with |v| <= 464, both signs: the device convert equals the oracle encoder."""
    top = int(np.array([464.0], np.float32).view(np.uint32)[0])
    chunk = 1 << 27
    log(f"[cvt-e4m3] {2 * (top + 1)} values")
    pool = ThreadPoolExecutor(16)
    bad = 0
    out = torch.empty(chunk, dtype=torch.uint8, device=DEV)
    for lo in range(0, top + 1, chunk):
        n = min(chunk, top + 1 - lo)
        for sign in (0, 0x80000000):
            bits = torch.arange(lo, lo + n, dtype=torch.int64, device=DEV) | sign
            v = bits.to(torch.int32).view(torch.float32) if sign == 0 else \
                (bits - (1 << 32)).to(torch.int32).view(torch.float32)
            ep.ep_check_cvt_e4m3(v, out[:n])
            got = out[:n].cpu().numpy()
            vh = v.cpu().numpy()
            parts = np.array_split(np.arange(n), 16)
            want = np.concatenate(list(pool.map(lambda ix: oracle.e4m3_encode(vh[ix]), parts)))
            bad += int((got != want).sum())
    pool.shutdown()
    assert bad == 0


def test_fp8_quantiser_exhaustive():
    """Every pair (block amax, BF16 x) with 0 < amax finite and |x| <= amax, both signs of x
    (~1.07e9 pairs): the dispatch kernels' quantiser (device division and E4M3 convert)
    gives the oracle's code of x / s under that amax's block scale."""
    amax = np.arange(1, 0x7F80, dtype=np.int64)          # positive finite BF16 magnitudes
    s_of = (np.maximum(wl.bf16_bits_to_f32(amax.astype(np.uint16)), np.float32(1e-4)) /
            np.float32(448.0)).astype(np.float32)        # block scale per amax (fp32, as the oracle)
    counts = 2 * (amax + 1)                                # x in [0, amax] and [-amax, -0]
    pool = ThreadPoolExecutor(16)
    bad, total, a0 = 0, 0, 0
    out = torch.empty(1 << 27, dtype=torch.uint8, device=DEV)
    while a0 < len(amax):
        a1 = a0
        n = 0
        while a1 < len(amax) and n + counts[a1] <= (1 << 27):
            n += int(counts[a1])
            a1 += 1
        c = counts[a0:a1]
        start = np.repeat(np.cumsum(c) - c, c)
        p = np.arange(n, dtype=np.int64) - start
        am = np.repeat(amax[a0:a1], c)
        x = np.where(p <= am, p, 0x8000 | (p - am - 1)).astype(np.uint16)
        s = np.repeat(s_of[a0:a1], c)
        ep.ep_check_quant_e4m3(torch.from_numpy(x.view(np.int16)).to(DEV), torch.from_numpy(s).to(DEV), out[:n])
        got = out[:n].cpu().numpy()
        parts = np.array_split(np.arange(n), 16)
        want = np.concatenate(list(pool.map(lambda ix: oracle.fp8_quantize(x[ix], s[ix]), parts)))
        bad += int((got != want).sum())
        total += n
        a0 = a1
    pool.shutdown()
    log(f"[quant-e4m3] {total} pairs, {bad} mismatches")
    assert total == int(counts.sum()) and bad == 0


def test_bf16_conversion_sweep():
    rng = np.random.default_rng(17)
    bits = rng.integers(0, 1 << 32, 1 << 25, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]  # finite only
    ties = ((rng.integers(0, 1 << 15, 1 << 20, dtype=np.uint32) << 17)
            | (rng.integers(0, 2, 1 << 20, dtype=np.uint32) << 16) | 0x8000)
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    sub = rng.integers(0, 1 << 23, 1 << 20, dtype=np.uint32) | (rng.integers(0, 2, 1 << 20, dtype=np.uint32) << 31)
    v = np.concatenate([bits, ties, sub]).view(np.float32)
    out = torch.empty(v.size, dtype=torch.int16, device=DEV)
    ep.ep_check_cvt_bf16(dev_f32(v), out)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(out), oracle.bf16_rne(v))
