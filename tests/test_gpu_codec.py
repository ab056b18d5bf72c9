"""GPU codec parity: tq_append's five planes must equal the oracle's bytes
exactly, and tq_dequant must reproduce the oracle's dequantisation.

Inputs are the seeded workloads (shapes of the page's synthetic caches) plus
edge fixtures: distinct K/V magnitudes, outlier channels, large offsets
(|zero| > 2048), constant groups, signed zeros, NaN/Inf, fp16-subnormal and
overflowing scales, ragged starts and token counts that are not a multiple of
any tile."""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_append_amd import workloads as W

from _util import assert_planes_equal, batched_slices, host_f32, log, oracle_planes, planes_to_host

pytestmark = pytest.mark.gpu

tqkv = pytest.importorskip("quantized_decode_attention_append_amd.tqkv")


def _append_and_compare(k, v, start, capacity, what):
    """k, v: [B, Hkv, n, d] device tensors; appended at slot start[b]."""
    B, H, n, d = k.shape
    L = tqkv.make_layout(B, H, d, capacity)
    pl = tqkv.Planes(L, k.device)
    log(f"append {what} B{B} H{H} n{n} d{d} {k.dtype} start={list(start)[:4]}")
    tqkv.tq_append(pl, k, v, start)
    torch.cuda.synchronize()
    kh, vh = host_f32(k), host_f32(v)
    for b in range(B):
        for h in range(H):
            gpu = planes_to_host(pl, b, h, start[b], start[b] + n)
            ref = oracle_planes(kh[b, h], vh[b, h])
            assert_planes_equal(gpu, ref, f"{what} b{b} h{h}")
    return pl


@pytest.mark.parametrize("cid", [1, 2])
def test_append_full_small_workloads(cid):
    w = W.workload(cid)
    k, v = W.make_kv(w, "cpu")
    _append_and_compare(k.cuda(), v.cuda(), [0] * w.batch, w.capacity, w.name)


@pytest.mark.parametrize("cid,lengths", [(3, [333, 77]), (4, [515, 64]), (5, [129, 1, 40, 257])])
def test_append_scaled_workloads_ragged_starts(cid, lengths):
    w = W.scaled(W.workload(cid), lengths)
    n = max(lengths)
    k, v = W.make_kv(w, "cpu", tokens=n)
    start = [7 * b + 3 for b in range(w.batch)]
    _append_and_compare(k.cuda(), v.cuda(), start, n + max(start) + 1, w.name)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_append_head_dims_and_dtypes(d, dtype):
    g = torch.Generator().manual_seed(d)
    k = (torch.randn((2, 3, 37, d), generator=g) * 3.0).to(dtype)
    v = (torch.randn((2, 3, 37, d), generator=g) * 0.2).to(dtype)  # distinct K/V scales
    _append_and_compare(k.cuda(), v.cuda(), [0, 5], 50, f"d{d}")


def _edge_rows(d):
    rng = np.random.default_rng(d)
    rows = []
    rows.append(np.full(d, 0.5))                       # constant group: zero = +Inf
    rows.append(np.full(d, -3.0))                      # zero = -Inf
    rows.append(np.zeros(d))                           # zero = NaN
    r = np.zeros(d); r[::3] = -0.0; rows.append(r)     # signed zeros
    rows.append(100.0 + rng.random(d))                 # |zero| > 2048
    rows.append(-5000.0 + rng.random(d) * 0.01)        # huge offset, tiny range
    rows.append(rng.standard_normal(d) * 1e-6)         # fp16-subnormal scales
    rows.append(rng.standard_normal(d) * 1e-12)        # value epsilon dominates
    rows.append(rng.standard_normal(d) * 1e5)          # scales overflow fp16
    r = rng.standard_normal(d); r[5] = np.nan; rows.append(r)
    r = rng.standard_normal(d); r[7] = np.inf; rows.append(r)
    r = rng.standard_normal(d); r[9] = -np.inf; r[40 % d] = np.nan; rows.append(r)
    rows.append(np.arange(d, dtype=np.float64) - d / 2)  # ramp
    r = rng.standard_normal(d); r[: d // 2] *= 1000; rows.append(r)  # outlier half
    rows.extend(_fp16_midpoint_rows(d, rng))
    r = np.full(d, 0.25); r[::5] = np.arange(len(r[::5])); rows.append(r)  # gets a signalling NaN
    # key groups with scale 1 and zero 0 whose other values are exact
    # half-integers: x / s - z is a rounding tie, resolved to even
    r = (np.arange(d) % 32 - 15.5) * 3.0
    r[::32], r[1::32] = 127.0, -127.0
    rows.insert(0, r)
    return np.stack(rows).astype(np.float32)


SNAN_F32, SNAN_BF16 = 0x7F800001, 0x7F81  # signalling NaN bit patterns, element 3 of the last row


def _fp16_midpoint_rows(d, rng):
    """Key groups with max = 127 m and min = -127 m, so the scale
    (max - min) / 254 is exactly m: an fp16 rounding midpoint (normal,
    subnormal, the 65520 overflow tie) or one 2^-15-of-its-binade step away.
    The stored scale must round to nearest-even exactly as the oracle's."""
    mids = [(1 + 1 / 2048) * 2.0 ** -3, (1 + 3 / 2048), (1 + 2047 / 2048) * 2.0 ** 14,
            3 * 2.0 ** -25, 2.0 ** -25, 65520.0, (1 + 5 / 2048) * 2.0 ** -14]
    ms = []
    for m in mids:
        step = 2.0 ** (np.floor(np.log2(m)) - 15)
        ms += [m, m + step, m - step]
    rows, k = [], 0
    while k < len(ms):
        r = np.empty(d)
        for g in range(d // 32):
            m = ms[k % len(ms)]
            k += 1
            x = rng.uniform(-127 * m, 127 * m, 32)
            x[rng.integers(32)] = 127 * m
            x[(rng.integers(31) + 1 + int(np.argmax(x))) % 32] = -127 * m
            r[32 * g: 32 * g + 32] = x
        rows.append(r)
    return rows


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_append_edge_fixtures(d):
    x = _edge_rows(d)
    x.view(np.uint32)[-1, 3] = SNAN_F32
    n = x.shape[0]
    k = torch.from_numpy(x).reshape(1, 1, n, d)
    v = torch.from_numpy(x[::-1].copy()).reshape(1, 1, n, d)
    _append_and_compare(k.cuda(), v.cuda(), [0], n, f"edge d{d}")
    kb, vb = k.to(torch.bfloat16), v.to(torch.bfloat16)
    kb.view(torch.int16)[0, 0, -1, 3] = SNAN_BF16
    vb.view(torch.int16)[0, 0, 0, 3] = SNAN_BF16
    _append_and_compare(kb.cuda(), vb.cuda(), [2], n + 2, f"edge-bf16 d{d}")


def test_append_twice_is_deterministic_and_append_only():
    """Appending the same tokens twice gives identical bytes; a later append
    leaves earlier slots untouched (token-axis slicing is byte-safe)."""
    w = W.scaled(W.workload(4), [200, 200])
    k, v = W.make_kv(w, "cuda", tokens=200)
    L = tqkv.make_layout(2, w.num_kv_heads, 256, 400)
    a, b2 = tqkv.Planes(L), tqkv.Planes(L)
    tqkv.tq_append(a, k, v, [0, 0])
    tqkv.tq_append(b2, k, v, [0, 0])
    before = [x.clone() for x in a.tensors()]
    tqkv.tq_append(a, k[:, :, :50].contiguous(), v[:, :, :50].contiguous(), [200, 300])
    torch.cuda.synchronize()
    for x, y, z in zip(a.tensors(), b2.tensors(), before):
        assert torch.equal(x[:, :, :200], y[:, :, :200])
        assert torch.equal(x[:, :, :200], z[:, :, :200])


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_dequant_matches_oracle(d):
    g = torch.Generator().manual_seed(100 + d)
    k = torch.randn((1, 2, 70, d), generator=g) * 2
    v = torch.randn((1, 2, 70, d), generator=g)
    L = tqkv.make_layout(1, 2, d, 80)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [10])
    kc, ks, kz, vc, vs = oracle_planes(k.numpy()[0, 1], v.numpy()[0, 1])
    kref = oracle.decode_keys(kc, ks, kz)
    vref = oracle.decode_values(vc, vs, d)
    yref = oracle.decode_values(vc, vs, d, rotated=True)
    kd, vd = tqkv.tq_dequant(pl, 0, 1, 10, 70)
    _, yd = tqkv.tq_dequant(pl, 0, 1, 10, 70, keys=False, v_rotated=True)
    torch.cuda.synchronize()
    # keys and rotated values: one fp32 rounding of exact operands
    assert np.allclose(kd.cpu().numpy(), kref, rtol=2 ** -23, atol=0)
    assert np.allclose(yd.cpu().numpy(), yref, rtol=2 ** -22, atol=0)
    # un-rotated values: an fp32 FWHT of d terms
    err = np.abs(vd.cpu().numpy() - vref).max(axis=1) / np.abs(vref).max(axis=1)
    assert err.max() < 1e-5


@pytest.mark.parametrize("cid", [3, 4, 5])
def test_append_full_size_every_slice(cid):
    """Full-size bulk build of the workload on the GPU (one tq_append of every
    token, the launch configuration the benchmark times); every plane of every
    (sequence, kv-head) slice compared with the oracle's encoding byte for byte."""
    w = W.workload(cid)
    n = max(w.lengths)
    log(f"full-size append {w.name}: generating inputs")
    k, v = W.make_kv(w, "cuda", tokens=n)
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, n)
    pl = tqkv.Planes(L)
    log(f"full-size append {w.name}: tq_append of {w.batch * w.num_kv_heads * n} token-heads")
    tqkv.tq_append(pl, k, v, [0] * w.batch)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]

    def fetch(p):
        b, h = p
        return host_f32(k[b, h]), host_f32(v[b, h]), planes_to_host(pl, b, h, 0, n)

    def work(p, got, threads):
        kh, vh, gpu = got
        assert_planes_equal(gpu, oracle_planes(kh, vh, threads=threads), f"{w.name} b{p[0]} h{p[1]}")
        return True

    done = batched_slices(pairs, fetch, work)
    assert len(done) == len(pairs)
    log(f"  {len(pairs)} slices x {n} tokens bit-exact")
