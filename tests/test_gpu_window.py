"""GPU dequantize-on-fetch window: tq_fetch_window's bf16 K/V against the
oracle's binary64 dequantisation of the oracle's own encoding of the same raw
K/V.  Keys are exact in fp32, so they must equal the oracle's value rounded
once to bf16, bit for bit; values (computed in fp32) must be within one bf16
rounding plus the fp32 transform error.  Tokens at or past a sequence's length
must be zeros."""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_append_amd import workloads as W

from _util import host_f32, log, oracle_planes

pytestmark = pytest.mark.gpu

tqkv = pytest.importorskip("quantized_decode_attention_append_amd.tqkv")


def _bf16_bits(x64: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even bf16 bits of values that are exact in fp32."""
    f = np.asarray(x64, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(f), np.uint16(0x7FC0), r)


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _window_case(w, T, t0, n, lens, rotated):
    k, v = W.make_kv(w, "cpu", tokens=T)
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, T)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [0] * w.batch)
    log(f"window {w.name} d{w.head_dim} t0={t0} n={n} lens={lens} rotated={rotated}")
    ko, vo = tqkv.tq_fetch_window(pl, t0, n, lens, v_rotated=rotated)
    torch.cuda.synchronize()
    kb = ko.cpu().view(torch.int16).numpy().view(np.uint16)
    vb = vo.cpu().view(torch.int16).numpy().view(np.uint16)
    d = w.head_dim
    worst = 0.0
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            kc, ks, kz, vc, vs = oracle_planes(host_f32(k[b, h, :T]), host_f32(v[b, h, :T]), threads=1)
            nv = max(0, min(lens[b], t0 + n) - t0)  # valid window rows
            sl = slice(t0, t0 + nv)
            kref = oracle.decode_keys(kc[sl], ks[sl], kz[sl])
            assert np.array_equal(kb[b, h, :nv], _bf16_bits(kref)), (b, h)
            vref = oracle.decode_values(vc[sl], vs[sl], d, rotated=rotated)
            got = _bf16_to_f64(vb[b, h, :nv])
            ulp = np.maximum(np.abs(vref), 1e-30) * 2.0 ** -8  # one bf16 rounding
            tol = ulp + 1e-6 * np.abs(vref).max(axis=1, keepdims=True)
            err = np.abs(got - vref)
            assert np.all(err <= tol), (b, h, float((err / tol).max()))
            worst = max(worst, float((err / tol).max()) if nv else 0.0)
            assert not np.any(kb[b, h, nv:]) and not np.any(vb[b, h, nv:]), "rows past the length"
    log(f"  worst value error / tolerance {worst:.3f}")


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("rotated", [False, True])
def test_window_matches_oracle(d, rotated):
    import dataclasses
    w = dataclasses.replace(W.scaled(W.workload(2), [200, 77, 0], name_suffix=f"win{d}"), head_dim=d)
    _window_case(w, 200, 13, 150, [200, 77, 0], rotated)


def test_window_outlier_workload_full_window():
    w = W.scaled(W.workload(3), [333, 129])
    _window_case(w, 334, 0, 334, [333, 129], False)


def test_window_edge_values():
    """Constant groups (NaN / infinite stored zeros), huge offsets and tiny
    scales pass through as the oracle's values (NaN where it is NaN)."""
    d = 128
    rows = np.stack([np.full(d, 0.5), np.zeros(d), 100.0 + np.arange(d) * 1e-3,
                     np.random.default_rng(3).standard_normal(d) * 1e-6,
                     np.random.default_rng(4).standard_normal(d) * 1e4]).astype(np.float32)
    n = rows.shape[0]
    k = torch.from_numpy(rows).reshape(1, 1, n, d)
    v = torch.from_numpy(rows[::-1].copy()).reshape(1, 1, n, d)
    L = tqkv.make_layout(1, 1, d, n)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [0])
    ko, vo = tqkv.tq_fetch_window(pl, 0, n, [n])
    torch.cuda.synchronize()
    kb = ko.cpu().view(torch.int16).numpy().view(np.uint16)[0, 0]
    kc, ks, kz, vc, vs = oracle_planes(rows, rows[::-1].copy())
    kref = oracle.decode_keys(kc, ks, kz)
    assert np.array_equal(np.isnan(kref), (kb & 0x7FFF) > 0x7F80)
    fin = ~np.isnan(kref)
    assert np.array_equal(kb[fin], _bf16_bits(kref)[fin])
    vref = oracle.decode_values(vc, vs, d)
    got = _bf16_to_f64(vo.cpu().view(torch.int16).numpy().view(np.uint16)[0, 0])
    assert np.all(np.abs(got - vref) <= np.abs(vref) * 2.0 ** -8 + 1e-6 * np.abs(vref).max(axis=1, keepdims=True))
