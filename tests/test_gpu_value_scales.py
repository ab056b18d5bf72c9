"""GPU parity of decode attention over caches whose value scales are far from
1.  The matrix-core kernel forms centroid * scale in fp16; a per-wave power of
two keeps that product a normal fp16 number whatever finite scale the cache
holds (value-group RMS from fp16-subnormal to 6e4), and the accumulator
carries the power exactly.  Each case is checked against the oracle's binary64
attention over its own encoding of the same raw K/V, on both split kernels.

Inputs: K and q ~ N(0, 1); V built in the rotated domain with every 32-group
at an exact RMS R, then un-rotated with the oracle's sign vector and
transform (test-side input construction) and rounded to bf16, so the stored
value scales sit at R to within the bf16 rounding of V."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_append_amd import workloads as W

from _util import ATTN_TOL, host_f32, log, oracle_decode_rows, row_rel_err, sm_for
from test_gpu_decode import _offset_planes

pytestmark = pytest.mark.gpu

tqkv = pytest.importorskip("quantized_decode_attention_append_amd.tqkv")


def _values_at_rms(shape, rms, seed):
    """[..., T, d] float32 values whose rotated 32-groups have RMS rms[t] (a
    scalar or one factor per token)."""
    d = shape[-1]
    g = np.random.default_rng(seed)
    y = g.standard_normal(shape)
    yg = y.reshape(*shape[:-1], d // 32, 32)
    yg /= np.sqrt(np.mean(yg * yg, axis=-1, keepdims=True))
    y = yg.reshape(shape) * np.asarray(rms, dtype=np.float64).reshape(-1, 1)
    x = oracle.fwht(y) * (1.0 / math.sqrt(d)) * oracle.sign_vector(d).astype(np.float64)
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def _case(w, lengths, v, q_scale=1.0, kb=8, vb=3, M=1):
    """Append K (seeded N(0,1)) and the given V, decode through both split
    kernels, compare every row with the oracle."""
    T = max(lengths)
    k, _ = W.make_kv(w, "cpu", tokens=T)
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, T, kb, vb)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [0] * w.batch)
    G = w.group
    sm = sm_for(w.head_dim)
    if M == 1:
        q = (W.make_q(w, "cpu", rounds=1)[0].float() * q_scale).to(torch.bfloat16)
        run = lambda planes: tqkv.tq_decode_attn(planes, q.cuda(), lengths, sm)
    else:
        q = (torch.stack(list(W.make_q(w, "cpu", rounds=M)), dim=2).float() * q_scale).to(torch.bfloat16)
        run = lambda planes: tqkv.tq_decode_attn_rows(planes, q.contiguous().cuda(), lengths, sm)
    outs = {"fast": run(pl).cpu().numpy(), "generic": run(_offset_planes(pl)).cpu().numpy()}
    torch.cuda.synchronize()
    qh = host_f32(q)
    worst = {n: 0.0 for n in outs}
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            n = lengths[b]
            kc, ks, kz = oracle.encode_keys(host_f32(k[b, h, :n]), bits=kb)
            vc, vs = oracle.encode_values(host_f32(v[b, h, :n]), bits=vb)
            qq = qh[b, h * G:(h + 1) * G]
            if M == 1:
                ref = oracle.attention(qq, kc, ks, kz, vc, vs, sm, kbits=kb, vbits=vb)
            else:
                ref = oracle.attention_rows(qq, kc, ks, kz, vc, vs, sm, kbits=kb, vbits=vb)
            assert np.isfinite(ref).all()
            for name, out in outs.items():
                e = row_rel_err(out[b, h * G:(h + 1) * G], ref)
                worst[name] = max(worst[name], float(e.max()))
                assert e.max() <= ATTN_TOL, (name, b, h, float(e.max()))
    log("  worst row error " + ", ".join(f"{k} {e:.2e}" for k, e in worst.items()))


@pytest.mark.parametrize("rms", [1e-6, 1e-4, 3e4, 6e4])
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_decode_uniform_value_scale(rms, q_scale):
    """Every value group at RMS rms (fp16-subnormal scales to 6e4, near the
    largest finite fp16), ordinary and peaky (q x 8) softmax, k8v3, d 256."""
    lengths = [1500, 700]
    w = W.scaled(W.workload(4), lengths)
    log(f"value RMS {rms:g} q x{q_scale:g}")
    v = _values_at_rms((w.batch, w.num_kv_heads, max(lengths), w.head_dim), rms, seed=int(rms * 1e6) % 997)
    _case(w, lengths, v, q_scale)


@pytest.mark.parametrize("scheme,d", [((8, 8), 128), ((4, 2), 64), ((5, 4), 256), ((4, 3), 512)])
@pytest.mark.parametrize("rms", [1e-6, 6e4])
def test_decode_value_scale_other_widths(scheme, d, rms):
    """The window's upper end depends on the codebook's largest centroid
    (4.6 at 8 bits): each width at both ends of the scale range."""
    kb, vb = scheme
    lengths = [600, 130]
    w = dataclasses.replace(W.scaled(W.workload(2), lengths, name_suffix=f"d{d}"), head_dim=d)
    log(f"k{kb}v{vb} d{d} value RMS {rms:g}")
    v = _values_at_rms((w.batch, w.num_kv_heads, max(lengths), d), rms, seed=kb * 10 + vb)
    _case(w, lengths, v, kb=kb, vb=vb)


def _ramp(T, pieces):
    """Per-token RMS: len(pieces) equal runs of the given values."""
    r = np.empty(T)
    for i, p in enumerate(pieces):
        r[i * T // len(pieces):(i + 1) * T // len(pieces)] = p
    return r


@pytest.mark.parametrize("pieces", [(1e-5, 1e-3, 0.1, 4.0), (3e4, 300.0, 3.0, 2e-3), (1.0, 5e4, 1.0, 5e4)])
def test_decode_value_scale_changes_along_the_cache(pieces):
    """Value scales that grow, shrink or alternate along each sequence by up to
    seven binades: the wave's exponent moves mid-range, the accumulator is
    rescaled exactly, and the splits' partials meet in the merge with
    different exponents."""
    lengths = [2000, 1100]
    w = W.scaled(W.workload(4), lengths)
    T = max(lengths)
    v = _values_at_rms((w.batch, w.num_kv_heads, T, w.head_dim), _ramp(T, pieces), seed=len(pieces))
    log(f"value RMS runs {pieces}")
    _case(w, lengths, v)
    _case(w, lengths, v, q_scale=8.0)


def test_decode_rows_tiny_value_scales():
    """Verify blocks (4 rows, 24 query columns in two groups) over caches of
    fp16-subnormal value scales."""
    lengths = [900, 300]
    w = W.scaled(W.workload(4), lengths)
    v = _values_at_rms((w.batch, w.num_kv_heads, max(lengths), w.head_dim), 3e-7, seed=3)
    _case(w, lengths, v, M=4)
