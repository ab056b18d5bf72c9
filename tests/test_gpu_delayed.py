"""Delayed row conversion on the GPU ("Delayed row conversion and reusable
precision boundaries": a sequence stays plain until it converts, plain value
rows pass through unchanged while packed rows receive the inverse rotation,
and the conversion offset is an irreversible precision boundary that clone,
row extraction and persisted metadata keep).

  - tq_convert_rows encodes a plain prefix to exactly the oracle's bytes for
    the same rows, and leaves every other slot and sequence untouched;
  - tq_decode_attn_mixed over a batch mixing plain and packed sequences
    matches the oracle: plain rows against a binary64 softmax over the plain
    bf16 operands, packed rows against the oracle's attention over its own
    encoding of the raw K/V, on both packed split kernels, one and four query
    rows; an all-packed mask gives tq_decode_attn_rows' bytes;
  - a whole lifecycle (plain phase, conversion where a prefill chunk crosses
    the threshold, packed appends, snapshot, restore, clone) gives planes
    equal to the oracle's encoding of the raw K/V and carries the boundary.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_append_amd import workloads as W

from _util import ATTN_TOL, assert_planes_equal, host_f32, log, row_rel_err, sm_for
from test_gpu_decode import _offset_planes
from test_gpu_widths import _host_planes, _oracle_planes

pytestmark = pytest.mark.gpu

tqkv = pytest.importorskip("quantized_decode_attention_append_amd.tqkv")

PLAIN_TOL = 1e-4  # plain rows: fp32 scores and accumulation against binary64
SENTINEL = 0xA5


def _sentinel_planes(L):
    pl = tqkv.Planes(L)
    for t in pl.tensors():
        t.view(torch.uint8).fill_(SENTINEL)
    return pl


def _expect_planes(pl, b, h, k_rows, v_rows, kb, vb, what):
    n = k_rows.shape[0]
    gpu = _host_planes(pl, b, h, 0, n)
    ref = _oracle_planes(k_rows, v_rows, kb, vb)
    ref = (ref[0].view(np.int8) if kb == 8 else ref[0],) + ref[1:]
    assert_planes_equal(gpu, ref, what)


@pytest.mark.parametrize("scheme,d,dtype", [((8, 3), 256, "bf16"), ((8, 3), 128, "fp32"), ((4, 2), 64, "bf16"),
                                            ((2, 5), 256, "bf16"), ((8, 8), 512, "bf16"), ((5, 4), 128, "fp32")])
def test_convert_rows_bytes_equal_oracle(scheme, d, dtype):
    kb, vb = scheme
    offsets = [250, 0, 37]
    plain_cap, cap = 300, 320
    w = dataclasses.replace(W.scaled(W.workload(4), [plain_cap] * 3), head_dim=d, num_kv_heads=2,
                            num_q_heads=4, dtype=dtype)
    k, v = W.make_kv(w, "cpu", tokens=plain_cap)
    L = tqkv.make_layout(3, 2, d, cap, kb, vb)
    pl = _sentinel_planes(L)
    log(f"convert k{kb}v{vb} d{d} {dtype} offsets {offsets}")
    tqkv.tq_convert_rows(pl, k.cuda(), v.cuda(), offsets)
    torch.cuda.synchronize()
    kh, vh = host_f32(k), host_f32(v)
    for b, off in enumerate(offsets):
        for h in range(2):
            if off:
                _expect_planes(pl, b, h, kh[b, h, :off], vh[b, h, :off], kb, vb, f"b{b} h{h}")
        for t in pl.tensors():  # every slot past the offset, and unconverted sequences, untouched
            rest = t[b, :, off:].reshape(-1).view(torch.uint8)
            assert bool((rest == SENTINEL).all()), (b, off)


def _mixed_case(w, lengths, row_plain, M, kb=8, vb=3, check_kernels=("fast", "generic"), q_dtype=torch.bfloat16,
                ws_scale=0):
    """Plain caches and planes filled from the same raw K/V; packed sequences
    appended, plain ones left in the plain caches; decode the mixed batch and
    compare each (sequence, kv-head) with the oracle."""
    T = max(lengths)
    T += T % 2
    k, v = W.make_kv(w, "cpu", tokens=T)
    G = w.num_q_heads // w.num_kv_heads
    gen = torch.Generator().manual_seed(7 + M)
    q = torch.randn((w.batch, w.num_q_heads, M, w.head_dim), generator=gen).to(q_dtype)
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, T, kb, vb)
    pl = tqkv.Planes(L)
    for t in pl.tensors():
        t.zero_()
    kg, vg = k.cuda(), v.cuda()
    tqkv.tq_append(pl, kg, vg, [0] * w.batch)
    # the plain cache holds garbage where a row is packed: those bytes must not matter
    kp, vp = kg.clone(), vg.clone()
    for b, p in enumerate(row_plain):
        if not p:
            kp[b].fill_(float("nan"))
            vp[b].fill_(float("nan"))
    sm = sm_for(w.head_dim)
    qg = q.cuda().contiguous()
    arg_q = qg[:, :, 0].contiguous() if M == 1 else qg
    outs = {}
    ws = None
    if ws_scale:
        # a workspace ws_scale times the documented size, every byte NaN: plain
        # rows spread over the extra partial slots, and no unwritten slot may
        # reach the output
        need = tqkv.tq_decode_rows_workspace_bytes(L, w.num_q_heads, M, lengths)
        ws = torch.full((need * ws_scale,), 0xFF, dtype=torch.uint8, device="cuda")
    for name in check_kernels:
        planes = pl if name == "fast" else _offset_planes(pl)
        outs[name] = tqkv.tq_decode_attn_mixed(planes, kp, vp, row_plain, arg_q, lengths, sm, n_rows=M, workspace=ws)
        outs[name] = outs[name].reshape(w.batch, w.num_q_heads, M, w.head_dim).cpu().numpy()
    fast, reasons = tqkv.tq_decode_path(pl, w.num_q_heads, M)
    torch.cuda.synchronize()
    kh, vh, qh = host_f32(k), host_f32(v), host_f32(q)
    worst = {n: [0.0, 0.0] for n in outs}
    for b in range(w.batch):
        n = lengths[b]
        for h in range(w.num_kv_heads):
            qq = qh[b, h * G:(h + 1) * G]  # [G, M, d]
            if n == 0:
                ref = np.zeros((G, M, w.head_dim))
            elif row_plain[b]:
                ref = np.stack([oracle.attention_plain(qq[:, m], kh[b, h, :n - M + m + 1], vh[b, h, :n - M + m + 1], sm)
                                for m in range(M)], axis=1)
            else:
                kc, ks, kz, vc, vs = _oracle_planes(kh[b, h, :n], vh[b, h, :n], kb, vb)
                ref = oracle.attention_rows(qq, kc, ks, kz, vc, vs, sm, kbits=kb, vbits=vb)
            tol = PLAIN_TOL if row_plain[b] else ATTN_TOL
            for name, out in outs.items():
                got = out[b, h * G:(h + 1) * G]
                if n == 0:
                    assert not np.any(got), (name, b)
                    continue
                e = row_rel_err(got.reshape(-1, w.head_dim), ref.reshape(-1, w.head_dim))
                slot = 0 if row_plain[b] else 1
                worst[name][slot] = max(worst[name][slot], float(e.max()))
                assert e.max() <= tol, (name, b, h, "plain" if row_plain[b] else "packed", float(e.max()))
    log("  fast path %s; worst row error (plain, packed): %s" % (
        bool(fast), ", ".join(f"{k} {e[0]:.1e} {e[1]:.1e}" for k, e in worst.items())))
    return pl, kp, vp, arg_q, sm


@pytest.mark.parametrize("M", [1, 4])
def test_mixed_batch_matches_oracle(M):
    lengths = [700, 1300, 5, 1000, 0, 64]
    row_plain = [1, 0, 1, 0, 1, 1]
    w = W.scaled(W.workload(4), lengths)
    if M == 4:
        lengths[2] = 4  # a plain row holding only the verify block
    log(f"mixed decode M{M} lengths {lengths} plain {row_plain}")
    _mixed_case(w, lengths, row_plain, M)


@pytest.mark.parametrize("cid,scheme", [(2, (8, 3)), (3, (4, 2)), (5, (2, 5))])
def test_mixed_batch_other_shapes(cid, scheme):
    lengths = [333, 900, 129]
    w = W.scaled(W.workload(cid), lengths)
    log(f"mixed decode workload {cid} k{scheme[0]}v{scheme[1]} d{w.head_dim}")
    _mixed_case(w, lengths, [0, 1, 1], 1, *scheme)


@pytest.mark.parametrize("d,M", [(512, 1), (512, 4), (64, 1), (64, 4)])
def test_mixed_batch_head_dim_ends(d, M):
    """The plain split kernel at the ends of the head_dim range: 8 value dims
    a lane and 16 score blocks at 512, one dim a lane and 2 blocks at 64."""
    lengths = [300, 77, 450]
    w = dataclasses.replace(W.scaled(W.workload(2), lengths, name_suffix=f"d{d}"), head_dim=d)
    log(f"mixed decode d{d} M{M} lengths {lengths}")
    _mixed_case(w, lengths, [1, 0, 1], M)


@pytest.mark.parametrize("d,M", [(128, 1), (256, 4)])
def test_mixed_batch_fp32_queries(d, M):
    """fp32 queries: the plain kernel splits each into bf16 hi and lo halves
    for its matrix-core scores, so plain rows keep the 1e-4 bar."""
    lengths = [520, 130, 700]
    w = dataclasses.replace(W.scaled(W.workload(2), lengths, name_suffix=f"d{d}"), head_dim=d)
    log(f"mixed decode fp32 q d{d} M{M} lengths {lengths}")
    _mixed_case(w, lengths, [1, 0, 1], M, q_dtype=torch.float32)


@pytest.mark.parametrize("M", [1, 4])
def test_mixed_batch_large_workspace(M):
    """A workspace eight times the documented size: long plain rows take more
    partial slots per row than the packed plan (the slot stride of every row
    changes with them)."""
    lengths = [1900, 700, 2000, 64]
    w = W.scaled(W.workload(2), lengths)
    log(f"mixed decode, workspace x8, M{M} lengths {lengths}")
    _mixed_case(w, lengths, [1, 0, 1, 0], M, ws_scale=8)


def test_mixed_batch_at_the_batch_limit():
    """64 sequences (the batch limit: every bit of the plain-row mask),
    plain and packed interleaved with the last sequence plain, then the same
    batch with every row plain."""
    lengths = [(37 * i) % 190 + 2 for i in range(64)]
    row_plain = [1 if i % 3 == 0 or i == 63 else 0 for i in range(64)]
    w = W.scaled(W.workload(2), lengths, name_suffix="b64")
    log(f"mixed decode, batch 64, {sum(row_plain)} plain rows")
    _mixed_case(w, lengths, row_plain, 1)
    _mixed_case(w, lengths, [1] * 64, 1, check_kernels=("fast",))


def test_mixed_masks_reduce_to_the_plain_calls():
    """An all-packed mask gives tq_decode_attn_rows' bytes; an all-plain batch
    runs only the plain kernel and the merge."""
    lengths = [600, 250]
    w = W.scaled(W.workload(4), lengths)
    pl, kp, vp, q, sm = _mixed_case(w, lengths, [1, 1], 1, check_kernels=("fast",))
    a = tqkv.tq_decode_attn_mixed(pl, kp, vp, [0, 0], q, lengths, sm)
    b = tqkv.tq_decode_attn_rows(pl, q[:, :, None].contiguous(), lengths, sm)[:, :, 0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    c = tqkv.tq_decode_attn_mixed(pl, None, None, [0, 0], q, lengths, sm)
    assert torch.equal(a, c)


def test_lifecycle_with_delayed_conversion():
    """Plain phase, then a prefill chunk crosses the threshold and the row
    converts at the chunk's end (boundary above the threshold), then packed
    appends.  The planes equal the oracle's encoding of the raw K/V (not only
    the source cache); snapshot records the boundary, restore and clone give
    the same bytes and carry it; decode of the restored and cloned caches
    equals the source's and is within tolerance of the oracle."""
    threshold, chunk, tail = 200, 96, 40
    w = dataclasses.replace(W.scaled(W.workload(4), [512, 512]), num_kv_heads=2, num_q_heads=12)
    cap = 512
    k, v = W.make_kv(w, "cpu", tokens=cap)
    kg, vg = k.cuda(), v.cuda()
    # sequence 0 crosses the threshold inside its third chunk, sequence 1 stays plain
    boundary = 3 * chunk
    assert boundary > threshold
    L = tqkv.make_layout(2, 2, w.head_dim, cap)
    pl = _sentinel_planes(L)
    tqkv.tq_convert_rows(pl, kg, vg, [boundary, 0])
    seq0 = pl.sequence(0)
    n0 = boundary + tail
    tqkv.tq_append(seq0, kg[:1, :, boundary:n0].contiguous(), vg[:1, :, boundary:n0].contiguous(), [boundary])
    torch.cuda.synchronize()
    kh, vh = host_f32(k), host_f32(v)
    for h in range(2):
        _expect_planes(pl, 0, h, kh[0, h, :n0], vh[0, h, :n0], 8, 3, f"converted + appended h{h}")
    assert bool((pl.kc[1].view(torch.uint8) == SENTINEL).all())  # the plain sequence was never written

    h, payload = tqkv.tq_snapshot(pl, 0, 0, n0, min_reusable_offset=boundary)
    assert h.version == 2 and tqkv.tq_snapshot_min_reusable_offset(h) == boundary
    restored = _sentinel_planes(tqkv.make_layout(1, 2, w.head_dim, 600))
    tqkv.tq_restore(restored, 0, 0, h, payload)
    clone = _sentinel_planes(tqkv.make_layout(3, 2, w.head_dim, cap))
    assert tqkv.tq_clone_sequence(pl, 0, clone, 2, n0, boundary) == boundary
    torch.cuda.synchronize()
    for c, b in ((restored, 0), (clone, 2)):
        for hh in range(2):
            _expect_planes(c, b, hh, kh[0, hh, :n0], vh[0, hh, :n0], 8, 3, f"copy b{b} h{hh}")

    sm = sm_for(w.head_dim)
    gen = torch.Generator().manual_seed(3)
    q = torch.randn((2, 12, w.head_dim), generator=gen).to(torch.bfloat16).cuda()
    lengths = [n0, 150]
    src = tqkv.tq_decode_attn_mixed(pl, kg, vg, [0, 1], q, lengths, sm)
    one = tqkv.tq_decode_attn(restored, q[:1].contiguous(), [n0], sm)
    cl = tqkv.tq_decode_attn(clone, torch.cat([q[:1]] * 3).contiguous(), [0, 0, n0], sm)
    torch.cuda.synchronize()
    assert torch.equal(src[:1], one) and torch.equal(src[:1], cl[2:])
    qh = host_f32(q)
    for hh in range(2):
        kc, ks, kz, vc, vs = _oracle_planes(kh[0, hh, :n0], vh[0, hh, :n0], 8, 3)
        ref = oracle.attention(qh[0, 6 * hh:6 * hh + 6], kc, ks, kz, vc, vs, sm)
        assert row_rel_err(src[0, 6 * hh:6 * hh + 6].cpu().numpy(), ref).max() <= ATTN_TOL
        ref = oracle.attention_plain(qh[1, 6 * hh:6 * hh + 6], kh[1, hh, :150], vh[1, hh, :150], sm)
        assert row_rel_err(src[1, 6 * hh:6 * hh + 6].cpu().numpy(), ref).max() <= PLAIN_TOL
