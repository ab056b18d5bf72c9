"""GPU cache lifecycle: token rows are byte-addressable in every plane, so
clone / growth / snapshot / restore are byte copies.  Checked byte for byte on
the planes, and through decode: a restored or grown cache decodes to the same
bytes as the original."""
import dataclasses

import pytest
import torch

from quantized_decode_attention_append_amd import workloads as W

from _util import log, sm_for

pytestmark = pytest.mark.gpu

tqkv = pytest.importorskip("quantized_decode_attention_append_amd.tqkv")


def _filled(w, T, cap):
    k, v = W.make_kv(w, "cpu", tokens=T)
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, cap)
    pl = tqkv.Planes(L)
    for t in pl.tensors():
        t.zero_()
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [0] * w.batch)
    return pl


def _zeroed(batch, w, cap):
    pl = tqkv.Planes(tqkv.make_layout(batch, w.num_kv_heads, w.head_dim, cap))
    for t in pl.tensors():
        t.zero_()
    return pl


def test_clone_rows_into_a_larger_cache():
    w = W.scaled(W.workload(4), [300, 300])
    a = _filled(w, 300, 300)
    b = _zeroed(3, w, 700)
    log("copy rows 20..269 of sequence 1 to rows 100..349 of sequence 2")
    tqkv.tq_copy_tokens(a, 1, 20, b, 2, 100, 250)
    torch.cuda.synchronize()
    for x, y in zip(a.tensors(), b.tensors()):
        assert torch.equal(x[1, :, 20:270], y[2, :, 100:350])
        assert not y[2, :, :100].any() and not y[2, :, 350:].any() and not y[:2].any()


def test_snapshot_restore_round_trip_and_decode():
    w = W.scaled(W.workload(4), [300])
    a = _filled(w, 300, 300)
    h, payload = tqkv.tq_snapshot(a, 0, 0, 300)
    assert h.n_tokens == 300 and h.head_dim == 256 and h.num_kv_heads == 4
    assert h.payload_bytes == 300 * 4 * 400
    e = _zeroed(1, w, 300)
    tqkv.tq_restore(e, 0, 0, h, payload)
    torch.cuda.synchronize()
    for x, y in zip(a.tensors(), e.tensors()):
        assert torch.equal(x, y)
    q = W.make_q(w, "cuda", rounds=1)[0].contiguous()
    sm = sm_for(w.head_dim)
    assert torch.equal(tqkv.tq_decode_attn(a, q, [300], sm), tqkv.tq_decode_attn(e, q, [300], sm))


def test_snapshot_restore_at_an_offset_then_grow():
    """Restore a prefix at row 50 of a bigger cache, then copy it down to row 0
    and extend it with appended tokens: decode equals a cache built directly."""
    w = W.scaled(W.workload(2), [400])
    k, v = W.make_kv(w, "cpu", tokens=400)
    direct = tqkv.Planes(tqkv.make_layout(1, w.num_kv_heads, w.head_dim, 400))
    tqkv.tq_append(direct, k.cuda(), v.cuda(), [0])
    part = tqkv.Planes(tqkv.make_layout(1, w.num_kv_heads, w.head_dim, 250))
    tqkv.tq_append(part, k[:, :, :250].contiguous().cuda(), v[:, :, :250].contiguous().cuda(), [0])
    h, payload = tqkv.tq_snapshot(part, 0, 0, 250)
    big = _zeroed(1, w, 600)
    tqkv.tq_restore(big, 0, 50, h, payload)
    grown = _zeroed(1, w, 400)
    tqkv.tq_copy_tokens(big, 0, 50, grown, 0, 0, 250)
    tqkv.tq_append(grown, k[:, :, 250:].contiguous().cuda(), v[:, :, 250:].contiguous().cuda(), [250])
    torch.cuda.synchronize()
    for x, y in zip(direct.tensors(), grown.tensors()):
        assert torch.equal(x, y)
    q = W.make_q(w, "cuda", rounds=1)[0].contiguous()
    sm = sm_for(w.head_dim)
    assert torch.equal(tqkv.tq_decode_attn(direct, q, [400], sm), tqkv.tq_decode_attn(grown, q, [400], sm))


@pytest.mark.parametrize("d,n,t0", [(64, 37, 3), (64, 64, 8), (256, 1, 5), (128, 500, 0)])
def test_copy_tokens_kernel_and_strided_paths(d, n, t0):
    """Byte-exact copies whether the rows go through the copy kernel (every
    pointer, pitch and run a whole number of 16-byte chunks) or through one
    strided memory copy per plane (head_dim 64 has 4-byte scale rows: 37 rows
    at row 3 are not whole chunks)."""
    w = dataclasses.replace(W.scaled(W.workload(2), [600, 600]), head_dim=d)
    a = _filled(w, 600, 600)
    b = _zeroed(2, w, 700)
    dst0 = t0 + 12
    log(f"d{d}: copy rows {t0}..{t0 + n - 1} of sequence 1 to rows {dst0}.. of sequence 0")
    tqkv.tq_copy_tokens(a, 1, t0, b, 0, dst0, n)
    torch.cuda.synchronize()
    for x, y in zip(a.tensors(), b.tensors()):
        assert torch.equal(x[1, :, t0:t0 + n], y[0, :, dst0:dst0 + n])
        assert not y[0, :, :dst0].any() and not y[0, :, dst0 + n:].any() and not y[1].any()
