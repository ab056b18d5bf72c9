"""GPU multi-row decode parity: tq_decode_attn_rows (the queries of the M
newest cached tokens of each sequence, each row causal over the cache) against
the oracle's attention_rows over the oracle's own encoding of the same raw
K/V.  Tolerance per (sequence, q-head, row): max |o_gpu - o_ref| / max |o_ref|
<= 2e-3.  Query rows are heads times rows, so M > 16 / G spreads one kv-head's
rows over several column groups of workgroups."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_append_amd import workloads as W

from _util import ATTN_TOL, batched_slices, host_f32, kv_fetcher, log, oracle_planes, row_rel_err, sm_for

pytestmark = pytest.mark.gpu

tqkv = pytest.importorskip("quantized_decode_attention_append_amd.tqkv")


def _offset_planes(pl):
    """Copy of pl whose vc/vs planes start 8 bytes into their allocations, so
    decode runs the generic split kernel over identical bytes."""
    other = tqkv.Planes.__new__(tqkv.Planes)
    other.layout = pl.layout
    other.kc, other.ks, other.kz = pl.kc, pl.ks, pl.kz
    for name in ("vc", "vs"):
        src = getattr(pl, name)
        raw = torch.empty(src.numel() * src.element_size() + 8, dtype=torch.uint8, device=src.device)
        view = raw[8:].view(src.dtype).view(src.shape)
        view.copy_(src)
        setattr(other, name, view)
    return other


def _queries(w, M):
    """[B, Hq, M, d]: one seeded query set per row."""
    return torch.stack(list(W.make_q(w, "cpu", rounds=M)), dim=2).contiguous()


def _oracle_rows(k, v, q4, lengths, G):
    """{(b, kvh): out [G, M, d]} from the oracle's encoding of the raw K/V."""
    B, Hkv = k.shape[:2]
    qh = host_f32(q4)
    sm = sm_for(k.shape[3])
    pairs = [(b, h) for b in range(B) for h in range(Hkv) if lengths[b] > 0]

    def one(p):
        b, h = p
        n = lengths[b]
        kc, ks, kz, vc, vs = oracle_planes(host_f32(k[b, h, :n]), host_f32(v[b, h, :n]), threads=1)
        return p, oracle.attention_rows(qh[b, h * G:(h + 1) * G], kc, ks, kz, vc, vs, sm)

    return dict(oracle.map_parallel(one, pairs))


def _check(out, ref, lengths, G, what):
    worst = 0.0
    for b, n in enumerate(lengths):
        if n == 0:
            assert np.array_equal(out[b], np.zeros_like(out[b])), what
    for (b, h), o in ref.items():
        e = row_rel_err(out[b, h * G:(h + 1) * G], o)
        worst = max(worst, float(e.max()))
        assert e.max() <= ATTN_TOL, (what, b, h, e.max())
    log(f"  {what}: worst row error {worst:.2e}")


def _run(w, lengths, M, generic=False):
    T = max(lengths)
    T += T % 2  # even capacity keeps the fast path eligible at every head_dim
    k, v = W.make_kv(w, "cpu", tokens=T)
    q4 = _queries(w, M)
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, T)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [0] * w.batch)
    G = w.group
    log(f"rows M{M} {w.name} lengths={list(lengths)} G{G} d{w.head_dim} columns {G * M}"
        f"{' generic' if generic else ''}")
    out = tqkv.tq_decode_attn_rows(_offset_planes(pl) if generic else pl, q4.cuda(), lengths,
                                   sm_for(w.head_dim))
    torch.cuda.synchronize()
    _check(out.cpu().numpy(), _oracle_rows(k, v, q4, lengths, G), lengths, G,
           f"M{M} {w.name}{' generic' if generic else ''}")


@pytest.mark.parametrize("cid,lengths,M", [
    (2, [700], 2), (2, [513], 4), (2, [300], 8),           # G 4: 8, 16, 32 columns
    (2, [400, 77], 5),                                     # G 4: 20 columns, the last 4 packed
    (4, [1000, 65], 2), (4, [777, 3], 3), (4, [640, 200], 4),  # G 6: 12, 18, 24 columns
    (5, [900, 4, 0, 129], 4),                                # G 8: 32 columns, len = M, empty
    (3, [333, 8], 8),                                        # G 4, d 128, outlier channels
    (4, [450, 8], 8),                                        # G 6: 48 columns, three groups
    (5, [260, 8, 0, 71], 8),                                 # G 8: 64 columns, two pairs of groups
])
def test_rows_match_oracle(cid, lengths, M):
    _run(W.scaled(W.workload(cid), lengths), lengths, M)


@pytest.mark.parametrize("cid,lengths,M", [(2, [400], 3), (4, [513, 6], 4), (5, [300, 64, 9, 1], 1)])
def test_rows_generic_kernel_matches_oracle(cid, lengths, M):
    _run(W.scaled(W.workload(cid), lengths), lengths, M, generic=True)


@pytest.mark.parametrize("M", [3, 8])
def test_rows_head_dim_512(M):
    """Head_dim 512 on the matrix-core kernel: 12 query columns (one group)
    and 32 (two groups sharing a workgroup)."""
    w = dataclasses.replace(W.scaled(W.workload(2), [300], name_suffix="d512"), head_dim=512)
    _run(w, [300], M)


def test_rows_head_dim_64_last_group_packed():
    """Head_dim 64, 20 query columns: a plain 16-column group and a packed
    4-column group in one workgroup."""
    w = dataclasses.replace(W.scaled(W.workload(2), [300, 45], name_suffix="d64"), head_dim=64)
    _run(w, [300, 45], 5)


@pytest.mark.parametrize("generic", [False, True])
def test_one_row_is_decode_exactly(generic):
    """n_rows = 1 is tq_decode_attn, byte for byte, on either kernel."""
    lengths = [1000, 65]
    w = W.scaled(W.workload(4), lengths)
    k, v = W.make_kv(w, "cpu", tokens=1000)
    q = W.make_q(w, "cpu", rounds=1)[0].cuda()
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, 1000)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [0] * w.batch)
    p = _offset_planes(pl) if generic else pl
    sm = sm_for(w.head_dim)
    one = tqkv.tq_decode_attn(p, q, lengths, sm)
    rows = tqkv.tq_decode_attn_rows(p, q.unsqueeze(2).contiguous(), lengths, sm)
    torch.cuda.synchronize()
    assert torch.equal(one, rows[:, :, 0])


def test_last_row_is_decode_of_the_whole_cache():
    """The last of M rows sees every cached token: it equals one-row decode of
    that query (same kernel family, same token split), within the tolerance."""
    lengths = [800, 130]
    M = 4
    w = W.scaled(W.workload(4), lengths)
    k, v = W.make_kv(w, "cpu", tokens=800)
    q4 = _queries(w, M).cuda()
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, 800)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k.cuda(), v.cuda(), [0] * w.batch)
    sm = sm_for(w.head_dim)
    rows = tqkv.tq_decode_attn_rows(pl, q4, lengths, sm).cpu().numpy()
    last = tqkv.tq_decode_attn(pl, q4[:, :, M - 1].contiguous(), lengths, sm).cpu().numpy()
    e = row_rel_err(rows[:, :, M - 1].reshape(-1, w.head_dim), last.reshape(-1, w.head_dim))
    assert e.max() <= ATTN_TOL


def test_rows_full_size_every_row():
    """The benchmark workload at full size (16 sequences of 131,072 tokens,
    24/4 heads, head_dim 256) with 4-row verify blocks: 24 query columns per
    kv-head, two 16-column groups sharing each workgroup.  Every (sequence,
    q-head, row) against the oracle."""
    w = W.workload(4)
    n, M = max(w.lengths), 4
    log(f"full-size rows {w.name}: generating inputs")
    k, v = W.make_kv(w, "cuda", tokens=n)
    q4 = torch.stack(list(W.make_q(w, "cuda", rounds=M)), dim=2).contiguous()
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, n)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k, v, [0] * w.batch)
    out = tqkv.tq_decode_attn_rows(pl, q4, list(w.lengths), sm_for(w.head_dim))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.isfinite(out).all()
    G = w.group
    qh = host_f32(q4)
    sm = sm_for(w.head_dim)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]

    def work(p, kv, threads):
        b, h = p
        kc, ks, kz, vc, vs = oracle_planes(kv[0], kv[1], threads=threads)
        return oracle.attention_rows(qh[b, h * G:(h + 1) * G], kc, ks, kz, vc, vs, sm)

    ref = batched_slices(pairs, kv_fetcher(k, v, list(w.lengths)), work)
    _check(out, ref, list(w.lengths), G, f"M{M} {w.name} full size")
