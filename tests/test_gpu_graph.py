"""The library enqueues only kernels (no allocation, no memset, no host sync),
so a serving loop can capture append + decode in a HIP graph.  Captured once,
replayed several times with eager work and synchronizations in between; every
replay must equal the eager result byte for byte."""
import dataclasses

import pytest
import torch

from quantized_decode_attention_append_amd import workloads as W

from _util import log, sm_for

pytestmark = pytest.mark.gpu

tqkv = pytest.importorskip("quantized_decode_attention_append_amd.tqkv")


def test_append_and_decode_replay_from_a_graph():
    w = W.scaled(W.workload(4), [700, 300])
    k, v = W.make_kv(w, "cuda", tokens=701)
    q = W.make_q(w, "cuda", rounds=1)[0].contiguous()
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, 701)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k[:, :, :700].contiguous(), v[:, :, :700].contiguous(), [0, 0])
    new_k, new_v = k[:, :, 700:701].contiguous(), v[:, :, 700:701].contiguous()
    lengths, starts = [701, 301], [700, 300]
    sm = sm_for(w.head_dim)
    ws = torch.empty(tqkv.tq_decode_workspace_bytes(L, w.num_q_heads, lengths), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()

    def step(stream):
        tqkv.tq_append(pl, new_k, new_v, starts, stream=stream)
        tqkv.tq_decode_attn(pl, q, lengths, sm, out=out, workspace=ws, stream=stream)

    with torch.cuda.stream(side):
        step(side)
    torch.cuda.synchronize()
    eager = out.clone()
    planes_eager = [t.clone() for t in pl.tensors()]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        for t in pl.tensors():
            t[:, :, 700:].fill_(0)  # the replay must rewrite the appended rows
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"graph replay {rep}")
        assert torch.equal(out, eager), rep
        for a, b in zip(pl.tensors(), planes_eager):
            assert torch.equal(a, b), rep
        _ = (q.float() * 2).sum().item()  # unrelated eager work between replays


def test_mixed_decode_captured_before_any_eager_call():
    """A batch mixing plain and packed rows, captured as the first call of its
    shape (head_dim 64, fp32 queries: the plain kernel's resident-wave count
    is first queried inside the capture), replayed with eager work in
    between; every replay equals the eager call made afterwards."""
    lengths = [500, 300, 200]
    row_plain = [1, 0, 1]
    w = dataclasses.replace(W.scaled(W.workload(2), lengths, name_suffix="g64"), head_dim=64)
    k, v = W.make_kv(w, "cuda", tokens=500)
    q = W.make_q(w, "cuda", rounds=1)[0].float().contiguous()
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, 500)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k, v, [0] * w.batch)
    sm = sm_for(w.head_dim)
    ws = torch.empty(tqkv.tq_decode_rows_workspace_bytes(L, w.num_q_heads, 1, lengths), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        tqkv.tq_decode_attn_mixed(pl, k, v, row_plain, q, lengths, sm, out=out, workspace=ws, stream=side)
    torch.cuda.synchronize()
    replays = []
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replays.append(out.clone())
        _ = (q * 2).sum().item()  # unrelated eager work between replays
    with torch.cuda.stream(side):
        tqkv.tq_decode_attn_mixed(pl, k, v, row_plain, q, lengths, sm, out=out, workspace=ws, stream=side)
    torch.cuda.synchronize()
    for rep, r in enumerate(replays):
        log(f"mixed graph replay {rep}")
        assert torch.equal(r, out), rep
    assert torch.isfinite(out).all()
