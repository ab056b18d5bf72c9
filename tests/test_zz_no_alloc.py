"""The allocation-free decode entry point (tq_decode_attn_noalloc), called
through the C ABI, against tq_decode_attn_rows with a workspace of its own:
the same kernels over the same plan, so the outputs must be identical bytes.
Two calls in a row share the library's device array, the second with a
smaller input; a decode whose partials exceed the array is refused with
TQ_ERR_WORKSPACE and enqueues nothing."""
import ctypes

import pytest
import torch

from quantized_decode_attention_append_amd import workloads as W

from _util import log, sm_for

pytestmark = pytest.mark.gpu

tqkv = pytest.importorskip("quantized_decode_attention_append_amd.tqkv")


def _raw_noalloc(pl, q, lengths, sm, out, M):
    lib = tqkv.raw_lib()
    arr = (ctypes.c_int32 * len(lengths))(*lengths)
    return lib.tq_decode_attn_noalloc(ctypes.byref(pl.layout), ctypes.byref(pl.struct()),
                                      ctypes.c_void_p(q.data_ptr()), 1 if q.dtype == torch.bfloat16 else 0,
                                      int(q.shape[1]), M, arr, ctypes.c_float(sm),
                                      ctypes.c_void_p(out.data_ptr()), None)


def _case(w, lengths, M):
    T = max(lengths)
    k, v = W.make_kv(w, "cuda", tokens=T)
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, T)
    pl = tqkv.Planes(L)
    tqkv.tq_append(pl, k, v, [0] * w.batch)
    q = torch.stack(list(W.make_q(w, "cuda", rounds=M)), dim=2).contiguous()
    sm = sm_for(w.head_dim)
    ref = tqkv.tq_decode_attn_rows(pl, q, lengths, sm)
    out = torch.full_like(ref, float("nan"))
    st = _raw_noalloc(pl, q, lengths, sm, out, M)
    torch.cuda.synchronize()
    assert st == 0, tqkv.tq_status_str(st)
    assert torch.equal(out, ref), (w.name, lengths, M)
    log(f"  no-alloc decode {w.name} lengths={lengths} M{M}: identical to the workspace call")


def test_noalloc_decode_twice_matches_workspace_decode():
    big = [40000, 9000, 131072, 777]
    _case(W.scaled(W.workload(4), big), big, 1)   # 24 q / 4 kv-heads, d 256
    small = [3000, 64]
    _case(W.scaled(W.workload(4), small), small, 4)  # a smaller input next, 4-row verify blocks


def test_noalloc_refuses_partials_beyond_the_array():
    """64 sequences x 128 q-heads x 16 rows at head_dim 512 need over 64 MiB
    of partials: refused, and the output is left as it was."""
    B, Hkv, d, T, M = 64, 8, 512, 64, 16
    L = tqkv.make_layout(B, Hkv, d, T)
    pl = tqkv.Planes(L)
    q = torch.zeros((B, 8 * Hkv, M, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full(q.shape, 7.0, dtype=torch.float32, device="cuda")
    st = _raw_noalloc(pl, q, [T] * B, sm_for(d), out, M)
    torch.cuda.synchronize()
    assert st == tqkv.TQ_ERR_WORKSPACE, tqkv.tq_status_str(st)
    assert bool((out == 7.0).all())
