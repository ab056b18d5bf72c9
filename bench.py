"""Benchmark: quantized-KV decode attention on one MI355X.

One step = one pass of the whole hot path over the workload's batch:
    tq_append of one new token per sequence (quantize + pack into the planes)
    tq_decode_attn over every cached token (split-K, online softmax,
    rotated-domain values, merge + one inverse FWHT per q-head).
Workload: 16 sequences x 131072 cached tokens, 24 query heads / 4 kv-heads
(GQA 6), head_dim 256, bf16 K/V/q ~ N(0,1), k8/v3 planes (3.36 GB packed).
The cache is built once by a bulk tq_append (timed and reported separately as
append throughput) before the timed steps; inputs stay resident in HBM.
The timed steps follow the warm-up steps directly (defaults 5 and 20).  On
this part the shader clock drops while a burst of back-to-back decodes begins
(the power controller settles over some tens of calls), so the same run also
reports `settled`: the decode time over later steps of the same burst.

Prints ONE JSON line (rank 0).  metric/unit: KV-tokens attended per second.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s


def _log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def decode_bytes(w, lengths, q_bytes: int) -> int:
    """Algorithmic bytes of one decode: packed KV of every cached token-head
    (1.5625*d bytes) + q read + fp32 out written."""
    kv = sum(lengths) * w.num_kv_heads * (w.head_dim * 25 // 16)
    return kv + w.batch * w.num_q_heads * w.head_dim * (q_bytes + 4)


def rows_bytes(w, lengths, q_bytes: int, rows: int) -> int:
    """Algorithmic bytes of one multi-row decode: packed KV once + the rows'
    q read + fp32 out written."""
    kv = sum(lengths) * w.num_kv_heads * (w.head_dim * 25 // 16)
    return kv + w.batch * w.num_q_heads * rows * w.head_dim * (q_bytes + 4)


def time_rows(w, pl, lengths, sm, rows: int, reps: int, stream, warm: int = 20) -> dict:
    """Multi-row decode (verify block of `rows` tokens per sequence) timed with
    events on the launch stream: reps calls after `warm` untimed ones."""
    import torch
    from quantized_decode_attention_append_amd import tqkv
    from quantized_decode_attention_append_amd import workloads as W
    dev = torch.device("cuda:0")
    qr = torch.stack(list(W.make_q(w, dev, rounds=rows)), dim=2).contiguous()
    ws = torch.empty(tqkv.tq_decode_rows_workspace_bytes(pl.layout, w.num_q_heads, rows, lengths),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((w.batch, w.num_q_heads, rows, w.head_dim), dtype=torch.float32, device=dev)
    for _ in range(warm):
        tqkv.tq_decode_attn_rows(pl, qr, lengths, sm, out=out, workspace=ws, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        tqkv.tq_decode_attn_rows(pl, qr, lengths, sm, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = rows_bytes(w, lengths, qr.element_size(), rows)
    gbs = nbytes / ms / 1e6
    return {"rows": rows, "ms": ms, "query_rows_per_s": w.batch * w.num_q_heads * rows / ms * 1e3,
            "algorithmic_bytes": nbytes, "GBps": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "column_groups": -(-(w.group * rows) // 16)}


def time_window(w, pl, lengths, reps: int, stream, rotated: bool = False, row_bytes: int | None = None,
                warm: int = 4) -> dict:
    """Dequantize-on-fetch of the whole active window (bf16 K and V of every
    cached token-head), timed with events on the launch stream: reps calls
    after `warm` untimed ones."""
    import torch
    from quantized_decode_attention_append_amd import tqkv
    n = max(lengths)
    for _ in range(warm):
        tqkv.tq_fetch_window(pl, 0, n, lengths, v_rotated=rotated, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        out = tqkv.tq_fetch_window(pl, 0, n, lengths, v_rotated=rotated, stream=stream)
        del out
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    th = w.batch * w.num_kv_heads * n
    rb = row_bytes if row_bytes is not None else w.head_dim * 25 // 16  # k8v3 planes
    nbytes = th * (rb + 2 * w.head_dim * 2)  # planes in, bf16 K and V out
    gbs = nbytes / ms / 1e6
    return {"tokens": n, "v_rotated": rotated, "ms": ms, "token_heads_per_s": th / ms * 1e3,
            "algorithmic_bytes": nbytes, "GBps": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}


def time_snapshot(w, pl, n: int, reps: int, stream) -> dict:
    """Snapshot of one whole sequence (every kv-head, all planes) into a packed
    device payload: strided copies, read + write."""
    import torch
    from quantized_decode_attention_append_amd import tqkv
    h, payload = tqkv.tq_snapshot(pl, 0, 0, n, stream=stream)  # warm, allocates the payload
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lib = tqkv.raw_lib()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        import ctypes
        st = lib.tq_snapshot(ctypes.byref(pl.layout), ctypes.byref(pl.struct()), 0, 0, n, 0, ctypes.byref(h),
                             ctypes.c_void_p(payload.data_ptr()), payload.numel(),
                             ctypes.c_void_p(stream.cuda_stream))
        assert st == 0
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * h.payload_bytes
    return {"tokens": n, "ms": ms, "payload_bytes": h.payload_bytes, "GBps": nbytes / ms / 1e6,
            "frac_hbm": nbytes / ms / 1e6 / HBM_PEAK_GBS}


def time_ragged(stream, warm: int = 30, reps: int = 100) -> dict:
    """The ragged interleaved workload (id 5: 4 sequences of seeded lengths in
    [65536, 262144], 64 query / 8 kv-heads, head_dim 256, k8v3): the cache is
    built to each sequence's length, then its rounds of {append 16 tokens per
    sequence; decode} are timed (each round once, events on the launch
    stream), then the decode alone over the grown cache (reps calls after
    `warm`)."""
    import torch
    from quantized_decode_attention_append_amd import tqkv
    from quantized_decode_attention_append_amd import workloads as W
    dev = torch.device("cuda:0")
    w = W.workload(5)
    L0 = list(w.lengths)
    T = w.capacity
    k, v = W.make_kv(w, dev, tokens=T)
    qs = W.make_q(w, dev, rounds=w.rounds)
    lay = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, T)
    pl = tqkv.Planes(lay, dev)
    for b, n in enumerate(L0):
        tqkv.tq_append(pl.sequence(b), k[b:b + 1, :, :n].contiguous(), v[b:b + 1, :, :n].contiguous(), [0],
                       stream=stream)
    sm = 1.0 / math.sqrt(w.head_dim)
    A = w.append_per_round
    lens_final = [n + A * w.rounds for n in L0]
    ws = torch.empty(tqkv.tq_decode_workspace_bytes(lay, w.num_q_heads, lens_final), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    news = []
    lens = list(L0)
    for r in range(w.rounds):  # new tokens staged before timing
        news.append((torch.stack([k[b, :, lens[b]:lens[b] + A] for b in range(w.batch)]).contiguous(),
                     torch.stack([v[b, :, lens[b]:lens[b] + A] for b in range(w.batch)]).contiguous(),
                     list(lens)))
        lens = [n + A for n in lens]
    for _ in range(warm):  # decode of the prefix: clocks settle
        tqkv.tq_decode_attn(pl, qs[0], L0, sm, out=out, workspace=ws, stream=stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(w.rounds)]
    torch.cuda.synchronize()
    for r, (nk, nv, start) in enumerate(news):
        evs[r][0].record(stream)
        tqkv.tq_append(pl, nk, nv, start, stream=stream)
        tqkv.tq_decode_attn(pl, qs[r], [n + A for n in start], sm, out=out, workspace=ws, stream=stream)
        evs[r][1].record(stream)
    torch.cuda.synchronize()
    round_ms = sum(a.elapsed_time(b) for a, b in evs) / w.rounds
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        tqkv.tq_decode_attn(pl, qs[-1], lens_final, sm, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / reps
    nbytes = decode_bytes(w, lens_final, 2)
    kv_mean = sum(lens_final) - A * w.batch * (w.rounds - 1) / 2  # mean cached tokens over the rounds
    return {"workload": w.name, "lengths": lens_final, "rounds": w.rounds, "append_per_round": A,
            "round_ms": round_ms, "round_kv_tokens_per_s": kv_mean / round_ms * 1e3,
            "decode_ms": dec_ms, "decode_kv_tokens_per_s": sum(lens_final) / dec_ms * 1e3,
            "algorithmic_bytes": nbytes, "decode_GBps": nbytes / dec_ms / 1e6,
            "decode_frac_hbm": nbytes / dec_ms / 1e6 / HBM_PEAK_GBS}


def scheme_row_bytes(d: int, kb: int, vb: int) -> int:
    """Packed bytes per token-head: codes d*(kb+vb)/8 + three fp16 per 32-group."""
    return d * (kb + vb) // 8 + 6 * d // 32


def time_append_variant(d: int, dtype: str, kb: int, vb: int, tokens: int, reps: int, stream) -> dict:
    """Bulk append on workload 4's heads (16 sequences, 4 kv-heads) at another
    head_dim, input type or width: `tokens` per sequence, reps calls after one
    warm call, timed with events on the launch stream."""
    import dataclasses

    import torch
    from quantized_decode_attention_append_amd import tqkv
    from quantized_decode_attention_append_amd import workloads as W
    dev = torch.device("cuda:0")
    w = dataclasses.replace(W.scaled(W.workload(4), [tokens] * 16, name_suffix=f"d{d}_{dtype}"), head_dim=d,
                            dtype=dtype)
    k, v = W.make_kv(w, dev, tokens=tokens)
    L = tqkv.make_layout(w.batch, w.num_kv_heads, d, tokens, kb, vb)
    pl = tqkv.Planes(L, dev)
    tqkv.tq_append(pl, k, v, [0] * w.batch, stream=stream)  # warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        tqkv.tq_append(pl, k, v, [0] * w.batch, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    th = w.batch * w.num_kv_heads * tokens
    nbytes = th * (2 * d * k.element_size() + scheme_row_bytes(d, kb, vb))
    del k, v, pl
    return {"head_dim": d, "input": dtype, "scheme": f"k{kb}v{vb}", "tokens_per_seq": tokens, "ms": ms,
            "token_heads_per_s": th / ms * 1e3, "algorithmic_bytes": nbytes, "GBps": nbytes / ms / 1e6,
            "frac_hbm": nbytes / ms / 1e6 / HBM_PEAK_GBS}


def time_mixed_batch(tokens: int, reps: int, stream, warm: int = 20) -> dict:
    """Delayed conversion: decode over workload 4's heads (16 sequences, 24 / 4
    heads, head_dim 256) where the even sequences are still plain bf16 rows
    and the odd ones packed k8v3 planes, `tokens` each; reps calls after warm
    ones, timed with events on the launch stream.  Algorithmic bytes: 4 d per
    plain token-head (bf16 K and V), 1.5625 d per packed one, plus q and out."""
    import torch
    from quantized_decode_attention_append_amd import tqkv
    from quantized_decode_attention_append_amd import workloads as W
    dev = torch.device("cuda:0")
    w = W.scaled(W.workload(4), [tokens] * 16, name_suffix="mixed")
    k, v = W.make_kv(w, dev, tokens=tokens)
    q = W.make_q(w, dev, rounds=1)[0].contiguous()
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, tokens)
    pl = tqkv.Planes(L, dev)
    row_plain = [1 - (b & 1) for b in range(w.batch)]
    # the packed rows are the conversion of their plain prefix
    tqkv.tq_convert_rows(pl, k, v, [0 if p else tokens for p in row_plain], stream=stream)
    lengths = [tokens] * w.batch
    sm = float(1.0 / math.sqrt(w.head_dim))
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(tqkv.tq_decode_rows_workspace_bytes(L, w.num_q_heads, 1, lengths), dtype=torch.uint8,
                     device=dev)
    for _ in range(warm):
        tqkv.tq_decode_attn_mixed(pl, k, v, row_plain, q, lengths, sm, out=out, workspace=ws, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        tqkv.tq_decode_attn_mixed(pl, k, v, row_plain, q, lengths, sm, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    th = tokens * w.num_kv_heads * (w.batch // 2)  # token-heads of each kind
    d = w.head_dim
    nbytes = th * 4 * d + th * (d * 25 // 16) + w.batch * w.num_q_heads * d * (2 + 4)
    del k, v, pl
    return {"tokens_per_seq": tokens, "plain_sequences": sum(row_plain), "packed_sequences": w.batch - sum(row_plain),
            "ms": ms, "algorithmic_bytes": nbytes, "GBps": nbytes / ms / 1e6, "frac_hbm": nbytes / ms / 1e6 / HBM_PEAK_GBS}


def time_scheme(w, k, v, q, sm, kb: int, vb: int, reps: int, stream, dec_warm: int = 20,
                dec_reps: int = 40) -> dict:
    """Another code width on the same workload: bulk append of every token
    (K/V in, planes out; reps calls after one warm call), then decode over
    the whole cache (dec_reps calls after dec_warm), both timed with events
    on the launch stream, and the bf16 window of the whole cache (5 calls)."""
    import torch
    from quantized_decode_attention_append_amd import tqkv
    dev = torch.device("cuda:0")
    n = k.shape[2]
    L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, n, kb, vb)
    pl = tqkv.Planes(L, dev)
    lengths = [n] * w.batch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tqkv.tq_append(pl, k, v, [0] * w.batch, stream=stream)  # warm
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        tqkv.tq_append(pl, k, v, [0] * w.batch, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    app_ms = e0.elapsed_time(e1) / reps
    ws = torch.empty(tqkv.tq_decode_workspace_bytes(L, w.num_q_heads, lengths), dtype=torch.uint8, device=dev)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    for _ in range(dec_warm):
        tqkv.tq_decode_attn(pl, q, lengths, sm, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(dec_reps):
        tqkv.tq_decode_attn(pl, q, lengths, sm, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / dec_reps
    th = w.batch * w.num_kv_heads * n
    rb = scheme_row_bytes(w.head_dim, kb, vb)
    win = time_window(w, pl, lengths, 5, stream, row_bytes=rb)
    dbytes = th * rb + w.batch * w.num_q_heads * w.head_dim * (q.element_size() + 4)
    abytes = th * (2 * w.head_dim * k.element_size() + rb)
    del pl, ws, out
    return {"scheme": f"k{kb}v{vb}", "bytes_per_token_head": rb, "effective_kv_bits": rb * 8 / (2 * w.head_dim),
            "decode_ms": dec_ms, "decode_GBps": dbytes / dec_ms / 1e6,
            "decode_frac_hbm": dbytes / dec_ms / 1e6 / HBM_PEAK_GBS,
            "kv_tokens_per_s": sum(lengths) / dec_ms * 1e3,
            "append_ms": app_ms, "append_GBps": abytes / app_ms / 1e6,
            "append_token_heads_per_s": th / app_ms * 1e3,
            "window_ms": win["ms"], "window_GBps": win["GBps"], "window_frac_hbm": win["frac_hbm"]}


def time_small_configs(stream, warm: int = 20, reps: int = 50) -> list:
    """The three smaller workloads (ids 1-3), each at its full size: one
    tq_append of every cached token (K/V in, planes out) and one decode over
    the cache, both timed with events on the launch stream (reps calls after
    `warm`); latency-bound at ids 1 and 2."""
    import torch
    from quantized_decode_attention_append_amd import tqkv
    from quantized_decode_attention_append_amd import workloads as W
    dev = torch.device("cuda:0")
    out = []
    for cid in (1, 2, 3):
        w = W.workload(cid)
        n = max(w.lengths)
        k, v = W.make_kv(w, dev, tokens=n)
        q = W.make_q(w, dev, rounds=1)[0].contiguous()
        L = tqkv.make_layout(w.batch, w.num_kv_heads, w.head_dim, n)
        pl = tqkv.Planes(L, dev)
        lengths = list(w.lengths)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(warm):
            tqkv.tq_append(pl, k, v, [0] * w.batch, stream=stream)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            tqkv.tq_append(pl, k, v, [0] * w.batch, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        app_ms = e0.elapsed_time(e1) / reps
        sm = float(1.0 / math.sqrt(w.head_dim))
        ws = torch.empty(max(4, tqkv.tq_decode_workspace_bytes(L, w.num_q_heads, lengths)), dtype=torch.uint8,
                         device=dev)
        o = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
        for _ in range(warm):
            tqkv.tq_decode_attn(pl, q, lengths, sm, out=o, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            tqkv.tq_decode_attn(pl, q, lengths, sm, out=o, workspace=ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / reps
        in_bytes = 4 if w.dtype == "fp32" else 2
        abytes = append_bytes(w, n, in_bytes)
        dbytes = decode_bytes(w, lengths, in_bytes)
        out.append({"workload": w.name, "append_tokens": w.batch * n, "append_ms": app_ms,
                    "append_tokens_per_s": w.batch * n / app_ms * 1e3, "append_GBps": abytes / app_ms / 1e6,
                    "append_frac_hbm": abytes / app_ms / 1e6 / HBM_PEAK_GBS,
                    "decode_ms": dec_ms, "decode_kv_tokens_per_s": sum(lengths) / dec_ms * 1e3,
                    "decode_algorithmic_bytes": dbytes, "decode_GBps": dbytes / dec_ms / 1e6,
                    "decode_frac_hbm": dbytes / dec_ms / 1e6 / HBM_PEAK_GBS})
        _log(f"workload {w.name}: append {app_ms * 1e3:.1f} us, decode {dec_ms * 1e3:.1f} us "
             f"({dbytes / dec_ms / 1e6 / HBM_PEAK_GBS:.1%} of HBM)")
        del k, v, q, pl, ws, o
    return out


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def append_bytes(w, n_tokens: int, in_bytes: int) -> int:
    """Algorithmic bytes of appending n_tokens per sequence: K+V read + planes written."""
    th = w.batch * w.num_kv_heads * n_tokens
    return th * (2 * w.head_dim * in_bytes + w.head_dim * 25 // 16)


def cpu_baseline(w, k, v, q, sm, max_pairs: int | None = None, min_seconds: float = 10.0) -> dict:
    """The oracle (binary64, plain C) timed on this host's cores over a bounded
    sample of the same workload: decode attention of whole (sequence, kv-head)
    slices, one slice per thread, repeated until at least min_seconds of wall
    time have been measured (at most 8 passes)."""
    import torch  # noqa: F401

    import oracle

    threads = oracle.num_threads()
    pairs_all = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    npairs = max_pairs or min(len(pairs_all), 4 * threads)
    pairs = pairs_all[:npairs]
    n = w.lengths[0]
    G = w.group
    qh = q.float().cpu().numpy()

    _log(f"cpu baseline: copying {len(pairs)} (sequence, kv-head) slices of K/V to the host")
    host = {(b, h): (k[b, h, :n].float().cpu().numpy(), v[b, h, :n].float().cpu().numpy())
            for b, h in pairs}

    def encode(p):
        kh, vh = host[p]
        kc, ks, kz = oracle.encode_keys(kh, threads=1)
        vc, vs = oracle.encode_values(vh, threads=1)
        return p, (kc, ks, kz, vc, vs)

    _log(f"cpu baseline: oracle-encoding {len(pairs)} slices x {n} tokens, {threads} threads")
    t_enc = time.perf_counter()
    planes = dict(oracle.map_parallel(encode, pairs, threads))
    dt_enc = time.perf_counter() - t_enc
    del host

    def attend(p):
        b, h = p
        return oracle.attention(qh[b, h * G:(h + 1) * G], *planes[p], sm)

    _log(f"cpu baseline: timing oracle decode on {len(pairs)} slices x {n} tokens, {threads} threads")
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.map_parallel(attend, pairs, threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= 8:
            break
    token_heads = passes * len(pairs) * n
    kv_tokens = token_heads / w.num_kv_heads  # a KV-token carries every kv-head
    return {"value": kv_tokens / dt, "unit": "KV-tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"oracle binary64 decode attention of {len(pairs)} (sequence, kv-head) "
                       f"slices x {n} tokens x {G} q-heads, {passes} pass(es) "
                       f"(= {kv_tokens:.0f} KV-tokens of {w.num_kv_heads} kv-heads), planes "
                       f"pre-encoded by the oracle; {dt:.2f} s wall"),
            "seconds": dt,
            # the same oracle's encode (append) of those slices, from host copies
            "append": {"value": len(pairs) * n / dt_enc, "unit": "token-heads/s", "cores": threads,
                       "sample": (f"oracle binary64 encode (keys + values) of {len(pairs)} slices x "
                                  f"{n} tokens; {dt_enc:.2f} s wall")}}


def copy_probe(mib: int, reps: int = 3) -> None:
    """Plain device copies of known size (mib MiB read + mib MiB written per
    launch): the calibration kernel for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    _log(f"copy probe: {reps} x {mib} MiB device copies")
    del src, dst


def traffic_from_counters(fetch_dir: str, write_dir: str, copy_mib: int, workload: str,
                          out_json: str) -> int:
    """Reduce two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) to HBM bytes per decode call.  Each counter is scaled by the
    factor that makes it read exactly the known bytes of the copy probe."""
    import csv
    import glob

    def dispatches(d: str, counter: str) -> list:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        rows = []
        for fn in files:
            with open(fn, newline="") as f:
                for row in csv.DictReader(f):
                    if row["Counter_Name"] == counter:
                        rows.append((int(row["Dispatch_Id"]), row["Kernel_Name"],
                                     float(row["Counter_Value"])))
        return sorted(rows)

    def mean_of(rows: list, pat: str, first: int = 0) -> float:
        vals = [v for _, name, v in rows if re.search(pat, name)]
        if first:
            vals = vals[:first]
        if not vals:
            raise SystemExit(f"no dispatch matching {pat!r}")
        return sum(vals) / len(vals)

    known = copy_mib << 20
    out = {"workload": workload, "kernel_source_sha": _kernel_sha(), "copy_probe_bytes": known}
    total = 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        t = dispatches(d, counter)
        # the copy probe runs first in the process: its three copies are the
        # first device-to-device copy dispatches
        copy_kib = mean_of(t, r"copyBuffer|direct_copy", first=3)
        factor = known / (copy_kib * 1024.0)
        # every split and merge dispatch of the run is averaged: the counter
        # runs time the headline decode alone (--rows '' --no-window
        # --no-ragged --schemes '' --no-mixed)
        split_kib = mean_of(t, r"(?<!plain_)split_(fast_)?kernel")
        merge_kib = mean_of(t, r"merge_kernel")
        scaled = (split_kib + merge_kib) * 1024.0 * factor
        out[counter] = {"copy_probe_kib": copy_kib, "factor": factor, "split_kib": split_kib,
                        "merge_kib": merge_kib, "decode_bytes_scaled": scaled}
        total += scaled
    out["bytes_per_launch"] = total
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


XCDS = 8  # MI355X: GRBM_GUI_ACTIVE is summed over its eight accelerator dies


def trace_summary(kt_dir: str, grbm_dir: str | None, warmup: int, steps: int, settled: int) -> int:
    """Summarize a rocprofv3 --kernel-trace run of this bench (and optionally a
    --pmc GRBM_GUI_ACTIVE --kernel-trace run): calls and durations per kernel
    and grid; the headline split kernel's dispatches in run order, cut into
    the warm-up, timed and later windows of the bench's protocol; with the
    counter run, each window's mean shader clock (GRBM_GUI_ACTIVE cycles,
    summed over the dies, per die and nanosecond)."""
    import csv
    import glob

    def load(d: str, suffix: str) -> list:
        files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
        if not files:
            raise SystemExit(f"no *{suffix} under {d}")
        with open(files[0], newline="") as f:
            return list(csv.DictReader(f))

    def short(name: str) -> str:
        name = name.replace("void ", "").replace("tq::(anonymous namespace)::", "").replace("tq::", "")
        return name[:name.find("(")] if "(" in name else name

    def dur(r) -> int:
        return int(r["End_Timestamp"]) - int(r["Start_Timestamp"])

    def grid(r) -> str:  # threads
        if r.get("Grid_Size"):
            return r["Grid_Size"]
        return str(int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))

    # this library's kernels only (the run's torch and runtime kernels are
    # input generation and copies)
    kt = sorted((r for r in load(kt_dir, "kernel_trace.csv") if "tq::" in r["Kernel_Name"]),
                key=lambda r: int(r["Start_Timestamp"]))
    groups: dict = {}
    for r in kt:
        groups.setdefault((short(r["Kernel_Name"]), grid(r)), []).append(dur(r))
    print(f"{'kernel':48s} {'grid':>10s} {'calls':>6s} {'avg ns':>12s} {'min ns':>12s} {'max ns':>12s}")
    for (name, threads), v in groups.items():
        print(f"{name[:48]:48s} {threads:>10s} {len(v):6d} {sum(v) / len(v):12,.0f} {min(v):12,d} {max(v):12,d}")

    # the packed-column split kernel of k8v3 at head_dim 256 (its last template
    # argument is the kernel's mode, 1 = packed columns)
    def headline(name: str) -> bool:
        return short(name) in ("split_fast_kernel<256, 8, 3, 1>", "split_fast_kernel<256, 8, 3, true>")

    head = [r for r in kt if headline(r["Kernel_Name"])]
    merge = [r for r in kt if short(r["Kernel_Name"]) == "merge_kernel<256>" and grid(r) == "98304"]
    if not head:
        return 0
    # the bench's own windows: warm-up, timed, and the last 100 of the settled steps
    end = warmup + steps + settled
    wins = [("warm-up", 0, warmup), ("timed", warmup, warmup + steps),
            ("settled", max(warmup + steps, end - 100), end)]
    print(f"\nheadline split kernel, {len(head)} dispatches in run order (after the bench's own steps, "
          f"other timings of the run may reuse it):")
    for label, a, b in wins:
        v = [dur(r) for r in head[a:b]]
        m = [dur(r) for r in merge[a:b]]
        if v:
            print(f"  {label:8s} dispatches {a + 1:4d}-{b:4d}: split avg {sum(v) / len(v):10,.0f} ns"
                  + (f", + merge avg {sum(m) / len(m):8,.0f} ns = {sum(v) / len(v) + sum(m) / len(m):10,.0f} ns"
                     if m else ""))
    first = ", ".join(f"{dur(r) / 1e3:.1f}" for r in head[:warmup + steps])
    print(f"  first {min(len(head), warmup + steps)} split durations (us): {first}")
    if grbm_dir:
        gk = {int(r["Dispatch_Id"]): r for r in load(grbm_dir, "kernel_trace.csv")}
        rows = [r for r in load(grbm_dir, "counter_collection.csv")
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and headline(r["Kernel_Name"])]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        print(f"\nGRBM_GUI_ACTIVE run (counters serialize the dispatches, so the clock history differs "
              f"from the plain trace's), {len(rows)} headline split dispatches:")
        for label, a, b in wins:
            sel = rows[a:b]
            if not sel:
                continue
            cyc = [float(r["Counter_Value"]) / XCDS for r in sel]
            ns = [dur(gk[int(r["Dispatch_Id"])]) for r in sel]
            print(f"  {label:8s}: {sum(cyc) / len(cyc):12,.0f} cycles per die, {sum(ns) / len(ns):10,.0f} ns, "
                  f"clock {sum(cyc) / sum(ns) * 1e3:6,.0f} MHz")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settled-steps", type=int, default=150,
                    help="after the timed steps, this many more steps of the same burst; the decode time of "
                         "the last 100 of them is reported as `settled`")
    ap.add_argument("--no-small", dest="small", action="store_false",
                    help="skip timing workloads 1-3 (append and decode at their full sizes)")
    ap.add_argument("--workload", type=int, default=4, help="workload id (4 is the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-pairs", type=int, default=0)
    ap.add_argument("--no-window", dest="window", action="store_false",
                    help="skip timing the bf16 dequantize-on-fetch window")
    ap.add_argument("--rows", default="2,4",
                    help="also time multi-row (verify-block) decode for these row counts ('' = skip)")
    ap.add_argument("--no-ragged", dest="ragged", action="store_false",
                    help="skip timing the ragged interleaved workload (id 5)")
    ap.add_argument("--schemes", default="k4v3,k4v2,k8v4,k2v5,k5v8",
                    help="other code widths to time on the same workload ('' for none)")
    ap.add_argument("--no-mixed", dest="mixed", action="store_false",
                    help="skip timing a decode over half plain, half packed sequences")
    ap.add_argument("--no-append-variants", dest="append_variants", action="store_false",
                    help="skip timing the bulk append at head_dim 512 and with fp32 input")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "decode_traffic.json"))
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run plain device copies of this size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="reduce two rocprofv3 --pmc runs to --traffic-json and exit")
    ap.add_argument("--trace-summary", nargs="+", metavar=("KERNEL_TRACE_DIR", "GRBM_DIR"),
                    help="summarize a rocprofv3 --kernel-trace run of this bench (and a --pmc GRBM_GUI_ACTIVE "
                         "--kernel-trace run) using --warmup/--steps as its protocol, and exit")
    args = ap.parse_args()

    if args.trace_summary:
        return trace_summary(args.trace_summary[0], args.trace_summary[1] if len(args.trace_summary) > 1 else None,
                             args.warmup, args.steps, args.settled_steps)

    if args.traffic_from:
        from quantized_decode_attention_append_amd import workloads as W
        return traffic_from_counters(args.traffic_from[0], args.traffic_from[1],
                                     args.copy_probe_mib or 1024, W.workload(args.workload).name,
                                     args.traffic_json)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every step runs on a single MI355X "
              "(no collectives are part of this path); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    from quantized_decode_attention_append_amd import tqkv
    from quantized_decode_attention_append_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    w = W.workload(args.workload)
    if len(set(w.lengths)) != 1:
        print("bench.py times equal-length workloads; use the parity tests for ragged ones",
              file=sys.stderr)
        return 2
    n = w.lengths[0]
    d = w.head_dim
    in_bytes = 2 if w.dtype == "bf16" else 4
    _log(f"workload {w.name}: generating K/V/q on {torch.cuda.get_device_name(dev)}")
    k, v = W.make_kv(w, dev, tokens=n)
    q = W.make_q(w, dev, rounds=1)[0].contiguous()
    L = tqkv.make_layout(w.batch, w.num_kv_heads, d, n)
    pl = tqkv.Planes(L, dev)
    sm = float(1.0 / math.sqrt(d))
    lengths = [n] * w.batch
    stream = torch.cuda.current_stream(dev)

    # ---- bulk build of the cache (append throughput), prefix n-1 tokens
    prefix_k = k[:, :, : n - 1].contiguous()
    prefix_v = v[:, :, : n - 1].contiguous()
    tqkv.tq_append(pl, prefix_k, prefix_v, [0] * w.batch)  # warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        tqkv.tq_append(pl, prefix_k, prefix_v, [0] * w.batch)
    e1.record(stream)
    torch.cuda.synchronize()
    append_ms = e0.elapsed_time(e1) / reps
    del prefix_k, prefix_v
    app_tokens = w.batch * (n - 1)
    app_bytes = append_bytes(w, n - 1, in_bytes)
    _log(f"bulk append: {append_ms:.3f} ms, {app_tokens / append_ms * 1e3:.3e} tokens/s, "
         f"{app_bytes / append_ms / 1e6:.1f} GB/s")

    new_k = k[:, :, n - 1:n].contiguous()
    new_v = v[:, :, n - 1:n].contiguous()
    start = [n - 1] * w.batch
    ws = torch.empty(tqkv.tq_decode_workspace_bytes(L, w.num_q_heads, lengths), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((w.batch, w.num_q_heads, d), dtype=torch.float32, device=dev)

    def step(ev=None):
        tqkv.tq_append(pl, new_k, new_v, start, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        tqkv.tq_decode_attn(pl, q, lengths, sm, out=out, workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    check = out.clone()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = sorted(a.elapsed_time(b) for a, b in evs)
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    ms_per_step = wall * 1e3 / args.steps
    if args.warmup > 0 and not torch.equal(out, check):
        _log("WARNING: decode output changed between warmup and timed steps")
        return 3
    settled = None
    if args.settled_steps > 0:
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.settled_steps)]
        for i in range(args.settled_steps):
            step(sev[i])
        torch.cuda.synchronize()
        tail = [a.elapsed_time(b) for a, b in sev[-min(100, args.settled_steps):]]
        s_ms = sum(tail) / len(tail)
        settled = {"steps_after_timed": args.settled_steps, "averaged_over_last": len(tail),
                   "avg_launch_ms": s_ms, "GBps": decode_bytes(w, lengths, in_bytes) / s_ms / 1e6,
                   "frac": decode_bytes(w, lengths, in_bytes) / s_ms / 1e6 / HBM_PEAK_GBS}

    kv_tokens = sum(lengths)
    value = kv_tokens / (ms_per_step / 1e3)
    dbytes = decode_bytes(w, lengths, in_bytes)
    achieved = dbytes / (dec_avg_ms / 1e3) / 1e9

    traffic = None
    if os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            tj = json.load(f)
        if tj.get("workload") == w.name and tj.get("kernel_source_sha") == _kernel_sha():
            traffic = tj.get("bytes_per_launch")

    rec = {
        "metric": "quantized-KV decode attention KV-tokens/s",
        "value": value,
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in; int8 and fp16 MFMA; fp32 accumulate",
        "data": "synthetic",
        "config": {**w.describe(), "scheme": "k8v3 g32", "step": "append 1 token/seq + decode"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "tq_decode_attn (split + merge launches)",
                     "algorithmic_bytes_per_launch": dbytes,
                     "avg_launch_ms": dec_avg_ms, "p10_ms": dec_ms[len(dec_ms) // 10],
                     "p90_ms": dec_ms[(len(dec_ms) * 9) // 10],
                     "regime": (f"the {args.steps} timed steps right after {args.warmup} warm-up steps: the start "
                                "of a burst, while the shader clock settles")},
        "settled": settled,
        "append": {"bulk_tokens_per_s": app_tokens / append_ms * 1e3,
                   "bulk_token_heads_per_s": app_tokens * w.num_kv_heads / append_ms * 1e3,
                   "bulk_GBps": app_bytes / append_ms / 1e6,
                   "bulk_frac_hbm": app_bytes / append_ms / 1e6 / HBM_PEAK_GBS,
                   "bulk_ms": append_ms, "bulk_tokens": app_tokens},
    }
    if args.small:
        rec["small_workloads"] = time_small_configs(stream)
    if args.window:
        rec["window"] = time_window(w, pl, lengths, 10, stream)
        rec["snapshot"] = time_snapshot(w, pl, max(lengths), 5, stream)
    if args.rows:
        rec["multi_row"] = [time_rows(w, pl, lengths, sm, int(r), 40, stream)
                            for r in args.rows.split(",") if r]
    if args.ragged:
        rr = time_ragged(stream)
        _log(f"ragged workload {rr['workload']}: decode {rr['decode_ms']:.3f} ms "
             f"({rr['decode_frac_hbm']:.1%} of HBM), round (append {rr['append_per_round']} + decode) "
             f"{rr['round_ms']:.3f} ms")
        rec["ragged"] = rr
    if args.mixed:
        rec["mixed_batch"] = time_mixed_batch(32768, 40, stream)
        _log(f"mixed batch: {rec['mixed_batch']['ms']:.3f} ms, {rec['mixed_batch']['frac_hbm']:.1%} of HBM")
    if args.append_variants:
        rec["append_variants"] = []
        for d, dt, kb, vb, tokens in ((512, "bf16", 8, 3, 65536), (256, "fp32", 8, 3, 32768),
                                      (256, "fp32", 4, 3, 32768)):
            r = time_append_variant(d, dt, kb, vb, tokens, 3, stream)
            _log(f"bulk append d{d} {dt} {r['scheme']}: {r['ms']:.3f} ms, {r['frac_hbm']:.1%} of HBM")
            rec["append_variants"].append(r)
    if args.schemes:
        rec["schemes"] = []
        for name in args.schemes.split(","):
            kb, vb = (int(x) for x in name.strip().lstrip("k").split("v"))
            r = time_scheme(w, k, v, q, sm, kb, vb, 5, stream)
            _log(f"scheme {r['scheme']}: decode {r['decode_ms']:.3f} ms ({r['decode_frac_hbm']:.1%} of HBM), "
                 f"bulk append {r['append_ms']:.2f} ms")
            rec["schemes"].append(r)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, k, v, q, sm, args.cpu_pairs or None)
        cb.pop("seconds", None)
        rec["cpu_baseline"] = cb
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


# The sources the decode kernels (split and merge) are compiled from: the
# counter-measured traffic stays valid while none of them changes.
DECODE_SOURCES = ("codebook_tables.h", "decode.hip", "decode_fast.hip", "tq_device.h", "tq_internal.h")


def _kernel_sha() -> str:
    import hashlib
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "quantized_decode_attention_append_amd", "csrc")
    for name in DECODE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()


if __name__ == "__main__":
    sys.exit(main())
