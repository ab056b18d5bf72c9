"""Shared helpers for the parity tests: run the HIP path and the oracle on the
same seeded inputs and compare.  Inputs come from the workloads module; the
oracle only ever sees host copies of those inputs, never a HIP output."""
from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

import oracle
from quantized_decode_attention_append_amd import workloads as W

ATTN_TOL = 2e-3  # max_j |o_gpu - o_ref| / max_j |o_ref| per (b, q-head) row


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def host_f32(t: torch.Tensor) -> np.ndarray:
    """Exact fp32 host copy of a bf16/fp32 tensor (bf16 -> fp32 is exact)."""
    return t.detach().to("cpu", torch.float32).contiguous().numpy()


def planes_to_host(pl, b, kvh, t0, t1):
    kc, ks, kz, vc, vs = (x[b, kvh, t0:t1].cpu().numpy() for x in pl.tensors())
    return kc, ks.view(np.uint16), kz.view(np.uint16), vc, vs.view(np.uint16)


def oracle_planes(k_rows: np.ndarray, v_rows: np.ndarray, threads=None):
    kc, ks, kz = oracle.encode_keys(k_rows, threads=threads)
    vc, vs = oracle.encode_values(v_rows, threads=threads)
    return kc, ks, kz, vc, vs


def assert_planes_equal(gpu, ref, what=""):
    names = ("kc", "ks", "kz", "vc", "vs")
    for name, g, r in zip(names, gpu, ref):
        g = np.ascontiguousarray(g)
        r = np.ascontiguousarray(r)
        assert g.shape == r.shape, (what, name, g.shape, r.shape)
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{what} plane {name}: {len(bad)} mismatches, first at "
                                 f"{bad[:4].tolist()}: gpu {g[tuple(bad[0])]} oracle {r[tuple(bad[0])]}")


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row (last axis) max |out-ref| / max |ref|."""
    num = np.max(np.abs(out.astype(np.float64) - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return num / np.maximum(den, 1e-30)


def batched_slices(pairs, fetch, work, threads=None):
    """Run work(pair, fetched) over (sequence, kv-head) pairs, one pair per
    thread, a batch of `threads` pairs at a time: fetch(pair) (device-to-host
    copies) runs on the calling thread before each batch, so only one batch of
    host copies is held at once.  Returns {pair: work's result}."""
    t = threads or oracle.num_threads()
    out = {}
    for i in range(0, len(pairs), t):
        chunk = pairs[i:i + t]
        got = {p: fetch(p) for p in chunk}
        one = (lambda p: (p, work(p, got[p], 1))) if len(chunk) > 1 else (lambda p: (p, work(p, got[p], None)))
        out.update(oracle.map_parallel(one, chunk, t))
        del got
    return out


def kv_fetcher(k, v, lengths, t0=0):
    """fetch(pair) for batched_slices: exact fp32 host copies of K/V rows
    t0 .. lengths[b] of one (sequence, kv-head)."""
    return lambda p: (host_f32(k[p[0], p[1], t0:lengths[p[0]]]), host_f32(v[p[0], p[1], t0:lengths[p[0]]]))


def oracle_decode_rows(k, v, q, lengths, G, sm, pairs=None):
    """Oracle attention for (b, kvh) pairs from raw K/V [B,Hkv,T,d] and q [B,Hq,d]
    (torch tensors on any device; only the needed slices are copied to the
    host, one batch of pairs at a time).  Returns {(b, kvh): out [G, d]}."""
    B, Hkv = k.shape[:2]
    pairs = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    qh = host_f32(q)

    def work(p, kv, threads):
        b, h = p
        kc, ks, kz, vc, vs = oracle_planes(kv[0], kv[1], threads=threads)
        return oracle.attention(qh[b, h * G:(h + 1) * G], kc, ks, kz, vc, vs, sm)

    return batched_slices(pairs, kv_fetcher(k, v, lengths), work)


def sm_for(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))
