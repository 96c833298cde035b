"""Non-head-aware variant (one index set shared by all heads) against the fp64
oracle through the C ABI: decode and causal prefill anchors, reuse over the
oracle's shared sets, GPU anchor sets feeding GPU reuse, and the reduction to
head-aware selection at one KV head (bit-identical there)."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import check_close, check_index_band, host64, log  # noqa: E402

from long_context_amd import kascade as K  # noqa: E402
from long_context_amd import synth  # noqa: E402
from long_context_amd.synth import to_oracle  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _decode(name, **kw):
    base = dict(name=name, wid=990, phase="decode", batch=2, hq=8, hkv=2, d=128, n=4133, k=256,
                tile=1, dtype="bf16", layers=2, planted=16, share=0.7)
    base.update(kw)
    return synth.Workload(**base)


def _prefill(name, **kw):
    base = dict(name=name, wid=995, phase="prefill", batch=1, hq=8, hkv=2, d=128, n=1088, k=256,
                tile=128, dtype="bf16", layers=2, planted=8, share=0.7, sinks=4)
    base.update(kw)
    return synth.Workload(**base)


DECODE = {
    "bf16_d128_ragged": _decode("bf16_d128_ragged"),
    "f32_d64_hkv4": _decode("f32_d64_hkv4", wid=991, hkv=4, d=64, n=777, k=65, dtype="f32"),
    "bf16_hq32_hkv8": _decode("bf16_hq32_hkv8", wid=992, hq=32, hkv=8, n=2000, k=128),
    "bf16_40k_spill": _decode("bf16_40k_spill", wid=993, batch=1, n=40000, k=512),
    "bf16_k_eq_n": _decode("bf16_k_eq_n", wid=994, n=300, k=300),
}
PREFILL = {
    "d128_ragged": _prefill("d128_ragged"),
    "d64_batch2_hkv4": _prefill("d64_batch2_hkv4", wid=996, batch=2, hkv=4, d=64, n=700, k=100),
    "k_below_tile": _prefill("k_below_tile", wid=997, n=450, k=40),
    "t64_ragged": _prefill("t64_ragged", wid=989, n=700, k=100, tile=64),
}


@pytest.mark.parametrize("case", sorted(DECODE))
def test_shared_decode(lib, orc, case):
    w = DECODE[case]
    log(f"[shared decode] case={case} B={w.batch} Hq={w.hq} Hkv={w.hkv} d={w.d} N={w.n} k={w.k} {w.dtype}")
    (q0, k0, v0), (q1, k1, v1) = synth.make_stack(w, device="cpu")
    dt = w.torch_dtype
    idx = K.anchor_decode(q0.to(DEV), k0.to(DEV), None, w.k, shared=True)
    torch.cuda.synchronize()
    assert tuple(idx.shape) == (w.batch, 1, 1, w.k)
    idx_o, pooled_o = orc.anchor_decode(to_oracle(q0), to_oracle(k0), w.k, shared=True)
    gi = idx.cpu().numpy().reshape(w.batch, w.k)
    same = [check_index_band(gi[b], idx_o[b], pooled_o[b], w.k, w.n, f"{case} b{b}") for b in range(w.batch)]
    # reuse over the oracle's shared sets, every head through its batch row's set
    idx_o4 = idx_o.reshape(w.batch, 1, 1, w.k)
    q1d, k1d, v1d = q1.to(DEV), k1.to(DEV), v1.to(DEV)
    out = K.reuse_decode(q1d, k1d, v1d, torch.from_numpy(idx_o4).to(DEV), shared=True)
    torch.cuda.synchronize()
    ref = orc.reuse_decode(to_oracle(q1), to_oracle(k1), to_oracle(v1), idx_o4, shared=True)
    check_close(host64(out).reshape(-1, w.d), ref, dt, f"{case} reuse")
    # GPU sets feeding GPU reuse, for the batch rows whose sets equal the oracle's
    out_c = K.reuse_decode(q1d, k1d, v1d, idx, shared=True)
    torch.cuda.synchronize()
    for b, s in enumerate(same):
        if s:
            rows = slice(b * w.hq, (b + 1) * w.hq)
            check_close(host64(out_c).reshape(-1, w.d)[rows], ref[rows], dt, f"{case} chain b{b}")
    assert any(same)


@pytest.mark.parametrize("case", sorted(PREFILL))
def test_shared_prefill(lib, orc, case):
    w = PREFILL[case]
    T, tiles = w.tile, -(-w.n // w.tile)
    log(f"[shared prefill] case={case} B={w.batch} Hq={w.hq} Hkv={w.hkv} d={w.d} N={w.n} k={w.k}")
    (q0, k0, v0), (q1, k1, v1) = synth.make_stack(w, device="cpu")
    idx = K.anchor_prefill(q0.to(DEV), k0.to(DEV), None, w.k, T, shared=True)
    torch.cuda.synchronize()
    assert tuple(idx.shape) == (w.batch, 1, tiles, w.k)
    idx_o, pooled_o = orc.anchor_prefill(to_oracle(q0), to_oracle(k0), w.k, T, shared=True)
    gi = idx.cpu().numpy().reshape(-1, w.k)
    same = []
    for u in range(gi.shape[0]):
        t = u % tiles
        prefix = min((t + 1) * T, w.n)
        same.append(check_index_band(gi[u], idx_o[u], pooled_o[u], min(w.k, prefix), prefix, f"{case} unit {u}"))
    idx_o4 = idx_o.reshape(w.batch, 1, tiles, w.k)
    q1d, k1d, v1d = q1.to(DEV), k1.to(DEV), v1.to(DEV)
    out = K.reuse_prefill(q1d, k1d, v1d, torch.from_numpy(idx_o4).to(DEV), T, shared=True)
    torch.cuda.synchronize()
    ref = orc.reuse_prefill(to_oracle(q1), to_oracle(k1), to_oracle(v1), idx_o4, T, shared=True)
    check_close(host64(out).reshape(-1, w.d), ref, torch.bfloat16, f"{case} reuse")
    out_c = host64(K.reuse_prefill(q1d, k1d, v1d, idx, T, shared=True)).reshape(w.batch, w.hq, w.n, w.d)
    torch.cuda.synchronize()
    ref4 = ref.reshape(w.batch, w.hq, w.n, w.d)
    for u, s in enumerate(same):
        if s:
            b, t = u // tiles, u % tiles
            rows = slice(t * T, min((t + 1) * T, w.n))
            check_close(out_c[b, :, rows], ref4[b, :, rows], torch.bfloat16, f"{case} chain unit {u}")
    assert any(same)


def test_shared_equals_head_aware_with_one_kv_head(lib):
    """With one KV head both selections pool the same heads in the same order,
    so index sets and reuse outputs agree bit for bit."""
    log("[shared] one KV head: decode and prefill")
    w = _decode("one_kv", wid=998, hq=8, hkv=1, n=3000, k=200)
    (q0, k0, v0), (q1, k1, v1) = [tuple(t.to(DEV) for t in layer) for layer in synth.make_stack(w, device="cpu")]
    a = K.anchor_decode(q0, k0, None, w.k)
    s = K.anchor_decode(q0, k0, None, w.k, shared=True)
    torch.cuda.synchronize()
    assert torch.equal(a, s)
    assert torch.equal(K.reuse_decode(q1, k1, v1, a), K.reuse_decode(q1, k1, v1, s, shared=True))
    w = _prefill("one_kv_prefill", wid=999, hq=4, hkv=1, n=600, k=128)
    (q0, k0, v0), (q1, k1, v1) = [tuple(t.to(DEV) for t in layer) for layer in synth.make_stack(w, device="cpu")]
    a = K.anchor_prefill(q0, k0, None, w.k, w.tile)
    s = K.anchor_prefill(q0, k0, None, w.k, w.tile, shared=True)
    torch.cuda.synchronize()
    assert torch.equal(a, s)
    assert torch.equal(K.reuse_prefill(q1, k1, v1, a, w.tile), K.reuse_prefill(q1, k1, v1, s, w.tile, shared=True))
