"""Non-finite inputs: the calls still return well-formed index sets.

With NaN or infinite keys the scores are undefined, so there is nothing to
compare against the oracle; what must hold is the shape of the result. Each
index set has exactly min(k, candidates) distinct keys, ascending and inside
the candidate range, padded with -1, and the reuse calls run over it. The
selection keys are float bit patterns with the sign cleared, so a NaN of
either sign still leaves exactly k keys selected.
"""
import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import log  # noqa: E402

from long_context_amd import kascade as K  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"

# bf16 bit patterns: -NaN, +NaN, +inf, -inf
_BITS = {"-nan": -64, "+nan": 32704, "+inf": 32640, "-inf": -128}


def _poison(t, rows):
    """Overwrite whole key rows of t [B, H, N, d] (bf16) with non-finite values."""
    bits = t.view(torch.int16)
    for row, kind in rows.items():
        bits[:, :, row, :] = _BITS[kind]
    return t


def _tensors(b, hq, hkv, n, d, q_len, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(b, hq, q_len, d, generator=g).to(torch.bfloat16)
    k = torch.randn(b, hkv, n, d, generator=g).to(torch.bfloat16)
    v = torch.randn(b, hkv, n, d, generator=g).to(torch.bfloat16)
    return q, k, v


def _check_set(row, count, limit, k):
    """row: one index set of length k (host int64)."""
    head, tail = row[:count], row[count:]
    assert torch.all(tail == -1), "slots past the selected count must hold -1"
    assert torch.all((head >= 0) & (head < limit)), "selected keys outside the candidate range"
    assert torch.all(head[1:] > head[:-1]), "selected keys must be distinct and ascending"


DECODE = {
    "n4096_k64": dict(n=4096, k=64, shared=False),
    "n40000_k100_two_subsegments": dict(n=40000, k=100, shared=False),
    "n640_k_eq_n": dict(n=640, k=640, shared=False),
    "n4096_k64_shared": dict(n=4096, k=64, shared=True),
}


@pytest.mark.parametrize("case", sorted(DECODE))
def test_decode_nonfinite_keys(lib, case):
    c = DECODE[case]
    n, k, shared = c["n"], c["k"], c["shared"]
    log(f"[nonfinite decode] case={case} N={n} k={k} shared={shared}")
    q, kk, v = _tensors(2, 8, 2, n, 128, 1, seed=11)
    _poison(kk, {3: "-nan", n // 3: "+nan", n // 2: "+inf", n - 1: "-inf"})
    qd, kd, vd = q.to(DEV), kk.to(DEV), v.to(DEV)
    out = torch.empty_like(qd)
    idx = K.anchor_decode(qd, kd, vd, k, out=out, shared=shared)
    o1 = K.reuse_decode(qd, kd, vd, idx, shared=shared)
    torch.cuda.synchronize()
    assert o1.shape == qd.shape
    h = idx.cpu().long()
    for b in range(h.shape[0]):
        for s in range(h.shape[1]):
            _check_set(h[b, s, 0], k, n, k)


PREFILL = {
    "n600_t128_k64": dict(n=600, tile=128, k=64),
    "n600_t64_k300": dict(n=600, tile=64, k=300),
}


@pytest.mark.parametrize("case", sorted(PREFILL))
def test_prefill_nonfinite_keys(lib, case):
    c = PREFILL[case]
    n, tile, k = c["n"], c["tile"], c["k"]
    log(f"[nonfinite prefill] case={case} N={n} T={tile} k={k}")
    q, kk, v = _tensors(1, 4, 1, n, 128, n, seed=12)
    _poison(kk, {2: "-nan", 130: "+nan", 300: "+inf", 599: "-inf"})
    qd, kd, vd = q.to(DEV), kk.to(DEV), v.to(DEV)
    out = torch.empty_like(qd)
    idx = K.anchor_prefill(qd, kd, vd, k, tile, out=out)
    o1 = K.reuse_prefill(qd, kd, vd, idx, tile)
    torch.cuda.synchronize()
    assert o1.shape == qd.shape
    h = idx.cpu().long()
    tiles = (n + tile - 1) // tile
    assert h.shape == (1, 1, tiles, k)
    for t in range(tiles):
        prefix = min((t + 1) * tile, n)
        _check_set(h[0, 0, t], min(k, prefix), prefix, k)
