"""CPU checks of the accuracy-sweep measures in bench.py: pooled attention
against a direct per-row computation, captured mass and planted recall on
hand-built sets."""
import math

import numpy as np
import pytest
import torch

import bench


def _softmax_rows(s):
    e = np.exp(s - s.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


def test_pooled_decode_matches_per_head_loop():
    g = torch.Generator().manual_seed(5)
    B, Hq, Hkv, N, d = 2, 6, 2, 37, 16
    q = torch.randn((B, Hq, 1, d), generator=g)
    k = torch.randn((B, Hkv, N, d), generator=g)
    got = bench.pooled_decode(q, k).numpy()
    G = Hq // Hkv
    for b in range(B):
        for kv in range(Hkv):
            want = np.zeros(N)
            for h in range(kv * G, (kv + 1) * G):
                s = k[b, kv].double().numpy() @ q[b, h, 0].double().numpy() / math.sqrt(d)
                want += _softmax_rows(s) / G
            np.testing.assert_allclose(got[b, kv], want, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("n,tile", [(40, 16), (48, 16), (7, 16)])
def test_pooled_prefill_matches_causal_loop(n, tile):
    g = torch.Generator().manual_seed(n)
    B, Hq, Hkv, d = 1, 4, 2, 8
    q = torch.randn((B, Hq, n, d), generator=g)
    k = torch.randn((B, Hkv, n, d), generator=g)
    got = bench.pooled_prefill(q, k, tile).numpy()
    G = Hq // Hkv
    tiles = -(-n // tile)
    assert got.shape == (B, Hkv, tiles, n)
    for kv in range(Hkv):
        for t in range(tiles):
            rows = range(t * tile, min((t + 1) * tile, n))
            want = np.zeros(n)
            for h in range(kv * G, (kv + 1) * G):
                for i in rows:
                    s = k[0, kv, : i + 1].double().numpy() @ q[0, h, i].double().numpy() / math.sqrt(d)
                    want[: i + 1] += _softmax_rows(s)
            want /= G * len(rows)
            np.testing.assert_allclose(got[0, kv, t], want, rtol=1e-5, atol=1e-7)
            assert abs(got[0, kv, t].sum() - 1.0) < 1e-5
            assert np.all(got[0, kv, t, (t + 1) * tile:] == 0.0)


def test_captured_mass_skips_padding():
    pooled = torch.tensor([[[0.1, 0.2, 0.3, 0.4]], [[0.25, 0.25, 0.25, 0.25]]])
    idx = torch.tensor([[[3, 1]], [[0, -1]]], dtype=torch.int32)
    assert bench.captured_mass(pooled, idx) == pytest.approx((0.6 + 0.25) / 2)


def test_planted_recall_decode_and_causal_tiles():
    pos = [[np.array([1, 5, 9])]]
    idx = np.array([[[[5, 9, 2]]]])
    assert bench.planted_recall(pos, idx, 1, 16) == pytest.approx(2 / 3)
    # prefill, tile 4, n 12: tile 0 sees {1}, tile 1 sees {1, 5}, tile 2 sees {1, 5, 9}
    idx = np.array([[[[1, -1], [1, 2], [5, 9]]]])
    assert bench.planted_recall(pos, idx, 4, 12) == pytest.approx((1 + 0.5 + 2 / 3) / 3)


def test_rel_error():
    a = torch.tensor([3.0, 4.0])
    assert bench.rel_error(a, a) == 0.0
    assert bench.rel_error(torch.tensor([3.0, 5.0]), a) == pytest.approx(0.2)


def test_measures_of_a_shared_set():
    """A set shared by all KV heads is scored against each head's own rows."""
    pooled = torch.tensor([[[[0.5, 0.5, 0.0]], [[0.0, 0.2, 0.8]]]])      # [B=1, Hkv=2, 1, N=3]
    idx = torch.tensor([[[[1, 2]]]], dtype=torch.int32)                  # [1, 1, 1, 2]
    assert bench.captured_mass(pooled, idx) == pytest.approx((0.5 + 1.0) / 2)
    pos = [[np.array([0, 1]), np.array([2])]]
    assert bench.planted_recall(pos, idx.numpy(), 1, 3) == pytest.approx((0.5 + 1.0) / 2)
