"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin takes an `Oracle` instance so that the same checks can also be run
against copies of the oracle with a deliberate mistake planted in them
(tests/test_oracle_mutants.py): every planted mistake must make at least one
pin fail.

What the pins rest on (the pages print no worked example or value table):
  * hand-derived closed forms (tests/golden/*.json),
  * torch.nn.functional.scaled_dot_product_attention in float64 on the CPU, a
    library routine, used (a) as textbook dense attention, (b) with a boolean
    mask as softmax restricted to a key set, (c) with V = identity to expose the
    post-softmax probability matrix that the anchor pools,
  * brute-force enumeration of k-subsets on tiny inputs,
  * invariants: probabilities sum to 1, V = 1 gives O = 1, permutation and
    order invariance, uniform keys, one-hot keys, tile 0 selecting everything.
"""
import itertools
import json
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---- helpers -----------------------------------------------------------------

def _rand(shape, seed, dtype=torch.float32, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g)).to(dtype)


def _host(t):
    """What the oracle reads: float32 array, or bf16 bit patterns."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _sdpa(q, k, v, causal=False, mask=None, scale=None):
    """Library attention in float64; GQA maps query head h to KV head h // G."""
    return F.scaled_dot_product_attention(q.double(), k.double(), v.double(), attn_mask=mask,
                                          is_causal=causal, scale=scale, enable_gqa=True)


def _probabilities(q, k, causal=False):
    """Post-softmax probability matrix [B,Hq,L,N] via attention with V = I."""
    B, Hkv, N, _ = k.shape
    eye = torch.eye(N, dtype=torch.float64).expand(B, Hkv, N, N).contiguous()
    return _sdpa(q, k, eye, causal=causal)


def _close(a, b, atol, rtol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    assert np.all(err <= lim), f"{what}: max err {err.max():.3e} (limit {atol}+{rtol}|b|)"


def _check_topk(idx_row, score, kt, what):
    """idx_row holds the kt largest of score (ties to lower index), ascending, then -1."""
    sel = idx_row[:kt]
    assert np.all(idx_row[kt:] == -1), f"{what}: padding"
    assert np.all(np.diff(sel) > 0), f"{what}: not strictly ascending"
    chosen = set(sel.tolist())
    rest = [j for j in range(len(score)) if j not in chosen]
    for j in sel:
        for r in rest:
            assert score[j] > score[r] or (score[j] == score[r] and j < r), \
                f"{what}: key {j} ({score[j]}) selected over {r} ({score[r]})"


# ---- closed forms ---------------------------------------------------------------

def pin_golden_decode(orc):
    g = json.load(open(os.path.join(GOLDEN, "closed_form_decode.json")))
    a, b = np.array(g["a"], float), np.array(g["b"], float)
    N = len(a)
    q = np.zeros((1, 2, 1, 4), np.float32)
    q[0, 0, 0, 0] = 2.0
    q[0, 1, 0, 1] = 2.0
    k = np.zeros((1, 1, N, 4), np.float32)
    k[0, 0, :, 0] = np.log(a)
    k[0, 0, :, 1] = np.log(b)
    k[0, 0, :, 2:] = np.array(g["k_extra_columns"], np.float32)
    v = np.zeros((1, 1, N, 4), np.float32)
    v[0, 0, :, 0] = np.arange(N)
    v[0, 0, :, 1] = np.arange(N) ** 2
    v[0, 0, :, 2] = 1.0
    idx, pooled = orc.anchor_decode(q, k, g["top_k"])
    assert idx[0].tolist() == g["expected_idx"], idx
    _close(pooled[0], g["expected_pooled"], 1e-6, what="golden decode pooled")
    out = orc.reuse_decode(q, k, v, idx.reshape(1, 1, 1, -1))
    _close(out, g["expected_reuse_out"], 1e-6, what="golden decode reuse")
    dense, lse = orc.dense(q, k, v, causal=False)
    _close(dense, g["expected_dense_out"], 1e-6, what="golden decode dense")
    _close(lse, g["expected_lse"], 1e-6, what="golden decode lse")


def pin_golden_prefill(orc):
    g = json.load(open(os.path.join(GOLDEN, "closed_form_prefill.json")))
    w = np.array(g["w"], float)
    N = len(w)
    q = np.zeros((1, 1, N, 2), np.float32)
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, N, 2), np.float32)
    k[0, 0, :, 0] = np.log(w)
    v = np.array(g["v"], np.float32).reshape(1, 1, N, 2)
    T = g["q_tile"]
    idx, pooled = orc.anchor_prefill(q, k, g["top_k"], T, scale=1.0)
    assert idx.tolist() == g["expected_idx"], idx
    _close(pooled, g["expected_pooled"], 1e-6, what="golden prefill pooled")
    out = orc.reuse_prefill(q, k, v, idx.reshape(1, 1, -1, g["top_k"]), T, scale=1.0)
    _close(out, g["expected_reuse_out"], 1e-6, what="golden prefill reuse")
    dense, lse = orc.dense(q, k, v, causal=True, scale=1.0)
    _close(dense, g["expected_dense_out"], 1e-6, what="golden prefill dense")
    _close(lse, g["expected_lse"], 1e-6, what="golden prefill lse")


def pin_lse_closed_form(orc):
    """Constant logits c over n keys: lse = c + ln n (decode n = N, causal n = i + 1)."""
    d, N, c = 4, 21, 0.75
    q = np.zeros((1, 2, N, d), np.float32)
    q[..., 0] = c * 2.0                 # scale 1/sqrt(4) = 1/2: logit c, all exact in float32
    k = np.zeros((1, 1, N, d), np.float32)
    k[..., 0] = 1.0
    _, lse = orc.dense(q, k, None, causal=True, want_out=False)
    expect = np.tile(c + np.log(np.arange(1, N + 1)), 2)
    _close(lse, expect, 1e-12, what="causal lse")
    _, lse = orc.dense(q[:, :, :1], k, None, causal=False, want_out=False)
    _close(lse, [c + np.log(N)] * 2, 1e-12, what="decode lse")


# ---- library routine: dense attention --------------------------------------------

def pin_dense_vs_sdpa(orc):
    for dtype in (torch.float32, torch.bfloat16):
        q = _rand((2, 4, 1, 32), 1, dtype)
        k = _rand((2, 2, 70, 32), 2, dtype)
        v = _rand((2, 2, 70, 32), 3, dtype)
        out, _ = orc.dense(_host(q), _host(k), _host(v), causal=False)
        _close(out, _sdpa(q, k, v).reshape(-1, 32), 1e-12, what=f"dense decode {dtype}")
        q = _rand((1, 6, 33, 16), 4, dtype)
        k = _rand((1, 3, 33, 16), 5, dtype)
        v = _rand((1, 3, 33, 16), 6, dtype)
        out, _ = orc.dense(_host(q), _host(k), _host(v), causal=True)
        _close(out, _sdpa(q, k, v, causal=True).reshape(-1, 16), 1e-12, what=f"dense causal {dtype}")


# ---- library routine: post-softmax probabilities pooled by the anchor --------------

def pin_decode_pooled_vs_sdpa(orc):
    for dtype in (torch.float32, torch.bfloat16):
        B, Hq, Hkv, d, N = 2, 6, 2, 16, 40
        q = _rand((B, Hq, 1, d), 11, dtype)
        k = _rand((B, Hkv, N, d), 12, dtype)
        P = _probabilities(q, k)                                   # [B,Hq,1,N]
        ref = P.reshape(B, Hkv, Hq // Hkv, N).mean(2).reshape(B * Hkv, N).numpy()
        idx, pooled = orc.anchor_decode(_host(q), _host(k), 7)
        _close(pooled, ref, 1e-13, what=f"decode pooled {dtype}")
        _close(pooled.sum(1), np.ones(B * Hkv), 1e-12, what="decode pooled sums to 1")
        for u in range(B * Hkv):
            _check_topk(idx[u], ref[u], 7, f"decode top-k unit {u}")


def pin_prefill_pooled_vs_sdpa(orc):
    for dtype in (torch.float32, torch.bfloat16):
        B, Hq, Hkv, d, N, T, K = 1, 4, 2, 8, 37, 8, 11   # 5 tiles, the last one ragged
        G = Hq // Hkv
        q = _rand((B, Hq, N, d), 21, dtype)
        k = _rand((B, Hkv, N, d), 22, dtype)
        P = _probabilities(q, k, causal=True)[0]                     # [Hq,N,N]
        tiles = -(-N // T)
        idx, pooled = orc.anchor_prefill(_host(q), _host(k), K, T)
        for kv in range(Hkv):
            for t in range(tiles):
                r0, r1 = t * T, min((t + 1) * T, N)
                ref = P[kv * G:(kv + 1) * G, r0:r1, :].mean((0, 1)).numpy()
                u = kv * tiles + t
                _close(pooled[u], ref, 1e-13, what=f"prefill pooled kv{kv} t{t} {dtype}")
                assert abs(pooled[u].sum() - 1) < 1e-12
                _check_topk(idx[u], ref[:r1], min(K, r1), f"prefill top-k kv{kv} t{t}")


def pin_topk_brute_force(orc):
    """Tiny case: the selected set maximises the pooled mass over all k-subsets."""
    B, Hq, Hkv, d, N, K = 1, 2, 1, 8, 12, 5
    q = _rand((B, Hq, 1, d), 31)
    k = _rand((B, Hkv, N, d), 32, scale=2.0)
    score = _probabilities(q, k).reshape(Hq, N).mean(0).numpy()
    best = max(itertools.combinations(range(N), K), key=lambda s: sum(score[list(s)]))
    idx, _ = orc.anchor_decode(_host(q), _host(k), K)
    assert idx[0].tolist() == list(best), (idx[0], best)
    # prefill, tile of 6 rows with prefix 12
    q = _rand((1, 1, N, d), 33)
    k = _rand((1, 1, N, d), 34, scale=2.0)
    P = _probabilities(q, k, causal=True)[0, 0]
    score = P[6:12].mean(0).numpy()
    best = max(itertools.combinations(range(N), K), key=lambda s: sum(score[list(s)]))
    idx, _ = orc.anchor_prefill(_host(q), _host(k), K, 6)
    assert idx[1].tolist() == list(best), (idx[1], best)


def pin_ties_go_to_lower_index(orc):
    """Three heavy keys and nine identical light keys, k = 5: the two lowest light ones fill up."""
    d, N = 8, 12
    q = np.zeros((1, 1, 1, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d), np.float32)
    k[0, 0, :, 1] = 0.3            # light keys: logit 0
    for j, s in ((8, 9.0), (9, 7.0), (1, 8.0)):
        k[0, 0, j, 0] = s
    idx, _ = orc.anchor_decode(q, k, 5)
    assert idx[0].tolist() == [0, 1, 2, 8, 9], idx
    # all keys identical: every score ties and the first k keys win
    k[:] = 0.5
    idx, pooled = orc.anchor_decode(q, k, 4)
    assert idx[0].tolist() == [0, 1, 2, 3]
    _close(pooled[0], np.full(N, 1.0 / N), 1e-15, what="uniform pooled")


# ---- library routine with a mask: softmax restricted to the saved set --------------

def _random_sets(rng, n_sets, limit, K, pad_prob=0.3):
    sets = np.full((n_sets, K), -1, np.int32)
    for s in range(n_sets):
        lim = limit[s] if np.ndim(limit) else limit
        cnt = min(K, lim)
        cnt = max(1, cnt - int(rng.random() < pad_prob) * rng.integers(0, cnt))
        sel = rng.choice(lim, size=cnt, replace=False)
        sets[s, :cnt] = sel                      # unsorted on purpose
        rng.shuffle(sets[s])                     # padding scattered too
    return sets


def pin_reuse_decode_vs_masked_sdpa(orc):
    rng = np.random.default_rng(5)
    for dtype in (torch.float32, torch.bfloat16):
        B, Hq, Hkv, d, N, K = 2, 8, 2, 32, 100, 20
        q = _rand((B, Hq, 1, d), 41, dtype)
        k = _rand((B, Hkv, N, d), 42, dtype)
        v = _rand((B, Hkv, N, d), 43, dtype)
        idx = _random_sets(rng, B * Hkv, N, K).reshape(B, Hkv, 1, K)
        mask = torch.zeros((B, Hq, 1, N), dtype=torch.bool)
        for b in range(B):
            for h in range(Hq):
                sel = idx[b, h // (Hq // Hkv), 0]
                mask[b, h, 0, sel[sel >= 0]] = True
        out = orc.reuse_decode(_host(q), _host(k), _host(v), idx)
        _close(out, _sdpa(q, k, v, mask=mask).reshape(-1, d), 1e-12, what=f"reuse decode {dtype}")


def pin_reuse_prefill_vs_masked_sdpa(orc):
    rng = np.random.default_rng(6)
    for dtype in (torch.float32, torch.bfloat16):
        B, Hq, Hkv, d, N, T, K = 1, 4, 2, 16, 45, 8, 6
        G, tiles = Hq // Hkv, -(-N // T)
        q = _rand((B, Hq, N, d), 51, dtype)
        k = _rand((B, Hkv, N, d), 52, dtype)
        v = _rand((B, Hkv, N, d), 53, dtype)
        prefix = [min((t + 1) * T, N) for t in range(tiles)] * Hkv
        idx = _random_sets(rng, Hkv * tiles, prefix, K).reshape(B, Hkv, tiles, K)
        mask = torch.zeros((B, Hq, N, N), dtype=torch.bool)
        for h in range(Hq):
            for i in range(N):
                sel = idx[0, h // G, i // T]
                sel = sel[(sel >= 0) & (sel <= i)]
                mask[0, h, i, sel] = True
        out = orc.reuse_prefill(_host(q), _host(k), _host(v), idx, T).reshape(Hq, N, d)
        empty = ~mask[0].any(-1)
        ref = _sdpa(q, k, v, mask=mask)[0]
        ref[empty] = 0.0                         # fully masked rows: no keys, output 0
        assert empty.any() and (~empty).any()
        _close(out, ref.numpy(), 1e-12, what=f"reuse prefill {dtype}")


# ---- identities and invariants ------------------------------------------------------

def pin_k_equals_n_is_dense(orc):
    B, Hq, Hkv, d, N = 1, 4, 2, 16, 50
    q = _rand((B, Hq, 1, d), 61)
    k = _rand((B, Hkv, N, d), 62)
    v = _rand((B, Hkv, N, d), 63)
    idx, _ = orc.anchor_decode(_host(q), _host(k), N)
    assert np.all(idx == np.arange(N))
    out = orc.reuse_decode(_host(q), _host(k), _host(v), idx.reshape(B, Hkv, 1, N))
    _close(out, _sdpa(q, k, v).reshape(-1, d), 1e-12, what="k=N decode")
    q = _rand((B, Hq, N, d), 64)
    T = 16
    idx, _ = orc.anchor_prefill(_host(q), _host(k), N, T)
    out = orc.reuse_prefill(_host(q), _host(k), _host(v), idx.reshape(B, Hkv, -1, N), T)
    _close(out, _sdpa(q, k, v, causal=True).reshape(-1, d), 1e-12, what="k=N prefill")


def pin_v_ones_gives_ones(orc):
    B, Hq, Hkv, d, N, T, K = 1, 4, 2, 16, 30, 8, 9
    q = _rand((B, Hq, N, d), 71)
    k = _rand((B, Hkv, N, d), 72)
    ones = np.ones((B, Hkv, N, d), np.float32)
    idx, _ = orc.anchor_prefill(_host(q), _host(k), K, T)
    out = orc.reuse_prefill(_host(q), _host(k), ones, idx.reshape(B, Hkv, -1, K), T)
    _close(out, np.ones_like(out), 1e-13, what="prefill V=1")
    idx, _ = orc.anchor_decode(_host(q[:, :, :1]), _host(k), K)
    out = orc.reuse_decode(_host(q[:, :, :1]), _host(k), ones, idx.reshape(B, Hkv, 1, K))
    _close(out, np.ones_like(out), 1e-13, what="decode V=1")
    out, _ = orc.dense(_host(q), _host(k), ones, causal=True)
    _close(out, np.ones_like(out), 1e-13, what="dense V=1")


def pin_uniform_keys_give_mean_v(orc):
    B, Hq, Hkv, d, N, K = 1, 2, 1, 8, 40, 10
    q = _rand((B, Hq, 1, d), 81)
    k = np.tile(_host(_rand((1, 1, 1, d), 82)), (1, 1, N, 1))
    v = _host(_rand((B, Hkv, N, d), 83))
    idx, _ = orc.anchor_decode(_host(q), k, K)
    assert idx[0].tolist() == list(range(K))
    out = orc.reuse_decode(_host(q), k, v, idx.reshape(1, 1, 1, K))
    _close(out, np.tile(v[0, 0, :K].astype(np.float64).mean(0), (Hq, 1)), 1e-12, what="mean of V")


def pin_one_hot_key(orc):
    B, Hq, Hkv, d, N, K = 1, 1, 1, 16, 64, 8
    q = _host(_rand((B, Hq, 1, d), 91))
    k = _host(_rand((B, Hkv, N, d), 92, scale=0.1))
    v = _host(_rand((B, Hkv, N, d), 93))
    qhat = q[0, 0, 0] / np.linalg.norm(q[0, 0, 0])
    k[0, 0, 37] = (100.0 * qhat).astype(np.float32)
    idx, _ = orc.anchor_decode(q, k, K)
    assert 37 in idx[0]
    out = orc.reuse_decode(q, k, v, idx.reshape(1, 1, 1, K))
    _close(out[0], v[0, 0, 37], 1e-6, what="one-hot key")


def pin_head_permutation(orc):
    B, Hq, Hkv, d, N, K = 1, 6, 3, 8, 30, 5
    G = Hq // Hkv
    q = _host(_rand((B, Hq, 1, d), 101))
    k = _host(_rand((B, Hkv, N, d), 102))
    perm = [2, 0, 1]
    qp = np.concatenate([q[:, p * G:(p + 1) * G] for p in perm], axis=1)
    kp = k[:, perm]
    idx, _ = orc.anchor_decode(q, k, K)
    idxp, _ = orc.anchor_decode(qp, kp, K)
    for new, old in enumerate(perm):
        assert idxp[new].tolist() == idx[old].tolist()


def pin_tile0_selects_prefix(orc):
    B, Hq, Hkv, d, N, T, K = 1, 2, 1, 8, 40, 16, 20
    q = _host(_rand((B, Hq, N, d), 111))
    k = _host(_rand((B, Hkv, N, d), 112))
    idx, _ = orc.anchor_prefill(q, k, K, T)
    assert idx[0].tolist() == list(range(T)) + [-1] * (K - T)
    assert np.all(idx[1] >= 0) and np.all(idx[1] < 2 * T)


def pin_index_order_invariance(orc):
    rng = np.random.default_rng(12)
    B, Hq, Hkv, d, N, K = 1, 2, 1, 16, 60, 12
    q = _host(_rand((B, Hq, 1, d), 121))
    k = _host(_rand((B, Hkv, N, d), 122))
    v = _host(_rand((B, Hkv, N, d), 123))
    idx = np.sort(rng.choice(N, K, replace=False)).astype(np.int32).reshape(1, 1, 1, K)
    a = orc.reuse_decode(q, k, v, idx)
    b = orc.reuse_decode(q, k, v, idx[..., rng.permutation(K)].copy())
    _close(a, b, 1e-12, what="order invariance")


def pin_bf16_same_as_f32_values(orc):
    B, Hq, Hkv, d, N, K = 1, 4, 2, 16, 33, 6
    q = _rand((B, Hq, 1, d), 131, torch.bfloat16)
    k = _rand((B, Hkv, N, d), 132, torch.bfloat16)
    v = _rand((B, Hkv, N, d), 133, torch.bfloat16)
    i1, p1 = orc.anchor_decode(_host(q), _host(k), K)
    i2, p2 = orc.anchor_decode(_host(q.float()), _host(k.float()), K)
    assert np.array_equal(i1, i2) and np.array_equal(p1, p2)
    o1 = orc.reuse_decode(_host(q), _host(k), _host(v), i1.reshape(B, Hkv, 1, K))
    o2 = orc.reuse_decode(_host(q.float()), _host(k.float()), _host(v.float()), i1.reshape(B, Hkv, 1, K))
    assert np.array_equal(o1, o2)



# ---- the non-head-aware variant: one index set shared by every head ---------------

def pin_shared_pooled_vs_sdpa(orc):
    """Shared sets rank the mean over ALL query heads (and tile rows) of the
    post-softmax probabilities; every head's probabilities come from its own
    KV head."""
    for dtype in (torch.float32, torch.bfloat16):
        B, Hq, Hkv, d, N, K = 2, 6, 3, 16, 40, 7
        q = _rand((B, Hq, 1, d), 141, dtype)
        k = _rand((B, Hkv, N, d), 142, dtype)
        ref = _probabilities(q, k)[:, :, 0, :].mean(1).numpy()        # [B, N]
        idx, pooled = orc.anchor_decode(_host(q), _host(k), K, shared=True)
        assert idx.shape == (B, K)
        _close(pooled, ref, 1e-13, what=f"shared decode pooled {dtype}")
        for b in range(B):
            _check_topk(idx[b], ref[b], K, f"shared decode top-k b{b}")
        # differs from every per-KV-head ranking on this input
        per_kv, _ = orc.anchor_decode(_host(q), _host(k), K)
        assert not any(np.array_equal(idx[0], per_kv[kv]) for kv in range(Hkv))
    B, Hq, Hkv, d, N, T, K = 1, 4, 2, 8, 37, 8, 11
    q = _rand((B, Hq, N, d), 143)
    k = _rand((B, Hkv, N, d), 144)
    P = _probabilities(q, k, causal=True)[0]                           # [Hq, N, N]
    tiles = -(-N // T)
    idx, pooled = orc.anchor_prefill(_host(q), _host(k), K, T, shared=True)
    assert idx.shape == (tiles, K)
    for t in range(tiles):
        r0, r1 = t * T, min((t + 1) * T, N)
        ref = P[:, r0:r1, :].mean((0, 1)).numpy()
        _close(pooled[t], ref, 1e-13, what=f"shared prefill pooled t{t}")
        _check_topk(idx[t], ref[:r1], min(K, r1), f"shared prefill top-k t{t}")


def pin_shared_topk_brute_force(orc):
    """Two KV heads, one shared set: it maximises the all-head mean mass over all k-subsets."""
    B, Hq, Hkv, d, N, K = 1, 4, 2, 8, 11, 4
    q = _rand((B, Hq, 1, d), 151)
    k = _rand((B, Hkv, N, d), 152, scale=2.0)
    score = _probabilities(q, k).reshape(Hq, N).mean(0).numpy()
    best = max(itertools.combinations(range(N), K), key=lambda s: sum(score[list(s)]))
    idx, _ = orc.anchor_decode(_host(q), _host(k), K, shared=True)
    assert idx[0].tolist() == list(best), (idx[0], best)


def pin_shared_reuse_vs_masked_sdpa(orc):
    """Every head attends through the one set of its batch row (and tile)."""
    rng = np.random.default_rng(16)
    B, Hq, Hkv, d, N, K = 2, 6, 3, 16, 50, 9
    q = _rand((B, Hq, 1, d), 161)
    k = _rand((B, Hkv, N, d), 162)
    v = _rand((B, Hkv, N, d), 163)
    idx = _random_sets(rng, B, N, K).reshape(B, 1, 1, K)
    mask = torch.zeros((B, Hq, 1, N), dtype=torch.bool)
    for b in range(B):
        sel = idx[b, 0, 0]
        mask[b, :, 0, sel[sel >= 0]] = True
    out = orc.reuse_decode(_host(q), _host(k), _host(v), idx, shared=True)
    _close(out, _sdpa(q, k, v, mask=mask).reshape(-1, d), 1e-12, what="shared reuse decode")
    B, N, T, K = 1, 29, 8, 5
    tiles = -(-N // T)
    q = _rand((B, Hq, N, d), 164)
    k = _rand((B, Hkv, N, d), 165)
    v = _rand((B, Hkv, N, d), 166)
    idx = _random_sets(rng, tiles, [min((t + 1) * T, N) for t in range(tiles)], K).reshape(B, 1, tiles, K)
    mask = torch.zeros((B, Hq, N, N), dtype=torch.bool)
    for i in range(N):
        sel = idx[0, 0, i // T]
        mask[0, :, i, sel[(sel >= 0) & (sel <= i)]] = True
    out = orc.reuse_prefill(_host(q), _host(k), _host(v), idx, T, shared=True).reshape(Hq, N, d)
    empty = ~mask[0].any(-1)
    ref = _sdpa(q, k, v, mask=mask)[0]
    ref[empty] = 0.0
    _close(out, ref.numpy(), 1e-12, what="shared reuse prefill")


def pin_shared_is_head_aware_with_one_kv_head(orc):
    """With one KV head the shared set is the head-aware set."""
    B, Hq, Hkv, d, N, T, K = 2, 4, 1, 16, 33, 8, 6
    q = _host(_rand((B, Hq, 1, d), 171))
    k = _host(_rand((B, Hkv, N, d), 172))
    v = _host(_rand((B, Hkv, N, d), 173))
    a, pa = orc.anchor_decode(q, k, K)
    s, ps = orc.anchor_decode(q, k, K, shared=True)
    assert np.array_equal(a, s) and np.array_equal(pa, ps)
    ia = a.reshape(B, 1, 1, K)
    assert np.array_equal(orc.reuse_decode(q, k, v, ia), orc.reuse_decode(q, k, v, ia, shared=True))
    qp = _host(_rand((B, Hq, N, d), 174))
    a, pa = orc.anchor_prefill(qp, k, K, T)
    s, ps = orc.anchor_prefill(qp, k, K, T, shared=True)
    assert np.array_equal(a, s) and np.array_equal(pa, ps)


ALL_PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]
