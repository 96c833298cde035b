"""Causal prefill parity: the HIP library against the fp64 oracle, through the C ABI."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import (check_close, check_index_band, check_lse, host64, log,  # noqa: E402
                    random_index_sets)

from long_context_amd import kascade as K  # noqa: E402
from long_context_amd import synth  # noqa: E402
from long_context_amd.synth import to_oracle  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16 = torch.bfloat16


def _small(name, **kw):
    base = dict(name=name, wid=950, phase="prefill", batch=1, hq=8, hkv=2, d=128, n=1000, k=256,
                tile=128, dtype="bf16", layers=2, planted=8, share=1.0, sinks=4)
    base.update(kw)
    return synth.Workload(**base)


CASES = {
    "d128_ragged": _small("d128_ragged"),
    "d64_g8": _small("d64_g8", wid=951, hq=16, hkv=2, d=64, n=700, k=160),
    "batch2_g1": _small("batch2_g1", wid=952, batch=2, hq=2, hkv=2, n=520, k=200),
    "k_ge_n": _small("k_ge_n", wid=953, n=300, k=512),
    "k_below_tile": _small("k_below_tile", wid=954, n=450, k=40),
    "single_short_tile": _small("single_short_tile", wid=955, n=77, k=32, planted=2),
    "n1": _small("n1", wid=956, n=1, k=1, planted=0, sinks=0),
    # 64-row selection tiles: four heads per reuse workgroup (G = 4, 8), two
    # heads (G = 2), one head (G = 1)
    "t64_d128_ragged": _small("t64_d128_ragged", wid=957, tile=64),
    "t64_d64_g8": _small("t64_d64_g8", wid=958, hq=16, hkv=2, d=64, n=700, k=160, tile=64),
    "t64_g2": _small("t64_g2", wid=959, hq=4, hkv=2, n=520, k=100, tile=64),
    "t64_g1_batch2": _small("t64_g1_batch2", wid=962, batch=2, hq=2, hkv=2, n=300, k=50, tile=64),
    "t64_k_below_tile": _small("t64_k_below_tile", wid=963, n=450, k=40, tile=64),
}


def _tiles(w):
    return -(-w.n // w.tile)


@pytest.mark.parametrize("case", sorted(CASES))
def test_prefill_anchor_and_reuse(lib, orc, case):
    w = CASES[case]
    T, tiles, G = w.tile, _tiles(w), w.group
    log(f"[prefill] case={case} B={w.batch} Hq={w.hq} Hkv={w.hkv} d={w.d} N={w.n} k={w.k}")
    (q0, k0, v0), (q1, k1, v1) = synth.make_stack(w, device="cpu")
    # ---- anchor ---------------------------------------------------------------
    qd, kd, vd = q0.to(DEV), k0.to(DEV), v0.to(DEV)
    out = torch.empty_like(qd)
    lse = torch.empty((w.batch, w.hq, w.n), dtype=torch.float32, device=DEV)
    idx = K.anchor_prefill(qd, kd, vd, w.k, T, out=out, lse=lse)
    torch.cuda.synchronize()
    idx_o, pooled_o = orc.anchor_prefill(to_oracle(q0), to_oracle(k0), w.k, T)
    dense_o, lse_o = orc.dense(to_oracle(q0), to_oracle(k0), to_oracle(v0), causal=True)
    gi = idx.cpu().numpy().reshape(-1, w.k)
    same = []
    for u in range(gi.shape[0]):
        t = u % tiles
        prefix = min((t + 1) * T, w.n)
        kt = min(w.k, prefix)
        same.append(check_index_band(gi[u], idx_o[u], pooled_o[u], kt, prefix, f"{case} unit {u} t{t}"))
        if kt == prefix:
            assert gi[u, :kt].tolist() == list(range(prefix)), f"{case} tile {t} keeps everything"
    check_close(host64(out).reshape(-1, w.d), dense_o, BF16, f"{case} anchor dense out")
    check_lse(host64(lse).reshape(-1), lse_o, f"{case} anchor lse")
    # ---- reuse with the oracle's sets ----------------------------------------
    idx_o4 = idx_o.reshape(w.batch, w.hkv, tiles, w.k)
    q1d, k1d, v1d = q1.to(DEV), k1.to(DEV), v1.to(DEV)
    out_r = K.reuse_prefill(q1d, k1d, v1d, torch.from_numpy(idx_o4).to(DEV), T)
    torch.cuda.synchronize()
    ref_r = orc.reuse_prefill(to_oracle(q1), to_oracle(k1), to_oracle(v1), idx_o4, T)
    check_close(host64(out_r).reshape(-1, w.d), ref_r, BF16, f"{case} reuse out")
    # ---- chained ----------------------------------------------------------------
    out_c = host64(K.reuse_prefill(q1d, k1d, v1d, idx, T)).reshape(w.batch, w.hq, w.n, w.d)
    torch.cuda.synchronize()
    ref_r = ref_r.reshape(w.batch, w.hq, w.n, w.d)
    for u, s in enumerate(same):
        if not s:
            continue
        b, kv, t = u // (w.hkv * tiles), (u // tiles) % w.hkv, u % tiles
        rows = slice(t * T, min((t + 1) * T, w.n))
        heads = slice(kv * G, (kv + 1) * G)
        check_close(out_c[b, heads, rows], ref_r[b, heads, rows], BF16, f"{case} chain unit {u}")


def test_prefill_reuse_k_eq_n_is_dense(lib, orc):
    w = _small("kn", wid=960, n=400, k=400)
    log("[prefill] case=reuse_k_eq_n_is_dense")
    (q, k, v), _ = synth.make_stack(w, device="cpu")
    tiles = _tiles(w)
    idx = np.full((1, w.hkv, tiles, w.k), -1, np.int32)
    for t in range(tiles):
        p = min((t + 1) * w.tile, w.n)
        idx[:, :, t, :p] = np.arange(p)
    out = K.reuse_prefill(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(idx).to(DEV), w.tile)
    torch.cuda.synchronize()
    dense_o, _ = orc.dense(to_oracle(q), to_oracle(k), to_oracle(v), causal=True)
    check_close(host64(out).reshape(-1, w.d), dense_o, BF16, "k=N reuse vs dense")


def test_prefill_deterministic(lib):
    w = _small("det", wid=961)
    log("[prefill] case=determinism")
    (q, k, v), _ = synth.make_stack(w, device="cpu")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = [K.anchor_prefill(qd, kd, vd, w.k, w.tile) for _ in range(2)]
    o = [K.reuse_prefill(qd, kd, vd, a[0], w.tile) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(a[0], a[1]) and torch.equal(o[0], o[1])


def _sampled_full(orc, w, tiles_sample, n_rows, seed):
    """Full-size prefill workload on the GPU; oracle on sampled tiles and rows."""
    T, tiles, G = w.tile, _tiles(w), w.group
    pos = synth.planted_positions(w.scaled(layers=2))
    q0, k0, v0 = synth.make_layer(w, 0, DEV, pos)
    q1, k1, v1 = synth.make_layer(w, 1, DEV, pos)
    out = torch.empty_like(q0)
    lse = torch.empty((w.batch, w.hq, w.n), dtype=torch.float32, device=DEV)
    idx = K.anchor_prefill(q0, k0, v0, w.k, T, out=out, lse=lse)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    Q0, K0, V0 = to_oracle(q0), to_oracle(k0), to_oracle(v0)
    units = np.array([(0, kv, t) for kv, t in tiles_sample], np.int32)
    io, po = orc.anchor_prefill(Q0, K0, w.k, T, units=units)
    for u, (_, kv, t) in enumerate(units):
        prefix = min((t + 1) * T, w.n)
        check_index_band(gi[0, kv, t], io[u], po[u], min(w.k, prefix), prefix, f"{w.name} (kv{kv},t{t})")
    rng = np.random.default_rng(seed)
    rows = np.stack([np.zeros(n_rows, int), rng.integers(0, w.hq, n_rows), rng.integers(0, w.n, n_rows)], 1)
    rows = rows.astype(np.int32)
    drows = rows[:2048]
    do, lo = orc.dense(Q0, K0, V0, causal=True, units=drows)
    oh, lh = host64(out), host64(lse)
    check_close(oh[drows[:, 0], drows[:, 1], drows[:, 2]], do, BF16, f"{w.name} dense rows")
    check_lse(lh[drows[:, 0], drows[:, 1], drows[:, 2]], lo, f"{w.name} lse rows")
    # reuse: sampled tiles carry the oracle's sets, the rest seeded random sets
    prefixes = np.minimum((np.arange(tiles) + 1) * T, w.n)
    idx_r = random_index_sets(rng, (1, w.hkv, tiles), np.broadcast_to(prefixes, (1, w.hkv, tiles)), w.k)
    for u, (_, kv, t) in enumerate(units):
        idx_r[0, kv, t] = io[u]
    out_r = K.reuse_prefill(q1, k1, v1, torch.from_numpy(idx_r).to(DEV), T)
    torch.cuda.synchronize()
    ro = orc.reuse_prefill(to_oracle(q1), to_oracle(k1), to_oracle(v1), idx_r, T, units=rows)
    check_close(host64(out_r)[rows[:, 0], rows[:, 1], rows[:, 2]], ro, BF16, f"{w.name} reuse rows")
    # rows of the sampled tiles specifically
    trows = []
    for (_, kv, t) in units:
        for h in range(kv * G, (kv + 1) * G):
            for i in rng.choice(np.arange(t * T, min((t + 1) * T, w.n)), 4, replace=False):
                trows.append((0, h, i))
    trows = np.array(trows, np.int32)
    ro = orc.reuse_prefill(to_oracle(q1), to_oracle(k1), to_oracle(v1), idx_r, T, units=trows)
    check_close(host64(out_r)[trows[:, 0], trows[:, 1], trows[:, 2]], ro, BF16, f"{w.name} reuse tile rows")


def test_prefill_8k_sampled(lib, orc):
    w = synth.WORKLOADS["prefill_8k"]
    log("[prefill] case=prefill_8k full size, sampled tiles and rows")
    _sampled_full(orc, w, [(0, 0), (0, 7), (3, 8), (5, 31), (7, 63)], 2048, seed=31)


def test_prefill_8k_t64_sampled(lib, orc):
    w = synth.WORKLOADS["prefill_8k"].scaled(tile=64)
    log("[prefill] case=prefill_8k with 64-row tiles, sampled tiles and rows")
    _sampled_full(orc, w, [(0, 0), (1, 15), (3, 16), (5, 63), (7, 127)], 2048, seed=33)


def test_prefill_32k_sampled(lib, orc):
    w = synth.WORKLOADS["prefill_32k"]
    log("[prefill] case=prefill_32k full size, sampled tiles and 1% of rows")
    n_rows = (w.hq * w.n) // 100
    _sampled_full(orc, w, [(0, 0), (2, 15), (4, 100), (6, 200), (7, 255)], n_rows, seed=32)
