"""Causal prefill parity: the HIP library against the fp64 oracle, through the C ABI."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import check_close, check_index_band, check_lse, host64, log  # noqa: E402

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
    # d = 64 with a last tile that ends inside its second 64-row half
    "d64_half_tile": _small("d64_half_tile", wid=964, hq=8, hkv=2, d=64, n=1000, k=256),
    # last tile of exactly 64 rows (one staged unit), and of 65 (a second unit
    # holding a single row)
    "d128_tile_64_rows": _small("d128_tile_64_rows", wid=965, n=576, k=200),
    "d64_tile_65_rows": _small("d64_tile_65_rows", wid=966, hq=8, hkv=2, d=64, n=577, k=200),
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


@pytest.mark.parametrize("tile,d,group", [(128, 128, 4), (64, 64, 2), (128, 64, 1), (64, 128, 1)])
def test_prefill_reuse_unsorted_padded_lists(lib, orc, tile, d, group):
    """Reuse lists in any order, with duplicate keys and -1 padding anywhere
    among a tile's first min(k, prefix) positions, and one tile all padding
    (its rows give zeros): the kernel must mask per key wherever a key above a
    row or a padding entry sits, not only in a list's last chunk."""
    w = _small(f"lists_t{tile}_d{d}_g{group}", wid=964 + tile + d + group, hq=2 * group, hkv=2, d=d,
               n=1000, k=200, tile=tile)
    log(f"[prefill] case=unsorted_padded_lists T={tile} d={d} G={group} N={w.n} k={w.k}")
    (q, k, v), _ = synth.make_stack(w, device="cpu")
    tiles = _tiles(w)
    rng = np.random.default_rng(17 + tile + d + group)
    idx = np.full((w.batch, w.hkv, tiles, w.k), -1, np.int32)
    for kv in range(w.hkv):
        for t in range(tiles):
            prefix = min((t + 1) * tile, w.n)
            kt = min(w.k, prefix)
            keys = rng.integers(0, prefix, size=kt).astype(np.int32)  # unsorted, duplicates allowed
            keys[rng.random(kt) < 0.15] = -1
            idx[0, kv, t, :kt] = keys
    empty_t = tiles // 2
    idx[0, 1, empty_t, :] = -1
    out = K.reuse_prefill(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(idx).to(DEV), tile)
    torch.cuda.synchronize()
    ref = orc.reuse_prefill(to_oracle(q), to_oracle(k), to_oracle(v), idx, tile)
    got = host64(out)
    check_close(got.reshape(-1, d), ref, BF16, f"unsorted padded lists T={tile} d={d}")
    rows = slice(empty_t * tile, min((empty_t + 1) * tile, w.n))
    assert np.all(got[0, group:2 * group, rows] == 0.0), "an all-padding list gives zeros"


def test_prefill_deterministic(lib):
    w = _small("det", wid=961)
    log("[prefill] case=determinism")
    (q, k, v), _ = synth.make_stack(w, device="cpu")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = [K.anchor_prefill(qd, kd, vd, w.k, w.tile) for _ in range(2)]
    o = [K.reuse_prefill(qd, kd, vd, a[0], w.tile) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(a[0], a[1]) and torch.equal(o[0], o[1])


def _anchor_tiles(w, per_kv, seed):
    """(KV head, tile) pairs for the anchor check: per_kv tiles of every KV
    head, seeded, each KV head including the first tile (even heads) or the
    last one (odd heads). per_kv=None takes every tile."""
    tiles = _tiles(w)
    if per_kv is None or per_kv >= tiles:
        return [(kv, t) for kv in range(w.hkv) for t in range(tiles)]
    rng = np.random.default_rng(seed)
    pairs = []
    for kv in range(w.hkv):
        forced = 0 if kv % 2 == 0 else tiles - 1
        rest = rng.choice(np.setdiff1d(np.arange(tiles), [forced]), per_kv - 1, replace=False)
        pairs += [(kv, int(t)) for t in sorted([forced, *rest.tolist()])]
    return pairs


def _full_workload(orc, w, per_kv, row_frac, seed):
    """Full-size prefill workload on the GPU against the oracle:
      * anchor index band on the (KV head, tile) pairs of _anchor_tiles;
      * dense output and lse on a seeded row_frac share of the (head, row) rows;
      * each reuse layer (own K/V, the anchor's GPU index sets) on a seeded
        row_frac share of the rows plus 4 rows per head of every checked tile,
        against the oracle's reuse over the same sets."""
    T, tiles, G = w.tile, _tiles(w), w.group
    pos = synth.planted_positions(w)
    q0, k0, v0 = synth.make_layer(w, 0, DEV, pos)
    out = torch.empty_like(q0)
    lse = torch.empty((w.batch, w.hq, w.n), dtype=torch.float32, device=DEV)
    idx = K.anchor_prefill(q0, k0, v0, w.k, T, out=out, lse=lse)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    Q0, K0, V0 = to_oracle(q0), to_oracle(k0), to_oracle(v0)
    oh, lh = host64(out), host64(lse)
    del q0, k0, v0, out, lse
    pairs = _anchor_tiles(w, per_kv, seed)
    log(f"[prefill] {w.name}: oracle anchor over {len(pairs)} of {w.hkv * tiles} (KV head, tile) pairs")
    units = np.array([(0, kv, t) for kv, t in pairs], np.int32)
    io, po = orc.anchor_prefill(Q0, K0, w.k, T, units=units, want_pooled=True)
    same = 0
    for u, (_, kv, t) in enumerate(units):
        prefix = min((t + 1) * T, w.n)
        kt = min(w.k, prefix)
        same += check_index_band(gi[0, kv, t], io[u], po[u], kt, prefix, f"{w.name} (kv{kv},t{t})")
        if kt == prefix:
            assert gi[0, kv, t, :kt].tolist() == list(range(prefix)), f"{w.name} tile {t} keeps everything"
    del po
    log(f"[prefill] {w.name}: anchor checked on {len(pairs)} (KV head, tile) pairs ({same} index sets "
        f"identical, the rest within the band)")
    rng = np.random.default_rng(seed + 1)
    total_rows = w.hq * w.n
    n_rows = max(1, int(round(row_frac * total_rows)))
    flat = np.sort(rng.choice(total_rows, n_rows, replace=False))
    rows = np.stack([np.zeros(n_rows, np.int64), flat // w.n, flat % w.n], 1).astype(np.int32)
    do, lo = orc.dense(Q0, K0, V0, causal=True, units=rows)
    check_close(oh[rows[:, 0], rows[:, 1], rows[:, 2]], do, BF16, f"{w.name} dense rows")
    check_lse(lh[rows[:, 0], rows[:, 1], rows[:, 2]], lo, f"{w.name} lse rows")
    log(f"[prefill] {w.name}: dense output and lse checked on {n_rows} of {total_rows} rows")
    del Q0, K0, V0, oh, lh
    trows = []
    for (_, kv, t) in units:
        for h in range(kv * G, (kv + 1) * G):
            for i in rng.choice(np.arange(t * T, min((t + 1) * T, w.n)), min(4, w.n - t * T), replace=False):
                trows.append((0, h, int(i)))
    rrows = np.concatenate([rows, np.array(trows, np.int32).reshape(-1, 3)])
    for layer in range(1, w.layers):
        q, k, v = synth.make_layer(w, layer, DEV, pos)
        o = K.reuse_prefill(q, k, v, idx, T)
        torch.cuda.synchronize()
        ro = orc.reuse_prefill(to_oracle(q), to_oracle(k), to_oracle(v), gi, T, units=rrows)
        check_close(host64(o)[rrows[:, 0], rrows[:, 1], rrows[:, 2]], ro, BF16, f"{w.name} reuse layer {layer}")
        log(f"[prefill] {w.name}: reuse layer {layer} checked on {len(rrows)} rows "
            f"({n_rows} seeded, {len(trows)} in the checked tiles)")
        del q, k, v, o


def test_prefill_8k_full(lib, orc):
    """Every (KV head, tile) anchor set of the 8K workload; 1/8 of the rows."""
    w = synth.WORKLOADS["prefill_8k"]
    log("[prefill] case=prefill_8k full size, every anchor tile")
    _full_workload(orc, w, per_kv=None, row_frac=1 / 8, seed=31)


def test_prefill_8k_t64_sampled(lib, orc):
    w = synth.WORKLOADS["prefill_8k"].scaled(tile=64)
    log("[prefill] case=prefill_8k with 64-row tiles, sampled tiles and rows")
    _full_workload(orc, w, per_kv=6, row_frac=1 / 64, seed=33)


def test_prefill_32k_sampled(lib, orc):
    """A seeded 1 % of the rows (the workload's own sample size) and 8 anchor
    tiles per KV head, the first and the last tile among them."""
    w = synth.WORKLOADS["prefill_32k"]
    log("[prefill] case=prefill_32k full size, 64 anchor tiles and 1% of rows")
    _full_workload(orc, w, per_kv=8, row_frac=1 / 100, seed=32)


@pytest.mark.parametrize("case", ["d128_ragged", "d64_g8", "n1"])
def test_prefill_dense_only(lib, orc, case):
    """The anchor call without an index buffer is dense causal attention."""
    w = CASES[case]
    log(f"[prefill] case=dense_only {case}")
    (q, k, v), _ = synth.make_stack(w, device="cpu")
    out = torch.empty_like(q, device=DEV)
    lse = torch.empty((w.batch, w.hq, w.n), dtype=torch.float32, device=DEV)
    assert K.anchor_prefill(q.to(DEV), k.to(DEV), v.to(DEV), w.k, w.tile, out=out, lse=lse,
                            dense_only=True) is None
    torch.cuda.synchronize()
    do, lo = orc.dense(to_oracle(q), to_oracle(k), to_oracle(v), causal=True)
    check_close(host64(out).reshape(-1, w.d), do, BF16, f"{case} dense-only out")
    check_lse(host64(lse).reshape(-1), lo, f"{case} dense-only lse")
