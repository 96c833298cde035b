"""Decode parity: the HIP library against the fp64 oracle, through the C ABI."""
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
    base = dict(name=name, wid=900, phase="decode", batch=2, hq=8, hkv=2, d=128, n=4133, k=256,
                tile=1, dtype="bf16", layers=2, planted=16, share=0.7)
    base.update(kw)
    return synth.Workload(**base)


CASES = {
    "decode_f32_1k": synth.WORKLOADS["decode_f32_1k"],
    "bf16_d128_ragged": _small("bf16_d128_ragged"),
    "bf16_d64_g8": _small("bf16_d64_g8", wid=901, hq=16, hkv=2, d=64, n=2000, k=100),
    "f32_d128_g2": _small("f32_d128_g2", wid=902, hq=4, hkv=2, dtype="f32", n=777, k=65),
    "bf16_g1": _small("bf16_g1", wid=903, hq=4, hkv=4, n=1500, k=129),
    "bf16_g16": _small("bf16_g16", wid=904, hq=16, hkv=1, n=3000, k=300, batch=1),
    "bf16_k_eq_n": _small("bf16_k_eq_n", wid=905, n=640, k=640),
    "bf16_tiny": _small("bf16_tiny", wid=906, n=5, k=3, planted=1, batch=1),
    "bf16_n1": _small("bf16_n1", wid=907, n=1, k=1, planted=0, batch=1),
    # Group sizes that do not divide the anchor's eight-row store groups, with
    # a ragged last chunk: (chunk, head) score rows straddle store instructions.
    "bf16_g3_ragged": _small("bf16_g3_ragged", wid=908, hq=6, hkv=2, n=2021, k=200),
    "bf16_g6_d64": _small("bf16_g6_d64", wid=909, hq=12, hkv=2, d=64, n=1111, k=77),
    # Long lists over few (batch, KV head) units: the reuse gather spreads a
    # unit over several workgroups whose partials the last one to finish
    # merges, and the last workgroup holds wavefronts with no entries.
    "bf16_many_workgroups": _small("bf16_many_workgroups", wid=915, batch=1, hq=4, hkv=1, n=9000, k=4000),
    "bf16_g16_d64_many_workgroups": _small("bf16_g16_d64_many_workgroups", wid=916, batch=1, hq=16, hkv=1,
                                           d=64, n=5000, k=2500),
    "bf16_g3_many_workgroups": _small("bf16_g3_many_workgroups", wid=917, batch=2, hq=6, hkv=2, n=7000,
                                      k=3001),
}


def _layers(w):
    """Anchor and first reuse layer, drawn on the CPU and copied to the GPU."""
    stack = synth.make_stack(w.scaled(layers=2), device="cpu")
    return stack[0], stack[1]


@pytest.mark.parametrize("case", sorted(CASES))
def test_decode_anchor_and_reuse(lib, orc, case):
    w = CASES[case]
    log(f"[decode] case={case} B={w.batch} Hq={w.hq} Hkv={w.hkv} d={w.d} N={w.n} k={w.k} {w.dtype}")
    (q0, k0, v0), (q1, k1, v1) = _layers(w)
    dt = w.torch_dtype
    # ---- anchor layer -------------------------------------------------------
    qd, kd, vd = q0.to(DEV), k0.to(DEV), v0.to(DEV)
    out = torch.empty_like(qd)
    lse = torch.empty((w.batch, w.hq, 1), dtype=torch.float32, device=DEV)
    idx = K.anchor_decode(qd, kd, vd, w.k, out=out, lse=lse)
    torch.cuda.synchronize()
    idx_o, pooled_o = orc.anchor_decode(to_oracle(q0), to_oracle(k0), w.k)
    dense_o, lse_o = orc.dense(to_oracle(q0), to_oracle(k0), to_oracle(v0), causal=False)
    gi = idx.cpu().numpy().reshape(-1, w.k)
    same = [check_index_band(gi[u], idx_o[u], pooled_o[u], w.k, w.n, f"{case} unit {u}")
            for u in range(gi.shape[0])]
    check_close(host64(out).reshape(-1, w.d), dense_o, dt, f"{case} anchor dense out")
    check_lse(host64(lse).reshape(-1), lse_o, f"{case} anchor lse")
    if w.k == w.n:
        assert np.array_equal(gi, np.tile(np.arange(w.n, dtype=np.int32), (gi.shape[0], 1)))
    # ---- reuse layer, oracle's index sets -------------------------------------
    idx_o4 = idx_o.reshape(w.batch, w.hkv, 1, w.k)
    q1d, k1d, v1d = q1.to(DEV), k1.to(DEV), v1.to(DEV)
    out_r = K.reuse_decode(q1d, k1d, v1d, torch.from_numpy(idx_o4).to(DEV))
    torch.cuda.synchronize()
    ref_r = orc.reuse_decode(to_oracle(q1), to_oracle(k1), to_oracle(v1), idx_o4)
    check_close(host64(out_r).reshape(-1, w.d), ref_r, dt, f"{case} reuse out")
    # ---- chained: GPU anchor indices feed the GPU reuse ----------------------
    out_c = K.reuse_decode(q1d, k1d, v1d, idx)
    torch.cuda.synchronize()
    G = w.hq // w.hkv
    for u, s in enumerate(same):
        if s:
            rows = slice(u * G, (u + 1) * G)
            check_close(host64(out_c).reshape(-1, w.d)[rows], ref_r[rows], dt, f"{case} chain unit {u}")


def test_decode_reuse_padding_anywhere(lib, orc):
    """-1 entries are skipped wherever they sit; an all -1 list gives zeros."""
    w = _small("pad", wid=910, n=1000, k=96)
    log("[decode] case=padding_anywhere")
    (q, k, v), _ = _layers(w)
    rng = np.random.default_rng(3)
    idx = random_index_sets(rng, (w.batch, w.hkv, 1), w.n, w.k)
    idx[0, 0, 0, rng.choice(w.k, 30, replace=False)] = -1
    idx[1, 1, 0, :] = -1
    out = K.reuse_decode(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    ref = orc.reuse_decode(to_oracle(q), to_oracle(k), to_oracle(v), idx)
    check_close(host64(out).reshape(-1, w.d), ref, torch.bfloat16, "padding")
    assert np.all(host64(out)[1, 4:8] == 0.0)


def test_decode_ties_go_to_lower_index(lib):
    """All keys identical: every pooled score ties, the first k keys win."""
    log("[decode] case=ties")
    B, Hq, Hkv, d, N, k = 1, 4, 1, 128, 700, 50
    g = torch.Generator().manual_seed(11)
    q = torch.randn((B, Hq, 1, d), generator=g).to(torch.bfloat16)
    row = torch.randn((1, 1, 1, d), generator=g).to(torch.bfloat16)
    kk = row.expand(B, Hkv, N, d).contiguous()
    idx = K.anchor_decode(q.to(DEV), kk.to(DEV), None, k)
    torch.cuda.synchronize()
    assert idx.cpu().numpy().reshape(-1).tolist() == list(range(k))


def test_decode_deterministic(lib):
    w = _small("det", wid=911)
    log("[decode] case=determinism")
    (q, k, v), _ = _layers(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = [K.anchor_decode(qd, kd, vd, w.k) for _ in range(2)]
    o = [K.reuse_decode(qd, kd, vd, a[0]) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(a[0], a[1]) and torch.equal(o[0], o[1])


def _full_workload(orc, w):
    """Full-size decode workload, drawn on the GPU, checked against the oracle
    on every unit: the anchor's index band, dense output and lse for all
    B*Hkv (batch, KV head) units, then every query row of each reuse layer
    (own K/V, the anchor's GPU index sets) against the oracle's reuse over
    the same sets. Layers are drawn one at a time to bound memory."""
    G = w.group
    pos = synth.planted_positions(w)
    q0, k0, v0 = synth.make_layer(w, 0, DEV, pos)
    out = torch.empty_like(q0)
    lse = torch.empty((w.batch, w.hq, 1), dtype=torch.float32, device=DEV)
    idx = K.anchor_decode(q0, k0, v0, w.k, out=out, lse=lse)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    Q0, K0, V0 = to_oracle(q0), to_oracle(k0), to_oracle(v0)
    del q0, k0, v0
    units = w.batch * w.hkv
    log(f"[decode] {w.name}: oracle anchor over all {units} (batch, KV head) units")
    io, po = orc.anchor_decode(Q0, K0, w.k)
    flat = gi.reshape(-1, w.k)
    same = sum(check_index_band(flat[u], io[u], po[u], w.k, w.n, f"{w.name} anchor unit {u}")
               for u in range(units))
    del po
    do, lo = orc.dense(Q0, K0, V0, causal=False)
    check_close(host64(out).reshape(-1, w.d), do, w.torch_dtype, f"{w.name} dense out")
    check_lse(host64(lse).reshape(-1), lo, f"{w.name} lse")
    log(f"[decode] {w.name}: anchor checked on {units} of {units} units ({same} index sets identical, "
        f"the rest within the band), dense output and lse on {w.batch * w.hq} of {w.batch * w.hq} rows")
    del Q0, K0, V0
    for layer in range(1, w.layers):
        q, k, v = synth.make_layer(w, layer, DEV, pos)
        o = K.reuse_decode(q, k, v, idx)
        torch.cuda.synchronize()
        ro = orc.reuse_decode(to_oracle(q), to_oracle(k), to_oracle(v), gi)
        check_close(host64(o).reshape(-1, w.d), ro, w.torch_dtype, f"{w.name} reuse layer {layer}")
        log(f"[decode] {w.name}: reuse layer {layer} checked on {w.batch * w.hq} of {w.batch * w.hq} rows")
        del q, k, v, o


def test_decode_llama8b_32k_full(lib, orc):
    w = synth.WORKLOADS["decode_llama8b_32k"]
    log("[decode] case=decode_llama8b_32k full size, every unit and every reuse layer")
    _full_workload(orc, w)


def test_decode_128k_full(lib, orc):
    w = synth.WORKLOADS["decode_128k"]
    log("[decode] case=decode_128k full size, every unit and every reuse layer")
    _full_workload(orc, w)


def test_graph_replay_matches_eager(lib):
    """Decode and prefill anchor + reuse captured in a HIP graph: every replay,
    with eager work and synchronisations between replays, reproduces the eager
    results bit for bit."""
    log("[graph] case=replay_matches_eager")
    wd = _small("graph_dec", wid=912)
    (q0, k0, v0), (q1, k1, v1) = [tuple(t.to(DEV) for t in layer) for layer in _layers(wd)]
    wp = synth.Workload("graph_pre", 913, "prefill", 1, 8, 2, 128, 700, 192, 128, "bf16", 2, 8, 1.0, 4)
    (p0, pk0, pv0), (p1, pk1, pv1) = [tuple(t.to(DEV) for t in layer) for layer in synth.make_stack(wp, "cpu")]
    outs = {n: torch.empty_like(t) for n, t in (("da", q0), ("dr", q1), ("pa", p0), ("pr", p1))}
    didx = torch.empty((wd.batch, wd.hkv, 1, wd.k), dtype=torch.int32, device=DEV)
    pidx = torch.empty((1, wp.hkv, wp.tiles, wp.k), dtype=torch.int32, device=DEV)
    ws = {
        "ad": K.workspace(K.problem(q0, k0, wd.k, 1), K.OP_ANCHOR_DECODE, DEV),
        "rd": K.workspace(K.problem(q1, k1, wd.k, 1), K.OP_REUSE_DECODE, DEV),
        "ap": K.workspace(K.problem(p0, pk0, wp.k, wp.tile), K.OP_ANCHOR_PREFILL, DEV),
    }

    def run():
        K.anchor_decode(q0, k0, v0, wd.k, out=outs["da"], idx=didx, ws=ws["ad"])
        K.reuse_decode(q1, k1, v1, didx, out=outs["dr"], ws=ws["rd"])
        K.anchor_prefill(p0, pk0, pv0, wp.k, wp.tile, out=outs["pa"], idx=pidx, ws=ws["ap"])
        K.reuse_prefill(p1, pk1, pv1, pidx, wp.tile, out=outs["pr"])

    run()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in outs.items()}
    ref_idx = (didx.clone(), pidx.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(3):
        for t in list(outs.values()) + [didx, pidx]:
            t.zero_()                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in outs:
            assert torch.equal(outs[n], ref[n]), n
        assert torch.equal(didx, ref_idx[0]) and torch.equal(pidx, ref_idx[1])


# ---- selection across 32768-key sub-segments ----------------------------------

@pytest.mark.parametrize("n,k", [(70000, 100), (70001, 40000)])
def test_decode_ties_across_subsegments(lib, n, k):
    """All keys identical over three sub-segments: the k lowest keys win,
    including when k exceeds a sub-segment and the merge reads its
    candidates from memory."""
    log(f"[decode] case=ties_across_subsegments n={n} k={k}")
    B, Hq, Hkv, d = 1, 2, 1, 64
    g = torch.Generator().manual_seed(12)
    q = torch.randn((B, Hq, 1, d), generator=g).to(torch.bfloat16)
    row = torch.randn((1, 1, 1, d), generator=g).to(torch.bfloat16)
    kk = row.expand(B, Hkv, n, d).contiguous()
    idx = K.anchor_decode(q.to(DEV), kk.to(DEV), None, k)
    torch.cuda.synchronize()
    assert idx.cpu().numpy().reshape(-1).tolist() == list(range(k))


@pytest.mark.parametrize("n,k", [(40000, 40000), (40000, 33000), (65537, 1000)])
def test_decode_long_segments_against_oracle(lib, orc, n, k):
    """Segments over one sub-segment: k = N keeps every key; k above a
    sub-segment sends the merge through memory; a ragged last sub-segment of
    one key."""
    w = _small(f"long_{n}_{k}", wid=914, batch=1, hq=4, hkv=2, d=64, n=n, k=k, planted=32)
    log(f"[decode] case=long_segments n={n} k={k}")
    (q, kk, v), _ = _layers(w)
    idx = K.anchor_decode(q.to(DEV), kk.to(DEV), None, k)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy().reshape(-1, k)
    io, po = orc.anchor_decode(to_oracle(q), to_oracle(kk), k)
    for u in range(gi.shape[0]):
        check_index_band(gi[u], io[u], po[u], k, n, f"long n={n} k={k} unit {u}")
    if k == n:
        assert np.array_equal(gi, np.tile(np.arange(n, dtype=np.int32), (gi.shape[0], 1)))


@pytest.mark.parametrize("case", ["bf16_d128_ragged", "f32_d128_g2", "bf16_g16"])
def test_decode_dense_only(lib, orc, case):
    """The anchor call without an index buffer is dense attention: output and
    lse against the oracle's dense attention, and no index buffer is touched."""
    w = CASES[case]
    log(f"[decode] case=dense_only {case}")
    (q, k, v), _ = _layers(w)
    out = torch.empty_like(q, device=DEV)
    lse = torch.empty((w.batch, w.hq, 1), dtype=torch.float32, device=DEV)
    assert K.anchor_decode(q.to(DEV), k.to(DEV), v.to(DEV), w.k, out=out, lse=lse, dense_only=True) is None
    torch.cuda.synchronize()
    do, lo = orc.dense(to_oracle(q), to_oracle(k), to_oracle(v), causal=False)
    check_close(host64(out).reshape(-1, w.d), do, w.torch_dtype, f"{case} dense-only out")
    check_lse(host64(lse).reshape(-1), lo, f"{case} dense-only lse")
    lse2 = torch.empty_like(lse)
    K.anchor_decode(q.to(DEV), k.to(DEV), None, w.k, lse=lse2, dense_only=True)
    torch.cuda.synchronize()
    check_lse(host64(lse2).reshape(-1), lo, f"{case} dense-only lse without output")


def test_decode_reuse_one_workspace_many_calls(lib, orc):
    """One decode workspace, zero-filled once, serves reuse calls of different
    sizes in a row (the arrival counters the gather's merge uses go back to
    zero after every call), interleaved with an anchor call on the same
    workspace; every output against the oracle."""
    log("[decode] case=one_workspace_many_calls")
    big = _small("ws_big", wid=918, batch=2, hq=8, hkv=2, n=9000, k=4000)
    small = _small("ws_small", wid=919, batch=1, hq=8, hkv=2, n=3000, k=700)
    ws = K.workspace(K.problem(torch.empty((2, 8, 1, 128), dtype=BF16), torch.empty((2, 2, 9000, 128), dtype=BF16),
                               4000, 1), K.OP_ANCHOR_DECODE, DEV)
    for w in (big, small, big, small):
        (q0, k0, v0), (q1, k1, v1) = _layers(w)
        idx = K.anchor_decode(q0.to(DEV), k0.to(DEV), None, w.k, ws=ws)
        out = K.reuse_decode(q1.to(DEV), k1.to(DEV), v1.to(DEV), idx, ws=ws)
        torch.cuda.synchronize()
        ref = orc.reuse_decode(to_oracle(q1), to_oracle(k1), to_oracle(v1), idx.cpu().numpy())
        check_close(host64(out).reshape(-1, w.d), ref, BF16, f"{w.name} reuse on a shared workspace")
    assert not ws[:256].any(), "arrival counters left non-zero"
