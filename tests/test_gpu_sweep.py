"""Accuracy sweep over k on small drifting stacks (decode and ragged causal
prefill): properties that hold whatever the data, since the exact top-k sets
of one anchor are nested as k grows, hold the most pooled attention of any
k keys, and at k = N select every key."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import log  # noqa: E402

import bench  # noqa: E402
from long_context_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    "decode": synth.Workload(name="sweep_decode", wid=981, phase="decode", batch=2, hq=8, hkv=2, d=128,
                             n=4096, k=256, tile=1, dtype="bf16", layers=3, planted=32, share=0.7),
    "prefill": synth.Workload(name="sweep_prefill", wid=982, phase="prefill", batch=1, hq=8, hkv=2, d=128,
                              n=1088, k=256, tile=128, dtype="bf16", layers=3, planted=32, share=0.7, sinks=4),
    "prefill_t64": synth.Workload(name="sweep_prefill_t64", wid=983, phase="prefill", batch=1, hq=8, hkv=2,
                                  d=128, n=1000, k=256, tile=64, dtype="bf16", layers=3, planted=32, share=0.7,
                                  sinks=4),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_accuracy_sweep_properties(lib, case):
    w = CASES[case]
    fractions = (64, 16, 4, 1)
    log(f"[sweep] {case} N={w.n} fractions={fractions}")
    rows = bench.accuracy_sweep(w, fractions)
    assert all("shared_set_layers" in r for r in rows)
    assert [r["top_k"] for r in rows] == [max(1, w.n // f) for f in fractions]
    for r in rows:
        log(f"[sweep] {case} k={r['top_k']} " + " ".join(
            f"L{x['layer']}:rec={x['planted_recall']},mass={x['attention_mass']},err={x['rel_error_vs_dense']}"
            for x in r["layers"]))
    for key in ("layers", "shared_set_layers"):
        for l in range(w.layers):
            mass = [r[key][l]["attention_mass"] for r in rows]
            recall = [r[key][l]["planted_recall"] for r in rows]
            # nested index sets: captured mass and planted recall never fall as k grows
            assert all(b >= a - 1e-4 for a, b in zip(mass, mass[1:])), (key, l, mass)
            assert all(b >= a for a, b in zip(recall, recall[1:])), (key, l, recall)
            full = rows[-1][key][l]
            # k = N: every key of every prefix is selected, so reuse is dense attention
            assert full["attention_mass"] == pytest.approx(1.0, abs=1e-4)
            assert full["planted_recall"] == 1.0
            assert full["rel_error_vs_dense"] < 1e-2
    # per KV head, its own top-k holds at least as much of the anchor layer's
    # pooled attention as the shared set of the same size does
    for r in rows:
        assert r["layers"][0]["attention_mass"] >= r["shared_set_layers"][0]["attention_mass"] - 2e-3
    # the anchor's sets are its exact top-k: no other set of k keys per segment
    # holds more of the anchor layer's own pooled attention
    q, k, _ = synth.make_layer(w, 0, "cuda")
    pooled = bench.pooled_decode(q, k).unsqueeze(2) if w.phase == "decode" else bench.pooled_prefill(q, k, w.tile)
    for r in rows:
        kk = min(r["top_k"], w.n)
        best = float(pooled.topk(kk, dim=-1).values.sum(-1).mean())
        assert r["layers"][0]["attention_mass"] == pytest.approx(best, rel=2e-3, abs=1e-4), r["top_k"]
