"""Anchor selection on a synthetic layer stack whose planted keys drift from
layer to layer (70% kept per layer): the overlap of top-k sets falls with
layer distance, and the chosen schedule scores at least as well as evenly
spaced anchors."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import log  # noqa: E402

from long_context_amd import schedule as S  # noqa: E402
from long_context_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu


def test_select_anchors_on_a_drifting_stack(lib):
    w = synth.Workload(name="sched", wid=980, phase="decode", batch=2, hq=8, hkv=2, d=128, n=4096, k=64,
                       tile=1, dtype="bf16", layers=8, planted=64, share=0.7)
    log(f"[schedule] layers={w.layers} N={w.n} k={w.k} planted={w.planted}")
    layers = synth.make_stack(w, device="cuda")
    qs = [q for q, _, _ in layers]
    ks = [k for _, k, _ in layers]
    anchors, score, sim = S.select_anchors(qs, ks, w.k, 3)
    log(f"[schedule] anchors={anchors} score={score:.3f} sim[0]={np.round(sim[0], 3).tolist()}")
    assert anchors[0] == 0 and len(anchors) == 3
    # overlaps fall with distance from each layer (on average over the stack)
    for dist in range(1, w.layers - 1):
        near = np.mean([sim[a, a + dist] for a in range(w.layers - dist)])
        far = np.mean([sim[a, a + dist + 1] for a in range(w.layers - dist - 1)])
        assert near >= far - 0.02, (dist, near, far)
    assert sim[0, 1] > 0.3  # adjacent layers share many of their top keys
    even = [0, 3, 6]
    assert score >= S.schedule_score(sim, even) - 1e-12
    assert score == pytest.approx(S.brute_force_schedule(sim, 3)[1])
