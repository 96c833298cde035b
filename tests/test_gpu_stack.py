"""A layer stack under an anchor schedule through kascade_attention, against
the oracle layer by layer: dense and anchor layers against dense attention,
reuse layers against the oracle's reuse over the oracle's indices of the
nearest preceding anchor (units whose GPU and oracle index sets agree)."""
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
BF16 = torch.bfloat16

STACKS = {
    "decode": (synth.Workload(name="stack_decode", wid=970, phase="decode", batch=2, hq=8, hkv=2, d=128,
                              n=3000, k=256, tile=1, dtype="bf16", layers=6, planted=16, share=0.7), [1, 4]),
    "prefill": (synth.Workload(name="stack_prefill", wid=971, phase="prefill", batch=1, hq=8, hkv=2, d=128,
                               n=700, k=256, tile=128, dtype="bf16", layers=4, planted=8, share=1.0,
                               sinks=4), [1]),
}


@pytest.mark.parametrize("case", sorted(STACKS))
def test_stack_follows_the_anchor_schedule(lib, orc, case):
    w, anchors = STACKS[case]
    log(f"[stack] case={case} layers={w.layers} anchors={anchors} N={w.n} k={w.k}")
    decode = w.phase == "decode"
    layers = synth.make_stack(w, device="cpu")
    qs = [q.to(DEV) for q, _, _ in layers]
    ks = [k.to(DEV) for _, k, _ in layers]
    vs = [v.to(DEV) for _, _, v in layers]
    outs, saved = K.kascade_attention(qs, ks, vs, w.k, anchors, q_tile=w.tile if not decode else 128)
    torch.cuda.synchronize()
    assert sorted(saved) == sorted(anchors)
    tiles = 1 if decode else -(-w.n // w.tile)
    G = w.hq // w.hkv
    oracle_sets = {}
    for l, (role, src) in enumerate(K.anchor_schedule(w.layers, anchors)):
        Q, Kt, V = (to_oracle(t) for t in layers[l])
        got = host64(outs[l]).reshape(w.batch, w.hq, -1, w.d)
        if role in ("dense", "anchor"):
            ref, _ = orc.dense(Q, Kt, V, causal=not decode)
            check_close(got.reshape(-1, w.d), ref, BF16, f"{case} layer {l} ({role}) dense out")
            if role == "anchor":
                idx_o, pooled_o = (orc.anchor_decode(Q, Kt, w.k) if decode
                                   else orc.anchor_prefill(Q, Kt, w.k, w.tile))
                gi = saved[l].cpu().numpy().reshape(-1, w.k)
                same = []
                for u in range(gi.shape[0]):
                    prefix = w.n if decode else min((u % tiles + 1) * w.tile, w.n)
                    same.append(check_index_band(gi[u], idx_o[u], pooled_o[u], min(w.k, prefix), prefix,
                                                 f"{case} anchor {l} unit {u}"))
                oracle_sets[l] = (idx_o.reshape(w.batch, w.hkv, tiles, w.k), same)
        else:
            idx_o4, same = oracle_sets[src]
            ref = (orc.reuse_decode(Q, Kt, V, idx_o4) if decode
                   else orc.reuse_prefill(Q, Kt, V, idx_o4, w.tile)).reshape(w.batch, w.hq, -1, w.d)
            checked = 0
            for u, s in enumerate(same):
                if not s:
                    continue
                b, kv, t = u // (w.hkv * tiles), (u // tiles) % w.hkv, u % tiles
                rows = slice(0, 1) if decode else slice(t * w.tile, min((t + 1) * w.tile, w.n))
                heads = slice(kv * G, (kv + 1) * G)
                check_close(got[b, heads, rows].reshape(-1, w.d), ref[b, heads, rows].reshape(-1, w.d), BF16,
                            f"{case} layer {l} reuse of {src} unit {u}")
                checked += 1
            assert checked > 0, f"{case} layer {l}: no unit with identical index sets to check"
