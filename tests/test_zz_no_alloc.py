"""kascade_reuse_decode_noalloc, the allocation-free reuse decode, against
kascade_reuse_decode (the workspace entry point), both through the C ABI:
calls in a row on one GPU, each after the first smaller than the one before,
outputs bit-identical to the workspace entry point's and within the bfloat16 /
float32 tolerances of the oracle; then the same call captured in a HIP graph
and replayed."""
import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import check_close, host64, log  # noqa: E402

from long_context_amd import kascade as K  # noqa: E402
from long_context_amd import synth  # noqa: E402
from long_context_amd.synth import to_oracle  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _w(name, wid, **kw):
    base = dict(name=name, wid=wid, phase="decode", batch=4, hq=32, hkv=8, d=128, n=8192, k=2048,
                tile=1, dtype="bf16", layers=2, planted=16, share=0.7)
    base.update(kw)
    return synth.Workload(**base)


# Several workgroups per (batch, KV head) whose partials sit in the library's
# scratch, then a smaller problem on the same scratch, then float32.
CALLS = [
    _w("noalloc_big", 980),
    _w("noalloc_small", 981, batch=1, hq=8, hkv=2, d=64, n=3000, k=700),
    _w("noalloc_f32", 982, batch=1, hq=4, hkv=1, d=128, n=1500, k=300, dtype="f32"),
]


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _noalloc(lib, q, k, v, idx, out):
    prob = K.problem(q, k, idx.shape[-1], 1)
    return lib.reuse_decode_noalloc_raw(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                        out.data_ptr(), _stream())


def test_noalloc_matches_the_workspace_entry_point(lib, orc):
    for w in CALLS:
        log(f"[noalloc] case={w.name} B={w.batch} Hq={w.hq} Hkv={w.hkv} d={w.d} N={w.n} k={w.k} {w.dtype}")
        (q0, k0, _), (q1, k1, v1) = synth.make_stack(w, device="cpu")
        q1d, k1d, v1d = q1.to(DEV), k1.to(DEV), v1.to(DEV)
        idx = K.anchor_decode(q0.to(DEV), k0.to(DEV), None, w.k)
        out_na = torch.empty_like(q1d)
        assert _noalloc(lib, q1d, k1d, v1d, idx, out_na) == K.OK
        out_ws = K.reuse_decode(q1d, k1d, v1d, idx)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), f"{w.name}: allocation-free output differs from the workspace call"
        ref = orc.reuse_decode(to_oracle(q1), to_oracle(k1), to_oracle(v1), idx.cpu().numpy())
        check_close(host64(out_na).reshape(-1, w.d), ref, w.torch_dtype, f"{w.name} against the oracle")


def test_noalloc_under_graph_capture(lib, orc):
    w = CALLS[0]
    log(f"[noalloc] case=graph_capture {w.name}")
    (q0, k0, _), (q1, k1, v1) = synth.make_stack(w, device="cpu")
    q1d, k1d, v1d = q1.to(DEV), k1.to(DEV), v1.to(DEV)
    idx = K.anchor_decode(q0.to(DEV), k0.to(DEV), None, w.k)
    out = torch.empty_like(q1d)
    assert _noalloc(lib, q1d, k1d, v1d, idx, out) == K.OK   # set-up outside the capture
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert _noalloc(lib, q1d, k1d, v1d, idx, out) == K.OK
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
