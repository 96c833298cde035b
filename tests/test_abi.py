"""The C ABI on the host: exports, validation, workspace sizing, argument errors.

No GPU is needed: every call here is rejected (or answered) by host code
before anything is enqueued, and no pointer passed here is dereferenced.
"""
import ctypes
import os
import re

import pytest

from long_context_amd import kascade as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kascade.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced by the checks exercised here


@pytest.fixture(scope="module")
def L():
    return K.library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(kascade_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    declared = _declared()
    assert declared == sorted(K.EXPORTS)
    for name in declared:
        assert hasattr(L.lib, name), name


def _prob(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, q_len=1, kv_len=4096,
                top_k=256, q_tile=128, scale=0.0, dtype=K.BF16)
    base.update(kw)
    return K.Problem(**base)


def _prefill(**kw):
    base = dict(q_len=1000, kv_len=1000)
    base.update(kw)
    return _prob(**base)


def test_validate_accepts_supported_problems(L):
    for dt in (K.F32, K.BF16):
        for d in (64, 128):
            assert L.validate(_prob(dtype=dt, head_dim=d), K.OP_ANCHOR_DECODE) == K.OK
            assert L.validate(_prob(dtype=dt, head_dim=d), K.OP_REUSE_DECODE) == K.OK
    for d in (64, 128):
        for tile in (64, 128):
            assert L.validate(_prefill(head_dim=d, q_tile=tile), K.OP_ANCHOR_PREFILL) == K.OK
            assert L.validate(_prefill(head_dim=d, q_tile=tile), K.OP_REUSE_PREFILL) == K.OK
    assert L.validate(_prob(top_k=4096), K.OP_ANCHOR_DECODE) == K.OK          # k = N
    assert L.validate(_prefill(top_k=5000), K.OP_ANCHOR_PREFILL) == K.OK      # k > N is fine in prefill
    assert L.validate(_prob(num_q_heads=32, num_kv_heads=2), K.OP_REUSE_DECODE) == K.OK  # G = 16


@pytest.mark.parametrize("kw,op,status", [
    (dict(num_q_heads=6, num_kv_heads=4), K.OP_REUSE_DECODE, K.ERR_INVALID),
    (dict(batch=0), K.OP_REUSE_DECODE, K.ERR_INVALID),
    (dict(top_k=0), K.OP_ANCHOR_DECODE, K.ERR_INVALID),
    (dict(top_k=4097), K.OP_ANCHOR_DECODE, K.ERR_INVALID),
    (dict(q_len=2), K.OP_REUSE_DECODE, K.ERR_INVALID),
    (dict(dtype=7), K.OP_REUSE_DECODE, K.ERR_INVALID),
    (dict(head_dim=96), K.OP_REUSE_DECODE, K.ERR_UNSUPPORTED),
    (dict(num_q_heads=34, num_kv_heads=2), K.OP_REUSE_DECODE, K.ERR_UNSUPPORTED),
    (dict(scale=float("nan")), K.OP_REUSE_DECODE, K.ERR_INVALID),
    (dict(q_len=1000, kv_len=999), K.OP_ANCHOR_PREFILL, K.ERR_INVALID),
    (dict(q_len=1000, kv_len=1000, dtype=K.F32), K.OP_ANCHOR_PREFILL, K.ERR_UNSUPPORTED),
    (dict(q_len=1000, kv_len=1000, q_tile=32), K.OP_REUSE_PREFILL, K.ERR_UNSUPPORTED),
    (dict(q_len=1000, kv_len=1000, q_tile=96), K.OP_ANCHOR_PREFILL, K.ERR_UNSUPPORTED),
    (dict(q_len=1000, kv_len=1000, q_tile=0), K.OP_REUSE_PREFILL, K.ERR_INVALID),
])
def test_validate_rejects(L, kw, op, status):
    assert L.validate(_prob(**kw), op) == status
    assert L.workspace_bytes(_prob(**kw), op) == 0


def test_validate_null_problem_and_bad_op(L):
    assert L.lib.kascade_validate(None, 0) == K.ERR_INVALID
    assert L.validate(_prob(), 9) == K.ERR_INVALID


def test_workspace_sizes(L):
    ad = L.workspace_bytes(_prob(), K.OP_ANCHOR_DECODE)
    rd = L.workspace_bytes(_prob(), K.OP_REUSE_DECODE)
    ap = L.workspace_bytes(_prefill(), K.OP_ANCHOR_PREFILL)
    rp = L.workspace_bytes(_prefill(), K.OP_REUSE_PREFILL)
    assert ad > 0 and rd > 0 and ap > 0 and rp == 0
    assert ad % 256 == 0 and rd % 256 == 0 and ap % 256 == 0
    # anchor decode holds at least the fp32 logits
    assert ad >= 4 * (2 * 8 * 4096)
    # past one 32768-key sub-segment it also holds the selection candidates:
    # per (b, KV head) and sub-segment, min(k, 32768) (score, key) pairs
    ws_k = {kk: L.workspace_bytes(_prob(kv_len=131072, top_k=kk), K.OP_ANCHOR_DECODE) for kk in (1024, 2048)}
    assert ws_k[2048] - ws_k[1024] == 2 * 2 * 4 * 1024 * 8          # B * Hkv * 4 sub-segments * 1024 * 8 B
    short = {kk: L.workspace_bytes(_prob(kv_len=32768, top_k=kk), K.OP_ANCHOR_DECODE) for kk in (1024, 2048)}
    assert short[2048] == short[1024]                              # one sub-segment: no candidates
    # anchor prefill holds the row lse and the ragged pooled scores
    tiles = -(-1000 // 128)
    ragged = 128 * (tiles - 1) * tiles // 2 + 1000
    assert ap >= 4 * (2 * 8 * 1000 + 2 * 2 * ragged)
    # 64-row tiles: twice the tiles, and a longer ragged layout
    ap64 = L.workspace_bytes(_prefill(q_tile=64), K.OP_ANCHOR_PREFILL)
    tiles = -(-1000 // 64)
    ragged64 = 64 * (tiles - 1) * tiles // 2 + 1000
    assert ap64 >= 4 * (2 * 8 * 1000 + 2 * 2 * ragged64) and ap64 > ap


def test_status_strings(L):
    for s in (K.OK, K.ERR_INVALID, K.ERR_UNSUPPORTED, K.ERR_WORKSPACE, K.ERR_HIP, K.ERR_SCRATCH):
        assert L.status_string(s) and L.status_string(s) != "unknown status"
    assert L.status_string(99) == "unknown status"


def test_entry_points_reject_before_launch(L):
    p = _prob()
    ws_ad = L.workspace_bytes(p, K.OP_ANCHOR_DECODE)
    ws_rd = L.workspace_bytes(p, K.OP_REUSE_DECODE)
    bad = _prob(num_q_heads=6, num_kv_heads=4)
    # invalid problem
    assert L.anchor_decode_raw(bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_ad, None) == K.ERR_INVALID
    assert L.reuse_decode_raw(bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_rd, None) == K.ERR_INVALID
    # null required pointers
    assert L.anchor_decode_raw(p, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_ad, None) == K.ERR_INVALID
    assert L.anchor_decode_raw(p, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, ws_ad, None) == K.ERR_INVALID
    assert L.reuse_decode_raw(p, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws_rd, None) == K.ERR_INVALID
    assert L.reuse_decode_raw(p, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_rd, None) == K.ERR_INVALID
    # misaligned tensors
    assert L.reuse_decode_raw(p, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, ws_rd, None) == K.ERR_INVALID
    assert L.reuse_decode_raw(p, FAKE, FAKE, FAKE, FAKE + 1, FAKE, FAKE, ws_rd, None) == K.ERR_INVALID
    # workspace missing, short or misaligned
    assert L.reuse_decode_raw(p, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws_rd, None) == K.ERR_WORKSPACE
    assert L.reuse_decode_raw(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_rd - 1, None) == K.ERR_WORKSPACE
    assert L.reuse_decode_raw(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, ws_rd, None) == K.ERR_WORKSPACE
    pp = _prefill()
    ws_ap = L.workspace_bytes(pp, K.OP_ANCHOR_PREFILL)
    # without an index buffer the anchor call is dense attention only: it needs out or lse
    assert L.anchor_prefill_raw(pp, FAKE, FAKE, FAKE, None, None, None, FAKE, ws_ap, None) == K.ERR_INVALID
    assert L.anchor_decode_raw(p, FAKE, FAKE, FAKE, None, None, None, FAKE, ws_ad, None) == K.ERR_INVALID
    assert L.anchor_prefill_raw(pp, FAKE, FAKE, None, FAKE, None, None, FAKE, ws_ap, None) == K.ERR_INVALID
    assert L.anchor_decode_raw(p, FAKE, FAKE, FAKE, FAKE, None, FAKE + 1, FAKE, ws_ad, None) == K.ERR_INVALID
    assert L.anchor_prefill_raw(pp, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_ap - 256, None) == K.ERR_WORKSPACE
    assert L.reuse_prefill_raw(pp, FAKE, FAKE, None, FAKE, FAKE, None, 0, None) == K.ERR_INVALID
    assert L.reuse_prefill_raw(_prefill(dtype=K.F32), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == K.ERR_UNSUPPORTED


def test_shared_index_set_flag(L):
    """One index set for all heads: 0 and 1 are the only valid values; the
    prefill anchor needs room for the summed rows, decode needs nothing more."""
    for op in range(4):
        mk = _prob if op in (K.OP_ANCHOR_DECODE, K.OP_REUSE_DECODE) else _prefill
        assert L.validate(mk(shared_index_set=1), op) == K.OK
        assert L.validate(mk(shared_index_set=2), op) == K.ERR_INVALID
        assert L.validate(mk(shared_index_set=-1), op) == K.ERR_INVALID
    # the shared decode anchor keeps one pooled row per batch row (B x N floats)
    assert L.workspace_bytes(_prob(shared_index_set=1), K.OP_ANCHOR_DECODE) == \
        L.workspace_bytes(_prob(), K.OP_ANCHOR_DECODE) + 2 * 4096 * 4
    ragged = 128 * 7 * 8 // 2 + 1000           # 8 tiles of 128 over N = 1000
    grow = L.workspace_bytes(_prefill(shared_index_set=1), K.OP_ANCHOR_PREFILL) - \
        L.workspace_bytes(_prefill(), K.OP_ANCHOR_PREFILL)
    assert grow >= 2 * ragged * 4 and grow < 2 * ragged * 4 + 256
    assert L.validate(_prob(batch=65536, num_q_heads=1, num_kv_heads=1, kv_len=16, top_k=4),
                      K.OP_ANCHOR_DECODE) == K.ERR_UNSUPPORTED


def test_binding_checks_index_set_shape():
    """The binding refuses an idx whose shape does not match the problem
    before any call reaches the library (host tensors: nothing is launched)."""
    import torch
    q = torch.zeros((2, 8, 1, 128), dtype=torch.bfloat16)
    k = torch.zeros((2, 2, 300, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="idx must be int32"):
        K.reuse_decode(q, k, k, torch.zeros((2, 1, 1, 16), dtype=torch.int32))            # per-KV-head expected
    with pytest.raises(ValueError, match="idx must be int32"):
        K.reuse_decode(q, k, k, torch.zeros((2, 2, 1, 16), dtype=torch.int32), shared=True)
    with pytest.raises(ValueError, match="idx must be int32"):
        K.reuse_decode(q, k, k, torch.zeros((2, 2, 1, 16), dtype=torch.int64))
    qp = torch.zeros((1, 8, 300, 128), dtype=torch.bfloat16)
    kp = torch.zeros((1, 2, 300, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="idx must be int32"):
        K.reuse_prefill(qp, kp, kp, torch.zeros((1, 2, 2, 16), dtype=torch.int32))         # 3 tiles expected
    assert K.idx_shape(K.problem(qp, kp, 16, 128, shared=True)) == (1, 1, 3, 16)


def test_noalloc_rejects_before_launch(L):
    """The allocation-free reuse decode refuses, on the host, a problem whose
    workspace exceeds its scratch, and the usual argument errors."""
    big = _prob(batch=512, num_q_heads=32, num_kv_heads=8, kv_len=32768, top_k=2048)
    assert L.workspace_bytes(big, K.OP_REUSE_DECODE) > K.NOALLOC_SCRATCH_BYTES
    assert L.reuse_decode_noalloc_raw(big, FAKE, FAKE, FAKE, FAKE, FAKE, None) == K.ERR_SCRATCH
    p = _prob()
    assert L.workspace_bytes(p, K.OP_REUSE_DECODE) <= K.NOALLOC_SCRATCH_BYTES
    assert L.reuse_decode_noalloc_raw(_prob(num_q_heads=6, num_kv_heads=4), FAKE, FAKE, FAKE, FAKE, FAKE,
                                      None) == K.ERR_INVALID
    assert L.reuse_decode_noalloc_raw(p, FAKE, FAKE, None, FAKE, FAKE, None) == K.ERR_INVALID
    assert L.reuse_decode_noalloc_raw(p, FAKE, FAKE, FAKE, FAKE + 1, FAKE, None) == K.ERR_INVALID
