"""Comparison rules between the GPU library and the fp64 oracle.

Floating point outputs:
  * float32 inputs: per output row, |gpu - ref| <= 1e-5 |ref| + 1e-5 max|ref_row|
    (a purely elementwise relative test is meaningless for entries near 0,
    and O is an average of zero-mean values); and the pure relative error
    |gpu - ref| / |ref| <= 1e-5 on the entries with |ref| >= FP32_REL_FLOOR
    times their row's largest magnitude.
  * bfloat16 inputs, float32 accumulation: |gpu - ref| <= 2e-2 + 2e-2 |ref|.
Anchor index sets (exact top-k):
  * exactly k_t distinct entries in [0, prefix), ascending, -1 afterwards;
  * every key in the symmetric difference with the oracle's set has an oracle
    pooled score within 1e-3 relative of the oracle's k_t-th largest score
    (near-ties may legitimately fall either way under float32 arithmetic).
"""
import sys

import numpy as np
import torch


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host64(t):
    return t.detach().to("cpu").double().numpy()


# fp32: the pure relative error |gpu - ref| / |ref| is also bounded by 1e-5 on
# the entries whose magnitude is at least this share of their row's largest.
FP32_REL_FLOOR = 0.25


def check_close(gpu, ref, dtype, what):
    a = np.asarray(gpu, np.float64).reshape(ref.shape)
    b = np.asarray(ref, np.float64)
    err = np.abs(a - b)
    if dtype == torch.float32:
        rowmax = np.abs(b).max(axis=-1, keepdims=True)
        lim = 1e-5 * np.abs(b) + 1e-5 * rowmax
    else:
        lim = 2e-2 + 2e-2 * np.abs(b)
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance, "
                           f"max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
    if dtype == torch.float32:
        big = np.abs(b) >= FP32_REL_FLOOR * rowmax
        rel = float((err[big] / np.abs(b[big])).max()) if big.any() else 0.0
        log(f"{what}: fp32 relative error {rel:.2e} on the {int(big.sum())} entries with "
            f"|ref| >= {FP32_REL_FLOOR} max|ref_row|")
        assert rel <= 1e-5, f"{what}: fp32 relative error {rel:.3e} above 1e-5 on large entries"
    return float(err.max())


def check_lse(gpu, ref, what):
    a = np.asarray(gpu, np.float64).reshape(ref.shape)
    err = np.abs(a - ref)
    lim = 1e-4 + 1e-5 * np.abs(ref)
    assert (err <= lim).all(), f"{what}: lse max err {err.max():.3e}"


def check_index_band(gpu_row, orc_row, orc_pooled, kt, n_cand, what, rel=1e-3):
    """Compare one anchor index row; returns True when the sets are identical."""
    gpu_row = np.asarray(gpu_row)
    k = len(gpu_row)
    sel = gpu_row[:kt]
    assert np.all(gpu_row[kt:] == -1), f"{what}: padding"
    assert np.all(sel >= 0) and np.all(sel < n_cand), f"{what}: index out of range"
    assert np.all(np.diff(sel) > 0), f"{what}: not strictly ascending"
    ref = set(np.asarray(orc_row[:kt]).tolist())
    got = set(sel.tolist())
    diff = ref ^ got
    if not diff:
        return True
    pk = min(orc_pooled[j] for j in ref)
    far = [j for j in diff if abs(orc_pooled[j] - pk) > rel * pk]
    assert not far, (f"{what}: {len(diff)} keys differ, {len(far)} outside the 1e-3 band "
                     f"(k={k}, kt={kt}, e.g. key {far[0]} score {orc_pooled[far[0]]:.6e} vs kth {pk:.6e})")
    return False


def random_index_sets(rng, shape, limits, k):
    """Seeded ascending index lists with -1 padding, for units no check reads."""
    out = np.full(shape + (k,), -1, np.int32)
    flat = out.reshape(-1, k)
    lim = np.broadcast_to(np.asarray(limits), shape).reshape(-1)
    for u in range(flat.shape[0]):
        n = int(lim[u])
        kt = min(k, n)
        flat[u, :kt] = np.sort(rng.choice(n, size=kt, replace=False))
    return out
