"""Benchmark of the Kascade hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * decode at 32K context, Llama-3-8B attention shape (B=16, Hq=32, Hkv=8,
    d=128, k=2048, bf16): one anchor layer (dense scores, pooled top-k, dense
    output) and three reuse layers with their own K/V;
  * causal prefill at 8K (B=1, Hq=32, Hkv=8, d=128, T=128, k=1024, bf16): one
    anchor layer (row log-sum-exp and dense output, pooled tile scores, per
    tile top-k) and three reuse layers.
All inputs are resident in HBM before timing starts. The step is timed as HIP
graph replays (the same kernels, without host launch gaps); an eager pass
gives per-call times and, through the library's per-kernel HIP events, the
per-kernel times behind the roofline. Prints one JSON line.

value = decode attention microseconds per layer (mean of the four decode
layers); the decode reuse-layer HBM rate and the prefill tokens/s sit beside it.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

from long_context_amd import kascade as K
from long_context_amd import synth

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, vendor figure
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, vendor figure

METRIC = "decode attn µs/layer + HBM GB/s at 32K ctx; prefill attn tokens/s at 8K"

ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_decode32k_prefill8k.txt")
CSRC = os.path.join(ROOT, "long_context_amd", "csrc")
# library timing name -> the source files that hold its kernel
KERNEL_SOURCE = {
    "decode_attn_dense": ("decode.hip",), "decode_attn_gather": ("decode.hip",),
    "decode_combine": ("decode.hip",), "topk_decode": ("topk.hip",), "topk_prefill": ("topk.hip",),
    "prefill_dense": ("prefill.hip", "lds_stage.hpp"), "prefill_pool": ("prefill.hip", "lds_stage.hpp"),
    "prefill_gather": ("prefill_gather.hip", "prefill.hip", "lds_stage.hpp"),
}


def kernel_source_digest(name):
    """sha256 (first 16 hex digits) over the kernel's source file, the shared
    device headers and the build flags: a change to any of them makes stored
    counter readings stale."""
    h = hashlib.sha256()
    for path in (*[os.path.join(CSRC, f) for f in KERNEL_SOURCE[name]], os.path.join(CSRC, "device_common.hpp"),
                 os.path.join(CSRC, "kernels.hpp"), os.path.join(ROOT, "long_context_amd", "build.py")):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(name):
    """HBM bytes per launch of kernel `name` from the committed FETCH_SIZE /
    WRITE_SIZE summary, or None when there is none or its source changed since."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    marker = "--- per-launch traffic (json) ---"
    if marker not in text:
        return None
    table = json.loads(text.split(marker, 1)[1])
    entry = table.get("kernels", {}).get(name)
    if entry is None or entry.get("source_digest") != kernel_source_digest(name):
        return None
    return entry["hbm_bytes_per_launch"]


def bytes_of(*ts):
    return sum(t.numel() * t.element_size() for t in ts)


class DecodeStack:
    def __init__(self, w, dev):
        self.w = w
        pos = synth.planted_positions(w)
        self.layers = [synth.make_layer(w, l, dev, pos) for l in range(w.layers)]
        q0, k0, v0 = self.layers[0]
        self.out = [torch.empty_like(q) for q, _, _ in self.layers]
        self.lse = torch.empty((w.batch, w.hq, 1), dtype=torch.float32, device=dev)
        self.idx = torch.empty((w.batch, w.hkv, 1, w.k), dtype=torch.int32, device=dev)
        self.ws_a = K.workspace(K.problem(q0, k0, w.k, 1), K.OP_ANCHOR_DECODE, dev)
        self.ws_r = K.workspace(K.problem(q0, k0, w.k, 1), K.OP_REUSE_DECODE, dev)

    def run(self, marks=None):
        q, k, v = self.layers[0]
        K.anchor_decode(q, k, v, self.w.k, out=self.out[0], lse=self.lse, idx=self.idx, ws=self.ws_a)
        if marks is not None:
            marks.append(("decode_anchor", _record()))
        for l in range(1, len(self.layers)):
            q, k, v = self.layers[l]
            K.reuse_decode(q, k, v, self.idx, out=self.out[l], ws=self.ws_r)
            if marks is not None:
                marks.append(("decode_reuse", _record()))

    def run_dense(self):
        """Dense attention in every layer (the anchor call without an index buffer)."""
        for l, (q, k, v) in enumerate(self.layers):
            K.anchor_decode(q, k, v, self.w.k, out=self.out[l], ws=self.ws_a, dense_only=True)

    def reuse_bytes(self):
        """Algorithmic bytes of one reuse layer: gathered K and V rows, idx, Q and O."""
        w = self.w
        rows = w.batch * w.hkv * w.k
        q, _, _ = self.layers[1]
        return rows * w.d * 2 * 2 + self.idx.numel() * 4 + 2 * bytes_of(q)

    def anchor_bytes(self):
        """Algorithmic bytes of the anchor: K and V read once (dense output requested)."""
        _, k, v = self.layers[0]
        return bytes_of(k, v)


class PrefillStack:
    def __init__(self, w, dev):
        self.w = w
        pos = synth.planted_positions(w)
        self.layers = [synth.make_layer(w, l, dev, pos) for l in range(w.layers)]
        q0, k0, _ = self.layers[0]
        self.out = [torch.empty_like(q) for q, _, _ in self.layers]
        self.idx = torch.empty((w.batch, w.hkv, w.tiles, w.k), dtype=torch.int32, device=dev)
        self.ws_a = K.workspace(K.problem(q0, k0, w.k, w.tile), K.OP_ANCHOR_PREFILL, dev)

    def run(self, marks=None):
        q, k, v = self.layers[0]
        K.anchor_prefill(q, k, v, self.w.k, self.w.tile, out=self.out[0], idx=self.idx, ws=self.ws_a)
        if marks is not None:
            marks.append(("prefill_anchor", _record()))
        for l in range(1, len(self.layers)):
            q, k, v = self.layers[l]
            K.reuse_prefill(q, k, v, self.idx, self.w.tile, out=self.out[l])
            if marks is not None:
                marks.append(("prefill_reuse", _record()))

    def run_dense(self):
        """Dense causal attention in every layer (no pooled scores, no selection)."""
        for l, (q, k, v) in enumerate(self.layers):
            K.anchor_prefill(q, k, v, self.w.k, self.w.tile, out=self.out[l], ws=self.ws_a, dense_only=True)

    def qk_flops(self):
        """Tile-granular causal QK^T flops of one pass over the sequence:
        every tile's G*T rows against its whole prefix of keys."""
        w = self.w
        total = 0
        for t in range(w.tiles):
            rows = min(w.tile, w.n - t * w.tile)
            total += w.batch * w.hq * rows * min((t + 1) * w.tile, w.n) * 2 * w.d
        return total

    def reuse_flops(self):
        """Tile-granular QK^T plus PV flops of one reuse layer over the saved sets."""
        w = self.w
        total = 0
        for t in range(w.tiles):
            rows = min(w.tile, w.n - t * w.tile)
            total += w.batch * w.hq * rows * min(w.k, (t + 1) * w.tile, w.n) * 2 * w.d * 2
        return total


def _event():
    return torch.cuda.Event(enable_timing=True)


def _record():
    e = _event()
    e.record()
    return e


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return time.perf_counter() - t0, r


def cpu_baseline(dec, pre, threads, prefill_tiles=96, prefill_rows=8192):
    """The fp64 oracle, as it stands, timed on the host cores.

    Each op is one oracle call over all its units, so the oracle's OpenMP loop
    spreads them over `threads` threads (the count reported is what its
    parallel region actually ran with).
      * decode 32K: the whole anchor layer (pooled top-k over all B*Hkv units,
        dense output and lse over all B*Hq rows) and one whole reuse layer over
        the anchor's sets -- measured, not extrapolated; value = the mean of
        one anchor and three reuse layers, us per layer, like the GPU figure;
      * prefill 8K: the anchor's pooled top-k on `prefill_tiles` seeded
        (KV head, tile) pairs, dense output and lse on `prefill_rows` seeded
        rows, reuse on `prefill_rows` seeded rows; each scaled to the whole
        layer by its per-unit cost (keys visited times heads, rows or d),
        so the prefill figure is an extrapolation and is labelled so;
      * a single-thread run of one decode unit gives the per-core rate."""
    import oracle
    orc = oracle.default()
    used = orc.threads(threads)
    w = dec.w
    G = w.group
    q0, k0, v0 = (synth.to_oracle(t) for t in dec.layers[0])
    t_sel, (io, _) = _timed(lambda: orc.anchor_decode(q0, k0, w.k, threads=threads, want_pooled=False))
    t_dense, _ = _timed(lambda: orc.dense(q0, k0, v0, causal=False, threads=threads))
    t_one, _ = _timed(lambda: orc.anchor_decode(q0[:1, :G], k0[:1, :1], w.k, threads=1, want_pooled=False))
    t_one_d, _ = _timed(lambda: orc.dense(q0[:1, :G], k0[:1, :1], v0[:1, :1], causal=False, threads=1))
    del k0, v0
    q1, k1, v1 = (synth.to_oracle(t) for t in dec.layers[1])
    idx = io.reshape(w.batch, w.hkv, 1, w.k)
    t_reuse, _ = _timed(lambda: orc.reuse_decode(q1, k1, v1, idx, threads=threads))
    del q1, k1, v1
    anchor_s = t_sel + t_dense
    dec_us = (anchor_s + (w.layers - 1) * t_reuse) / w.layers * 1e6

    # prefill: sampled units, scaled to the layer by cost
    wp = pre.w
    T, tiles = wp.tile, wp.tiles
    P0, K0, V0 = (synth.to_oracle(t) for t in pre.layers[0])
    rng = np.random.default_rng(11)
    prefix = np.minimum((np.arange(tiles) + 1) * T, wp.n)
    rows_t = prefix - np.arange(tiles) * T
    pairs = np.array([(0, i % wp.hkv, t) for i, t in enumerate(rng.choice(tiles, prefill_tiles))], np.int32)
    t_pool, (ip, _) = _timed(lambda: orc.anchor_prefill(P0, K0, wp.k, T, units=pairs, threads=threads,
                                                        want_pooled=False))
    # pooled work of a tile ~ G * rows * prefix; the layer holds every (KV head, tile)
    cost_tile = G * rows_t * prefix
    pool_layer = t_pool * (wp.hkv * cost_tile.sum()) / cost_tile[pairs[:, 2]].sum()
    flat = rng.choice(wp.hq * wp.n, prefill_rows, replace=False)
    rows = np.stack([np.zeros(prefill_rows, np.int64), flat // wp.n, flat % wp.n], 1).astype(np.int32)
    t_pd, _ = _timed(lambda: orc.dense(P0, K0, V0, causal=True, units=rows, threads=threads))
    # dense work of row i ~ i + 1 keys
    dense_layer = t_pd * (wp.hq * (wp.n * (wp.n + 1) / 2)) / (rows[:, 2] + 1).sum()
    del P0, K0, V0
    P1, K1, V1 = (synth.to_oracle(t) for t in pre.layers[1])
    idxp = pre.idx.cpu().numpy()
    t_pr, _ = _timed(lambda: orc.reuse_prefill(P1, K1, V1, idxp, T, units=rows, threads=threads))
    # reuse work of row i ~ keys of its tile's set at or below i
    kept = (idxp[0][:, :, None, :] >= 0) & (idxp[0][:, :, None, :] <= np.arange(T)[None, None, :, None]
                                             + (np.arange(tiles) * T)[None, :, None, None])
    per_row = kept.sum(-1).reshape(wp.hkv, tiles * T)[:, :wp.n]          # [Hkv, N]
    row_cost = np.repeat(per_row, G, axis=0)                             # [Hq, N]
    reuse_layer = t_pr * row_cost.sum() / max(1, row_cost[rows[:, 1], rows[:, 2]].sum())
    del P1, K1, V1
    pre_anchor_s = pool_layer + dense_layer
    pre_tps = wp.batch * wp.n * wp.layers / (pre_anchor_s + (wp.layers - 1) * reuse_layer)
    return {
        "value": round(dec_us, 1), "unit": "us/layer", "cores": used, "kind": "oracle",
        "sample": (f"decode 32K: whole layers -- anchor top-k over all {w.batch * w.hkv} (batch, KV head) "
                   f"units and dense output/lse over all {w.batch * w.hq} rows, one reuse layer over all "
                   f"rows -- mean of 1 anchor + {w.layers - 1} reuse layers; prefill 8K: {prefill_tiles} "
                   f"(KV head, tile) anchor sets and {prefill_rows} rows each of dense and reuse attention, "
                   "scaled to whole layers by per-unit cost (extrapolated)"),
        "cpu_model": _cpu_model(),
        "threads_requested": threads,
        "decode_anchor_layer_s": round(anchor_s, 3),
        "decode_reuse_layer_s": round(t_reuse, 4),
        "decode_per_core_us_per_unit": round((t_one + t_one_d) * 1e6, 1),
        "decode_per_core_note": ("one (batch, KV head) unit of the anchor layer (top-k of its 4 heads plus their "
                                 "dense output) on one thread"),
        "prefill_tokens_per_s": round(pre_tps, 2),
        "prefill_tokens_per_s_kind": "extrapolated from the sampled units",
        "prefill_anchor_layer_s": round(pre_anchor_s, 2),
        "prefill_reuse_layer_s": round(reuse_layer, 2),
    }


def profile_pass(kind, reps, workloads=("decode_llama8b_32k", "prefill_8k")):
    """Short runs for hardware-counter and kernel-trace passes under rocprofv3.

    copy:    one plain elementwise kernel that reads 1 GiB and writes 1 GiB
             (negation of fp32), the known-size reference for FETCH_SIZE and
             WRITE_SIZE;
    kernels: `reps` eager passes of the layer stacks of `workloads` (by
             default the benchmark's decode and prefill stacks).
    """
    dev = "cuda"
    if kind == "copy":
        a = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": "copy", "read_bytes": 1 << 30, "write_bytes": 1 << 30}))
        return
    stacks = []
    for name in workloads:
        w = synth.WORKLOADS[name]
        stacks.append((DecodeStack if w.phase == "decode" else PrefillStack)(w, dev))
    torch.cuda.synchronize()
    for _ in range(reps):
        for st in stacks:
            st.run()
    torch.cuda.synchronize()
    print(json.dumps({"profile_pass": "kernels", "reps": reps, "workloads": list(workloads)}), flush=True)


def probe_mix(iters=4096, reps=3):
    """Vector/matrix overlap of the prefill kernels' inner mixes on registers
    and LDS only (long_context_amd/csrc/probe/mix_probe.hip): the pooled pass's
    16-row block at one to six wavefronts per SIMD, and the attention step with
    operands one step ahead or just in time, with no synchronisation, a
    workgroup barrier per step, or an LDS-counter wait that allows one step of
    slack, and once with K resident in registers. The grid puts the given number of wavefronts on each of the 1024
    SIMDs. Times are HIP events around each launch (median of `reps`, after a
    warm-up that brings the clock up); under rocprofv3 --kernel-trace the
    dispatches give the kernel durations. One JSON line per configuration."""
    import ctypes
    from long_context_amd import build as B
    lib = ctypes.CDLL(B.PROBE_LIBRARY)
    lib.kascade_probe_mix.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 2
    lib.kascade_probe_mix.restype = ctypes.c_int
    out = torch.empty(256 * 256 * 6, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    mfma_flops = {("pool", 128): 16 * 16 * 16 * 32 * 2, ("pool", 64): 8 * 16 * 16 * 32 * 2,
                  ("attn", 128): 16 * 32 * 32 * 16 * 2, ("attn", 64): 8 * 32 * 32 * 16 * 2}
    modes = {0: "operands one step ahead", 1: "ahead + barrier per step", 2: "just in time + barrier per step",
             3: "ahead + LDS-counter wait, one step of slack", 4: "ahead, K resident (V^T the only LDS reads)"}
    configs = [("pool", 0, d, wps) for d in (128, 64) for wps in range(1, 7)]
    configs += [("attn", m, 128, wps) for m, wps in ((0, 2), (1, 2), (2, 2), (2, 3), (3, 2), (4, 2))]
    configs += [("attn", m, 64, 3) for m in (0, 1, 2, 3, 4)]

    def launch(kind, mode, d, wps):
        rc = lib.kascade_probe_mix(0 if kind == "pool" else 1, mode, d, wps, iters, out.data_ptr(), stream)
        assert rc == 0, (kind, mode, d, wps, rc)

    for _ in range(20):  # clock warm-up
        launch("pool", 0, 128, 4)
    torch.cuda.synchronize()
    for kind, mode, d, wps in configs:
        launch(kind, mode, d, wps)
        times = []
        for _ in range(reps):
            a, b = _event(), _event()
            a.record()
            launch(kind, mode, d, wps)
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        t = float(np.median(times))
        waves = 256 * wps * 4
        frac = waves * iters * mfma_flops[(kind, d)] / t / (PEAK_BF16_TFLOPS * 1e12)
        row = {"probe": "mix", "kind": kind, "d": d, "waves_per_simd": wps, "ms": round(t * 1e3, 3),
               "of_bf16_peak": round(frac, 3)}
        if kind == "attn":
            row["mode"] = modes[mode]
        print(json.dumps(row), flush=True)


def probe_gather(reps=5, workload="decode_llama8b_32k"):
    """Cold-cache memory ceiling of the decode reuse layer's access pattern.

    A load-only probe (long_context_amd/csrc/probe/gather_probe.hip) reads the
    K and V rows that the anchor's index sets name -- the reuse gather's bytes
    without its arithmetic -- and the same number of rows read contiguously,
    over a sweep of wavefronts per (batch, KV head) and of row groups in
    flight per wavefront. Before every timed launch a 2 GiB buffer is read,
    which fills the 256 MB Infinity Cache with unrelated clean lines (a
    written flush would leave dirty lines to be written back during the timed
    kernel). The reuse call itself is timed the same way. Times are HIP events
    around the one launch; under rocprofv3 --kernel-trace the dispatches give
    the kernel durations alone. One JSON line per configuration, then a
    summary line."""
    import ctypes
    from long_context_amd import build as B
    lib = ctypes.CDLL(B.PROBE_LIBRARY)
    lib.kascade_probe_gather.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 6 + [ctypes.c_void_p] * 2
    lib.kascade_probe_gather.restype = ctypes.c_int
    dev = "cuda"
    w = synth.WORKLOADS[workload].scaled(layers=2)
    pos = synth.planted_positions(w)
    q0, k0, _ = synth.make_layer(w, 0, dev, pos)
    q1, k1, v1 = synth.make_layer(w, 1, dev, pos)
    idx = K.anchor_decode(q0, k0, None, w.k)
    del q0, k0
    units = w.batch * w.hkv
    assert w.d == 128 and k1.dtype == torch.bfloat16  # 256-byte rows
    flush = torch.ones((2 << 30) // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    gather_bytes = units * w.k * w.d * 2 * 2

    def cold(launch):
        times = []
        for _ in range(reps):
            flush.sum()
            torch.cuda.synchronize()
            a, b = _event(), _event()
            a.record()
            launch()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3)
        return float(np.median(times))

    out = torch.empty_like(q1)
    ws = K.workspace(K.problem(q1, k1, w.k, 1), K.OP_REUSE_DECODE, dev)
    t_reuse = cold(lambda: K.reuse_decode(q1, k1, v1, idx, out=out, ws=ws))
    rows = []
    for contiguous in (0, 1):
        for splits in (8, 16, 32, 64):
            for inflight in (1, 2, 4, 8):
                def launch():
                    rc = lib.kascade_probe_gather(k1.data_ptr(), v1.data_ptr(), idx.data_ptr(), units, w.n, w.k,
                                                  splits, inflight, contiguous, sink.data_ptr(), stream)
                    assert rc == 0, rc
                t = cold(launch)
                row = {"probe": "gather_ceiling", "workload": w.name, "rows": "contiguous" if contiguous else "gathered",
                       "waves_per_unit": splits, "row_groups_in_flight": inflight, "us": round(t, 2),
                       "gbs": round(gather_bytes / (t * 1e-6) / 1e9, 1)}
                rows.append(row)
                print(json.dumps(row), flush=True)
    best = {kind: max((r for r in rows if r["rows"] == kind), key=lambda r: r["gbs"]) for kind in ("gathered", "contiguous")}
    print(json.dumps({"probe": "gather_ceiling_summary", "workload": w.name, "bytes": gather_bytes,
                      "reuse_call_cold_us": round(t_reuse, 2),
                      "reuse_call_cold_gbs": round(dec_reuse_bytes(w) / (t_reuse * 1e-6) / 1e9, 1),
                      "best_gathered": best["gathered"], "best_contiguous": best["contiguous"],
                      "peak_gbs": PEAK_HBM_GBS}), flush=True)


def dec_reuse_bytes(w):
    """Algorithmic bytes of one decode reuse layer: gathered K and V rows, idx, Q and O."""
    esz = 4 if w.dtype == "f32" else 2
    return (w.batch * w.hkv * w.k * w.d * esz * 2 + w.batch * w.hkv * w.k * 4
            + 2 * w.batch * w.hq * w.d * esz)


# ---- accuracy against dense attention, swept over k -------------------------
#
# The pages leave k as a hyper-parameter picked with a small validation sweep
# (euno.news summary, "Limitations & Future Work") and fix the prefill
# selection to tiles (Kascade abstract, opentrain.ai page). This sweep runs the
# path at k = N/64 ... N/4 over a stack of synthetic layers whose planted heavy
# keys drift from layer to layer, and reports per layer how well the anchor's
# index set serves it against that layer's own dense attention.

SWEEP_K_FRACTIONS = (64, 32, 16, 8, 4)     # k = N / f


def pooled_decode(q, k):
    """Group-mean post-softmax attention of each KV head's decode queries over
    all keys, float32 [B, Hkv, N]."""
    B, Hq, _, d = q.shape
    Hkv = k.shape[1]
    qf = q.float().reshape(B, Hkv, Hq // Hkv, d)
    kt = k.float().transpose(2, 3).contiguous()
    return torch.softmax(torch.matmul(qf, kt) / math.sqrt(d), dim=-1).mean(dim=2)


def pooled_prefill(q, k, tile):
    """Causal post-softmax attention averaged over each query tile's rows and
    the group's heads, float32 [B, Hkv, tiles, N]; row t sums to 1."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    tiles = -(-N // tile)
    tile_of_row = torch.arange(N, device=q.device) // tile
    rows = torch.bincount(tile_of_row, minlength=tiles).float()
    future = torch.ones((N, N), dtype=torch.bool, device=q.device).triu(1)
    out = torch.zeros((B, Hkv, tiles, N), dtype=torch.float32, device=q.device)
    for b in range(B):
        for kv in range(Hkv):
            s = torch.matmul(q[b, kv * G:(kv + 1) * G].float(), k[b, kv].float().t().contiguous())
            s = (s / math.sqrt(d)).masked_fill_(future, float("-inf"))
            p = torch.softmax(s, dim=-1).sum(0)
            out[b, kv].index_add_(0, tile_of_row, p)
            del s, p
    return out / (G * rows)[None, None, :, None]


def captured_mass(pooled, idx):
    """Mean over index sets of the pooled attention mass the set holds
    (entries -1 hold none). pooled [..., N], idx [..., k]; a shared set
    (idx [B, 1, ...]) is scored against every KV head's pooled row."""
    idx = idx.expand(*pooled.shape[:-1], idx.shape[-1])
    take = pooled.gather(-1, idx.long().clamp_min(0)) * (idx >= 0)
    return float(take.sum(-1).mean())


def planted_recall(positions, idx, tile, n):
    """Mean over (b, KV head, tile) of the fraction of planted keys inside the
    tile's causal prefix that the index set holds. positions[b][kv] are one
    layer's planted rows; idx [B, S, tiles, k] on the host, S = Hkv or 1 (a
    set shared by all heads)."""
    fr = []
    for b, per_kv in enumerate(positions):
        for kv, pos in enumerate(per_kv):
            s = kv if idx.shape[1] > 1 else 0
            for t in range(idx.shape[2]):
                live = pos[pos < min((t + 1) * tile, n)] if idx.shape[2] > 1 else pos
                if live.size:
                    fr.append(np.isin(live, idx[b, s, t]).mean())
    return float(np.mean(fr))


def rel_error(out, ref):
    """Frobenius-norm error of `out` relative to `ref`, in float32."""
    o, r = out.float(), ref.float()
    return float(torch.linalg.vector_norm(o - r) / torch.linalg.vector_norm(r))


def accuracy_sweep(w, fractions=SWEEP_K_FRACTIONS, dev="cuda", shared=(False, True)):
    """For each k = N/f: the anchor (layer 0) selects its index sets once, then
    every layer of the stack (the anchor itself included) attends through the
    reuse call to those sets with its own Q, K and V. Per layer: planted-key
    recall, captured pooled attention mass, and the output's error relative to
    the layer's dense attention. With shared=(False, True) both head-aware sets
    ("layers") and one set shared by all heads ("shared_set_layers", the
    ablation) are measured. Returns one dict per k."""
    decode = w.phase == "decode"
    pos = synth.planted_positions(w)
    layers = [synth.make_layer(w, l, dev, pos) for l in range(w.layers)]
    dense, pooled = [], []
    for q, k, v in layers:
        o = torch.empty_like(q)
        if decode:
            K.anchor_decode(q, k, v, min(w.k, w.n), out=o)
            pooled.append(pooled_decode(q, k).unsqueeze(2))
        else:
            K.anchor_prefill(q, k, v, min(w.k, w.n), w.tile, out=o)
            pooled.append(pooled_prefill(q, k, w.tile))
        dense.append(o)
    rows = []
    q0, k0, v0 = layers[0]
    for f in fractions:
        kk = max(1, w.n // f)
        row = {"sweep": "accuracy_vs_k", "workload": w.name, "phase": w.phase, "n": w.n,
               "q_tile": w.tile if not decode else None, "top_k": kk, "k_over_n": f"1/{f}",
               "share": w.share, "gain": w.gain}
        for sh in shared:
            if decode:
                idx = K.anchor_decode(q0, k0, v0, kk, shared=sh)
            else:
                idx = K.anchor_prefill(q0, k0, v0, kk, w.tile, shared=sh)
            idx_host = idx.cpu().numpy()
            per_layer = []
            for l, (q, k, v) in enumerate(layers):
                if decode:
                    o = K.reuse_decode(q, k, v, idx, shared=sh)
                else:
                    o = K.reuse_prefill(q, k, v, idx, w.tile, shared=sh)
                per_layer.append({
                    "layer": l,
                    "planted_recall": round(planted_recall(pos[l], idx_host, w.tile, w.n), 4),
                    "attention_mass": round(captured_mass(pooled[l], idx), 4),
                    "rel_error_vs_dense": round(rel_error(o, dense[l]), 5),
                })
            row["shared_set_layers" if sh else "layers"] = per_layer
        rows.append(row)
    torch.cuda.synchronize()
    return rows


def sweep_workloads():
    """The decode workload at 32K and the 8K prefill workload, the latter with
    its planted keys drifting like the decode one's (70 % kept from layer to
    layer) so the reuse layers meet new heavy keys, and with 128- and 64-row
    selection tiles; each at the benchmarked planted-row gain (diffuse
    attention) and at gain 16 (most of the attention on the planted keys)."""
    dec = synth.WORKLOADS["decode_llama8b_32k"]
    pre = synth.WORKLOADS["prefill_8k"].scaled(share=0.7)
    pre64 = pre.scaled(tile=64)
    return [dec, dec.scaled(gain=16.0), pre, pre.scaled(gain=16.0), pre64, pre64.scaled(gain=16.0)]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-pass", choices=("copy", "kernels"),
                    help="run a short pass for rocprofv3 counters instead of the benchmark")
    ap.add_argument("--profile-workloads", default="decode_llama8b_32k,prefill_8k",
                    help="comma-separated synthetic workloads for --profile-pass kernels")
    ap.add_argument("--probe", choices=("gather", "mix"),
                    help="gather: cold-cache memory ceiling of the decode reuse gather (load-only probe "
                         "sweep); mix: vector/matrix overlap of the prefill kernels' inner mixes")
    ap.add_argument("--probe-workload", default="decode_llama8b_32k")
    ap.add_argument("--sweep", action="store_true",
                    help="accuracy against dense attention over k = N/64 ... N/4 (one JSON line per k)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    if args.profile_pass:
        profile_pass(args.profile_pass, max(args.steps, 1), tuple(args.profile_workloads.split(",")))
        return
    if args.probe == "gather":
        probe_gather(workload=args.probe_workload)
        return
    if args.probe == "mix":
        probe_mix()
        return
    if args.sweep:
        for w in sweep_workloads():
            for row in accuracy_sweep(w):
                print(json.dumps(row), flush=True)
        return
    dev = "cuda"
    lib = K.library()
    dec = DecodeStack(synth.WORKLOADS["decode_llama8b_32k"], dev)
    pre = PrefillStack(synth.WORKLOADS["prefill_8k"], dev)
    torch.cuda.synchronize()

    def step(marks=None):
        dec.run(marks)
        pre.run(marks)

    for _ in range(args.warmup):
        step()
        dec.run_dense()
        pre.run_dense()
    torch.cuda.synchronize()

    # The step as two HIP graphs (decode stack, prefill stack): replays carry
    # no host launch cost between the short kernels of a layer. The dense
    # baseline (every layer plain dense attention, same tensors) is captured
    # and timed the same way.
    graphs, dense_graphs = {}, {}
    for name, stack in (("decode", dec), ("prefill", pre)):
        for table, fn in ((graphs, stack.run), (dense_graphs, stack.run_dense)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            table[name] = g
    for _ in range(args.warmup):
        for g in list(graphs.values()) + list(dense_graphs.values()):
            g.replay()
    torch.cuda.synchronize()
    # K steps bracketed by events, with an event after every step for the spread
    start_g = _record()
    step_ev = []
    for _ in range(args.steps):
        for g in graphs.values():
            g.replay()
        step_ev.append(_record())
    torch.cuda.synchronize()
    total_ms = start_g.elapsed_time(step_ev[-1])
    per_step = np.array([(start_g if i == 0 else step_ev[i - 1]).elapsed_time(e) for i, e in enumerate(step_ev)])

    def time_graph(g):
        """Per-replay times (ms) of one graph over args.steps replays."""
        evs = [_record()]
        for _ in range(args.steps):
            g.replay()
            evs.append(_record())
        torch.cuda.synchronize()
        return np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])

    stack_ms = {n: time_graph(g) for n, g in graphs.items()}
    dense_ms = {n: time_graph(g) for n, g in dense_graphs.items()}
    gt = {n: float(v.mean()) for n, v in stack_ms.items()}

    # eager pass: per-call marks on the current stream and per-kernel events
    # inside the library
    lib.timing_collect()
    lib.timing_enable(True)
    marks = []
    start = _record()
    for _ in range(args.steps):
        marks.append(("step_start", _record()))
        step(marks)
    stop = _record()
    torch.cuda.synchronize()
    lib.timing_enable(False)
    kernels = lib.timing_collect()
    eager_ms_per_step = start.elapsed_time(stop) / args.steps
    ms_per_step = total_ms / args.steps

    calls = {}
    prev = None
    for name, ev in marks:
        if prev is not None and name != "step_start":
            calls.setdefault(name, []).append(prev.elapsed_time(ev))
        prev = ev
    avg = {n: float(np.mean(v)) for n, v in calls.items()}
    kern = {n: (ms / cnt) for n, (ms, cnt) in kernels.items()}

    wd, wp = dec.w, pre.w
    t_dec_layer_ms = gt["decode"] / wd.layers
    t_pre_stack_ms = gt["prefill"]
    prefill_tps = wp.batch * wp.n * wp.layers / (t_pre_stack_ms * 1e-3)
    reuse_gbs = dec.reuse_bytes() / (kern["decode_attn_gather"] * 1e-3) / 1e9
    reuse_call_gbs = dec.reuse_bytes() / (avg["decode_reuse"] * 1e-3) / 1e9
    anchor_gbs = dec.anchor_bytes() / (kern["decode_attn_dense"] * 1e-3) / 1e9
    pool_tflops = pre.qk_flops() / (kern["prefill_pool"] * 1e-3) / 1e12
    dense_tflops = 2 * pre.qk_flops() / (kern["prefill_dense"] * 1e-3) / 1e12
    gather_tflops = pre.reuse_flops() / (kern["prefill_gather"] * 1e-3) / 1e12

    # dense attention per layer: the graph of dense-only calls (no scores kept,
    # no selection) over the same four layers, per layer
    dense_dec_ms = float(dense_ms["decode"].mean()) / wd.layers
    dense_pre_ms = float(dense_ms["prefill"].mean()) / wp.layers

    # dominant kernel: the largest share of the step
    share = {n: kernels[n][0] / args.steps for n in kernels}
    dominant = max(share, key=share.get)
    rooflines = {
        "decode_attn_dense": ("hbm", anchor_gbs, PEAK_HBM_GBS, "GB/s", dec.anchor_bytes()),
        "decode_attn_gather": ("hbm", reuse_gbs, PEAK_HBM_GBS, "GB/s", dec.reuse_bytes()),
        "prefill_pool": ("mfma", pool_tflops, PEAK_BF16_TFLOPS, "TFLOP/s", pre.qk_flops()),
        "prefill_dense": ("mfma", dense_tflops, PEAK_BF16_TFLOPS, "TFLOP/s", 2 * pre.qk_flops()),
        "prefill_gather": ("mfma", gather_tflops, PEAK_BF16_TFLOPS, "TFLOP/s", pre.reuse_flops()),
    }
    bound, achieved, peak, unit, work = rooflines.get(dominant, rooflines["decode_attn_dense"])
    roofline = {"kernel": dominant, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4), "traffic": stored_traffic(dominant),
                "work_per_launch": work, "avg_launch_ms": round(kern[dominant], 5)}

    def spread(v, scale=1.0, nd=2):
        return {"mean": round(float(v.mean()) * scale, nd), "median": round(float(np.median(v)) * scale, nd),
                "min": round(float(v.min()) * scale, nd), "max": round(float(v.max()) * scale, nd)}

    result = {
        "metric": METRIC,
        "value": round(t_dec_layer_ms * 1e3, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode_llama8b_32k (anchor + 3 reuse layers) + prefill_8k (anchor + 3 reuse layers)",
            "decode": {"batch": wd.batch, "hq": wd.hq, "hkv": wd.hkv, "d": wd.d, "context": wd.n, "top_k": wd.k},
            "prefill": {"batch": wp.batch, "hq": wp.hq, "hkv": wp.hkv, "d": wp.d, "seq_len": wp.n,
                        "q_tile": wp.tile, "top_k": wp.k},
        },
        "roofline": roofline,
        "metrics": {
            "decode_us_per_layer": round(t_dec_layer_ms * 1e3, 3),
            "step_ms": spread(per_step, nd=4),
            "decode_stack_us_graph": spread(stack_ms["decode"], 1e3),
            "prefill_stack_us_graph": spread(stack_ms["prefill"], 1e3),
            "eager_ms_per_step": round(eager_ms_per_step, 4),
            "decode_anchor_us": round(avg["decode_anchor"] * 1e3, 2),
            "decode_reuse_us": round(avg["decode_reuse"] * 1e3, 2),
            "decode_reuse_hbm_gbs_kernel": round(reuse_gbs, 1),
            "decode_reuse_hbm_gbs_call": round(reuse_call_gbs, 1),
            "decode_anchor_hbm_gbs_kernel": round(anchor_gbs, 1),
            "prefill_tokens_per_s": round(prefill_tps, 1),
            # context: dense attention per layer (dense-only calls, no scores
            # kept, no selection, timed as a graph over the same four layers)
            # against the Kascade stack's mean layer
            "dense_decode_layer_us": round(dense_dec_ms * 1e3, 2),
            "dense_decode_stack_us_graph": spread(dense_ms["decode"], 1e3),
            "decode_speedup_vs_dense": round(dense_dec_ms / t_dec_layer_ms, 3),
            "dense_prefill_layer_us": round(dense_pre_ms * 1e3, 2),
            "dense_prefill_stack_us_graph": spread(dense_ms["prefill"], 1e3),
            "prefill_speedup_vs_dense": round(dense_pre_ms / (t_pre_stack_ms / wp.layers), 3),
            "speedup_vs_dense_by_layers": {
                str(L): {"decode": round(L * dense_dec_ms / (avg["decode_anchor"] + (L - 1) * avg["decode_reuse"]), 3),
                         "prefill": round(L * dense_pre_ms / (avg["prefill_anchor"] + (L - 1) * avg["prefill_reuse"]), 3)}
                for L in (2, 4, 8, 16, 32)},
            "prefill_anchor_us": round(avg["prefill_anchor"] * 1e3, 2),
            "prefill_reuse_us": round(avg["prefill_reuse"] * 1e3, 2),
            "prefill_pool_tflops": round(pool_tflops, 2),
            "prefill_dense_tflops": round(dense_tflops, 2),
            "prefill_gather_tflops": round(gather_tflops, 2),
            "kernel_avg_us": {n: round(v * 1e3, 2) for n, v in sorted(kern.items())},
            "rooflines": {n: {"bound": r[0], "achieved": round(r[1], 2), "peak": r[2], "unit": r[3],
                              "frac": round(r[1] / r[2], 4), "traffic": stored_traffic(n)}
                          for n, r in rooflines.items()},
        },
    }
    if not args.no_cpu_baseline:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        result["cpu_baseline"] = cpu_baseline(dec, pre, threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
