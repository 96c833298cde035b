"""Seeded synthetic inputs for Kascade's anchor/reuse attention.

Input plumbing only: this module draws Q, K, V and plants structure in them.
It holds none of the method's arithmetic, and both the GPU path's tests and
the oracle's tests draw their inputs from it.

Structure follows what the pages say the method exploits (Kascade abstract,
opentrain.ai page, "Abstract"; euno.news summary, "Overview"): post-softmax
attention is dominated by a few keys, and the identity of those keys is stable
across nearby layers. So each KV head gets a set of planted heavy keys whose
positions are shared (fully, or 70 % from one layer to the next) across layers,
plus, for prefill, a few leading "sink" rows with a larger norm.

Recipe (all normal draws are float32, then rounded to nearest-even bfloat16
unless the workload is float32):
  * Q, K, V ~ N(0, 1); generator seed 1000*workload_id + 10*layer + tensor_id
    (tensor_id 0 = Q, 1 = K, 2 = V, 3 = planted-row noise).
  * decode planted row p of KV head kv:  K[b,kv,p] = gain * q_dir + N(0, 0.1^2),
    q_dir the unit vector of the sum of the group's query vectors at that layer.
  * prefill planted row p:  K[b,kv,p] *= gain;  sink rows 0..3:  K[b,kv,0:4] *= 3.
  * gain = 4 for the workloads below; at d = 128 and 32K keys that leaves the
    attention diffuse (the planted keys hold a few per cent of it), a larger
    gain concentrates it on them.
  * positions come from numpy.random.default_rng(1000*workload_id + 7 + b):
    `share` = 1.0 keeps them for every layer, 0.7 keeps round(0.7*P) of the
    previous layer's P positions and redraws the rest disjoint from the kept.
"""
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # seed namespace
    phase: str          # "decode" | "prefill"
    batch: int
    hq: int
    hkv: int
    d: int
    n: int              # context (decode) or sequence (prefill) length
    k: int              # top-k
    tile: int           # query tile (prefill)
    dtype: str          # "f32" | "bf16"
    layers: int         # 1 anchor + (layers - 1) reuse
    planted: int        # planted heavy keys per KV head
    share: float        # fraction of planted positions kept layer to layer
    sinks: int = 0      # leading sink rows (prefill)
    gain: float = 4.0   # planted-row scale

    @property
    def group(self):
        return self.hq // self.hkv

    @property
    def tiles(self):
        return 1 if self.phase == "decode" else -(-self.n // self.tile)

    @property
    def q_len(self):
        return 1 if self.phase == "decode" else self.n

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def scaled(self, **kw):
        return replace(self, **kw)


# The five workloads the method is measured on.
WORKLOADS = {
    "decode_f32_1k": Workload("decode_f32_1k", 1, "decode", 1, 4, 1, 64, 1024, 64, 1, "f32", 2, 8, 1.0),
    "decode_llama8b_32k": Workload("decode_llama8b_32k", 2, "decode", 16, 32, 8, 128, 32768, 2048, 1,
                                   "bf16", 4, 64, 0.7),
    "prefill_8k": Workload("prefill_8k", 3, "prefill", 1, 32, 8, 128, 8192, 1024, 128, "bf16", 4, 32, 1.0, 4),
    "decode_128k": Workload("decode_128k", 4, "decode", 4, 64, 8, 128, 131072, 4096, 1, "bf16", 4, 128, 0.7),
    "prefill_32k": Workload("prefill_32k", 5, "prefill", 1, 64, 8, 64, 32768, 2048, 128, "bf16", 4, 64, 1.0, 4),
}


def planted_positions(w: Workload):
    """positions[layer][b][kv] -> sorted int64 array of w.planted key indices."""
    lo = w.sinks
    out = []
    for layer in range(w.layers):
        per_b = []
        for b in range(w.batch):
            rng = np.random.default_rng(1000 * w.wid + 7 + b + 100003 * layer)
            per_kv = []
            for kv in range(w.hkv):
                if layer == 0 or w.share >= 1.0:
                    if layer == 0:
                        base = np.random.default_rng(1000 * w.wid + 7 + b * 7919 + kv * 104729)
                        pos = base.choice(np.arange(lo, w.n), size=w.planted, replace=False)
                    else:
                        pos = out[0][b][kv]
                else:
                    prev = out[layer - 1][b][kv]
                    keep_n = int(round(w.share * w.planted))
                    kept = rng.choice(prev, size=keep_n, replace=False)
                    pool = np.setdiff1d(np.arange(lo, w.n), kept)
                    fresh = rng.choice(pool, size=w.planted - keep_n, replace=False)
                    pos = np.concatenate([kept, fresh])
                per_kv.append(np.sort(pos.astype(np.int64)))
            per_b.append(per_kv)
        out.append(per_b)
    return out


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_layer(w: Workload, layer: int, device="cpu", positions=None):
    """Q [B,Hq,q_len,d], K and V [B,Hkv,N,d] of one layer, in w's dtype, on `device`."""
    dev = torch.device(device)
    base = 1000 * w.wid + 10 * layer
    q = torch.randn((w.batch, w.hq, w.q_len, w.d), generator=_gen(base + 0, dev), device=dev)
    k = torch.randn((w.batch, w.hkv, w.n, w.d), generator=_gen(base + 1, dev), device=dev)
    v = torch.randn((w.batch, w.hkv, w.n, w.d), generator=_gen(base + 2, dev), device=dev)
    if positions is None:
        positions = planted_positions(w)
    noise_gen = _gen(base + 3, dev)
    if w.planted:
        for b in range(w.batch):
            for kv in range(w.hkv):
                pos = torch.as_tensor(positions[layer][b][kv], device=dev)
                if w.phase == "decode":
                    qsum = q[b, kv * w.group:(kv + 1) * w.group, 0, :].sum(0)
                    qdir = qsum / qsum.norm()
                    eps = 0.1 * torch.randn((pos.numel(), w.d), generator=noise_gen, device=dev)
                    k[b, kv, pos, :] = w.gain * qdir[None, :] + eps
                else:
                    k[b, kv, pos, :] *= w.gain
    if w.sinks:
        k[:, :, : w.sinks, :] *= 3.0
    dt = w.torch_dtype
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous()


def make_stack(w: Workload, device="cpu"):
    """All layers: list of (q, k, v); layer 0 is the anchor."""
    pos = planted_positions(w)
    return [make_layer(w, layer, device, pos) for layer in range(w.layers)]


def to_oracle(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a stored tensor as the oracle reads it (bf16 -> raw bits)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def checksum(t: torch.Tensor) -> str:
    """Order-sensitive 64-bit checksum of a tensor's stored bytes, for logs."""
    b = t.detach().to("cpu").contiguous().view(torch.uint8).numpy()
    import hashlib
    return hashlib.blake2b(b.tobytes(), digest_size=8).hexdigest()
