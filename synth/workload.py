"""Seeded synthetic inputs for one attention layer (Q, K, V) with planted head types.

This module only draws inputs; it contains none of FlexPrefill's arithmetic.
Both the CPU oracle tests and the GPU path read the tensors it returns.

The FlexPrefill pages evaluate on RULER and InfiniteBench with trained
Llama / GLM / Qwen weights; neither the datasets nor the weights are used
here.  Instead every query head carries one of four planted attention
behaviours, named after the patterns the method distinguishes (the
"Approach" paragraph of the atlas.scime.ai summary: vertical-slash versus
query-aware):

* vertical ("V"): a handful of sink keys that every query of the head
  attends to;
* slash ("S"): attention concentrated on a few diagonals (fixed offsets
  ``i - j``), made by a rotary-rotated shared low-rank Q/K component;
* query-aware ("QA"): each 128-token query segment attends to the key
  segments of two of eight clusters;
* noise ("N"): nothing planted on the query side.

Reading of the magnitudes (the workload text gives "norm 6", "scale 3",
"norm 4" without saying per what): a stated magnitude is the per-coordinate
contribution to q.k at an aligned query/key pair, split between a small
key-side plant (amplitude KEY_AMP per coordinate) and a query-side partner
that makes the pattern appear in attention.  The slash component is shared
by Q and K, so its contribution is the square of its scale.  The three
families live in disjoint coordinate blocks of the head dimension
(vertical: the first quarter, query-aware: the second quarter, slash: the
second half), so a head's partner does not couple to the other families'
key plants.  With grouped-query attention all key-side plants are
superposed in every key/value head; a query head's type is decided by the
partner it carries.  Unstructured parts: Q ~ N(0, 1), K ~ N(0, KEY_NOISE^2),
V ~ N(0, 1) per coordinate.

Recipe per key/value head (b, kv): sink positions {0} plus sinks-1 distinct
uniform positions in [1, N); a +-KEY_AMP sink vector s on the vertical
coordinates added to those keys; eight +-KEY_AMP cluster directions W_c on
the query-aware coordinates, one cluster id per 128-token key segment, W of
that id added to every key of the segment; a rank-16 vector a of
per-coordinate scale KEY_AMP on the slash coordinates, rotated by position
(rotary pairs (2t, 2t+1), base 10000) and added to every key, averaged over
``slash_width`` consecutive positions.  Per query head: vertical adds
s * SINK_MAG / KEY_AMP^2 to every query; slash adds the position-rotated
a * SLASH_SCALE^2 / KEY_AMP^2; query-aware adds (W_c1 + W_c2) * QA_MAG /
KEY_AMP^2 with two distinct clusters drawn per 128-token query segment.

Every random draw comes from ``numpy.random.default_rng`` seeded with a
tuple (config seed, stream id, batch, head), so any single head can be
regenerated on its own and gives the same values as a full generation.
Values are drawn in float32 and rounded to bfloat16 (round-to-nearest-even,
through torch) for bf16 configurations; the returned float32 arrays then
hold exactly the bf16 values the GPU receives.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .configs import HEAD_TYPES, NOISE, QUERY_AWARE, SLASH, VERTICAL, LayerConfig

SEGMENT = 128          # token granularity of the query-aware cluster structure
N_CLUSTERS = 8
# Stated magnitudes, read as the per-coordinate product of a query-side
# partner and its key-side plant (the contribution of one coordinate to q.k
# at an aligned query/key pair).
SINK_MAG = 6.0         # vertical: sink keys
QA_MAG = 4.0           # query-aware: cluster directions
SLASH_SCALE = 3.0      # slash: rotary low-rank component
KEY_AMP = 1.5          # per-coordinate amplitude of every key-side plant
KEY_NOISE = 0.5        # standard deviation of the unstructured part of K
SLASH_RANK = 16
ROPE_BASE = 10000.0

# stream ids of the seeded generators
_S_Q, _S_K, _S_V, _S_PLANT, _S_PARTNER, _S_TYPES = range(6)


def head_types(cfg: LayerConfig) -> List[str]:
    """Planted type of every query head.

    Explicit per-head types win; otherwise the fractions in ``cfg.mix`` are
    turned into counts by largest remainder (ties go to the earlier type in
    V, S, QA, N order) and spread over the heads by a seeded permutation.
    """
    if cfg.explicit_types:
        if len(cfg.explicit_types) != cfg.Hq:
            raise ValueError("explicit_types must list one type per query head")
        return list(cfg.explicit_types)
    raw = [f * cfg.Hq for f in cfg.mix]
    counts = [int(math.floor(r)) for r in raw]
    rem = sorted(range(4), key=lambda t: (-(raw[t] - counts[t]), t))
    for t in rem[: cfg.Hq - sum(counts)]:
        counts[t] += 1
    types: List[str] = []
    for t, c in zip(HEAD_TYPES, counts):
        types += [t] * c
    perm = np.random.default_rng([cfg.seed, _S_TYPES]).permutation(cfg.Hq)
    return [types[p] for p in perm]


def _rope(vec: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Rotate adjacent coordinate pairs (2t, 2t+1) of ``vec`` by pos * theta_t,
    theta_t = base^(-2t/len(vec)); one rotated copy per position."""
    dim = vec.shape[0]
    half = dim // 2
    theta = ROPE_BASE ** (-2.0 * np.arange(half, dtype=np.float64) / dim)
    ang = positions.astype(np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a0 = vec[0::2].astype(np.float64)[None, :]
    a1 = vec[1::2].astype(np.float64)[None, :]
    out = np.empty((positions.shape[0], dim), dtype=np.float64)
    out[:, 0::2] = a0 * c - a1 * s
    out[:, 1::2] = a0 * s + a1 * c
    return out


def _round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype}")
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


class LayerGen:
    """Generator for one layer's Q, K, V; heads can be produced one at a time."""

    def __init__(self, cfg: LayerConfig):
        if cfg.d % 8 != 0:
            raise ValueError("head dim must be a multiple of 8")
        self.cfg = cfg
        self.types = head_types(cfg)
        d = cfg.d
        self.dims_v = slice(0, d // 4)
        self.dims_qa = slice(d // 4, d // 2)
        self.dims_s = slice(d // 2, d)
        self._plants: Dict[Tuple[int, int], dict] = {}

    # ----------------------------------------------------------------- plants
    def plants(self, b: int, kv: int) -> dict:
        key = (b, kv)
        if key in self._plants:
            return self._plants[key]
        cfg = self.cfg
        rng = np.random.default_rng([cfg.seed, _S_PLANT, b, kv])
        n_sinks = min(cfg.sinks, cfg.N)
        others = rng.choice(np.arange(1, cfg.N), size=n_sinks - 1, replace=False) \
            if n_sinks > 1 else np.zeros(0, dtype=np.int64)
        sinks = np.sort(np.concatenate([[0], others]).astype(np.int64))
        dv = self.dims_v.stop - self.dims_v.start
        dq = self.dims_qa.stop - self.dims_qa.start
        ds = self.dims_s.stop - self.dims_s.start
        s_vec = rng.choice([-KEY_AMP, KEY_AMP], size=dv)
        w_cl = rng.choice([-KEY_AMP, KEY_AMP], size=(N_CLUSTERS, dq))
        n_seg = (cfg.N + SEGMENT - 1) // SEGMENT
        seg_cluster = rng.integers(0, N_CLUSTERS, size=n_seg)
        basis, _ = np.linalg.qr(rng.standard_normal((ds, SLASH_RANK)))
        z = rng.standard_normal(SLASH_RANK)
        a_vec = basis @ (KEY_AMP * z) * math.sqrt(ds / SLASH_RANK)
        p = dict(sinks=sinks, s_vec=s_vec, w_cl=w_cl, seg_cluster=seg_cluster,
                 a_vec=a_vec)
        self._plants[key] = p
        return p

    # ------------------------------------------------------------------ heads
    def k_head(self, b: int, kv: int) -> np.ndarray:
        cfg = self.cfg
        p = self.plants(b, kv)
        rng = np.random.default_rng([cfg.seed, _S_K, b, kv])
        k = rng.standard_normal((cfg.N, cfg.d), dtype=np.float32) * np.float32(KEY_NOISE)
        k[p["sinks"], self.dims_v] += p["s_vec"].astype(np.float32)
        seg = np.arange(cfg.N) // SEGMENT
        k[:, self.dims_qa] += p["w_cl"][p["seg_cluster"][seg]].astype(np.float32)
        w = cfg.slash_width
        pos = np.arange(cfg.N)
        acc = np.zeros((cfg.N, self.dims_s.stop - self.dims_s.start))
        for t in range(w):
            acc += _rope(p["a_vec"], pos + t)
        k[:, self.dims_s] += (acc / math.sqrt(w)).astype(np.float32)
        return _round_to(k, cfg.dtype)

    def v_head(self, b: int, kv: int) -> np.ndarray:
        cfg = self.cfg
        rng = np.random.default_rng([cfg.seed, _S_V, b, kv])
        return _round_to(rng.standard_normal((cfg.N, cfg.d), dtype=np.float32), cfg.dtype)

    def q_head(self, b: int, h: int) -> np.ndarray:
        cfg = self.cfg
        kv = h // cfg.group
        p = self.plants(b, kv)
        rng = np.random.default_rng([cfg.seed, _S_Q, b, h])
        q = rng.standard_normal((cfg.N, cfg.d), dtype=np.float32)
        t = self.types[h]
        if t == VERTICAL:
            q[:, self.dims_v] += (p["s_vec"] * (SINK_MAG / KEY_AMP ** 2)).astype(np.float32)
        elif t == SLASH:
            q[:, self.dims_s] += (_rope(p["a_vec"], np.arange(cfg.N))
                                  * (SLASH_SCALE ** 2 / KEY_AMP ** 2)).astype(np.float32)
        elif t == QUERY_AWARE:
            prng = np.random.default_rng([cfg.seed, _S_PARTNER, b, h])
            n_seg = (cfg.N + SEGMENT - 1) // SEGMENT
            picks = np.stack([prng.choice(N_CLUSTERS, size=2, replace=False)
                              for _ in range(n_seg)])
            dirs = (p["w_cl"][picks[:, 0]] + p["w_cl"][picks[:, 1]]) * (QA_MAG / KEY_AMP ** 2)
            seg = np.arange(cfg.N) // SEGMENT
            q[:, self.dims_qa] += dirs[seg].astype(np.float32)
        elif t != NOISE:
            raise ValueError(t)
        return _round_to(q, cfg.dtype)

    # ----------------------------------------------------------- whole layer
    def numpy_layer(self, q_heads: Optional[Sequence[int]] = None):
        """float32 arrays q [B, len(q_heads), N, d], k and v [B, Hkv, N, d].

        With ``q_heads`` given only those query heads are generated; k and v
        are still indexed by the full key/value head number."""
        cfg = self.cfg
        hs = list(range(cfg.Hq)) if q_heads is None else list(q_heads)
        q = np.stack([np.stack([self.q_head(b, h) for h in hs]) for b in range(cfg.B)])
        kvs = sorted({h // cfg.group for h in hs}) if q_heads is not None else range(cfg.Hkv)
        k = np.zeros((cfg.B, cfg.Hkv, cfg.N, cfg.d), np.float32)
        v = np.zeros((cfg.B, cfg.Hkv, cfg.N, cfg.d), np.float32)
        for b in range(cfg.B):
            for kv in kvs:
                k[b, kv] = self.k_head(b, kv)
                v[b, kv] = self.v_head(b, kv)
        return q, k, v

    def torch_layer(self, device="cuda"):
        """(q, k, v) torch tensors of the configuration's dtype on ``device``,
        contiguous [B, H, N, d], filled head by head."""
        import torch
        cfg = self.cfg
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        q = torch.empty((cfg.B, cfg.Hq, cfg.N, cfg.d), dtype=tdt, device=device)
        k = torch.empty((cfg.B, cfg.Hkv, cfg.N, cfg.d), dtype=tdt, device=device)
        v = torch.empty((cfg.B, cfg.Hkv, cfg.N, cfg.d), dtype=tdt, device=device)
        for b in range(cfg.B):
            for h in range(cfg.Hq):
                q[b, h].copy_(torch.from_numpy(self.q_head(b, h)).to(tdt))
            for kv in range(cfg.Hkv):
                k[b, kv].copy_(torch.from_numpy(self.k_head(b, kv)).to(tdt))
                v[b, kv].copy_(torch.from_numpy(self.v_head(b, kv)).to(tdt))
        return q, k, v
