"""Seeded synthetic workloads for relation-aware attention (inputs only).

This module holds shapes, value distributions and seeds, and nothing of the
method's arithmetic.  Tests, the benchmark and the smoke check draw their inputs
from here, so the fp64 oracle and the HIP path see bit-identical operands.

Inputs are drawn in fp32 on the CPU with ``torch.Generator().manual_seed(seed)``
in the fixed order q, k, v, key table, value table (or the T5 bias table), key
lengths, and are then cast once to the workload's dtype.

The shapes are those of the Transformer base and big models of "Self-Attention
with Relative Position Representations" (§5, Evaluation Methodology: d_z = 64,
8 or 16 heads), a long-sequence stress shape, and the T5 default bucketing
(B = 32, max_distance = 128) of "Relative position embeddings", section "T5".
The pages train on WMT14 translation data; these synthetic tensors of the same
attention shapes stand in for it (no data or trained weights are needed to time
or check the forward operator).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SEED_BASE = 20260000


@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    description: str
    batch: int
    heads: int
    n: int
    d: int
    clip: int = 0
    dtype: torch.dtype = torch.bfloat16
    qkv_std: float = 1.0
    table_std: float = 0.02
    use_key_table: bool = True
    use_value_table: bool = True
    causal: bool = False
    len_range: tuple | None = None          # inclusive [lo, hi] key lengths
    t5: dict | None = None                  # num_buckets, max_distance, bidirectional
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return SEED_BASE + self.config_id


WORKLOADS = {
    "tiny": Workload(
        name="tiny", config_id=1,
        description="tiny fp32 check: B1 H2 n32 d16 clip 4, key+value tables",
        batch=1, heads=2, n=32, d=16, clip=4, dtype=torch.float32,
        qkv_std=1.0, table_std=0.1),
    "base": Workload(
        name="base", config_id=2,
        description="Transformer-base encoder self-attention: B32 H8 n128 d64 "
                    "clip 16, key padding lengths U[64,128], key+value tables",
        batch=32, heads=8, n=128, d=64, clip=16, len_range=(64, 128)),
    "big_causal_k": Workload(
        name="big_causal_k", config_id=3,
        description="Transformer-big decoder causal self-attention: B16 H16 "
                    "n256 d64 clip 16, key table only",
        batch=16, heads=16, n=256, d=64, clip=16, causal=True,
        use_value_table=False),
    "big_causal_kv": Workload(
        name="big_causal_kv", config_id=3,
        description="Transformer-big decoder causal self-attention: B16 H16 "
                    "n256 d64 clip 16, key+value tables",
        batch=16, heads=16, n=256, d=64, clip=16, causal=True),
    "long": Workload(
        name="long", config_id=4,
        description="long-sequence causal stress: B2 H16 n4096 d128 clip 64, "
                    "key+value tables",
        batch=2, heads=16, n=4096, d=128, clip=64, causal=True),
    "t5": Workload(
        name="t5", config_id=5,
        description="T5 bucketed scalar bias: B8 H12 n1024 d64, bidirectional, "
                    "32 buckets, max_distance 128, no 1/sqrt(d), key padding "
                    "lengths U[512,1024]",
        batch=8, heads=12, n=1024, d=64, qkv_std=1.0 / 8.0, table_std=1.0,
        use_key_table=False, use_value_table=False, len_range=(512, 1024),
        t5={"num_buckets": 32, "max_distance": 128, "bidirectional": True}),
}


def make_inputs(w: Workload | str, *, batch=None, n=None, heads=None,
                seed=None) -> dict:
    """CPU tensors for workload ``w`` (optionally with a smaller batch/n/heads).

    Returns a dict with q, k, v ([B, H, n, d], workload dtype), key_table and
    value_table ([H, 2c+1, d] or None), t5_bias ([num_buckets, H] fp32 or None)
    and key_lens (int32 [B] or None).  Every tensor is drawn even when the
    workload drops it, so the draw order (and thus the bits of what is kept)
    does not depend on the variant.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = batch or w.batch
    H = heads or w.heads
    N = n or w.n
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)

    def normal(shape, std):
        return torch.randn(shape, generator=g, dtype=torch.float32) * std

    q = normal((B, H, N, w.d), w.qkv_std)
    k = normal((B, H, N, w.d), w.qkv_std)
    v = normal((B, H, N, w.d), w.qkv_std)
    out = {"q": q.to(w.dtype), "k": k.to(w.dtype), "v": v.to(w.dtype),
           "key_table": None, "value_table": None, "t5_bias": None,
           "key_lens": None}
    if w.t5 is None:
        rows = 2 * w.clip + 1
        kt = normal((H, rows, w.d), w.table_std)
        vt = normal((H, rows, w.d), w.table_std)
        if w.use_key_table:
            out["key_table"] = kt.to(w.dtype)
        if w.use_value_table:
            out["value_table"] = vt.to(w.dtype)
    else:
        out["t5_bias"] = normal((w.t5["num_buckets"], H), w.table_std)
    if w.len_range is not None:
        lo, hi = w.len_range
        lo, hi = min(lo, N), min(hi, N)
        out["key_lens"] = torch.randint(lo, hi + 1, (B,), generator=g,
                                        dtype=torch.int32)
    return out


def attention_kwargs(w: Workload | str) -> dict:
    """Non-tensor operator arguments of a workload."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    kw = {"causal": w.causal}
    if w.t5 is None:
        kw["clip"] = w.clip
    else:
        kw.update(w.t5)
    return kw


# ---------------------------------------------------------------------------
# Incremental decoding: the newest position(s) of each sequence over its
# key/value cache.  Beam search with the Transformer big model is the pages'
# inference setting ("Self-Attention with Relative Position Representations",
# §5); 16 sentences x 4 beams give 64 sequences.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    config_id: int
    description: str
    batch: int
    heads: int
    cache: int               # rows of the cache (L)
    d: int
    tq: int = 1              # new positions per sequence
    clip: int = 16
    dtype: torch.dtype = torch.bfloat16
    qkv_std: float = 1.0
    table_std: float = 0.02
    len_range: tuple = (512, 1024)

    @property
    def seed(self) -> int:
        return SEED_BASE + self.config_id


DECODE_WORKLOADS = {
    "decode": DecodeWorkload(
        name="decode", config_id=6,
        description="Transformer-big beam-search decoding step: B64 (16 sentences x 4 "
                    "beams) H16 d64 clip 16, key+value tables, cache of 1024 positions "
                    "with lengths U[512,1024], one new position per sequence",
        batch=64, heads=16, cache=1024, d=64),
}


def make_decode_inputs(w: DecodeWorkload | str, *, batch=None, heads=None, cache=None,
                       tq=None, seed=None) -> dict:
    """CPU tensors for a decode workload: q [B, H, Tq, d], the caches k and v
    [B, H, L, d], key_table and value_table [H, 2c+1, d] and cache_lens int32
    [B] (drawn in that order, fp32 then cast once to the workload dtype)."""
    if isinstance(w, str):
        w = DECODE_WORKLOADS[w]
    B, H = batch or w.batch, heads or w.heads
    L, Tq = cache or w.cache, tq or w.tq
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)

    def normal(shape, std):
        return torch.randn(shape, generator=g, dtype=torch.float32) * std

    q = normal((B, H, Tq, w.d), w.qkv_std)
    k = normal((B, H, L, w.d), w.qkv_std)
    v = normal((B, H, L, w.d), w.qkv_std)
    kt = normal((H, 2 * w.clip + 1, w.d), w.table_std)
    vt = normal((H, 2 * w.clip + 1, w.d), w.table_std)
    lo, hi = min(w.len_range[0], L), min(w.len_range[1], L)
    lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int32)
    return {"q": q.to(w.dtype), "k": k.to(w.dtype), "v": v.to(w.dtype),
            "key_table": kt.to(w.dtype), "value_table": vt.to(w.dtype), "cache_lens": lens}


# ---------------------------------------------------------------------------
# Transformer-XL relative logits.  The pages give no sizes (the transformer-xl
# page stops before its implementation); a language-model segment: B8 H16 n512
# d64 causal, the position table over every distance (window n - 1), per-head
# global biases.  R stands for the projected sinusoidal encodings W_R r.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class XLWorkload:
    name: str
    config_id: int
    description: str
    batch: int
    heads: int
    n: int
    d: int
    window: int
    causal: bool = True
    dtype: torch.dtype = torch.bfloat16
    qkv_std: float = 1.0
    table_std: float = 0.5

    @property
    def seed(self) -> int:
        return SEED_BASE + self.config_id


XL_WORKLOADS = {
    "xl": XLWorkload(
        name="xl", config_id=7,
        description="Transformer-XL relative logits on a language-model segment: B8 H16 "
                    "n512 d64 causal, position table over every distance (window 511), "
                    "per-head u and v",
        batch=8, heads=16, n=512, d=64, window=511),
    "xl128": XLWorkload(
        name="xl128", config_id=7,
        description="Transformer-XL relative logits with 128-wide heads: B8 H8 n512 d128 "
                    "causal, position table over every distance (window 511), per-head u "
                    "and v",
        batch=8, heads=8, n=512, d=128, window=511),
}


def make_xl_inputs(w: XLWorkload | str, *, batch=None, heads=None, n=None, seed=None) -> dict:
    """CPU tensors for an XL workload, drawn in this order: q, k, v [B, H, n, d],
    the position table R [H, 2W+1, d], u and v biases [H, d] (fp32 draws cast
    once to the workload dtype)."""
    if isinstance(w, str):
        w = XL_WORKLOADS[w]
    B, H, N = batch or w.batch, heads or w.heads, n or w.n
    W = min(w.window, N - 1)
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)

    def normal(shape, std):
        return torch.randn(shape, generator=g, dtype=torch.float32) * std

    q = normal((B, H, N, w.d), w.qkv_std)
    k = normal((B, H, N, w.d), w.qkv_std)
    v = normal((B, H, N, w.d), w.qkv_std)
    R = normal((H, 2 * W + 1, w.d), w.table_std)
    u = normal((H, w.d), w.table_std)
    vb = normal((H, w.d), w.table_std)
    return {"q": q.to(w.dtype), "k": k.to(w.dtype), "v": v.to(w.dtype), "R": R.to(w.dtype),
            "u": u.to(w.dtype), "vb": vb.to(w.dtype), "window": W}


# ---------------------------------------------------------------------------
# 2-D window bias (Swin).  The pages give no sizes; a first stage of a windowed
# vision transformer: 7 x 7 windows (n = 49), 3 heads of d = 32, 2048 windows.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class GridWorkload:
    name: str
    config_id: int
    description: str
    batch: int          # windows
    heads: int
    side: int           # M: n = M * M tokens per window
    d: int
    dtype: torch.dtype = torch.bfloat16
    qkv_std: float = 1.0
    table_std: float = 1.0

    @property
    def seed(self) -> int:
        return SEED_BASE + self.config_id


GRID_WORKLOADS = {
    "swin": GridWorkload(
        name="swin", config_id=8,
        description="2-D window relative position bias: 2048 windows of 7 x 7 tokens, "
                    "H3 d32, bias table [3, 169]",
        batch=2048, heads=3, side=7, d=32),
}


def make_grid_inputs(w: GridWorkload | str, *, batch=None, seed=None) -> dict:
    """CPU tensors for a 2-D window workload, drawn in this order: q, k, v
    [B, H, M*M, d] and the bias table [H, (2M-1)^2] fp32."""
    if isinstance(w, str):
        w = GRID_WORKLOADS[w]
    B, H, n = batch or w.batch, w.heads, w.side * w.side
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)

    def normal(shape, std):
        return torch.randn(shape, generator=g, dtype=torch.float32) * std

    q = normal((B, H, n, w.d), w.qkv_std)
    k = normal((B, H, n, w.d), w.qkv_std)
    v = normal((B, H, n, w.d), w.qkv_std)
    bias = normal((H, (2 * w.side - 1) ** 2), w.table_std)
    return {"q": q.to(w.dtype), "k": k.to(w.dtype), "v": v.to(w.dtype), "bias": bias}


# ---------------------------------------------------------------------------
# Per-pair edge labels.  The pages give no sizes; the Transformer-big attention
# shape (16 heads of d = 64) over 256-token inputs whose every (query, key)
# edge carries one of 64 labels (a relation vocabulary the size of a set of
# dependency or discourse types), drawn uniformly per pair.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class EdgeWorkload:
    name: str
    config_id: int
    description: str
    batch: int
    heads: int
    n: int
    d: int
    labels: int         # NL: label vocabulary
    tables: bool = False  # key and value tables [H, NL, d] instead of a bias table
    causal: bool = False
    dtype: torch.dtype = torch.bfloat16
    qkv_std: float = 1.0
    table_std: float = 1.0

    @property
    def seed(self) -> int:
        return SEED_BASE + self.config_id


EDGE_WORKLOADS = {
    "edge": EdgeWorkload(
        name="edge", config_id=9,
        description="per-pair edge labels: B16 H16 n256 d64, 64 labels uniform per pair, "
                    "bias table [16, 64], no mask",
        batch=16, heads=16, n=256, d=64, labels=64),
    "edge_kv": EdgeWorkload(
        name="edge_kv", config_id=10,
        description="relation-aware attention over a labeled graph: B16 H16 n256 d64, 64 "
                    "labels uniform per pair, key+value tables [16, 64, 64], no mask",
        batch=16, heads=16, n=256, d=64, labels=64, tables=True, table_std=0.02),
}


def make_edge_inputs(w: EdgeWorkload | str, *, batch=None, n=None, seed=None) -> dict:
    """CPU tensors for an edge-label workload, drawn in this order: q, k, v
    [B, H, n, d], the bias table [H, NL] fp32 (or the key and value tables [H,
    NL, d] in the workload dtype) and the labels [B, n, n] (int64, uniform in
    [0, NL))."""
    if isinstance(w, str):
        w = EDGE_WORKLOADS[w]
    B, H, n = batch or w.batch, w.heads, n or w.n
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)

    def normal(shape, std):
        return torch.randn(shape, generator=g, dtype=torch.float32) * std

    q = normal((B, H, n, w.d), w.qkv_std)
    k = normal((B, H, n, w.d), w.qkv_std)
    v = normal((B, H, n, w.d), w.qkv_std)
    if w.tables:
        wK = normal((H, w.labels, w.d), w.table_std)
        wV = normal((H, w.labels, w.d), w.table_std)
        labels = torch.randint(0, w.labels, (B, n, n), generator=g)
        return {"q": q.to(w.dtype), "k": k.to(w.dtype), "v": v.to(w.dtype),
                "wK": wK.to(w.dtype), "wV": wV.to(w.dtype), "labels": labels}
    bias = normal((H, w.labels), w.table_std)
    labels = torch.randint(0, w.labels, (B, n, n), generator=g)
    return {"q": q.to(w.dtype), "k": k.to(w.dtype), "v": v.to(w.dtype), "bias": bias,
            "labels": labels}
