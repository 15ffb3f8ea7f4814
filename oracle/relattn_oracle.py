"""fp64 CPU oracle for relation-aware self-attention and T5 bucketed bias.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never calls it, and this module shares
no code with that path: it imports nothing from the package.

Everything here is the plain definition of the method, written for a reader to
check against the pages by eye.  Inputs may be any real dtype (fp32, bf16 as
torch or numpy arrays); they are upcast exactly to float64 and all arithmetic
runs in float64.

Sources (page titles, then section / equation):

* "Self-Attention with Relative Position Representations" (paper summary page),
  §3.4 "Standard Self-Attention" (Eq. 1, Eq. 2 and the softmax), "Relation-Aware
  Self-Attention" (Eq. 3, Eq. 4), "Relative Position Representations: From
  Arbitrary Edges to Sequences" (the clip function and the 2k+1 tables),
  "Efficient Implementation" (Eq. 5, the split of the logit and of the output).
* "Shaw et al. Relative Position Representations" (tutorial page): the same
  equations in q, k, v notation with offset r = j - i.
* "Relative position embeddings" (survey page), section "T5": the scalar bias
  A_ij = q_i.k_j + b^(h)_beta(j-i), the bucket function beta, no 1/sqrt(d).

Readings where the pages are silent or garbled:

* offset sign is j - i, table row 0 holds offset -k;
* tables are [Ht, 2k+1, d] with Ht in {1, H} (Ht == 1: shared by all heads);
* the 1/sqrt(d) scale multiplies both terms of the logit (Eq. 5); a^V is unscaled;
* masks: causal hides keys j > i; key padding hides keys j >= len_b; masked
  keys contribute neither v_j nor a^V_ij; a row with no visible key outputs 0;
* T5 bidirectional: half of the buckets per sign, B_exact = half/2, the
  logarithmic part spans (half - B_exact) buckets and is capped at half - 1,
  keys after the query (delta > 0) use the upper half; unidirectional uses all
  B buckets for delta <= 0 and maps delta > 0 to bucket 0;
* the floor in beta is taken of the exact real number (rational comparison),
  not of a rounded floating-point logarithm;
* Transformer-XL (transformer-xl page, "Relative Position Encoding in
  Transformer-XL", and the survey page's "Transformer-XL" section): the score is
  the four terms (a) q.k, (b) q.R_{i-j}, (c) u.k, (d) v.R_{i-j}, with R the
  projected relative encodings, given as a table over i - j (clipped to +-W like
  the other tables; W >= n - 1 clips nothing); the attention scale (1/sqrt(d) by
  default) multiplies the whole score, as it does for the Shaw logit;
* Swin 2-D bias (survey page, "Relative position embeddings", Swin paragraph):
  the n = M*M tokens of a window are in raster order (token p at row p div M,
  column p mod M); the table has (2M-1)^2 entries per head, entry
  (dy + M - 1)(2M - 1) + (dx + M - 1) for the key-minus-query offset (dy, dx);
* per-pair edge labels ("Self-Attention with Relative Position Representations"
  summary page, the labeled-graph reading of section 3.1: any pairwise label
  may index the relation; survey page, "Placement in the taxonomy": a scalar
  bias table indexed per pair): labels are given per batch as an n x n integer
  matrix E[b, i, j] for the edge from query i to key j, shared by the heads; the
  bias table is [Hb, NL] with Hb in {1, H}; the attention scale (1/sqrt(d) by
  default) multiplies the content logit only, as for the offset bias;
* per-pair edge labels with vector tables (the same labeled-graph reading of
  Eq. 3 and Eq. 4): a^K_ij = w^K[h', E[b, i, j]] and a^V_ij = w^V[h', E[b, i, j]]
  with tables [Ht, NL, d], Ht in {1, H}; the scale multiplies both terms of the
  logit (as in Eq. 5) and a^V is unscaled, as for the clipped-offset tables;
* backward (no page prints it): the gradients of a scalar loss sum(dz * z) by
  the chain rule through the forward above; a table shared by all heads takes
  the sum over heads, and hidden pairs give no gradient.  Pinned by central
  finite differences of the forward, by library autograd where the tables
  vanish, and by the row-sum identities of the softmax.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = [
    "clip",
    "relative_labels",
    "visible",
    "t5_bucket",
    "t5_bucket_matrix",
    "shaw_logits",
    "relattn_bruteforce",
    "relattn_factored",
    "relattn_rows",
    "t5_attention",
    "t5_rows",
    "relattn_decode",
    "t5_decode",
    "offset_bias_attention",
    "offset_bias_decode",
    "relattn_backward",
    "t5_backward",
    "offset_bias_backward",
    "xl_attention",
    "xl_decode",
    "grid_bias_attention",
    "grid_bias_backward",
    "edge_label_attention",
    "edge_label_backward",
    "xl_backward",
    "edge_label_relattn_backward",
    "edge_label_relattn",
    "to_f64",
]


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def to_f64(x):
    """Exact upcast of a numpy array or torch tensor (any real dtype) to float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor; bf16 -> fp64 is exact
        import torch
        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _table_for_head(table, h):
    """Per-head slice of a [Ht, 2k+1, d] table; Ht == 1 means shared by all heads."""
    if table is None:
        return None
    return table[0] if table.shape[0] == 1 else table[h]


def _key_lengths(key_lens, batch, n):
    if key_lens is None:
        return [n] * batch
    lens = [int(x) for x in np.asarray(key_lens).reshape(-1)]
    return [max(0, min(n, x)) for x in lens]


# ---------------------------------------------------------------------------
# relative position labels (paper summary page, "Relative Position
# Representations: From Arbitrary Edges to Sequences")
# ---------------------------------------------------------------------------

def clip(x: int, k: int) -> int:
    """clip(x, k) = max(-k, min(k, x))."""
    return max(-k, min(k, x))


def relative_labels(n: int, k: int) -> np.ndarray:
    """R[i, j] = clip(j - i, k) for query i and key j (int64, n x n)."""
    by_delta = np.array([clip(x, k) for x in range(-(n - 1), n)], dtype=np.int64)
    delta = np.arange(n)[None, :] - np.arange(n)[:, None]  # j - i
    return by_delta[delta + (n - 1)]


def visible(n: int, causal: bool, key_len: int) -> np.ndarray:
    """Boolean n x n matrix: key j is visible to query i."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    ok = j < key_len
    if causal:
        ok = ok & (j <= i)
    return np.broadcast_to(ok, (n, n)).copy()


# ---------------------------------------------------------------------------
# T5 bucketing (survey page "Relative position embeddings", section "T5")
# ---------------------------------------------------------------------------

def t5_bucket(delta: int, num_buckets: int = 32, max_distance: int = 128,
              bidirectional: bool = True) -> int:
    """Bucket beta(delta) for offset delta = j - i.

    For a distance a below B_exact the bucket is a itself.  Otherwise it is
    B_exact + floor((nb) * ln(a / B_exact) / ln(D_max / B_exact)), clamped to the
    last bucket of its half, with nb the number of logarithmic buckets.  The
    floor is evaluated exactly: floor(x) >= t  <=>  (a/B_exact)^nb >=
    (D_max/B_exact)^t, a comparison of rationals.
    """
    if bidirectional:
        half = num_buckets // 2
        base = half if delta > 0 else 0
        a = abs(delta)
    else:
        half = num_buckets
        base = 0
        a = max(-delta, 0)
    exact = half // 2
    if a < exact:
        return base + a
    nb = half - exact
    lhs = Fraction(a, exact) ** nb
    step = Fraction(max_distance, exact)
    t = 0
    # largest t with (a/exact)^nb >= (D/exact)^t, stopping at the cap half-1
    while exact + t < half - 1 and lhs >= step ** (t + 1):
        t += 1
    return base + exact + t


def t5_bucket_matrix(n: int, num_buckets: int = 32, max_distance: int = 128,
                     bidirectional: bool = True) -> np.ndarray:
    """Bmat[i, j] = beta(j - i) (int64, n x n)."""
    by_delta = np.array([t5_bucket(x, num_buckets, max_distance, bidirectional)
                         for x in range(-(n - 1), n)], dtype=np.int64)
    delta = np.arange(n)[None, :] - np.arange(n)[:, None]  # j - i
    return by_delta[delta + (n - 1)]


# ---------------------------------------------------------------------------
# softmax over visible keys (paper summary page, §3.4 softmax under Eq. 2)
# ---------------------------------------------------------------------------

def _masked_softmax_rows(e: np.ndarray, ok: np.ndarray) -> np.ndarray:
    """alpha[i, j] = exp(e_ij) / sum_{visible j'} exp(e_ij'); 0 where hidden.

    A row with no visible key gets all-zero weights.
    """
    e_vis = np.where(ok, e, -np.inf)
    row_max = e_vis.max(axis=1, keepdims=True)
    row_max = np.where(np.isfinite(row_max), row_max, 0.0)  # rows with no key
    w = np.where(ok, np.exp(e_vis - row_max), 0.0)
    total = w.sum(axis=1, keepdims=True)
    return np.divide(w, total, out=np.zeros_like(w), where=total > 0)


# ---------------------------------------------------------------------------
# Shaw et al., brute force: materialise a^K_ij and a^V_ij (Eq. 3, Eq. 4)
# ---------------------------------------------------------------------------

def _default_scale(d: int, scale):
    return 1.0 / np.sqrt(d) if (scale is None or scale <= 0) else float(scale)


def shaw_logits(q, k, aK, clip_k: int, scale=None) -> np.ndarray:
    """e[i, j] = scale * q_i . (k_j + a^K_ij) for ONE head (q, k: [n, d]).

    a^K_ij = w^K_clip(j-i, k) (Eq. 4); no mask applied.
    """
    q = to_f64(q)
    k = to_f64(k)
    n, d = q.shape
    s = _default_scale(d, scale)
    R = relative_labels(n, clip_k)
    if aK is None:
        AK = np.zeros((n, n, d))
    else:
        AK = to_f64(aK)[R + clip_k]  # [n, n, d], row (i, j) = w^K_{clip(j-i)}
    keys = k[None, :, :] + AK  # relation-augmented key of j as seen from i
    return s * np.einsum("id,ijd->ij", q, keys)


def relattn_bruteforce(q, k, v, aK=None, aV=None, clip_k: int = 0, scale=None,
                       causal: bool = False, key_lens=None, return_alpha=False):
    """Relation-aware self-attention by its definition, all heads.

    q, k, v: [B, H, n, d]; aK, aV: [Ht, 2k+1, d] or None (None counts as zero).
    Materialises the n x n x d edge tensors per head (Eq. 3 and Eq. 4), then
    masked softmax, then z_i = sum_j alpha_ij (v_j + a^V_ij).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    aK, aV = to_f64(aK), to_f64(aV)
    B, H, n, d = q.shape
    lens = _key_lengths(key_lens, B, n)
    R = relative_labels(n, clip_k)
    z = np.zeros((B, H, n, v.shape[-1]))
    alphas = np.zeros((B, H, n, n)) if return_alpha else None
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            e = shaw_logits(q[b, h], k[b, h], _table_for_head(aK, h), clip_k, scale)
            alpha = _masked_softmax_rows(e, ok)
            if aV is None:
                AV = np.zeros((n, n, v.shape[-1]))
            else:
                AV = _table_for_head(aV, h)[R + clip_k]  # [n, n, d]
            vals = v[b, h][None, :, :] + AV  # value of j as seen from i
            z[b, h] = np.einsum("ij,ijd->id", alpha, vals)
            if return_alpha:
                alphas[b, h] = alpha
    return (z, alphas) if return_alpha else z


# ---------------------------------------------------------------------------
# Shaw et al., factored (Eq. 5 and the split of Eq. 3)
# ---------------------------------------------------------------------------

def relattn_factored(q, k, v, aK=None, aV=None, clip_k: int = 0, scale=None,
                     causal: bool = False, key_lens=None, return_bucket_sums=False):
    """Same result as ``relattn_bruteforce`` through the split of Eq. 5.

    e = scale * Q K^T + L[i, clip(j-i)+k] with L = scale * Q (w^K)^T, and
    z = alpha V + S W^V with S[i, r] = sum of alpha_ij over keys j whose label
    is r.  Nothing of size n x n x d is formed.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    aK, aV = to_f64(aK), to_f64(aV)
    B, H, n, d = q.shape
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    R = relative_labels(n, clip_k)
    nlab = 2 * clip_k + 1
    z = np.zeros((B, H, n, v.shape[-1]))
    S_all = np.zeros((B, H, n, nlab)) if return_bucket_sums else None
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            e = s * (q[b, h] @ k[b, h].T)  # content term (Eq. 2 form)
            if aK is not None:
                L = s * (q[b, h] @ _table_for_head(aK, h).T)  # [n, 2k+1]
                e = e + np.take_along_axis(L, R + clip_k, axis=1)
            alpha = _masked_softmax_rows(e, ok)
            out = alpha @ v[b, h]
            # S[i, r] = sum of alpha_ij over the keys j whose label row is r
            S = np.stack([np.bincount(R[i] + clip_k, weights=alpha[i], minlength=nlab)
                          for i in range(n)])
            if aV is not None:
                out = out + S @ _table_for_head(aV, h)
            z[b, h] = out
            if return_bucket_sums:
                S_all[b, h] = S
    return (z, S_all) if return_bucket_sums else z


def relattn_rows(q, k, v, aK=None, aV=None, clip_k: int = 0, scale=None,
                 causal: bool = False, key_lens=None, rows=()):
    """Brute-force output rows z[b, h, i] for a list of (b, h, i).

    For each row the n x d slab k_j + a^K_ij and v_j + a^V_ij is materialised
    (Eq. 4 and Eq. 3 for one query), so large shapes can be sampled row by row.
    Returns an array [len(rows), d].
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    aK, aV = to_f64(aK), to_f64(aV)
    B, H, n, d = q.shape
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    out = np.zeros((len(rows), v.shape[-1]))
    labels = np.array([clip(j, clip_k) for j in range(-(n - 1), n)]) + clip_k
    for t, (b, h, i) in enumerate(rows):
        idx = labels[np.arange(n) - i + (n - 1)]  # label row of (i, j) for all j
        tk = _table_for_head(aK, h)
        tv = _table_for_head(aV, h)
        keys = k[b, h] + (tk[idx] if tk is not None else 0.0)
        vals = v[b, h] + (tv[idx] if tv is not None else 0.0)
        e = s * (keys @ q[b, h, i])
        ok = np.arange(n) < lens[b]
        if causal:
            ok &= np.arange(n) <= i
        if not ok.any():
            continue
        w = np.exp(e[ok] - e[ok].max())
        out[t] = (w / w.sum()) @ vals[ok]
    return out


# ---------------------------------------------------------------------------
# T5 scalar bias (survey page "Relative position embeddings", section "T5")
# ---------------------------------------------------------------------------

def t5_attention(q, k, v, bias, num_buckets: int = 32, max_distance: int = 128,
                 bidirectional: bool = True, scale=None, causal: bool = False,
                 key_lens=None):
    """A_ij = scale * q_i.k_j + bias[beta(j-i), h], softmax, z_i = sum alpha_ij v_j.

    bias: [num_buckets, H]; T5 uses no 1/sqrt(d) scaling, so scale defaults to 1.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    bias = to_f64(bias)
    B, H, n, d = q.shape
    s = 1.0 if (scale is None or scale <= 0) else float(scale)
    lens = _key_lengths(key_lens, B, n)
    Bm = t5_bucket_matrix(n, num_buckets, max_distance, bidirectional)
    z = np.zeros((B, H, n, v.shape[-1]))
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            e = s * (q[b, h] @ k[b, h].T) + bias[Bm, h]
            z[b, h] = _masked_softmax_rows(e, ok) @ v[b, h]
    return z


def t5_rows(q, k, v, bias, num_buckets: int = 32, max_distance: int = 128,
            bidirectional: bool = True, scale=None, causal: bool = False,
            key_lens=None, rows=()):
    """T5 output rows z[b, h, i] for a list of (b, h, i)."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    bias = to_f64(bias)
    B, H, n, d = q.shape
    s = 1.0 if (scale is None or scale <= 0) else float(scale)
    lens = _key_lengths(key_lens, B, n)
    by_delta = np.array([t5_bucket(x, num_buckets, max_distance, bidirectional)
                         for x in range(-(n - 1), n)])
    out = np.zeros((len(rows), v.shape[-1]))
    for t, (b, h, i) in enumerate(rows):
        bk = by_delta[np.arange(n) - i + (n - 1)]
        e = s * (k[b, h] @ q[b, h, i]) + bias[bk, h]
        ok = np.arange(n) < lens[b]
        if causal:
            ok &= np.arange(n) <= i
        if not ok.any():
            continue
        w = np.exp(e[ok] - e[ok].max())
        out[t] = (w / w.sum()) @ v[b, h][ok]
    return out


# ---------------------------------------------------------------------------
# Incremental decoding over a key/value cache
# ---------------------------------------------------------------------------

def _decode_positions(Tq, L, cache_lens, B):
    """Position of query t of batch b: len_b - Tq + t, with len_b clamped to [0, L]."""
    lens = [L] * B if cache_lens is None else [min(max(int(x), 0), L) for x in cache_lens]
    return [[lens[b] - Tq + t for t in range(Tq)] for b in range(B)]


def relattn_decode(q, k, v, aK=None, aV=None, clip_k: int = 0, scale=None, cache_lens=None):
    """The newest Tq positions of each sequence attending over its cache.

    q: [B, H, Tq, d]; k, v: [B, H, L, d] (the cache); aK, aV: [Ht, 2k+1, d] or
    None; cache_lens: [B] valid cache rows per batch (None = L), the new
    positions included.  Query t of batch b sits at position i = len_b - Tq + t
    and sees the keys j <= i (the causal mask of a decoder).  Each output row
    is Eq. 3 with the logits of Eq. 4 (paper-summary page, section 3.4, with
    r = clip(j - i, k)), computed here key by key; a query with no visible key
    (i < 0) outputs zeros.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    aK, aV = to_f64(aK), to_f64(aV)
    B, H, Tq, d = q.shape
    L = k.shape[2]
    s = _default_scale(d, scale)
    pos = _decode_positions(Tq, L, cache_lens, B)
    z = np.zeros((B, H, Tq, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            tk, tv = _table_for_head(aK, h), _table_for_head(aV, h)
            for t in range(Tq):
                i = pos[b][t]
                if i < 0:
                    continue
                e = np.empty(i + 1)
                vals = np.empty((i + 1, v.shape[-1]))
                for j in range(i + 1):
                    r = clip(j - i, clip_k) + clip_k
                    key = k[b, h, j] + (tk[r] if tk is not None else 0.0)
                    e[j] = s * float(q[b, h, t] @ key)
                    vals[j] = v[b, h, j] + (tv[r] if tv is not None else 0.0)
                w = np.exp(e - e.max())
                z[b, h, t] = (w / w.sum()) @ vals
    return z


def t5_decode(q, k, v, bias, num_buckets: int = 32, max_distance: int = 128,
              bidirectional: bool = True, scale=None, cache_lens=None):
    """T5 bias (survey page, section "T5") for the newest Tq positions over a
    cache; positions and visibility as in ``relattn_decode``."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    bias = to_f64(bias)
    B, H, Tq, d = q.shape
    L = k.shape[2]
    s = 1.0 if (scale is None or scale <= 0) else float(scale)
    pos = _decode_positions(Tq, L, cache_lens, B)
    z = np.zeros((B, H, Tq, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            for t in range(Tq):
                i = pos[b][t]
                if i < 0:
                    continue
                e = np.array([s * float(q[b, h, t] @ k[b, h, j]) +
                              bias[t5_bucket(j - i, num_buckets, max_distance, bidirectional), h]
                              for j in range(i + 1)])
                w = np.exp(e - e.max())
                z[b, h, t] = (w / w.sum()) @ v[b, h, :i + 1]
    return z


# ---------------------------------------------------------------------------
# Scalar bias by clipped offset (survey page "Relative position embeddings",
# section "Placement in the taxonomy": the T5 bias with its bucket table
# replaced by a function of the offset, -m_h |delta| giving ALiBi)
# ---------------------------------------------------------------------------

def offset_bias_attention(q, k, v, bias, window: int, scale=None, causal: bool = False,
                          key_lens=None):
    """A_ij = scale * q_i.k_j + bias[h', clip(j - i, window) + window], softmax,
    z_i = sum_j alpha_ij v_j.

    bias: [Hb, 2*window + 1] with Hb in {1, H} (Hb == 1: one row for every
    head); entry window + delta holds offset delta; offsets beyond +-window
    take the end entries (the clip of the tables of Shaw et al.).  scale
    defaults to 1/sqrt(d), the attention this bias is added to.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    bias = to_f64(bias)
    B, H, n, d = q.shape
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    R = relative_labels(n, window) + window  # n x n entry index
    z = np.zeros((B, H, n, v.shape[-1]))
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            row = bias[0 if bias.shape[0] == 1 else h]
            e = s * (q[b, h] @ k[b, h].T) + row[R]
            z[b, h] = _masked_softmax_rows(e, ok) @ v[b, h]
    return z


def offset_bias_decode(q, k, v, bias, window: int, scale=None, cache_lens=None):
    """The offset-bias attention (ALiBi as a table) for the newest Tq positions
    over a cache: query t of batch b sits at position len_b - Tq + t and sees
    keys 0 .. that position; e_j = scale * q.k_j + bias[h', clip(j - i, W) + W].
    scale defaults to 1/sqrt(d); positions and visibility as in
    ``relattn_decode``."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    bias = to_f64(bias)
    B, H, Tq, d = q.shape
    L = k.shape[2]
    s = _default_scale(d, scale)
    pos = _decode_positions(Tq, L, cache_lens, B)
    z = np.zeros((B, H, Tq, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            row = bias[0 if bias.shape[0] == 1 else h]
            for t in range(Tq):
                i = pos[b][t]
                if i < 0:
                    continue
                e = np.array([s * float(q[b, h, t] @ k[b, h, j]) + row[clip(j - i, window) + window]
                              for j in range(i + 1)])
                w = np.exp(e - e.max())
                z[b, h, t] = (w / w.sum()) @ v[b, h, :i + 1]
    return z


# ---------------------------------------------------------------------------
# Backward: gradients of a loss through the forward of Eq. 3 and Eq. 4 (and of
# the T5 bias), by the chain rule written out term by term.  dz is the
# gradient of the loss with respect to the output z.
# ---------------------------------------------------------------------------

def relattn_backward(q, k, v, aK=None, aV=None, clip_k: int = 0, dz=None, scale=None,
                     causal: bool = False, key_lens=None):
    """Gradients (dq, dk, dv, daK, daV) of sum(dz * z), z = relattn_bruteforce(...).

    For one head, with alpha the masked softmax of e_ij = s q_i.(k_j + a^K_ij)
    and z_i = sum_j alpha_ij (v_j + a^V_ij):
      dalpha_ij = dz_i . (v_j + a^V_ij)
      de_ij     = alpha_ij (dalpha_ij - sum_j' alpha_ij' dalpha_ij')   (softmax)
      dq_i      = s sum_j de_ij (k_j + a^K_ij)
      dk_j      = s sum_i de_ij q_i            dv_j = sum_i alpha_ij dz_i
      da^K_r    = s sum_{(i,j): label r} de_ij q_i
      da^V_r    = sum_{(i,j): label r} alpha_ij dz_i
    Tables shared by all heads (Ht == 1) collect the sums of every head.
    Returns None for an absent table.
    """
    q, k, v, dz = to_f64(q), to_f64(k), to_f64(v), to_f64(dz)
    aK, aV = to_f64(aK), to_f64(aV)
    B, H, n, d = q.shape
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    R = relative_labels(n, clip_k) + clip_k
    nlab = 2 * clip_k + 1
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    daK = None if aK is None else np.zeros_like(aK)
    daV = None if aV is None else np.zeros_like(aV)
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            tk, tv = _table_for_head(aK, h), _table_for_head(aV, h)
            keys = k[b, h][None, :, :] + (tk[R] if tk is not None else 0.0)   # [n, n, d]
            vals = v[b, h][None, :, :] + (tv[R] if tv is not None else 0.0)
            e = s * np.einsum("id,ijd->ij", q[b, h], keys)
            alpha = _masked_softmax_rows(e, ok)
            dalpha = np.einsum("id,ijd->ij", dz[b, h], vals)
            de = alpha * (dalpha - (alpha * dalpha).sum(axis=1, keepdims=True))
            dq[b, h] = s * np.einsum("ij,ijd->id", de, keys)
            dk[b, h] = s * de.T @ q[b, h]
            dv[b, h] = alpha.T @ dz[b, h]
            hk = 0 if (aK is not None and aK.shape[0] == 1) else h
            hv = 0 if (aV is not None and aV.shape[0] == 1) else h
            for r in range(nlab):
                sel = R == r
                if daK is not None:
                    daK[hk, r] += s * (de * sel).sum(axis=1) @ q[b, h]
                if daV is not None:
                    daV[hv, r] += (alpha * sel).sum(axis=1) @ dz[b, h]
    return dq, dk, dv, daK, daV


def t5_backward(q, k, v, bias, num_buckets: int = 32, max_distance: int = 128,
                bidirectional: bool = True, dz=None, scale=None, causal: bool = False,
                key_lens=None):
    """Gradients (dq, dk, dv, dbias) of sum(dz * z) for the T5 bias attention:
    de as in ``relattn_backward`` with dalpha_ij = dz_i . v_j, and
    dbias[beta, h] = sum over the pairs of bucket beta of de_ij."""
    q, k, v, dz = to_f64(q), to_f64(k), to_f64(v), to_f64(dz)
    bias = to_f64(bias)
    B, H, n, d = q.shape
    s = 1.0 if (scale is None or scale <= 0) else float(scale)
    lens = _key_lengths(key_lens, B, n)
    Bm = t5_bucket_matrix(n, num_buckets, max_distance, bidirectional)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    db = np.zeros_like(bias)
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            e = s * (q[b, h] @ k[b, h].T) + bias[Bm, h]
            alpha = _masked_softmax_rows(e, ok)
            dalpha = dz[b, h] @ v[b, h].T
            de = alpha * (dalpha - (alpha * dalpha).sum(axis=1, keepdims=True))
            dq[b, h] = s * de @ k[b, h]
            dk[b, h] = s * de.T @ q[b, h]
            dv[b, h] = alpha.T @ dz[b, h]
            db[:, h] += np.bincount(Bm.ravel(), weights=de.ravel(), minlength=num_buckets)
    return dq, dk, dv, db


def offset_bias_backward(q, k, v, bias, window: int, dz=None, scale=None,
                         causal: bool = False, key_lens=None):
    """Gradients (dq, dk, dv, dbias) of sum(dz * z) for offset_bias_attention:
    de as in ``relattn_backward`` with dalpha_ij = dz_i . v_j, and dbias[h', w]
    = sum over the pairs whose clipped offset has entry w of de_ij (summed over
    the heads when one row serves every head)."""
    q, k, v, dz = to_f64(q), to_f64(k), to_f64(v), to_f64(dz)
    bias = to_f64(bias)
    B, H, n, d = q.shape
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    R = relative_labels(n, window) + window
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    db = np.zeros_like(bias)
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            hb = 0 if bias.shape[0] == 1 else h
            e = s * (q[b, h] @ k[b, h].T) + bias[hb][R]
            alpha = _masked_softmax_rows(e, ok)
            dalpha = dz[b, h] @ v[b, h].T
            de = alpha * (dalpha - (alpha * dalpha).sum(axis=1, keepdims=True))
            dq[b, h] = s * de @ k[b, h]
            dk[b, h] = s * de.T @ q[b, h]
            dv[b, h] = alpha.T @ dz[b, h]
            db[hb] += np.bincount(R.ravel(), weights=de.ravel(), minlength=2 * window + 1)
    return dq, dk, dv, db


def xl_attention(q, k, v, R, u, vb, window: int, scale=None, causal: bool = False,
                 key_lens=None):
    """Transformer-XL relative logits (transformer-xl page, the four-term score;
    survey page, section "Transformer-XL"):

        A_ij = s * [ q_i.k_j  +  q_i.R_{i-j}  +  u.k_j  +  v.R_{i-j} ]
                      (a)          (b)          (c)        (d)

    R: [Hr, 2*window + 1, d], row window + (i - j) holds distance i - j;
    distances beyond +-window take the end rows.  u, vb: [Hu, d] (Hr, Hu in
    {1, H}; 1 = shared by all heads).  Softmax over the visible keys, z = alpha V
    (no value term).  s defaults to 1/sqrt(d).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    R, u, vb = to_f64(R), to_f64(u), to_f64(vb)
    B, H, n, d = q.shape
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    dist = np.clip(i - j, -window, window) + window  # row of R for each pair
    z = np.zeros((B, H, n, v.shape[-1]))
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            Rh = R[0 if R.shape[0] == 1 else h][dist]          # [n, n, d]
            uh = u[0 if u.shape[0] == 1 else h]
            vh = vb[0 if vb.shape[0] == 1 else h]
            term_a = q[b, h] @ k[b, h].T
            term_b = np.einsum("id,ijd->ij", q[b, h], Rh)
            term_c = (k[b, h] @ uh)[None, :]
            term_d = np.einsum("d,ijd->ij", vh, Rh)
            e = s * (term_a + term_b + term_c + term_d)
            z[b, h] = _masked_softmax_rows(e, ok) @ v[b, h]
    return z


def xl_backward(q, k, v, R, u, vb, window: int, dz=None, scale=None, causal: bool = False,
                key_lens=None):
    """Gradients (dq, dk, dv, dR, du, dvb) of sum(dz * z) for xl_attention, by
    the chain rule through the four-term score written as
    e_ij = s [(q_i + u).k_j + (q_i + v).R_{i-j}]:
    de_ij = alpha_ij (dalpha_ij - sum_j' alpha_ij' dalpha_ij') with dalpha_ij =
    dz_i . v_j, and
        dq_i = s sum_j de_ij (k_j + R_{i-j})      dk_j = s sum_i de_ij (q_i + u)
        dv_j = sum_i alpha_ij dz_i
        dR_r = s sum over pairs with row r of de_ij (q_i + v)
        du = s sum_ij de_ij k_j                   dv_bias = s sum_ij de_ij R_{i-j}
    Tables shared by the heads (leading dimension 1) get the sum over heads."""
    q, k, v, dz = to_f64(q), to_f64(k), to_f64(v), to_f64(dz)
    R, u, vb = to_f64(R), to_f64(u), to_f64(vb)
    B, H, n, d = q.shape
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    dist = np.clip(i - j, -window, window) + window
    nrow = 2 * window + 1
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dR, du, dvb = np.zeros_like(R), np.zeros_like(u), np.zeros_like(vb)
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            hr = 0 if R.shape[0] == 1 else h
            hu = 0 if u.shape[0] == 1 else h
            hv = 0 if vb.shape[0] == 1 else h
            Rh = R[hr][dist]                                    # [n, n, d]
            a = q[b, h] + u[hu]                                 # content query
            c = q[b, h] + vb[hv]                                # position query
            e = s * (a @ k[b, h].T + np.einsum("id,ijd->ij", c, Rh))
            alpha = _masked_softmax_rows(e, ok)
            dalpha = dz[b, h] @ v[b, h].T
            de = alpha * (dalpha - (alpha * dalpha).sum(axis=1, keepdims=True))
            dq[b, h] = s * (de @ k[b, h] + np.einsum("ij,ijd->id", de, Rh))
            dk[b, h] = s * de.T @ a
            dv[b, h] = alpha.T @ dz[b, h]
            # per query, the sum of de over the pairs of each row of R
            G = np.zeros((n, nrow))
            for t in range(n):
                G[t] = np.bincount(dist[t], weights=de[t], minlength=nrow)
            dR[hr] += s * G.T @ c
            du[hu] += s * de.sum(axis=0) @ k[b, h]
            dvb[hv] += s * G.sum(axis=0) @ R[hr]
    return dq, dk, dv, dR, du, dvb


def xl_decode(q, k, v, R, u, vb, window: int, scale=None, cache_lens=None):
    """Transformer-XL logits for the newest Tq positions over a cache (the
    evaluation setting of the transformer-xl page: each new token attends over
    everything before it): query t of batch b at position i = len_b - Tq + t
    sees keys 0 .. i, e_j = s [q.k_j + q.R_{i-j} + u.k_j + v.R_{i-j}] with R's
    row window + (i - j), distances beyond the window taking the end row.
    Positions and visibility as in ``relattn_decode``."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    R, u, vb = to_f64(R), to_f64(u), to_f64(vb)
    B, H, Tq, d = q.shape
    L = k.shape[2]
    s = _default_scale(d, scale)
    pos = _decode_positions(Tq, L, cache_lens, B)
    z = np.zeros((B, H, Tq, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            Rh = R[0 if R.shape[0] == 1 else h]
            uh = u[0 if u.shape[0] == 1 else h]
            vh = vb[0 if vb.shape[0] == 1 else h]
            for t in range(Tq):
                i = pos[b][t]
                if i < 0:
                    continue
                e = np.array([s * (float(q[b, h, t] @ k[b, h, j])
                                   + float(q[b, h, t] @ Rh[clip(i - j, window) + window])
                                   + float(uh @ k[b, h, j])
                                   + float(vh @ Rh[clip(i - j, window) + window]))
                              for j in range(i + 1)])
                w = np.exp(e - e.max())
                z[b, h, t] = (w / w.sum()) @ v[b, h, :i + 1]
    return z


def grid_bias_attention(q, k, v, bias, window: int, scale=None, key_lens=None):
    """Swin-style relative position bias on an M x M window (survey page,
    "Relative position embeddings": the T5 scalar bias ported to a grid, the
    table indexed by the flattened 2-D offset):

        A_ij = s q_i.k_j + bias[h', (y_j - y_i + M - 1)(2M - 1) + (x_j - x_i + M - 1)]

    with token p at (y, x) = (p div M, p mod M), n = M * M.  bias: [Hb,
    (2M-1)^2], Hb in {1, H}.  s defaults to 1/sqrt(d).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    bias = to_f64(bias)
    B, H, n, d = q.shape
    M = int(window)
    assert n == M * M
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    y, x = np.divmod(np.arange(n), M)
    entry = (y[None, :] - y[:, None] + M - 1) * (2 * M - 1) + (x[None, :] - x[:, None] + M - 1)
    z = np.zeros((B, H, n, v.shape[-1]))
    for b in range(B):
        ok = visible(n, False, lens[b])
        for h in range(H):
            row = bias[0 if bias.shape[0] == 1 else h]
            e = s * (q[b, h] @ k[b, h].T) + row[entry]
            z[b, h] = _masked_softmax_rows(e, ok) @ v[b, h]
    return z


def grid_bias_backward(q, k, v, bias, window: int, dz=None, scale=None, key_lens=None):
    """Gradients (dq, dk, dv, dbias) of sum(dz * z) for grid_bias_attention, the
    2-D window bias as a function of its table (survey page, "Relative position
    embeddings", Swin paragraph): de_ij = alpha_ij (dalpha_ij - sum_j' alpha_ij'
    dalpha_ij') with dalpha_ij = dz_i . v_j, dq = s de k, dk = s de^T q,
    dv = alpha^T dz, and dbias[h', e] = the sum of de_ij over the pairs whose
    flattened 2-D offset is entry e (summed over the heads when one row serves
    every head)."""
    q, k, v, dz = to_f64(q), to_f64(k), to_f64(v), to_f64(dz)
    bias = to_f64(bias)
    B, H, n, d = q.shape
    M = int(window)
    assert n == M * M
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    y, x = np.divmod(np.arange(n), M)
    entry = (y[None, :] - y[:, None] + M - 1) * (2 * M - 1) + (x[None, :] - x[:, None] + M - 1)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    db = np.zeros_like(bias)
    for b in range(B):
        ok = visible(n, False, lens[b])
        for h in range(H):
            hb = 0 if bias.shape[0] == 1 else h
            e = s * (q[b, h] @ k[b, h].T) + bias[hb][entry]
            alpha = _masked_softmax_rows(e, ok)
            dalpha = dz[b, h] @ v[b, h].T
            de = alpha * (dalpha - (alpha * dalpha).sum(axis=1, keepdims=True))
            dq[b, h] = s * de @ k[b, h]
            dk[b, h] = s * de.T @ q[b, h]
            dv[b, h] = alpha.T @ dz[b, h]
            db[hb] += np.bincount(entry.ravel(), weights=de.ravel(),
                                  minlength=(2 * M - 1) ** 2)
    return dq, dk, dv, db


# ---------------------------------------------------------------------------
# Per-pair edge labels ("Self-Attention with Relative Position
# Representations" summary page: the input as a labeled, directed, fully
# connected graph whose edge labels need not be positions; survey page,
# "Relative position embeddings", section "Placement in the taxonomy": the
# scalar bias by a label of the pair)
# ---------------------------------------------------------------------------

def edge_label_attention(q, k, v, labels, bias, scale=None, causal: bool = False,
                         key_lens=None):
    """A_ij = scale * q_i.k_j + bias[h', E[b, i, j]], softmax, z_i = sum_j alpha_ij v_j.

    labels: [B, n, n] integers in [0, NL), the label of the edge from query i
    to key j, the same for every head of a batch entry.  bias: [Hb, NL] with
    Hb in {1, H} (Hb == 1: one row for every head).  scale defaults to
    1/sqrt(d).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    bias = to_f64(bias)
    E = np.asarray(labels).astype(np.int64)
    B, H, n, d = q.shape
    assert E.shape == (B, n, n)
    assert E.min(initial=0) >= 0 and E.max(initial=0) < bias.shape[1]
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    z = np.zeros((B, H, n, v.shape[-1]))
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            row = bias[0 if bias.shape[0] == 1 else h]
            e = s * (q[b, h] @ k[b, h].T) + row[E[b]]
            z[b, h] = _masked_softmax_rows(e, ok) @ v[b, h]
    return z


def edge_label_backward(q, k, v, labels, bias, dz=None, scale=None, causal: bool = False,
                        key_lens=None):
    """Gradients (dq, dk, dv, dbias) of sum(dz * z) for edge_label_attention, the
    scalar bias looked up by each pair's label, by the chain rule: de_ij =
    alpha_ij (dalpha_ij - sum_j' alpha_ij' dalpha_ij') with dalpha_ij = dz_i . v_j,
    dq = s de k, dk = s de^T q, dv = alpha^T dz, and dbias[h', l] = the sum of
    de_ij over the pairs labelled l (over the heads h' covers and the batch)."""
    q, k, v, dz = to_f64(q), to_f64(k), to_f64(v), to_f64(dz)
    bias = to_f64(bias)
    E = np.asarray(labels).astype(np.int64)
    B, H, n, d = q.shape
    assert E.shape == (B, n, n)
    assert E.min(initial=0) >= 0 and E.max(initial=0) < bias.shape[1]
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    db = np.zeros_like(bias)
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            hb = 0 if bias.shape[0] == 1 else h
            e = s * (q[b, h] @ k[b, h].T) + bias[hb][E[b]]
            alpha = _masked_softmax_rows(e, ok)
            dalpha = dz[b, h] @ v[b, h].T
            de = alpha * (dalpha - (alpha * dalpha).sum(axis=1, keepdims=True))
            dq[b, h] = s * de @ k[b, h]
            dk[b, h] = s * de.T @ q[b, h]
            dv[b, h] = alpha.T @ dz[b, h]
            db[hb] += np.bincount(E[b].ravel(), weights=de.ravel(), minlength=bias.shape[1])
    return dq, dk, dv, db


def edge_label_relattn(q, k, v, labels, aK=None, aV=None, scale=None, causal: bool = False,
                       key_lens=None):
    """Relation-aware self-attention (Eq. 4 and Eq. 3) over a labeled graph:
    a^K_ij = aK[h', E[b, i, j]], a^V_ij = aV[h', E[b, i, j]], materialised.

        e_ij = scale * q_i . (k_j + a^K_ij),   z_i = sum_j alpha_ij (v_j + a^V_ij)

    labels: [B, n, n] integers in [0, NL), shared by the heads; aK, aV: [Ht, NL,
    d] with Ht in {1, H}, either may be None (absent = zero).  scale defaults to
    1/sqrt(d).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    aK, aV = to_f64(aK), to_f64(aV)
    E = np.asarray(labels).astype(np.int64)
    B, H, n, d = q.shape
    assert E.shape == (B, n, n)
    for t in (aK, aV):
        if t is not None:
            assert E.min(initial=0) >= 0 and E.max(initial=0) < t.shape[1]
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    z = np.zeros((B, H, n, v.shape[-1]))
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            kk = k[b, h][None, :, :]                                  # [1, n, d]
            if aK is not None:
                kk = kk + _table_for_head(aK, h)[E[b]]                # [n, n, d]
            e = s * np.einsum("id,ijd->ij", q[b, h], np.broadcast_to(kk, (n, n, d)))
            alpha = _masked_softmax_rows(e, ok)
            vv = v[b, h][None, :, :]
            if aV is not None:
                vv = vv + _table_for_head(aV, h)[E[b]]
            z[b, h] = np.einsum("ij,ijd->id", alpha, np.broadcast_to(vv, (n, n, v.shape[-1])))
    return z


def edge_label_relattn_backward(q, k, v, labels, aK=None, aV=None, dz=None, scale=None,
                                causal: bool = False, key_lens=None):
    """Gradients (dq, dk, dv, daK, daV) of sum(dz * z) for edge_label_relattn,
    by the chain rule through Eq. 4 and Eq. 3 with each pair's tables read by
    its label: dalpha_ij = dz_i . (v_j + a^V_ij), de_ij = alpha_ij (dalpha_ij -
    sum_j' alpha_ij' dalpha_ij'), and
        dq_i = s sum_j de_ij (k_j + a^K_ij)     dk_j = s sum_i de_ij q_i
        dv_j = sum_i alpha_ij dz_i
        daK[l] = s sum over the pairs labelled l of de_ij q_i
        daV[l] = sum over the pairs labelled l of alpha_ij dz_i
    (summed over the heads for a shared table; None for an absent table)."""
    q, k, v, dz = to_f64(q), to_f64(k), to_f64(v), to_f64(dz)
    aK, aV = to_f64(aK), to_f64(aV)
    E = np.asarray(labels).astype(np.int64)
    B, H, n, d = q.shape
    assert E.shape == (B, n, n)
    s = _default_scale(d, scale)
    lens = _key_lengths(key_lens, B, n)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    daK = None if aK is None else np.zeros_like(aK)
    daV = None if aV is None else np.zeros_like(aV)
    for b in range(B):
        ok = visible(n, causal, lens[b])
        for h in range(H):
            kk = np.broadcast_to(k[b, h][None, :, :], (n, n, d))
            if aK is not None:
                kk = kk + _table_for_head(aK, h)[E[b]]
            vv = np.broadcast_to(v[b, h][None, :, :], (n, n, d))
            if aV is not None:
                vv = vv + _table_for_head(aV, h)[E[b]]
            e = s * np.einsum("id,ijd->ij", q[b, h], kk)
            alpha = _masked_softmax_rows(e, ok)
            dalpha = np.einsum("id,ijd->ij", dz[b, h], vv)
            de = alpha * (dalpha - (alpha * dalpha).sum(axis=1, keepdims=True))
            dq[b, h] = s * np.einsum("ij,ijd->id", de, kk)
            dk[b, h] = s * de.T @ q[b, h]
            dv[b, h] = alpha.T @ dz[b, h]
            for i in range(n):
                if aK is not None:
                    gk = np.bincount(E[b, i], weights=de[i], minlength=aK.shape[1])
                    daK[0 if aK.shape[0] == 1 else h] += s * gk[:, None] * q[b, h, i][None, :]
                if aV is not None:
                    gv = np.bincount(E[b, i], weights=alpha[i], minlength=aV.shape[1])
                    daV[0 if aV.shape[0] == 1 else h] += gv[:, None] * dz[b, h, i][None, :]
    return dq, dk, dv, daK, daV
