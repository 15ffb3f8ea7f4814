"""Pins of the fp64 oracle against what the pages and the mathematics fix.

No GPU.  Each test names the passage (page title, section / equation) it
checks.  Sources of stored values are the JSON files in tests/golden/, each with
its citation; none was produced by the HIP path.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import relattn_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rnd(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def sdpa(q, k, v, ok, scale):
    """Textbook attention (Eq. 1-2) by a library routine, fp64 on the CPU."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(ok), scale=scale).numpy()


# ---------------------------------------------------------------------------
# labels: paper summary page, "Relative Position Representations: From
# Arbitrary Edges to Sequences"
# ---------------------------------------------------------------------------

def test_clip_worked_values():
    g = golden("clip_worked_values.json")
    for x, want in g["clip_k4"]:
        assert oracle.clip(x, 4) == want
    d = g["direction"]
    R = oracle.relative_labels(8, 4)
    assert R[d["i"], d["j"]] == d["forward"]
    assert R[d["j"], d["i"]] == d["reverse"]


def test_label_counts():
    g = golden("clip_worked_values.json")
    for k, count in g["label_count"]:
        R = oracle.relative_labels(2 * k + 5, k)
        assert len(np.unique(R)) == count
    assert sorted(np.unique(oracle.relative_labels(12, 4)).tolist()) == g["labels_k4"]


def test_k0_single_label():
    # k = 0: every pair gets the same label (Table 2 discussion of k = 0).
    assert np.all(oracle.relative_labels(9, 0) == 0)


# ---------------------------------------------------------------------------
# T5 buckets: survey page "Relative position embeddings", section "T5"
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["default_bidirectional", "small_bidirectional",
                                  "small_unidirectional"])
def test_t5_bucket_hand_table(case):
    g = golden("t5_buckets.json")[case]
    for delta, want in g["delta_to_bucket"]:
        got = oracle.t5_bucket(delta, g["num_buckets"], g["max_distance"],
                               g["bidirectional"])
        assert got == want, (delta, got, want)


def test_t5_first_distance_per_bucket():
    g = golden("t5_buckets.json")["default_bidirectional"]
    for bucket, first in g["first_distance_of_bucket"]:
        assert oracle.t5_bucket(-first) == bucket
        assert oracle.t5_bucket(-(first - 1)) == bucket - 1


def test_t5_bucket_matches_real_formula_away_from_ties():
    """Exact floor equals the floating-point evaluation of the printed formula
    wherever the real value is not within 1e-9 of an integer."""
    for (B, D, bidir) in [(32, 128, True), (32, 128, False), (16, 64, True),
                          (64, 256, True), (8, 8, False)]:
        half = B // 2 if bidir else B
        ex = half // 2
        for a in range(ex, 3000):
            x = math.log(a / ex) / math.log(D / ex) * (half - ex)
            if abs(x - round(x)) < 1e-9:
                continue
            want = min(half - 1, ex + math.floor(x))
            assert oracle.t5_bucket(-a, B, D, bidir) == want, (B, D, a)


def test_t5_bucket_ties_are_exact():
    # a = 16, 32, 64 make 2*log2(a/8) exactly 2, 4, 6 (B=32, D=128).
    for a, want in [(16, 10), (32, 12), (64, 14)]:
        assert oracle.t5_bucket(-a) == want
        assert oracle.t5_bucket(a) == want + 16


def test_t5_param_count():
    # 32 buckets x 12 heads = 384 numbers (T5 section); the bias table of the
    # T5 workload is [num_buckets, H].
    import workloads
    t = workloads.make_inputs("t5", batch=1, n=8)["t5_bias"]
    assert t.shape == (32, 12) and t.numel() == 384


def test_edge_table_param_counts():
    # Per-head tables of the big model with k = 8: 16*17*64*2 = 34,816 numbers;
    # shared across heads: 17*64*2 = 2,176 ("Key Design Choices", per-head
    # versus shared edge representations).
    assert 16 * (2 * 8 + 1) * 64 * 2 == 34816
    assert (2 * 8 + 1) * 64 * 2 == 2176


# ---------------------------------------------------------------------------
# hand-worked examples (Eq. 3, Eq. 4; T5 logit)
# ---------------------------------------------------------------------------

def _softmax(x):
    x = np.asarray(x, dtype=np.float64)
    w = np.exp(x - x.max())
    return w / w.sum()


def test_shaw_worked_example():
    g = golden("shaw_worked_example.json")
    q, k, v = (np.array(g[x], dtype=np.float64) for x in "qkv")
    wK, wV = np.array(g["wK"], float), np.array(g["wV"], float)
    c = g["clip"]
    assert oracle.relative_labels(3, c).tolist() == g["labels"]
    e = oracle.shaw_logits(q, k, wK, c)
    np.testing.assert_allclose(e, g["logits"], rtol=0, atol=1e-15)
    u = np.array(g["value_plus_edge"], float)
    want = np.stack([_softmax(g["logits"][i]) @ u[i] for i in range(3)])
    Q, K, V = (x[None, None] for x in (q, k, v))
    for fn in (oracle.relattn_bruteforce, oracle.relattn_factored):
        z = fn(Q, K, V, wK[None], wV[None], c)[0, 0]
        np.testing.assert_allclose(z, want, rtol=0, atol=1e-15)
        np.testing.assert_allclose(z[1], g["z_row1_uniform"], rtol=0, atol=1e-15)
        zc = fn(Q, K, V, wK[None], wV[None], c, causal=True)[0, 0]
        np.testing.assert_allclose(zc[0], g["causal_z"]["row0"], atol=1e-15)
        np.testing.assert_allclose(zc[1], g["causal_z"]["row1"], atol=1e-15)
        np.testing.assert_allclose(zc[2], want[2], atol=1e-15)


def test_t5_worked_example():
    g = golden("t5_worked_example.json")
    q, k, v = (np.array(g[x], dtype=np.float64)[None, None] for x in "qkv")
    bias = np.array(g["bias"], float)[:, None]
    Bm = oracle.t5_bucket_matrix(3, g["num_buckets"], g["max_distance"],
                                 g["bidirectional"])
    assert Bm.tolist() == g["buckets"]
    want = np.stack([_softmax(g["logits"][i]) @ v[0, 0] for i in range(3)])
    z = oracle.t5_attention(q, k, v, bias, g["num_buckets"], g["max_distance"],
                            g["bidirectional"])[0, 0]
    np.testing.assert_allclose(z, want, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# special cases that reduce to textbook attention (Eq. 1, Eq. 2)
# ---------------------------------------------------------------------------

MASKS = [(False, None), (True, None), (False, [5, 11]), (True, [7, 11])]


@pytest.mark.parametrize("causal,lens", MASKS)
def test_zero_tables_equal_textbook_attention(causal, lens):
    B, H, n, d, c = 2, 3, 11, 8, 3
    q, k, v = rnd((B, H, n, d), 1), rnd((B, H, n, d), 2), rnd((B, H, n, d), 3)
    zeros = np.zeros((H, 2 * c + 1, d))
    for b in range(B):
        ok = oracle.visible(n, causal, n if lens is None else lens[b])
        ref = sdpa(q[b], k[b], v[b], ok, 1 / math.sqrt(d))
        for fn in (oracle.relattn_bruteforce, oracle.relattn_factored):
            for tables in ((zeros, zeros), (None, None)):
                z = fn(q, k, v, *tables, c, causal=causal, key_lens=lens)
                np.testing.assert_allclose(z[b], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal,lens", MASKS)
def test_t5_zero_bias_equals_unscaled_attention(causal, lens):
    B, H, n, d = 2, 3, 13, 8
    q, k, v = rnd((B, H, n, d), 4), rnd((B, H, n, d), 5), rnd((B, H, n, d), 6)
    z = oracle.t5_attention(q, k, v, np.zeros((32, H)), causal=causal, key_lens=lens)
    for b in range(B):
        ok = oracle.visible(n, causal, n if lens is None else lens[b])
        np.testing.assert_allclose(z[b], sdpa(q[b], k[b], v[b], ok, 1.0),
                                   rtol=1e-12, atol=1e-12)


def test_k0_closed_form():
    """k = 0: q_i.w^K_0 is constant per row, so alpha is vanilla attention and,
    since every row of alpha sums to 1, z = vanilla + w^V_0."""
    B, H, n, d = 1, 2, 10, 8
    q, k, v = rnd((B, H, n, d), 7), rnd((B, H, n, d), 8), rnd((B, H, n, d), 9)
    wK, wV = rnd((H, 1, d), 10), rnd((H, 1, d), 11)
    for causal in (False, True):
        ok = oracle.visible(n, causal, n)
        for fn in (oracle.relattn_bruteforce, oracle.relattn_factored):
            z = fn(q, k, v, wK, wV, 0, causal=causal)
            for h in range(H):
                want = sdpa(q[0, h], k[0, h], v[0, h], ok, 1 / math.sqrt(d)) + wV[h, 0]
                np.testing.assert_allclose(z[0, h], want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# invariants of alpha and of the bucket sums (softmax under Eq. 2; Eq. 5 split)
# ---------------------------------------------------------------------------

def test_alpha_rows_and_bucket_sums():
    B, H, n, d, c = 2, 2, 14, 8, 3
    q, k, v = rnd((B, H, n, d), 12), rnd((B, H, n, d), 13), rnd((B, H, n, d), 14)
    wK, wV = rnd((H, 2 * c + 1, d), 15), rnd((H, 2 * c + 1, d), 16)
    lens = [9, 0]
    _, alpha = oracle.relattn_bruteforce(q, k, v, wK, wV, c, causal=True,
                                         key_lens=lens, return_alpha=True)
    _, S = oracle.relattn_factored(q, k, v, wK, wV, c, causal=True, key_lens=lens,
                                   return_bucket_sums=True)
    np.testing.assert_allclose(alpha[0].sum(-1), 1.0, atol=1e-14)
    assert np.all(alpha[1] == 0)              # len 0: no visible key
    np.testing.assert_allclose(S[0].sum(-1), 1.0, atol=1e-14)
    assert np.all(alpha[0][..., :, 9:] == 0)  # padded keys get no weight
    for h in range(H):
        for i in range(n):
            for r in range(1, 2 * c):          # interior label: one key only
                j = i + r - c
                if 0 <= j < n:
                    assert S[0, h, i, r] == pytest.approx(alpha[0, h, i, j], abs=1e-15)


# ---------------------------------------------------------------------------
# Eq. 5: the factored form equals the definition
# ---------------------------------------------------------------------------

def _cases():
    rng = np.random.default_rng(2026)
    for t in range(40):
        n = int(rng.integers(1, 25))
        c = int(rng.integers(0, n + 3))
        d = int(rng.choice([2, 4, 8]))
        H = int(rng.integers(1, 4))
        B = int(rng.integers(1, 3))
        causal = bool(rng.integers(0, 2))
        lens = None if rng.integers(0, 2) else [int(x) for x in rng.integers(0, n + 1, B)]
        shared = bool(rng.integers(0, 2))
        which = int(rng.integers(0, 4))  # 0 K+V, 1 K only, 2 V only, 3 none
        yield t, n, c, d, H, B, causal, lens, shared, which


@pytest.mark.parametrize("case", list(_cases()), ids=lambda c: f"case{c[0]}")
def test_factored_matches_bruteforce(case):
    t, n, c, d, H, B, causal, lens, shared, which = case
    q, k, v = (rnd((B, H, n, d), 100 * t + s) for s in range(3))
    Ht = 1 if shared else H
    wK = rnd((Ht, 2 * c + 1, d), 100 * t + 3) if which in (0, 1) else None
    wV = rnd((Ht, 2 * c + 1, d), 100 * t + 4) if which in (0, 2) else None
    scale = None if t % 3 else 0.37
    zb = oracle.relattn_bruteforce(q, k, v, wK, wV, c, scale, causal, lens)
    zf = oracle.relattn_factored(q, k, v, wK, wV, c, scale, causal, lens)
    np.testing.assert_allclose(zf, zb, rtol=0, atol=1e-12)
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(n)]
    zr = oracle.relattn_rows(q, k, v, wK, wV, c, scale, causal, lens, rows=rows)
    np.testing.assert_allclose(zr, zb.reshape(-1, zb.shape[-1]), rtol=0, atol=1e-12)


def test_t5_rows_match_full():
    B, H, n, d = 2, 3, 40, 8
    q, k, v = rnd((B, H, n, d), 20), rnd((B, H, n, d), 21), rnd((B, H, n, d), 22)
    bias = rnd((32, H), 23)
    lens = [25, 40]
    for bidir in (True, False):
        z = oracle.t5_attention(q, k, v, bias, 32, 16, bidir, key_lens=lens)
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(n)]
        zr = oracle.t5_rows(q, k, v, bias, 32, 16, bidir, key_lens=lens, rows=rows)
        np.testing.assert_allclose(zr, z.reshape(-1, d), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# clipping (section "Relative Position Representations: From Arbitrary Edges to
# Sequences"): offsets range over -(n-1)..n-1, so k >= n-1 clips nothing
# ---------------------------------------------------------------------------

def _per_offset_attention(q, k, v, tK, tV):
    """Unclipped relative attention with one vector per offset j-i, written
    directly from Eq. 3 and Eq. 4 with a^X_ij = t[j - i + n - 1] (no clip)."""
    n, d = q.shape
    out = np.zeros_like(v)
    for i in range(n):
        e = np.array([q[i] @ (k[j] + tK[j - i + n - 1]) for j in range(n)]) / math.sqrt(d)
        a = _softmax(e)
        out[i] = sum(a[j] * (v[j] + tV[j - i + n - 1]) for j in range(n))
    return out


def test_no_clipping_when_k_at_least_n_minus_1():
    n, d = 7, 4
    q, k, v = rnd((1, 1, n, d), 30), rnd((1, 1, n, d), 31), rnd((1, 1, n, d), 32)
    tK, tV = rnd((2 * n - 1, d), 33), rnd((2 * n - 1, d), 34)
    want = _per_offset_attention(q[0, 0], k[0, 0], v[0, 0], tK, tV)
    for c in (n - 1, n, n + 3):
        pad = c - (n - 1)  # table rows for |offset| > n-1 are never reachable
        wK = np.concatenate([rnd((pad, d), 35), tK, rnd((pad, d), 36)])[None]
        wV = np.concatenate([rnd((pad, d), 37), tV, rnd((pad, d), 38)])[None]
        for fn in (oracle.relattn_bruteforce, oracle.relattn_factored):
            np.testing.assert_allclose(fn(q, k, v, wK, wV, c)[0, 0], want, atol=1e-12)


# ---------------------------------------------------------------------------
# causal masking (decoder self-attention): only offsets <= 0 are visible
# ---------------------------------------------------------------------------

def test_causal_ignores_positive_offset_rows():
    B, H, n, d, c = 1, 2, 12, 8, 4
    q, k, v = rnd((B, H, n, d), 40), rnd((B, H, n, d), 41), rnd((B, H, n, d), 42)
    wK, wV = rnd((H, 2 * c + 1, d), 43), rnd((H, 2 * c + 1, d), 44)
    wK2, wV2 = wK.copy(), wV.copy()
    wK2[:, c + 1:] += 5.0  # rows of offsets 1..k
    wV2[:, c + 1:] -= 3.0
    for fn in (oracle.relattn_bruteforce, oracle.relattn_factored):
        z1 = fn(q, k, v, wK, wV, c, causal=True)
        z2 = fn(q, k, v, wK2, wV2, c, causal=True)
        assert np.array_equal(z1, z2)


def test_causal_prefix_property():
    B, H, n, d, c = 1, 2, 15, 8, 3
    q, k, v = rnd((B, H, n, d), 50), rnd((B, H, n, d), 51), rnd((B, H, n, d), 52)
    wK, wV = rnd((H, 2 * c + 1, d), 53), rnd((H, 2 * c + 1, d), 54)
    full = oracle.relattn_factored(q, k, v, wK, wV, c, causal=True)
    m = 9
    pre = oracle.relattn_bruteforce(q[..., :m, :], k[..., :m, :], v[..., :m, :],
                                    wK, wV, c, causal=True)
    np.testing.assert_allclose(pre, full[..., :m, :], atol=1e-12)


# ---------------------------------------------------------------------------
# tables shared across heads ("Efficient Implementation", edge sharing)
# ---------------------------------------------------------------------------

def test_shared_tables_equal_replicated():
    B, H, n, d, c = 2, 3, 10, 4, 2
    q, k, v = rnd((B, H, n, d), 60), rnd((B, H, n, d), 61), rnd((B, H, n, d), 62)
    wK, wV = rnd((1, 2 * c + 1, d), 63), rnd((1, 2 * c + 1, d), 64)
    for fn in (oracle.relattn_bruteforce, oracle.relattn_factored):
        z1 = fn(q, k, v, wK, wV, c)
        z2 = fn(q, k, v, np.repeat(wK, H, 0), np.repeat(wV, H, 0), c)
        assert np.array_equal(z1, z2)


# ---------------------------------------------------------------------------
# one-hot probe of the offset sign (a^K_ij = w^K_clip(j-i))
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("offset", [-3, -1, 0, 2])
def test_one_hot_probe_offset_sign(offset):
    """Only the key-table row of ``offset`` is non-zero and q is parallel to it:
    each query attends (almost) entirely to key j = i + offset.  With value
    rows v_j = e_j the output row is that one-hot vector."""
    n, c = 10, 4
    d = n + 1
    q = np.zeros((1, 1, n, d)); q[..., n] = 1.0
    k = np.zeros((1, 1, n, d))
    v = np.eye(n, d)[None, None]
    wK = np.zeros((1, 2 * c + 1, d)); wK[0, offset + c, n] = 60.0
    z = oracle.relattn_factored(q, k, v, wK, None, c)[0, 0]
    zb = oracle.relattn_bruteforce(q, k, v, wK, None, c)[0, 0]
    for i in range(n):
        j = i + offset
        if 0 <= j < n:
            assert np.argmax(z[i]) == j and z[i, j] > 0.999
            assert np.argmax(zb[i]) == j


# ---------------------------------------------------------------------------
# the pins bite: plant a mistake in the oracle and watch a pin fail
# ---------------------------------------------------------------------------

def test_planted_sign_flip_is_caught(monkeypatch):
    monkeypatch.setattr(orc, "clip", lambda x, k: max(-k, min(k, -x)))
    with pytest.raises(AssertionError):
        test_shaw_worked_example()
    with pytest.raises(AssertionError):
        test_one_hot_probe_offset_sign(2)


def test_planted_unscaled_key_term_is_caught(monkeypatch):
    real = orc.shaw_logits

    def wrong(q, k, aK, clip_k, scale=None):  # scale only on the content term
        e = real(q, k, None, clip_k, scale)
        if aK is None:
            return e
        R = orc.relative_labels(len(q), clip_k)
        return e + np.einsum("id,ijd->ij", orc.to_f64(q), orc.to_f64(aK)[R + clip_k])

    monkeypatch.setattr(orc, "shaw_logits", wrong)
    with pytest.raises(AssertionError):
        test_shaw_worked_example()


def test_planted_dropped_value_term_is_caught(monkeypatch):
    real = orc.relattn_bruteforce
    wrong = lambda q, k, v, aK=None, aV=None, *a, **kw: real(q, k, v, aK, None, *a, **kw)
    monkeypatch.setattr(orc, "relattn_bruteforce", wrong)
    monkeypatch.setattr(oracle, "relattn_bruteforce", wrong)
    with pytest.raises(AssertionError):
        test_k0_closed_form()


# ---------------------------------------------------------------------------
# incremental decoding: each new position's row is the causal forward's row at
# that position (paper-summary page §3.4, Eq. 3 and Eq. 4; the causal reading
# of the mask); the decode oracle is pinned to the forward oracle's rows and to
# closed forms
# ---------------------------------------------------------------------------

def _decode_case(seed, B=3, H=2, L=23, d=8, Tq=2):
    q_full = rnd((B, H, L, d), seed)
    k, v = rnd((B, H, L, d), seed + 1), rnd((B, H, L, d), seed + 2)
    lens = [L, 11, 1][:B]
    return q_full, k, v, lens, Tq


@pytest.mark.parametrize("c", [0, 3, 30])
@pytest.mark.parametrize("tables", ["kv", "k", "v", "none", "shared"])
def test_decode_matches_forward_rows(c, tables):
    q_full, k, v, lens, Tq = _decode_case(40 + c)
    B, H, L, d = q_full.shape
    Ht = 1 if tables == "shared" else H
    wK = rnd((Ht, 2 * c + 1, d), 50, 0.3) if tables in ("kv", "k", "shared") else None
    wV = rnd((Ht, 2 * c + 1, d), 51, 0.3) if tables in ("kv", "v", "shared") else None
    # the decode queries are the full sequence's rows at positions len - Tq + t
    q = np.zeros((B, H, Tq, d))
    rows, where = [], []
    for b in range(B):
        for t in range(Tq):
            i = lens[b] - Tq + t
            if i >= 0:
                q[b, :, t] = q_full[b, :, i]
                for h in range(H):
                    rows.append((b, h, i))
                    where.append((b, h, t))
    z = oracle.relattn_decode(q, k, v, wK, wV, c, cache_lens=lens)
    zr = oracle.relattn_rows(q_full, k, v, wK, wV, c, causal=True, key_lens=lens, rows=rows)
    for (b, h, t), row in zip(where, zr):
        np.testing.assert_allclose(z[b, h, t], row, rtol=0, atol=1e-12)
    # a query with no visible key (position < 0) outputs zeros
    assert np.all(z[2, :, 0] == 0.0) and lens[2] - Tq + 0 < 0


@pytest.mark.parametrize("bidir", [True, False])
def test_t5_decode_matches_forward_rows(bidir):
    q_full, k, v, lens, Tq = _decode_case(60, L=40)
    B, H, L, d = q_full.shape
    bias = rnd((32, H), 61)
    q = np.zeros((B, H, Tq, d))
    rows, where = [], []
    for b in range(B):
        for t in range(Tq):
            i = lens[b] - Tq + t
            if i >= 0:
                q[b, :, t] = q_full[b, :, i]
                for h in range(H):
                    rows.append((b, h, i))
                    where.append((b, h, t))
    z = oracle.t5_decode(q, k, v, bias, 32, 16, bidir, cache_lens=lens)
    zr = oracle.t5_rows(q_full, k, v, bias, 32, 16, bidir, causal=True, key_lens=lens, rows=rows)
    for (b, h, t), row in zip(where, zr):
        np.testing.assert_allclose(z[b, h, t], row, rtol=0, atol=1e-12)


def test_decode_first_position_closed_form():
    """One cached key at offset 0 (label row k): alpha = 1, so the output is
    v_0 + a^V_0 (Eq. 3) whatever the logits are."""
    B, H, L, d, c = 1, 2, 5, 4, 2
    q, k, v = rnd((B, H, 1, d), 70), rnd((B, H, L, d), 71), rnd((B, H, L, d), 72)
    wK, wV = rnd((H, 2 * c + 1, d), 73), rnd((H, 2 * c + 1, d), 74)
    z = oracle.relattn_decode(q, k, v, wK, wV, c, cache_lens=[1])
    for h in range(H):
        np.testing.assert_allclose(z[0, h, 0], v[0, h, 0] + wV[h, c], rtol=0, atol=1e-14)


def test_decode_two_keys_closed_form():
    """Two cached keys at offsets -1 and 0 with clip 1: labels 0 and 1, so
    alpha_0 = 1 / (1 + exp(e_1 - e_0)) with e_j = q.(k_j + a^K) / sqrt(d)."""
    d, c = 4, 1
    q, k, v = rnd((1, 1, 1, d), 80), rnd((1, 1, 2, d), 81), rnd((1, 1, 2, d), 82)
    wK, wV = rnd((1, 3, d), 83), rnd((1, 3, d), 84)
    e0 = q[0, 0, 0] @ (k[0, 0, 0] + wK[0, 0]) / math.sqrt(d)
    e1 = q[0, 0, 0] @ (k[0, 0, 1] + wK[0, 1]) / math.sqrt(d)
    a0 = 1.0 / (1.0 + math.exp(e1 - e0))
    want = a0 * (v[0, 0, 0] + wV[0, 0]) + (1 - a0) * (v[0, 0, 1] + wV[0, 1])
    z = oracle.relattn_decode(q, k, v, wK, wV, c, cache_lens=[2])
    np.testing.assert_allclose(z[0, 0, 0], want, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# scalar bias by clipped offset (survey page "Relative position embeddings",
# section "Placement in the taxonomy")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bidir", [True, False])
@pytest.mark.parametrize("causal,lens", [(False, None), (True, None), (False, [9, 30])])
def test_offset_bias_from_t5_buckets_equals_t5(bidir, causal, lens):
    """A table filled with the T5 bias of each offset's bucket (window large
    enough to cover every offset) gives the T5 attention, scale 1."""
    B, H, n, d = 2, 3, 30, 8
    q, k, v = rnd((B, H, n, d), 90), rnd((B, H, n, d), 91), rnd((B, H, n, d), 92)
    t5b = rnd((32, H), 93)
    W = n - 1
    table = np.array([[t5b[oracle.t5_bucket(x, 32, 16, bidir), h] for x in range(-W, W + 1)]
                      for h in range(H)])
    z = oracle.offset_bias_attention(q, k, v, table, W, scale=1.0, causal=causal, key_lens=lens)
    want = oracle.t5_attention(q, k, v, t5b, 32, 16, bidir, causal=causal, key_lens=lens)
    np.testing.assert_allclose(z, want, rtol=0, atol=1e-12)


def test_offset_bias_constant_is_textbook():
    """A bias equal for every offset cancels in the softmax: textbook scaled
    attention (library routine)."""
    B, H, n, d = 1, 2, 12, 8
    q, k, v = rnd((B, H, n, d), 94), rnd((B, H, n, d), 95), rnd((B, H, n, d), 96)
    table = np.full((1, 9), 3.7)
    z = oracle.offset_bias_attention(q, k, v, table, 4)
    ok = np.ones((n, n), dtype=bool)
    np.testing.assert_allclose(z, sdpa(q, k, v, ok, 1 / math.sqrt(d)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("offset", [-3, 0, 2])
def test_offset_bias_one_hot_probe(offset):
    """A large bias at one offset makes each query attend to the key at that
    offset (j = i + offset) when it exists: the sign and centring of the
    table index."""
    n, d, W = 8, 4, 5
    q, k, v = rnd((1, 1, n, d), 97, 0.01), rnd((1, 1, n, d), 98, 0.01), rnd((1, 1, n, d), 99)
    table = np.zeros((1, 2 * W + 1))
    table[0, W + offset] = 60.0
    z = oracle.offset_bias_attention(q, k, v, table, W)
    for i in range(n):
        if 0 <= i + offset < n:
            np.testing.assert_allclose(z[0, 0, i], v[0, 0, i + offset], atol=1e-9)


def test_alibi_window_clips_to_end_entries():
    """ALiBi (-m |delta|) with window w: offsets beyond w take the bias of w,
    which equals ALiBi with the distance capped at w."""
    B, H, n, d, w = 1, 2, 16, 8, 5
    q, k, v = rnd((B, H, n, d), 100), rnd((B, H, n, d), 101), rnd((B, H, n, d), 102)
    slopes = [0.5, 0.125]
    table = np.array([[-m * abs(x) for x in range(-w, w + 1)] for m in slopes])
    big = np.array([[-m * min(abs(x), w) for x in range(-(n - 1), n)] for m in slopes])
    z = oracle.offset_bias_attention(q, k, v, table, w, causal=True)
    z2 = oracle.offset_bias_attention(q, k, v, big, n - 1, causal=True)
    np.testing.assert_allclose(z, z2, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# backward: the chain rule through Eq. 3 and Eq. 4, pinned by central finite
# differences of the (independently pinned) forward oracle, by library
# autograd when the tables vanish, and by closed-form sums
# ---------------------------------------------------------------------------

def _fd_check(f, x, grad, idx_list, eps=1e-6, tol=1e-6):
    for idx in idx_list:
        x0 = x[idx]
        x[idx] = x0 + eps
        fp = f()
        x[idx] = x0 - eps
        fm = f()
        x[idx] = x0
        fd = (fp - fm) / (2 * eps)
        assert abs(fd - grad[idx]) <= tol * max(1.0, abs(fd)), (idx, fd, grad[idx])


@pytest.mark.parametrize("causal,lens,shared", [(False, None, False), (True, None, False),
                                               (False, [5, 7], True)])
def test_backward_matches_finite_differences(causal, lens, shared):
    B, H, n, d, c = 2, 2, 7, 4, 2
    q, k, v = rnd((B, H, n, d), 110), rnd((B, H, n, d), 111), rnd((B, H, n, d), 112)
    Ht = 1 if shared else H
    aK, aV = rnd((Ht, 2 * c + 1, d), 113, 0.5), rnd((Ht, 2 * c + 1, d), 114, 0.5)
    dz = rnd((B, H, n, d), 115)
    grads = oracle.relattn_backward(q, k, v, aK, aV, c, dz, causal=causal, key_lens=lens)
    loss = lambda: float((dz * oracle.relattn_bruteforce(q, k, v, aK, aV, c, causal=causal,
                                                         key_lens=lens)).sum())
    rng = np.random.default_rng(116)
    for x, g in zip((q, k, v, aK, aV), grads):
        idx = [tuple(int(rng.integers(s)) for s in x.shape) for _ in range(6)]
        _fd_check(loss, x, g, idx)


@pytest.mark.parametrize("bidir", [True, False])
def test_t5_backward_matches_finite_differences(bidir):
    B, H, n, d = 1, 2, 20, 4
    q, k, v = rnd((B, H, n, d), 120), rnd((B, H, n, d), 121), rnd((B, H, n, d), 122)
    bias, dz = rnd((8, H), 123), rnd((B, H, n, d), 124)
    grads = oracle.t5_backward(q, k, v, bias, 8, 12, bidir, dz, causal=True)
    loss = lambda: float((dz * oracle.t5_attention(q, k, v, bias, 8, 12, bidir,
                                                   causal=True)).sum())
    rng = np.random.default_rng(125)
    for x, g in zip((q, k, v, bias), grads):
        idx = [tuple(int(rng.integers(s)) for s in x.shape) for _ in range(6)]
        _fd_check(loss, x, g, idx)


def test_backward_zero_tables_equals_library_autograd():
    """Zero tables: the gradients of textbook attention, by torch autograd of
    the library routine in fp64."""
    B, H, n, d = 2, 2, 9, 8
    q, k, v, dz = (rnd((B, H, n, d), 130 + i) for i in range(4))
    c = 3
    z0 = np.zeros((H, 2 * c + 1, d))
    dq, dk, dv, daK, daV = oracle.relattn_backward(q, k, v, z0, z0, c, dz, causal=True)
    t = [torch.tensor(x, requires_grad=True) for x in (q, k, v)]
    out = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True)
    out.backward(torch.tensor(dz))
    for mine, theirs in zip((dq, dk, dv), t):
        np.testing.assert_allclose(mine, theirs.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_closed_form_sums():
    """Every row's weights sum to 1: the value gradients summed over keys (and
    over labels) equal the output gradients summed over queries, and the
    logit gradients of a row sum to 0, so the key-table gradient summed over
    labels is s * sum_i (sum_j de_ij) q_i = 0."""
    B, H, n, d, c = 1, 2, 10, 4, 3
    q, k, v = rnd((B, H, n, d), 140), rnd((B, H, n, d), 141), rnd((B, H, n, d), 142)
    aK, aV = rnd((H, 2 * c + 1, d), 143), rnd((H, 2 * c + 1, d), 144)
    dz = rnd((B, H, n, d), 145)
    dq, dk, dv, daK, daV = oracle.relattn_backward(q, k, v, aK, aV, c, dz)
    for h in range(H):
        np.testing.assert_allclose(dv[0, h].sum(axis=0), dz[0, h].sum(axis=0), atol=1e-12)
        np.testing.assert_allclose(daV[h].sum(axis=0), dz[0, h].sum(axis=0), atol=1e-12)
        np.testing.assert_allclose(daK[h].sum(axis=0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dk[0, h].sum(axis=0), 0.0, atol=1e-12)


def test_t5_backward_bias_gradient_sums_to_zero():
    """sum over buckets of dbias[:, h] = sum_ij de_ij = 0; and a bias constant
    across buckets shifts every row by one value, which the softmax ignores, so
    q, k, v get the textbook gradients (torch autograd of the library routine)."""
    B, H, n, d = 1, 2, 12, 4
    q, k, v, dz = (rnd((B, H, n, d), 150 + i) for i in range(4))
    bias = rnd((16, H), 154)
    db = oracle.t5_backward(q, k, v, bias, 16, 40, True, dz, key_lens=[9])[3]
    np.testing.assert_allclose(db.sum(axis=0), 0.0, atol=1e-12)
    flat = np.repeat(rnd((1, H), 155), 8, axis=0)
    dq, dk, dv, db1 = oracle.t5_backward(q, k, v, flat, 8, 20, False, dz, scale=0.5,
                                         causal=True)
    t = [torch.tensor(x, requires_grad=True) for x in (q, k, v)]
    torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True, scale=0.5).backward(
        torch.tensor(dz))
    for mine, theirs in zip((dq, dk, dv), t):
        np.testing.assert_allclose(mine, theirs.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(db1.sum(axis=0), 0.0, atol=1e-12)


@pytest.mark.parametrize("shared,causal", [(False, False), (True, True)])
def test_offset_bias_backward_matches_finite_differences(shared, causal):
    B, H, n, d, W = 1, 2, 12, 4, 5
    q, k, v, dz = (rnd((B, H, n, d), 160 + i) for i in range(4))
    bias = rnd((1 if shared else H, 2 * W + 1), 164)
    grads = oracle.offset_bias_backward(q, k, v, bias, W, dz, causal=causal, key_lens=[9])
    loss = lambda: float((dz * oracle.offset_bias_attention(q, k, v, bias, W, causal=causal,
                                                           key_lens=[9])).sum())
    rng = np.random.default_rng(165)
    for x, g in zip((q, k, v, bias), grads):
        idx = [tuple(int(rng.integers(s)) for s in x.shape) for _ in range(6)]
        _fd_check(loss, x, g, idx)


@pytest.mark.parametrize("bidir", [True, False])
def test_offset_bias_backward_against_t5_backward(bidir):
    """A table holding each offset's T5 bucket bias is the T5 forward; its
    gradient summed over the offsets of each bucket is the T5 bias gradient,
    and q, k, v get the same gradients."""
    B, H, n, d, nb, maxd = 1, 2, 40, 8, 8, 12
    q, k, v, dz = (rnd((B, H, n, d), 170 + i) for i in range(4))
    tb = rnd((nb, H), 174)
    W = n - 1
    beta = np.array([oracle.t5_bucket(w - W, nb, maxd, bidir) for w in range(2 * W + 1)])
    table = tb[beta].T  # [H, 2W + 1]
    dq, dk, dv, dob = oracle.offset_bias_backward(q, k, v, table, W, dz, scale=1.0,
                                                  causal=True)
    tq, tk, tv, dtb = oracle.t5_backward(q, k, v, tb, nb, maxd, bidir, dz, causal=True)
    for a, b_ in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)
    for h in range(H):
        folded = np.bincount(beta, weights=dob[h], minlength=nb)
        np.testing.assert_allclose(folded, dtb[:, h], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dob.sum(axis=1), 0.0, atol=1e-12)


# ---------------------------------------------------------------------------
# Transformer-XL relative logits
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window,shared", [(False, 20, False), (True, 20, True),
                                                  (False, 3, False)])
def test_xl_without_global_biases_is_shaw_with_reversed_table(causal, window, shared):
    """u = v = 0 leaves terms (a) and (b): the Shaw key term with the table read
    by i - j instead of j - i, i.e. w^K[r] = R[2W - r]."""
    B, H, n, d = 2, 2, 11, 8
    q, k, v = (rnd((B, H, n, d), 180 + i) for i in range(3))
    R = rnd((1 if shared else H, 2 * window + 1, d), 183)
    zero = np.zeros((1, d))
    got = oracle.xl_attention(q, k, v, R, zero, zero, window, causal=causal, key_lens=[n, 7])
    want = oracle.relattn_bruteforce(q, k, v, R[:, ::-1].copy(), None, window, causal=causal,
                                     key_lens=[n, 7])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_xl_without_position_table_is_attention_of_shifted_queries():
    """R = 0 leaves terms (a) and (c): q_i.k_j + u.k_j = (q_i + u).k_j, i.e.
    library attention of q + u; term (d) vanishes whatever v is."""
    B, H, n, d, W = 1, 3, 9, 8, 4
    q, k, v = (rnd((B, H, n, d), 190 + i) for i in range(3))
    u, vb = rnd((H, d), 193), rnd((H, d), 194)
    got = oracle.xl_attention(q, k, v, np.zeros((H, 2 * W + 1, d)), u, vb, W, causal=True)
    qs = torch.tensor(q + u[None, :, None, :])
    want = torch.nn.functional.scaled_dot_product_attention(
        qs, torch.tensor(k), torch.tensor(v), is_causal=True).numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_xl_global_position_bias_is_an_offset_bias():
    """q = 0 and u = 0 leave term (d) alone: v.R_{i-j} is a scalar
    by distance, i.e. an offset bias with entry W + (j - i) = v.R[W - (j - i)]."""
    B, H, n, d, W = 1, 2, 10, 8, 6
    k, v = rnd((B, H, n, d), 200), rnd((B, H, n, d), 201)
    q = np.zeros((B, H, n, d))
    R, vb = rnd((H, 2 * W + 1, d), 202), rnd((H, d), 203)
    got = oracle.xl_attention(q, k, v, R, np.zeros((H, d)), vb, W, scale=0.5)
    bias = np.stack([0.5 * (R[h] @ vb[h])[::-1] for h in range(H)])  # entry W + (j - i)
    want = oracle.offset_bias_attention(q, k, v, bias, W, scale=0.5)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)



@pytest.mark.parametrize("causal,lens,window,shared", [(False, None, 2, False),
                                                       (True, None, 9, True),
                                                       (False, [6, 4], 3, False)])
def test_xl_backward_matches_finite_differences(causal, lens, window, shared):
    B, H, n, d = 2, 2, 6, 4
    q, k, v, dz = (rnd((B, H, n, d), 380 + i) for i in range(4))
    Hs = 1 if shared else H
    R, u, vb = rnd((Hs, 2 * window + 1, d), 384, 0.5), rnd((Hs, d), 385), rnd((Hs, d), 386)
    grads = oracle.xl_backward(q, k, v, R, u, vb, window, dz, causal=causal, key_lens=lens)
    loss = lambda: float((dz * oracle.xl_attention(q, k, v, R, u, vb, window, causal=causal,
                                                   key_lens=lens)).sum())
    rng = np.random.default_rng(387)
    for x, g in zip((q, k, v, R, u, vb), grads):
        idx = [tuple(int(rng.integers(s)) for s in x.shape) for _ in range(6)]
        _fd_check(loss, x, g, idx)


@pytest.mark.parametrize("causal,window,shared", [(False, 20, False), (True, 4, True)])
def test_xl_backward_without_global_biases_is_shaw_backward(causal, window, shared):
    """u = v = 0: dq, dk, dv are the Shaw key-table gradients with the table
    read by i - j (w^K[r] = R[2W - r]), and dR is that table's gradient
    reversed."""
    B, H, n, d = 2, 2, 11, 8
    q, k, v, dz = (rnd((B, H, n, d), 390 + i) for i in range(4))
    R = rnd((1 if shared else H, 2 * window + 1, d), 394)
    zero = np.zeros((1, d))
    got = oracle.xl_backward(q, k, v, R, zero, zero, window, dz, causal=causal, key_lens=[n, 7])
    want = oracle.relattn_backward(q, k, v, R[:, ::-1].copy(), None, window, dz, causal=causal,
                                   key_lens=[n, 7])
    for a, b_ in zip(got[:3], want[:3]):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[3], want[3][:, ::-1], rtol=0, atol=1e-12)


@pytest.mark.parametrize("shared", [False, True])
def test_xl_backward_global_bias_gradients_sum_to_the_query_gradients(shared):
    """q enters every logit through q + u and q + v, so du + dv_bias equals the
    query gradients summed over the batch and the positions (and over the heads
    for one shared pair), and the key gradients of each row sum to zero
    (softmax rows)."""
    B, H, n, d, W = 2, 3, 9, 8, 3
    q, k, v, dz = (rnd((B, H, n, d), 400 + i) for i in range(4))
    Hs = 1 if shared else H
    R, u, vb = rnd((Hs, 2 * W + 1, d), 404), rnd((Hs, d), 405), rnd((Hs, d), 406)
    dq, dk, dv, dR, du, dvb = oracle.xl_backward(q, k, v, R, u, vb, W, dz, causal=True,
                                                 key_lens=[n, 5])
    per_head = dq.sum(axis=(0, 2))
    want = per_head.sum(axis=0, keepdims=True) if shared else per_head
    np.testing.assert_allclose(du + dvb, want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)

# ---------------------------------------------------------------------------
# Swin 2-D window bias
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 3, 5])
def test_grid_bias_of_a_1d_offset_function_is_an_offset_bias(M):
    """A table whose entry (dy, dx) holds f(dy*M + dx) -- a function of the
    raster offset j - i alone -- is the offset-bias attention with entry f(j -
    i).  f is asymmetric, so a flipped sign or swapped dy/dx fails."""
    n = M * M
    B, H, d = 2, 2, 8
    q, k, v = (rnd((B, H, n, d), 210 + i) for i in range(3))
    W = n - 1
    f = rnd((H, 2 * W + 1), 213)                     # f[h, W + delta]
    dy, dx = np.meshgrid(np.arange(-(M - 1), M), np.arange(-(M - 1), M), indexing="ij")
    table = np.stack([f[h][W + (dy * M + dx)].ravel() for h in range(H)])
    got = oracle.grid_bias_attention(q, k, v, table, M, key_lens=[n, max(1, n - 2)])
    want = oracle.offset_bias_attention(q, k, v, f, W, key_lens=[n, max(1, n - 2)])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_grid_bias_constant_table_is_textbook_attention():
    M, B, H, d = 4, 1, 3, 8
    n = M * M
    q, k, v = (rnd((B, H, n, d), 220 + i) for i in range(3))
    table = np.full((1, (2 * M - 1) ** 2), 0.7)
    got = oracle.grid_bias_attention(q, k, v, table, M, scale=0.5)
    want = torch.nn.functional.scaled_dot_product_attention(
        *(torch.tensor(x) for x in (q, k, v)), scale=0.5).numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shared", [False, True])
def test_grid_bias_backward_matches_finite_differences(shared):
    M, B, H, d = 3, 2, 2, 4
    n = M * M
    q, k, v, dz = (rnd((B, H, n, d), 240 + i) for i in range(4))
    bias = rnd((1 if shared else H, (2 * M - 1) ** 2), 244)
    lens = [n, 5]
    grads = oracle.grid_bias_backward(q, k, v, bias, M, dz, key_lens=lens)
    loss = lambda: float((dz * oracle.grid_bias_attention(q, k, v, bias, M,
                                                          key_lens=lens)).sum())
    rng = np.random.default_rng(245)
    for x, g in zip((q, k, v, bias), grads):
        idx = [tuple(int(rng.integers(s)) for s in x.shape) for _ in range(6)]
        _fd_check(loss, x, g, idx)


@pytest.mark.parametrize("M", [2, 4])
def test_grid_bias_backward_of_a_1d_offset_function_is_the_offset_bias_backward(M):
    """With a table holding f(dy*M + dx), q, k and v get the offset-bias
    gradients, and the table's gradient summed over the entries of each raster
    offset is the offset table's gradient (an entry swap or a sign slip in the
    entry fails); each head's table gradient sums to zero (softmax rows)."""
    n = M * M
    B, H, d = 2, 2, 8
    q, k, v, dz = (rnd((B, H, n, d), 250 + i) for i in range(4))
    W = n - 1
    f = rnd((H, 2 * W + 1), 254)
    dy, dx = np.meshgrid(np.arange(-(M - 1), M), np.arange(-(M - 1), M), indexing="ij")
    delta = (dy * M + dx).ravel()
    table = np.stack([f[h][W + delta] for h in range(H)])
    lens = [n, max(1, n - 3)]
    gq, gk, gv, gdb = oracle.grid_bias_backward(q, k, v, table, M, dz, key_lens=lens)
    oq, ok_, ov, odb = oracle.offset_bias_backward(q, k, v, f, W, dz, key_lens=lens)
    for a, b_ in ((gq, oq), (gk, ok_), (gv, ov)):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)
    for h in range(H):
        folded = np.bincount(W + delta, weights=gdb[h], minlength=2 * W + 1)
        np.testing.assert_allclose(folded, odb[h], rtol=0, atol=1e-12)
    np.testing.assert_allclose(gdb.sum(axis=1), 0.0, atol=1e-12)


def test_grid_bias_entry_layout_probe():
    """A single large entry at (dy, dx) = (1, -2) with q = 0: each query's
    weights pile on the key one row down and two columns left when it exists,
    and are uniform otherwise."""
    M = 4
    n = M * M
    q = np.zeros((1, 1, n, n))
    k = rnd((1, 1, n, n), 231)
    v = np.eye(n)[None, None]          # z_i = the weight row of query i
    table = np.zeros((1, (2 * M - 1) ** 2))
    table[0, (1 + M - 1) * (2 * M - 1) + (-2 + M - 1)] = 50.0
    w = oracle.grid_bias_attention(q, k, v, table, M)[0, 0]
    for i in range(n):
        yi, xi = divmod(i, M)
        if yi + 1 < M and xi - 2 >= 0:
            j = (yi + 1) * M + (xi - 2)
            assert w[i, j] > 0.999
        else:
            np.testing.assert_allclose(w[i], 1.0 / n, atol=1e-12)


# ---------------------------------------------------------------------------
# scalar bias by a per-pair edge label (summary page of "Self-Attention with
# Relative Position Representations": any pairwise label may index the
# relation; survey page, "Placement in the taxonomy")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bidir", [True, False])
@pytest.mark.parametrize("causal,lens", [(False, None), (True, None), (False, [9, 30])])
def test_edge_labels_from_t5_buckets_equal_t5(bidir, causal, lens):
    """Labels E[i, j] = beta(j - i) with the T5 table as the bias rows give the
    T5 attention (scale 1).  Bidirectional buckets are not symmetric in the
    offset, so a transposed label matrix fails."""
    B, H, n, d = 2, 3, 30, 8
    q, k, v = rnd((B, H, n, d), 300), rnd((B, H, n, d), 301), rnd((B, H, n, d), 302)
    t5b = rnd((32, H), 303)
    E = np.array([[oracle.t5_bucket(j - i, 32, 16, bidir) for j in range(n)] for i in range(n)])
    z = oracle.edge_label_attention(q, k, v, np.stack([E] * B), t5b.T, scale=1.0,
                                    causal=causal, key_lens=lens)
    want = oracle.t5_attention(q, k, v, t5b, 32, 16, bidir, causal=causal, key_lens=lens)
    np.testing.assert_allclose(z, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shared", [False, True])
def test_edge_labels_from_clipped_offsets_equal_offset_bias(shared):
    """Labels clip(j - i, W) + W reproduce the offset bias with the same table."""
    B, H, n, d, W = 2, 3, 17, 8, 4
    q, k, v = rnd((B, H, n, d), 310), rnd((B, H, n, d), 311), rnd((B, H, n, d), 312)
    table = rnd((1 if shared else H, 2 * W + 1), 313)
    E = oracle.relative_labels(n, W) + W
    z = oracle.edge_label_attention(q, k, v, np.stack([E] * B), table, causal=True,
                                    key_lens=[n, 11])
    want = oracle.offset_bias_attention(q, k, v, table, W, causal=True, key_lens=[n, 11])
    np.testing.assert_allclose(z, want, rtol=0, atol=1e-12)


def test_edge_labels_constant_bias_is_textbook():
    """One bias value for every label cancels in the softmax: textbook scaled
    attention (library routine), whatever the labels."""
    B, H, n, d = 2, 2, 13, 8
    q, k, v = rnd((B, H, n, d), 320), rnd((B, H, n, d), 321), rnd((B, H, n, d), 322)
    E = np.random.default_rng(323).integers(0, 5, (B, n, n))
    z = oracle.edge_label_attention(q, k, v, E, np.full((1, 5), -1.3))
    ok = np.ones((n, n), dtype=bool)
    np.testing.assert_allclose(z, sdpa(q, k, v, ok, 1 / math.sqrt(d)), rtol=0, atol=1e-12)


def test_edge_labels_probe_per_batch():
    """A large bias on label 3 with q = 0 and v = I: query i of batch b spreads
    its weight evenly over exactly the keys j with E[b, i, j] == 3 (uniformly
    over all keys when there is none).  The two batch entries hold different
    labels, so reading another entry's matrix or its transpose fails."""
    B, n = 2, 12
    rng = np.random.default_rng(330)
    E = rng.integers(0, 6, (B, n, n))
    E[0, 5, :] = 0                      # a row without label 3
    q = np.zeros((B, 1, n, n))
    k = rnd((B, 1, n, n), 331)
    v = np.broadcast_to(np.eye(n), (B, 1, n, n)).copy()
    bias = np.zeros((1, 6))
    bias[0, 3] = 60.0
    w = oracle.edge_label_attention(q, k, v, E, bias)
    for b in range(B):
        for i in range(n):
            hit = E[b, i] == 3
            want = hit / hit.sum() if hit.any() else np.full(n, 1.0 / n)
            np.testing.assert_allclose(w[b, 0, i], want, rtol=0, atol=1e-12)


def test_edge_labels_two_tokens_closed_form():
    """n = 2: each row is a two-way softmax, alpha_i1 = 1 / (1 + exp(e_i0 - e_i1)),
    with e_ij = s q_i k_j + b[E_ij], written out per element."""
    rng = np.random.default_rng(340)
    q, k, v = (rng.standard_normal((1, 1, 2, 3)) for _ in range(3))
    E = np.array([[[2, 0], [1, 2]]])
    bias = np.array([[0.4, -1.1, 0.9]])
    s = 0.7
    z = oracle.edge_label_attention(q, k, v, E, bias, scale=s)[0, 0]
    for i in range(2):
        e = [s * float(np.dot(q[0, 0, i], k[0, 0, j])) + bias[0, E[0, i, j]] for j in range(2)]
        a1 = 1.0 / (1.0 + math.exp(e[0] - e[1]))
        np.testing.assert_allclose(z[i], (1 - a1) * v[0, 0, 0] + a1 * v[0, 0, 1], rtol=0,
                                   atol=1e-14)



@pytest.mark.parametrize("causal,lens,shared", [(False, None, False), (True, None, True),
                                               (False, [6, 3], False)])
def test_edge_label_backward_matches_finite_differences(causal, lens, shared):
    B, H, n, d, NL = 2, 2, 6, 4, 5
    q, k, v, dz = (rnd((B, H, n, d), 350 + i) for i in range(4))
    bias = rnd((1 if shared else H, NL), 354)
    E = np.random.default_rng(355).integers(0, NL, size=(B, n, n))
    grads = oracle.edge_label_backward(q, k, v, E, bias, dz, causal=causal, key_lens=lens)
    loss = lambda: float((dz * oracle.edge_label_attention(q, k, v, E, bias, causal=causal,
                                                           key_lens=lens)).sum())
    rng = np.random.default_rng(356)
    for x, g in zip((q, k, v, bias), grads):
        idx = [tuple(int(rng.integers(s)) for s in x.shape) for _ in range(6)]
        _fd_check(loss, x, g, idx)


@pytest.mark.parametrize("bidir", [True, False])
@pytest.mark.parametrize("causal,lens", [(False, None), (True, None), (False, [9, 30])])
def test_edge_label_backward_from_t5_buckets_is_t5_backward(bidir, causal, lens):
    """Labels E[i, j] = beta(j - i) with the T5 table as bias rows give the T5
    gradients, the bias gradient transposed ([H, NL] against [NL, H]); the
    buckets are not symmetric in the offset, so transposed labels fail."""
    B, H, n, d = 2, 3, 30, 8
    q, k, v, dz = (rnd((B, H, n, d), 360 + i) for i in range(4))
    t5b = rnd((32, H), 364)
    E = np.array([[oracle.t5_bucket(j - i, 32, 16, bidir) for j in range(n)] for i in range(n)])
    got = oracle.edge_label_backward(q, k, v, np.stack([E] * B), t5b.T, dz, scale=1.0,
                                     causal=causal, key_lens=lens)
    want = oracle.t5_backward(q, k, v, t5b, 32, 16, bidir, dz, scale=1.0, causal=causal,
                              key_lens=lens)
    for a, b_ in zip(got[:3], want[:3]):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[3], want[3].T, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shared", [False, True])
def test_edge_label_backward_from_clipped_offsets_is_offset_bias_backward(shared):
    """Labels clip(j - i, W) + W: the offset-bias gradients, table included; a
    table row that no pair reaches gets exactly 0, and each head's bias
    gradient sums to 0 (every softmax row's dS does)."""
    B, H, n, d, W = 2, 3, 17, 8, 4
    q, k, v, dz = (rnd((B, H, n, d), 370 + i) for i in range(4))
    table = rnd((1 if shared else H, 2 * W + 2), 374)  # one label more than any pair carries
    E = oracle.relative_labels(n, W) + W
    got = oracle.edge_label_backward(q, k, v, np.stack([E] * B), table, dz, causal=True,
                                     key_lens=[n, 11])
    want = oracle.offset_bias_backward(q, k, v, table[:, :2 * W + 1], W, dz, causal=True,
                                       key_lens=[n, 11])
    for a, b_ in zip(got[:3], want[:3]):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[3][:, :2 * W + 1], want[3], rtol=0, atol=1e-12)
    assert np.all(got[3][:, 2 * W + 1] == 0.0)
    np.testing.assert_allclose(got[3].sum(axis=1), 0.0, atol=1e-12)


# ---------------------------------------------------------------------------
# relation-aware attention with per-pair labels and vector tables (Eq. 3 and
# Eq. 4 over a labeled graph)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tables", ["KV", "K", "V"])
@pytest.mark.parametrize("causal,lens", [(False, None), (True, None), (False, [7, 15])])
def test_edge_relattn_with_clipped_offset_labels_is_shaw(tables, causal, lens):
    """Labels clip(j - i, k) + k with the 2k+1-row tables are Shaw's
    relation-aware attention (the brute-force oracle)."""
    B, H, n, d, kc = 2, 3, 15, 8, 3
    q, k, v = rnd((B, H, n, d), 400), rnd((B, H, n, d), 401), rnd((B, H, n, d), 402)
    aK = rnd((H, 2 * kc + 1, d), 403) if "K" in tables else None
    aV = rnd((1, 2 * kc + 1, d), 404) if "V" in tables else None
    E = np.stack([oracle.relative_labels(n, kc) + kc] * B)
    z = oracle.edge_label_relattn(q, k, v, E, aK, aV, causal=causal, key_lens=lens)
    want = oracle.relattn_bruteforce(q, k, v, aK, aV, kc, causal=causal, key_lens=lens)
    np.testing.assert_allclose(z, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("tables", ["KV", "K", "V"])
@pytest.mark.parametrize("causal,lens,shared", [(False, None, False), (True, None, True),
                                               (False, [6, 3], False)])
def test_edge_relattn_backward_matches_finite_differences(tables, causal, lens, shared):
    B, H, n, d, NL = 2, 2, 6, 4, 5
    q, k, v, dz = (rnd((B, H, n, d), 410 + i) for i in range(4))
    Ht = 1 if shared else H
    aK = rnd((Ht, NL, d), 414, 0.5) if "K" in tables else None
    aV = rnd((Ht, NL, d), 415, 0.5) if "V" in tables else None
    E = np.random.default_rng(416).integers(0, NL, size=(B, n, n))
    grads = oracle.edge_label_relattn_backward(q, k, v, E, aK, aV, dz, causal=causal,
                                               key_lens=lens)
    loss = lambda: float((dz * oracle.edge_label_relattn(q, k, v, E, aK, aV, causal=causal,
                                                         key_lens=lens)).sum())
    rng = np.random.default_rng(417)
    for x, g in zip((q, k, v, aK, aV), grads):
        if x is None:
            assert g is None
            continue
        idx = [tuple(int(rng.integers(s)) for s in x.shape) for _ in range(6)]
        _fd_check(loss, x, g, idx)


@pytest.mark.parametrize("causal,lens", [(False, None), (True, [11, 7])])
def test_edge_relattn_backward_with_clipped_offset_labels_is_shaw_backward(causal, lens):
    """Labels clip(j - i, k) + k: Shaw's backward, tables included (a
    transposed label matrix or a swapped table gradient fails)."""
    B, H, n, d, c = 2, 2, 11, 8, 3
    q, k, v, dz = (rnd((B, H, n, d), 420 + i) for i in range(4))
    aK, aV = rnd((H, 2 * c + 1, d), 424, 0.5), rnd((H, 2 * c + 1, d), 425, 0.5)
    E = np.stack([oracle.relative_labels(n, c) + c] * B)
    got = oracle.edge_label_relattn_backward(q, k, v, E, aK, aV, dz, causal=causal,
                                             key_lens=lens)
    want = oracle.relattn_backward(q, k, v, aK, aV, c, dz, causal=causal, key_lens=lens)
    for a, b_ in zip(got, want):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)


def test_edge_relattn_single_label_is_textbook_on_shifted_keys_and_values():
    """One label everywhere: a^K_ij = w^K, a^V_ij = w^V, i.e. attention over k_j + w^K
    and v_j + w^V (library routine)."""
    B, H, n, d = 2, 2, 11, 8
    q, k, v = rnd((B, H, n, d), 410), rnd((B, H, n, d), 411), rnd((B, H, n, d), 412)
    wK, wV = rnd((H, 1, d), 413), rnd((H, 1, d), 414)
    E = np.zeros((B, n, n), dtype=np.int64)
    z = oracle.edge_label_relattn(q, k, v, E, wK, wV, causal=True)
    ok = np.tril(np.ones((n, n), dtype=bool))
    want = sdpa(q, k + wK[None], v + wV[None], ok, 1 / math.sqrt(d))
    np.testing.assert_allclose(z, want, rtol=0, atol=1e-12)


def test_edge_relattn_value_histogram_probe():
    """q = 0 (uniform weights over the visible keys), value table only:
    z_i - mean_j v_j = sum_r (count of label r in row i of batch b / n) w^V_r.
    The batch entries hold different label matrices and the rows are not
    symmetric, so a transposed or another entry's matrix fails."""
    B, H, n, d, NL = 2, 2, 9, 5, 6
    rng = np.random.default_rng(420)
    E = rng.integers(0, NL, (B, n, n))
    q = np.zeros((B, H, n, d))
    k, v = rnd((B, H, n, d), 421), rnd((B, H, n, d), 422)
    aV = rnd((H, NL, d), 423)
    z = oracle.edge_label_relattn(q, k, v, E, None, aV)
    for b in range(B):
        for h in range(H):
            for i in range(n):
                hist = np.bincount(E[b, i], minlength=NL) / n
                np.testing.assert_allclose(z[b, h, i] - v[b, h].mean(axis=0), hist @ aV[h],
                                           rtol=0, atol=1e-12)


def test_edge_relattn_label_permutation_invariance():
    """Renaming the labels and permuting the table rows alike changes nothing."""
    B, H, n, d, NL = 2, 2, 10, 8, 7
    q, k, v = rnd((B, H, n, d), 430), rnd((B, H, n, d), 431), rnd((B, H, n, d), 432)
    aK, aV = rnd((H, NL, d), 433), rnd((H, NL, d), 434)
    E = np.random.default_rng(435).integers(0, NL, (B, n, n))
    perm = np.random.default_rng(436).permutation(NL)
    inv = np.argsort(perm)
    z1 = oracle.edge_label_relattn(q, k, v, E, aK, aV, causal=True)
    z2 = oracle.edge_label_relattn(q, k, v, perm[E], aK[:, inv], aV[:, inv], causal=True)
    np.testing.assert_allclose(z1, z2, rtol=0, atol=1e-12)


def test_edge_relattn_two_tokens_closed_form():
    """n = 2, d = 2, written out per element: e_ij = s q_i.(k_j + w^K_{E_ij}),
    alpha_i1 = 1 / (1 + exp(e_i0 - e_i1)), z_i = sum_j alpha_ij (v_j + w^V_{E_ij})."""
    rng = np.random.default_rng(440)
    q, k, v = (rng.standard_normal((1, 1, 2, 2)) for _ in range(3))
    E = np.array([[[1, 0], [2, 1]]])
    wK, wV = rng.standard_normal((1, 3, 2)), rng.standard_normal((1, 3, 2))
    s = 0.9
    z = oracle.edge_label_relattn(q, k, v, E, wK, wV, scale=s)[0, 0]
    for i in range(2):
        e = [s * sum(q[0, 0, i, c] * (k[0, 0, j, c] + wK[0, E[0, i, j], c]) for c in range(2))
             for j in range(2)]
        a1 = 1.0 / (1.0 + math.exp(e[0] - e[1]))
        want = [(1 - a1) * (v[0, 0, 0, c] + wV[0, E[0, i, 0], c])
                + a1 * (v[0, 0, 1, c] + wV[0, E[0, i, 1], c]) for c in range(2)]
        np.testing.assert_allclose(z[i], want, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# the edge-label pins bite: plant a mistake in either edge-label oracle and
# watch the named pin fail
# ---------------------------------------------------------------------------

def _plant(monkeypatch, name, wrong):
    monkeypatch.setattr(orc, name, wrong)
    monkeypatch.setattr(oracle, name, wrong)


@pytest.mark.parametrize("fault", ["transposed", "wrong_batch", "dropped_scale", "head0_row"])
def test_planted_edge_bias_mistakes_are_caught(monkeypatch, fault):
    """Scalar bias by edge label: a transposed label matrix, every batch entry
    reading entry 0's labels, the 1/sqrt(d) (or explicit) scale dropped from
    q.k, and head 0's bias row used for every head each fail a pin."""
    real = orc.edge_label_attention

    def wrong(q, k, v, labels, bias, scale=None, causal=False, key_lens=None):
        E = np.asarray(labels)
        b = orc.to_f64(bias)
        if fault == "transposed":
            E = np.swapaxes(E, 1, 2)
        elif fault == "wrong_batch":
            E = np.broadcast_to(E[:1], E.shape)
        elif fault == "dropped_scale":
            scale = 1.0
        elif fault == "head0_row":
            b = b[:1]
        return real(q, k, v, E, b, scale=scale, causal=causal, key_lens=key_lens)

    _plant(monkeypatch, "edge_label_attention", wrong)
    pin = {
        "transposed": lambda: test_edge_labels_from_t5_buckets_equal_t5(True, False, None),
        "wrong_batch": test_edge_labels_probe_per_batch,
        "dropped_scale": test_edge_labels_two_tokens_closed_form,
        "head0_row": lambda: test_edge_labels_from_clipped_offsets_equal_offset_bias(False),
    }[fault]
    with pytest.raises(AssertionError):
        pin()


def _edge_relattn_with(fault):
    """edge_label_relattn written out again with one planted mistake."""
    def f(q, k, v, labels, aK=None, aV=None, scale=None, causal=False, key_lens=None):
        q, k, v = orc.to_f64(q), orc.to_f64(k), orc.to_f64(v)
        aK, aV = orc.to_f64(aK), orc.to_f64(aV)
        E = np.asarray(labels).astype(np.int64)
        B, H, n, d = q.shape
        s = 1.0 / np.sqrt(d) if (scale is None or scale <= 0) else float(scale)
        EK = np.swapaxes(E, 1, 2) if fault == "key_transposed" else E
        EV = np.swapaxes(E, 1, 2) if fault == "value_transposed" else E
        if fault == "wrong_batch":
            EK = EV = np.broadcast_to(E[:1], E.shape)
        lens = [n] * B if key_lens is None else [max(0, min(n, int(x))) for x in key_lens]
        z = np.zeros((B, H, n, v.shape[-1]))
        for b in range(B):
            ok = orc.visible(n, causal, lens[b])
            for h in range(H):
                hh = 0 if fault == "head0_tables" else h
                kk = np.broadcast_to(k[b, h][None], (n, n, d))
                if aK is not None:
                    kk = kk + aK[0 if aK.shape[0] == 1 else hh][EK[b]]
                alpha = orc._masked_softmax_rows(np.einsum("id,ijd->ij", s * q[b, h], kk), ok)
                vv = np.broadcast_to(v[b, h][None], (n, n, v.shape[-1]))
                if aV is not None:
                    tv = aV[0 if aV.shape[0] == 1 else hh][EV[b]]
                    vv = vv + (s * tv if fault == "scaled_value" else tv)
                z[b, h] = np.einsum("ij,ijd->id", alpha, vv)
        return z
    return f


@pytest.mark.parametrize("fault", ["key_transposed", "value_transposed", "wrong_batch",
                                   "head0_tables", "scaled_value"])
def test_planted_edge_relattn_mistakes_are_caught(monkeypatch, fault):
    """Edge labels with key and value tables: a transposed label matrix on the
    key side or on the value side, every batch entry reading entry 0's labels,
    head 0's tables used for every head, and the 1/sqrt(d) scale applied to the
    value term each fail a pin.  The unplanted rewrite passes the same pins, so
    each failure is the planted mistake's."""
    pin = {
        "key_transposed": lambda: test_edge_relattn_with_clipped_offset_labels_is_shaw(
            "K", False, None),
        "value_transposed": test_edge_relattn_value_histogram_probe,
        "wrong_batch": test_edge_relattn_value_histogram_probe,
        "head0_tables": lambda: test_edge_relattn_with_clipped_offset_labels_is_shaw(
            "K", False, None),
        "scaled_value": test_edge_relattn_two_tokens_closed_form,
    }[fault]
    _plant(monkeypatch, "edge_label_relattn", _edge_relattn_with(None))
    pin()
    _plant(monkeypatch, "edge_label_relattn", _edge_relattn_with(fault))
    with pytest.raises(AssertionError):
        pin()


@pytest.mark.parametrize("window,shared", [(3, False), (40, True)])
def test_offset_bias_decode_matches_forward_rows(window, shared):
    """Decoding with an offset table reproduces the causal offset-bias
    attention's rows at the decoded positions (per-head and shared rows, a window
    that clips and one that does not)."""
    q_full, k, v, lens, Tq = _decode_case(70, L=40)
    B, H, L, d = q_full.shape
    bias = rnd((1 if shared else H, 2 * window + 1), 71)
    q = np.zeros((B, H, Tq, d))
    for b in range(B):
        for t in range(Tq):
            i = lens[b] - Tq + t
            if i >= 0:
                q[b, :, t] = q_full[b, :, i]
    z = oracle.offset_bias_decode(q, k, v, bias, window, cache_lens=lens)
    full = oracle.offset_bias_attention(q_full, k, v, bias, window, causal=True, key_lens=lens)
    for b in range(B):
        for t in range(Tq):
            i = lens[b] - Tq + t
            if i >= 0:
                np.testing.assert_allclose(z[b, :, t], full[b, :, i], rtol=0, atol=1e-12)
            else:
                assert np.all(z[b, :, t] == 0.0)


@pytest.mark.parametrize("window,shared", [(3, False), (40, True)])
def test_xl_decode_matches_forward_rows(window, shared):
    """Transformer-XL decoding reproduces the causal XL attention's rows at the
    decoded positions (per-head and shared R, u, v; a window that clips and one
    that does not)."""
    q_full, k, v, lens, Tq = _decode_case(80, L=40)
    B, H, L, d = q_full.shape
    Hr = 1 if shared else H
    R = rnd((Hr, 2 * window + 1, d), 81, 0.5)
    u, vb = rnd((Hr, d), 82, 0.5), rnd((Hr, d), 83, 0.5)
    q = np.zeros((B, H, Tq, d))
    for b in range(B):
        for t in range(Tq):
            i = lens[b] - Tq + t
            if i >= 0:
                q[b, :, t] = q_full[b, :, i]
    z = oracle.xl_decode(q, k, v, R, u, vb, window, cache_lens=lens)
    full = oracle.xl_attention(q_full, k, v, R, u, vb, window, causal=True, key_lens=lens)
    for b in range(B):
        for t in range(Tq):
            i = lens[b] - Tq + t
            if i >= 0:
                np.testing.assert_allclose(z[b, :, t], full[b, :, i], rtol=0, atol=1e-12)
            else:
                assert np.all(z[b, :, t] == 0.0)
