"""Pins for the fp64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: a library routine
(torch's fp64 scaled-dot-product attention), brute force written independently with
Python loops and math.exp, closed forms, hand-derived golden cases and invariants of
the retrieval / streaming split.  The mutation tests at the end plant plausible
mistakes in the oracle (on the CPU) and show that a pin catches each of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "attention_closed_forms.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def brute_force(q, K, V, i, retrieval, sink, recent, scale):
    """Independent dense attention for one row: explicit membership test, Python loops."""
    D = len(q)
    keys = []
    for j in range(i + 1):
        in_sink = j < sink
        in_window = (i - j) < recent
        if retrieval or in_sink or in_window:
            keys.append(j)
    scores = [scale * sum(q[d] * K[j][d] for d in range(D)) for j in keys]
    mx = max(scores)
    ex = [math.exp(s - mx) for s in scores]
    tot = sum(ex)
    return [sum(ex[a] / tot * V[j][d] for a, j in enumerate(keys)) for d in range(V.shape[1])]


# --- library routine -------------------------------------------------------------

@pytest.mark.parametrize("L,D,H", [(1, 8, 1), (37, 16, 3), (200, 64, 2)])
def test_all_retrieval_equals_torch_sdpa(L, D, H):
    rng = np.random.default_rng(L * 7 + D)
    Q, K, V = _rand(rng, L, H, D), _rand(rng, L, H, D), _rand(rng, L, H, D)
    mask = np.ones(H, dtype=bool)
    out = A.layer_attention(Q, np.arange(L), K, V, mask, sink=4, recent=8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).permute(1, 0, 2), torch.from_numpy(K).permute(1, 0, 2),
        torch.from_numpy(V).permute(1, 0, 2), is_causal=True).permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_streaming_equals_torch_sdpa_with_explicit_mask():
    """torch SDPA with a boolean mask built as the sink + window band."""
    L, D, S, R = 150, 32, 5, 17
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, L, D), _rand(rng, L, D), _rand(rng, L, D)
    ii, jj = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    band = (jj <= ii) & ((jj < S) | (ii - jj < R))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(band)[None]).numpy()[0]
    out = A.head_attention(q, np.arange(L), k, v, False, S, R)
    assert np.max(np.abs(out - ref)) < 1e-12


# --- brute force ----------------------------------------------------------------

@settings(max_examples=40, deadline=None)
@given(L=st.integers(1, 24), D=st.integers(1, 6), sink=st.integers(0, 6), recent=st.integers(1, 9),
       retrieval=st.booleans(), seed=st.integers(0, 2**16))
def test_brute_force_tiny(L, D, sink, recent, retrieval, seed):
    rng = np.random.default_rng(seed)
    q, K, V = _rand(rng, L, D), _rand(rng, L, D), _rand(rng, L, D)
    scale = 1.0 / math.sqrt(D)
    out = A.head_attention(q, np.arange(L), K, V, retrieval, sink, recent)
    for i in range(L):
        ref = brute_force(q[i], K, V, i, retrieval, sink, recent, scale)
        assert np.max(np.abs(out[i] - np.array(ref))) < 1e-12


# --- closed forms and golden cases ----------------------------------------------

def test_golden_closed_forms():
    for c in json.load(open(GOLDEN))["cases"]:
        K = np.array(c["K"], dtype=np.float64)
        V = np.array(c["V"], dtype=np.float64)
        q = np.array([c["q"]], dtype=np.float64)
        out = A.head_attention(q, [c["position"]], K, V, c["retrieval"], c["sink"], c["recent"],
                               scale=c["scale"])
        assert np.allclose(out[0], c["expected"], atol=1e-12, rtol=0), c["name"]


def test_gqa_golden_two_query_heads_share_kv():
    """Hq=2, Hkv=1: head 0 (q=0) weights keys 0,1 equally -> (2+6)/2 = 4; head 1 (q=ln3)
    weights them 1/4, 3/4 -> 5."""
    Q = np.array([[[0.0], [math.log(3.0)]]])
    K = np.array([[[0.0]], [[1.0]]])
    V = np.array([[[2.0]], [[6.0]]])
    out = A.layer_attention(Q, [1], K, V, np.array([True]), 0, 1, scale=1.0)
    assert np.allclose(out[0, :, 0], [4.0, 5.0], atol=1e-12)


@pytest.mark.parametrize("sink,recent", [(0, 1), (4, 16), (3, 1), (8, 8)])
def test_constant_keys_give_mean_of_visible_values(sink, recent):
    L, D = 60, 8
    rng = np.random.default_rng(sink * 31 + recent)
    q = _rand(rng, L, D)
    K = np.tile(_rand(rng, 1, D), (L, 1))
    V = _rand(rng, L, D)
    out = A.head_attention(q, np.arange(L), K, V, False, sink, recent)
    for i in range(L):
        n_vis = min(i + 1, sink + recent)
        keys = sorted(set(range(min(sink, i + 1))) | set(range(max(0, i - recent + 1), i + 1)))
        assert len(keys) == n_vis
        assert np.allclose(out[i], V[keys].mean(axis=0), atol=1e-12)


def test_one_hot_values_expose_the_weights():
    """V = identity (D >= L) makes O equal to the weight matrix: its support must be the
    visible set exactly, and its nonzero entries the softmax of the visible scores."""
    L, S, R = 40, 3, 7
    rng = np.random.default_rng(11)
    D = L
    q, K = _rand(rng, L, D), _rand(rng, L, D)
    V = np.eye(L)
    out = A.head_attention(q, np.arange(L), K, V, False, S, R)
    for i in range(L):
        support = set(np.nonzero(out[i] > 0)[0].tolist())
        assert support == {j for j in range(i + 1) if j < S or i - j < R}
        keys = sorted(support)
        s = (K[keys] @ q[i]) / math.sqrt(D)
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.allclose(out[i, keys], p, atol=1e-13)


# --- invariants -----------------------------------------------------------------

@pytest.mark.parametrize("L,S,R", [(50, 4, 64), (64, 0, 64), (33, 30, 3), (10, 10, 1)])
def test_streaming_with_large_cache_is_full_attention(L, S, R):
    assert S + R >= L
    rng = np.random.default_rng(L + S)
    q, K, V = _rand(rng, L, 16), _rand(rng, L, 16), _rand(rng, L, 16)
    a = A.head_attention(q, np.arange(L), K, V, False, S, R)
    b = A.head_attention(q, np.arange(L), K, V, True, S, R)
    assert np.max(np.abs(a - b)) < 1e-13


@pytest.mark.parametrize("retrieval", [True, False])
def test_weights_sum_to_one(retrieval):
    L = 90
    rng = np.random.default_rng(5)
    q, K, V = _rand(rng, L, 8) * 4, _rand(rng, L, 8) * 4, _rand(rng, L, 8)
    _, w = A.head_attention(q, np.arange(L), K, V, retrieval, 4, 10, return_weights=True)
    for i, (keys, p) in enumerate(w):
        assert abs(p.sum() - 1.0) < 1e-12
        assert len(keys) == (i + 1 if retrieval else min(i + 1, 14))


def test_streaming_ignores_tokens_outside_sink_and_window():
    L, S, R = 120, 4, 16
    rng = np.random.default_rng(9)
    q, K, V = _rand(rng, L, 16), _rand(rng, L, 16), _rand(rng, L, 16)
    base = A.head_attention(q, np.arange(L), K, V, False, S, R)
    K2, V2 = K.copy(), V.copy()
    i = L - 1
    hidden = [j for j in range(L) if not (j < S or i - j < R)]
    K2[hidden] += 5 * _rand(rng, len(hidden), 16)
    V2[hidden] -= 7
    pert = A.head_attention(q[i:], [i], K2, V2, False, S, R)
    assert np.array_equal(pert[0], base[i])
    full = A.head_attention(q[i:], [i], K2, V2, True, S, R)
    assert np.max(np.abs(full[0] - A.head_attention(q[i:], [i], K, V, True, S, R)[0])) > 1e-3


def test_gqa_equals_mha_with_repeated_kv():
    L, Hkv, G, D = 70, 3, 4, 16
    rng = np.random.default_rng(21)
    Q = _rand(rng, L, Hkv * G, D)
    K, V = _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    mask = np.array([True, False, True])
    gqa = A.layer_attention(Q, np.arange(L), K, V, mask, 2, 9)
    mha = A.layer_attention(Q, np.arange(L), np.repeat(K, G, axis=1), np.repeat(V, G, axis=1),
                            np.repeat(mask, G), 2, 9)
    assert np.max(np.abs(gqa - mha)) < 1e-14


def test_decode_row_equals_prefill_row():
    L, H, D = 80, 4, 16
    rng = np.random.default_rng(4)
    Q, K, V = _rand(rng, L, H, D), _rand(rng, L, H, D), _rand(rng, L, H, D)
    mask = np.array([True, False, False, True])
    full = A.layer_attention(Q, np.arange(L), K, V, mask, 3, 11)
    for t in (0, 5, 13, 14, 15, 79):
        row = A.layer_attention(Q[t:t + 1], [t], K[:t + 1], V[:t + 1], mask, 3, 11)
        assert np.max(np.abs(row[0] - full[t])) < 1e-14


def test_chunked_rows_equal_unchunked():
    """Rows computed in arbitrary groups (as a chunked prefill would) match."""
    L = 1100
    rng = np.random.default_rng(8)
    q, K, V = _rand(rng, L, 8), _rand(rng, L, 8), _rand(rng, L, 8)
    full = A.head_attention(q, np.arange(L), K, V, False, 6, 100)
    for a, b in [(0, 1), (1, 517), (517, 1100)]:
        part = A.head_attention(q[a:b], np.arange(a, b), K[:b], V[:b], False, 6, 100)
        assert np.max(np.abs(part - full[a:b])) < 1e-14


def test_bf16_upcast_is_exact():
    bits = np.array([0x3F80, 0xC040, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    assert A.upcast(bits, "bf16").tolist() == [1.0, -3.0, 2.0 ** -133, 3.3895313892515355e38, -0.0]


# --- planted mistakes -------------------------------------------------------------

def _brute_force_fails(monkeypatch_fn):
    rng = np.random.default_rng(2)
    L, D, S, R = 20, 3, 2, 5
    q, K, V = _rand(rng, L, D), _rand(rng, L, D), _rand(rng, L, D)
    out = A.head_attention(q, np.arange(L), K, V, False, S, R)
    worst = 0.0
    for i in range(L):
        ref = brute_force(q[i], K, V, i, False, S, R, 1 / math.sqrt(D))
        worst = max(worst, float(np.max(np.abs(out[i] - np.array(ref)))))
    return worst > 1e-9


@pytest.mark.parametrize("mutant", [
    lambda i, j, r, s, w: ((j >= 0) & (j <= i)) & (np.asarray(r) | (j < s) | ((i - j) < w - 1)),   # window one short
    lambda i, j, r, s, w: ((j >= 0) & (j <= i)) & (np.asarray(r) | (j < s - 1) | ((i - j) < w)),   # sink one short
    lambda i, j, r, s, w: ((j >= 0) & (j < i)) & (np.asarray(r) | (j < s) | ((i - j) < w)),        # self not visible
    lambda i, j, r, s, w: ((j >= 0) & (j <= i)) & (np.asarray(r) | (j < w) | ((i - j) < s)),       # sink / window swapped
])
def test_planted_mask_mistakes_are_caught(monkeypatch, mutant):
    # (a window or sink widened in ``visible`` alone is not a mistake the oracle can
    # make: the candidate keys bound each row independently, see the next test)
    monkeypatch.setattr(A, "visible", mutant)
    assert _brute_force_fails(None)


def test_planted_wide_candidates_are_caught(monkeypatch):
    """Widening both the candidate window and the rule by one key is caught."""
    orig = A._candidates

    def wide(positions, retrieval, sink, recent):
        return orig(positions, retrieval, sink, recent + 1)

    monkeypatch.setattr(A, "_candidates", wide)
    monkeypatch.setattr(A, "visible", lambda i, j, r, s, w: ((j >= 0) & (j <= i)) & (np.asarray(r) | (j < s) | ((i - j) <= w)))
    assert _brute_force_fails(None)


def test_planted_missing_scale_is_caught(monkeypatch):
    orig = A.head_attention

    def no_scale(q, positions, K, V, retrieval, sink, recent, scale=None, return_weights=False):
        return orig(q, positions, K, V, retrieval, sink, recent, 1.0, return_weights)

    monkeypatch.setattr(A, "head_attention", no_scale)
    rng = np.random.default_rng(0)
    L, H, D = 30, 2, 16
    Q, K, V = _rand(rng, L, H, D), _rand(rng, L, H, D), _rand(rng, L, H, D)
    out = A.layer_attention(Q, np.arange(L), K, V, np.ones(H, bool), 0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).permute(1, 0, 2), torch.from_numpy(K).permute(1, 0, 2),
        torch.from_numpy(V).permute(1, 0, 2), is_causal=True).permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) > 1e-3


def test_planted_gqa_mapping_mistake_is_caught(monkeypatch):
    """Mapping query head h to KV head h % Hkv instead of h // G breaks the GQA pin."""
    L, Hkv, G, D = 30, 2, 2, 8
    rng = np.random.default_rng(1)
    Q = _rand(rng, L, Hkv * G, D)
    K, V = _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    mask = np.array([True, False])
    mha = A.layer_attention(Q, np.arange(L), np.repeat(K, G, axis=1), np.repeat(V, G, axis=1),
                            np.repeat(mask, G), 2, 5)
    wrong = np.stack([A.head_attention(Q[:, h], np.arange(L), K[:, h % Hkv], V[:, h % Hkv],
                                       bool(mask[h % Hkv]), 2, 5) for h in range(Hkv * G)], axis=1)
    assert np.max(np.abs(wrong - mha)) > 1e-3



@pytest.mark.parametrize("retrieval", [True, False])
@pytest.mark.parametrize("t", [0, 5, 6, 7, 30, 34, 60])
def test_periodic_history_equals_the_explicit_history(retrieval, t):
    """head_attention_periodic against head_attention over the repeated history written
    out (period 7), below, at and past period boundaries, for both head kinds."""
    rng = np.random.default_rng(11)
    P, D = 7, 16
    Kp, Vp = rng.standard_normal((P, D)), rng.standard_normal((P, D))
    L = t + 1
    K = Kp[np.arange(L) % P]
    V = Vp[np.arange(L) % P]
    q = rng.standard_normal(D)
    ref = A.head_attention(q[None], [t], K, V, retrieval, 3, 4)[0]
    got = A.head_attention_periodic(q, t, Kp, Vp, retrieval, 3, 4)
    assert np.allclose(got, ref, atol=1e-12, rtol=1e-12)


def test_periodic_history_counts_classes_by_multiplicity():
    """A planted mistake (every class counted once, i.e. the history truncated to one
    period) fails the comparison."""
    rng = np.random.default_rng(12)
    P, D, t = 5, 8, 12
    Kp, Vp = rng.standard_normal((P, D)) * 3, rng.standard_normal((P, D))
    q = rng.standard_normal(D)
    K = Kp[np.arange(t + 1) % P]
    V = Vp[np.arange(t + 1) % P]
    ref = A.head_attention(q[None], [t], K, V, True, 0, 1)[0]
    once = A.head_attention(q[None], [P - 1], Kp, Vp, True, 0, 1)[0]
    assert not np.allclose(once, ref, atol=1e-6)
    assert np.allclose(A.head_attention_periodic(q, t, Kp, Vp, True, 0, 1), ref, atol=1e-12)
