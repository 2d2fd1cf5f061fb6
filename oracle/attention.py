"""Plain fp64 masked-softmax attention with the retrieval / streaming head split.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Slow on purpose: every
output row is the textbook softmax over the set of keys the row may see, computed in
float64 with NumPy.  There is no online softmax, no tiling beyond processing rows in
groups, no ring buffer and no constant-length cache: the oracle keeps the whole K/V
history of every head and expresses eviction purely as the visibility rule below, so
it is independent of how any cache lays out or evicts tokens.

What is computed (the plain definition)
---------------------------------------
For query head ``h`` with KV head ``g = h // G`` (``G = Hq / Hkv``) and a query at
absolute position ``i`` (0-based):

* retrieval head: the query sees every earlier token and itself, ``{j : j <= i}``.
  Source: hotpaper.ai page "DuoAttention: Efficient Long-Context LLM Inference with
  Retrieval and Streaming Heads", abstract (retrieval heads need full attention over
  all tokens and keep a full KV cache); nav.superapi.store "What is DuoAttention",
  Technical principles (retrieval heads do full attention on all tokens).
* streaming head: the query sees only the attention sinks and the recent tokens,
  ``{j : j <= i and (j < sink or i - j < recent)}``.  Source: same abstract
  (streaming heads attend to recent tokens and attention sinks and use a light,
  constant-length KV cache); the hotpaper.ai technical-approach section (each layer
  holds a full cache for retrieval heads and a fixed-length cache of recent tokens
  and sinks for streaming heads); cn.bg3.co, DuoAttention 的创新设计 section.
* scores ``s_ij = c * <q_i, k_j>`` with ``c = 1/sqrt(D)`` unless given, softmax over
  the visible set, output ``o_i = sum_j p_ij v_j``.

Readings where the pages are silent: sinks are the first
``sink`` positions; the recent window counts the current token (``i - j < recent``);
sink and window overlap is a set union; labels are per KV head and a query head takes
its KV head's label (MHA and GQA, hotpaper.ai technical-approach section); prefill is
causal; a decode token is appended before it attends, so it sees itself.
"""

from __future__ import annotations

import numpy as np

ROW_GROUP = 512  # rows per NumPy matrix product; only bounds host memory use


def upcast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored values to float64.

    ``dtype`` is "f32" (float32 array) or "bf16" (uint16 array holding bfloat16 bit
    patterns: the 16 high bits of an IEEE float32)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def visible(i, j, retrieval, sink: int, recent: int):
    """Visibility rule: may a query at position ``i`` see the key at position ``j``?

    Broadcasts over ``i`` and ``j``.  ``retrieval`` is a bool (or bool array that
    broadcasts).  See the module docstring for the passages this follows."""
    i = np.asarray(i)
    j = np.asarray(j)
    causal = (j >= 0) & (j <= i)
    streaming_ok = (j < sink) | ((i - j) < recent)
    return causal & (np.asarray(retrieval) | streaming_ok)


def _candidates(positions: np.ndarray, retrieval: bool, sink: int, recent: int):
    """Key positions a group of rows must be tested against, and which are valid.

    Retrieval rows test every key up to the largest row position.  Streaming rows test
    the sink positions ``0..sink-1`` and the ``recent`` positions ending at the row;
    every visible key is in one of the two groups, and a window position below
    ``sink`` is dropped as a duplicate of its sink entry.  Validity is decided by
    ``visible`` alone."""
    positions = np.asarray(positions, dtype=np.int64)
    if retrieval:
        cand = np.broadcast_to(np.arange(int(positions.max()) + 1), (len(positions), int(positions.max()) + 1))
        valid = visible(positions[:, None], cand, True, sink, recent)
        return cand, valid
    sinks = np.broadcast_to(np.arange(sink, dtype=np.int64), (len(positions), sink))
    window = positions[:, None] - recent + 1 + np.arange(recent, dtype=np.int64)[None, :]
    cand = np.concatenate([sinks, window], axis=1)
    valid = visible(positions[:, None], cand, False, sink, recent)
    duplicate = np.zeros_like(valid)
    duplicate[:, sink:] = window < sink
    return cand, valid & ~duplicate


def head_attention(q: np.ndarray, positions, K: np.ndarray, V: np.ndarray,
                   retrieval: bool, sink: int, recent: int, scale: float | None = None,
                   return_weights: bool = False):
    """Attention of query rows of ONE query head against ONE KV head's full history.

    q: [n, D] rows (float64) at absolute ``positions`` (length n).
    K, V: [L, D] float64 history with L > max(positions).
    Returns O [n, D] float64; with ``return_weights`` also a list of (keys, p) per row.
    """
    q = np.asarray(q, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64).reshape(-1)
    n, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if n and positions.max() >= K.shape[0]:
        raise ValueError("history shorter than the largest query position")
    out = np.empty((n, V.shape[1]), dtype=np.float64)
    weights = []
    for a in range(0, n, ROW_GROUP):
        b = min(n, a + ROW_GROUP)
        pos = positions[a:b]
        cand, valid = _candidates(pos, retrieval, sink, recent)
        safe = np.where(valid, cand, 0)
        if retrieval:
            kc = K[: cand.shape[1]]
            s = scale * (q[a:b] @ kc.T)
        else:
            kc = K[safe]  # [rows, cand, D]
            s = scale * np.einsum("rd,rcd->rc", q[a:b], kc)
        s = np.where(valid, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        if retrieval:
            out[a:b] = p @ V[: cand.shape[1]]
        else:
            out[a:b] = np.einsum("rc,rcd->rd", p, V[safe])
        if return_weights:
            for r in range(b - a):
                keys = cand[r][valid[r]]
                order = np.argsort(keys)
                weights.append((keys[order], p[r][valid[r]][order]))
    if return_weights:
        return out, weights
    return out


def layer_attention(Q: np.ndarray, positions, K: np.ndarray, V: np.ndarray,
                    retrieval_kv: np.ndarray, sink: int, recent: int,
                    scale: float | None = None, heads=None) -> np.ndarray:
    """Mixed-head attention of one layer.

    Q: [n, Hq, D] query rows at absolute ``positions``.
    K, V: [L, Hkv, D] full history of every KV head (streaming heads included).
    retrieval_kv: [Hkv] bool, True = retrieval head.  Query head h uses KV head
    h // (Hq // Hkv): the MHA (G = 1) and GQA (G > 1) mapping.
    heads: optional iterable of query heads to compute (others are left NaN).
    Returns O [n, Hq, D] float64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    n, Hq, D = Q.shape
    Hkv = K.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    out = np.full((n, Hq, V.shape[2]), np.nan)
    for h in (range(Hq) if heads is None else heads):
        g = h // G
        out[:, h] = head_attention(Q[:, h], positions, K[:, g], V[:, g],
                                   bool(retrieval_kv[g]), sink, recent, scale)
    return out


def head_attention_periodic(q: np.ndarray, t: int, K_period: np.ndarray, V_period: np.ndarray,
                            retrieval: bool, sink: int, recent: int, scale: float | None = None) -> np.ndarray:
    """Attention of ONE query row at position ``t`` over a history that repeats with
    period P: the key and value at position j are K_period[j mod P], V_period[j mod P].

    The visible set is the one ``visible`` defines (same passages as ``head_attention``).
    For a retrieval head it is every position 0..t: position class c (= j mod P) occurs
    n + [c < r] times, with t + 1 = n P + r, so the softmax over the set equals the
    softmax over one period with each class's weight multiplied by its count (a sum of
    equal terms, grouped).  For a streaming head the sink and window positions are listed
    explicitly.  This lets the oracle check contexts far longer than a history it could
    hold.  q: [D]; K_period, V_period: [P, D] float64.  Returns [D] float64."""
    q = np.asarray(q, dtype=np.float64)
    P, D = K_period.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if retrieval:
        n, r = divmod(int(t) + 1, P)
        count = np.full(P, float(n))
        count[:r] += 1.0
        s = scale * (K_period @ q)
        s = np.where(count > 0, s, -np.inf)
        m = s.max()
        w = count * np.exp(s - m)
        return (w @ V_period) / w.sum()
    cand, valid = _candidates(np.array([t]), False, sink, recent)
    keys = cand[0][valid[0]]
    kc = K_period[keys % P]
    s = scale * (kc @ q)
    e = np.exp(s - s.max())
    return (e @ V_period[keys % P]) / e.sum()
