"""Contiguous brute-force attention (numpy, fp64) — TEST INFRASTRUCTURE ONLY.

The textbook case the paged oracle must reduce to: before paging, each
request's K/V sat in one contiguous region ([P2] "vLLM internals (2)",
section on the two kinds of waste of contiguous allocation; [P1] "LLM
inference basics and vLLM internals" §4).  Here K and V of one sequence are
plain [c][H_kv][d] arrays; no block table, no pool layout.  GQA is expressed
as repeating each KV head for its group of query heads ([P1] §2).
"""
import numpy as np


def attention(q, k, v, scale):
    """q: [H][d]; k, v: [c][H_kv][d] (fp64) -> [H][d] fp64 softmax attention."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    H = q.shape[0]
    c, Hkv, _ = k.shape
    if c == 0:
        return np.zeros_like(q)
    group = H // Hkv
    k_rep = np.repeat(k, group, axis=1)          # [c][H][d], head h reads h // group
    v_rep = np.repeat(v, group, axis=1)
    logits = scale * np.einsum("hd,chd->hc", q, k_rep)
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=1, keepdims=True)
    return np.einsum("hc,chd->hd", w, v_rep)


def causal_chunk(q, k, v, scale):
    """The last n = q.shape[0] tokens of a sequence attending causally:
    q: [n][H][d]; k, v: [c][H_kv][d] with c >= n (the whole context, chunk
    included).  Token j sits at position c - n + j and sees keys 0 .. that
    position; each token is the textbook attention over its visible keys."""
    q = np.asarray(q, np.float64)
    c = k.shape[0]
    n = q.shape[0]
    return np.stack([attention(q[j], k[:c - n + j + 1], v[:c - n + j + 1], scale)
                     for j in range(n)])
