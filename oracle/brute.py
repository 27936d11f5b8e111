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
