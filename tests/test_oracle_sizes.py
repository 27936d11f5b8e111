"""Pins of the oracle's size formula to the pages' printed numbers.

"LLM inference basics and vLLM internals" (ttlab.hopto.org) §2 prints the
per-token KV size table and two cross-checks; the vToken page's "KV cache
basics" prints the Llama-2 7B figure.  Fixtures: tests/golden/kv_sizes.txt,
tests/golden/kv_size_crosschecks.txt.
"""
import os

import pytest

import oracle

G = os.path.join(os.path.dirname(__file__), "golden")


def rows(name):
    with open(os.path.join(G, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


@pytest.mark.parametrize("row", rows("kv_sizes.txt"), ids=lambda r: r[0])
def test_bytes_per_token_table(row):
    _, L, H, d, b, bpt, kib, gib32k = row
    got = oracle.bytes_per_token(int(L), int(H), int(d), int(b))
    assert got == int(bpt)
    assert got == int(kib) * 1024
    assert got * 32768 / 2**30 == pytest.approx(float(gib32k), rel=0, abs=1e-12)


@pytest.mark.parametrize("row", rows("kv_sizes.txt"), ids=lambda r: r[0])
def test_fp8_halves_bytes(row):
    # [P1] §2: FP8 KV cache makes b = 1, halving the size again.
    _, L, H, d, b, bpt, *_ = row
    assert oracle.bytes_per_token(int(L), int(H), int(d), 1) * 2 == int(bpt)


def test_worked_crosschecks():
    for r in rows("kv_size_crosschecks.txt"):
        if r[0] == "BLOCKS":
            tokens, bs, blocks, usable = map(int, r[1:])
            assert -(-tokens // bs) == blocks
            assert blocks - 1 == usable          # block 0 is the null block
            continue
        tokens, L, H, d, b = map(int, r[:5])
        gib, digits = float(r[5]), int(r[6])
        got = tokens * oracle.bytes_per_token(L, H, d, b) / 2**30
        assert round(got, digits) == gib


def test_gqa_ratio_7b():
    # [P1] §11 (interview answer): 7B's 28 query heads as MHA would be 7x.
    assert oracle.bytes_per_token(28, 28, 128, 2) == 7 * oracle.bytes_per_token(28, 4, 128, 2)
