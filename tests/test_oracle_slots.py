"""Pins of the oracle's block-table indexing to the pages' diagrams.

"LLM inference basics and vLLM internals" §4 diagram (request A: 38 tokens in
physical 7, 1, 3, the last 6/16 full; request B shares physical 7) and
"vLLM internals (2)", "Block table" diagram (0->7, 1->2, 2->19, 3->4).
Fixture: tests/golden/block_table_examples.txt.
"""
import os

import numpy as np

import oracle

G = os.path.join(os.path.dirname(__file__), "golden")


def examples():
    out = []
    for ln in open(os.path.join(G, "block_table_examples.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        name, bs, table, pos, slot = ln.split()
        out.append((name, int(bs), [int(x) for x in table.split(",")], int(pos), int(slot)))
    return out


def test_slot_examples():
    ex = examples()
    assert len(ex) >= 10
    for name, bs, table, pos, slot in ex:
        assert oracle.slot_of_position(np.array(table, np.int32), pos, bs) == slot, name


def test_request_a_waste_and_sharing():
    bs = 16
    a = np.array([7, 1, 3], np.int32)
    b = np.array([7], np.int32)
    # request A: 38 tokens -> 3 blocks, last block holds 6 of 16 -> waste 10 < bs
    assert -(-38 // bs) == 3 and 38 - 2 * bs == 6
    waste = 3 * bs - 38
    assert waste == 10 and waste <= bs - 1
    # A's and B's first token land on the same physical slot (shared block 7)
    assert oracle.slot_of_position(a, 0, bs) == oracle.slot_of_position(b, 0, bs)
    # decode slot of A's newest token (position 37): physical 3, row 5
    slots = oracle.decode_slots(a[None, :], np.array([38], np.int32), bs)
    assert slots[0] == 3 * 16 + 5


def test_decode_slots_edge_cases():
    bt = np.array([[5, 9], [2, 0]], np.int32)
    slots = oracle.decode_slots(bt, np.array([0, 33], np.int32), 16)
    assert slots[0] == -1           # empty context: no newest token
    assert slots[1] == -1           # position 32 lies past a 2-block table
    slots = oracle.decode_slots(bt, np.array([32, 1], np.int32), 16)
    assert list(slots) == [9 * 16 + 15, 2 * 16]
