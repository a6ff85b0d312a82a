"""Pins for the oracle's fixed-budget retention, slot layout and compaction.

KVpop summary: Sec. 3 (sinks + protected recent window + per-head top-k
long-range tokens; attention only over the retained set), App. C.1
(B = s + w + k), App. F (ranking and selection in float32).  Expected
values come from hand-worked fixtures, Python's ``sorted`` (a textbook sort,
a different route from the oracle's C ``qsort``), special cases with known
answers and invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f(x):
    return {"nan": float("nan"), "inf": float("inf"), "-inf": float("-inf"), "-0": -0.0}.get(x, x) \
        if isinstance(x, str) else float(x)


def _layout_positions(sp):
    return sorted(int(p) for p in sp if p >= 0)


def test_golden_hand_worked_layouts():
    g = json.load(open(os.path.join(GOLD, "select_hand.json")))
    for c in g["cases"]:
        sc = np.array([[[_f(x) for x in c["scores"]]]], np.float32)
        sp, ss = oracle.select(sc, c["s"], c["w"], c["budget"])
        assert sp[0, 0].tolist() == c["slot_pos"], c["name"]
        for j, p in enumerate(c["slot_pos"]):
            if p < 0:
                assert ss[0, 0, j] == -np.inf
            else:
                np.testing.assert_array_equal(ss[0, 0, j], sc[0, 0, p])


KINDS = ["normal", "ties", "special", "const", "ramp", "nan"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("S,s,w,budget", [(256, 4, 16, 64), (100, 0, 0, 10), (50, 4, 16, 64),
                                          (300, 1, 7, 200), (33, 33, 0, 40), (1000, 4, 128, 140)])
def test_select_matches_textbook_sort(kind, S, s, w, budget):
    sc = synth.scores((2, 3, S), seed=S + budget, kind=kind).numpy()
    sp, _ = oracle.select(sc, s, w, budget)
    k = budget - s - w
    for b in range(2):
        for h in range(3):
            row = sp[b, h]
            R, chosen = brute.select_positions(sc[b, h], s, w, budget)
            assert _layout_positions(row) == R
            # canonical layout
            assert row[:min(s, S)].tolist() == list(range(min(s, S)))
            pool = row[s:s + k]
            assert [int(p) for p in pool if p >= 0] == chosen
            assert all(p < 0 for p in pool[len(chosen):])
            for p in range(max(S - w, s), S):
                assert row[s + k + p % w] == p


@pytest.mark.parametrize("kind", KINDS)
def test_selection_invariants(kind):
    S, s, w, budget = 512, 4, 32, 100
    k = budget - s - w
    sc = synth.scores((1, 4, S), seed=77, kind=kind).numpy()
    sp, _ = oracle.select(sc, s, w, budget)

    def rank_key(t, row):
        x = float(row[t])
        return (0 if math.isnan(x) else 1, -math.inf if math.isnan(x) else x, -t)

    for h in range(4):
        row = sp[0, h]
        kept = set(int(p) for p in row if p >= 0)
        assert len(kept) == (row >= 0).sum() == min(budget, S)  # no duplicates, full budget
        assert set(range(s)) <= kept and set(range(S - w, S)) <= kept
        pool = [int(p) for p in row[s:s + k] if p >= 0]
        rest = [t for t in range(s, S - w) if t not in kept]
        # every kept long-range token ranks before every dropped eligible token
        worst_kept = min(rank_key(t, sc[0, h]) for t in pool)
        best_dropped = max(rank_key(t, sc[0, h]) for t in rest)
        assert worst_kept > best_dropped


def test_special_cases():
    S, s, w, budget = 200, 4, 16, 50
    k = budget - s - w
    for kind, expect in (("const", list(range(s, s + k))),
                         ("nan", list(range(s, s + k))),
                         ("ramp", list(range(S - w - k, S - w)))):
        sc = synth.scores((1, 1, S), seed=1, kind=kind).numpy()
        sp, _ = oracle.select(sc, s, w, budget)
        assert sp[0, 0, s:s + k].tolist() == expect, kind


def test_permutation_equivariance_distinct_scores():
    S, s, w, budget = 300, 4, 20, 90
    r = np.random.default_rng(3)
    sc = r.permutation(np.arange(S, dtype=np.float32) * 0.37 - 20.0)[None, None]
    sp, _ = oracle.select(sc, s, w, budget)
    # permute the eligible region; the kept *scores* must be the same multiset
    perm = np.arange(S)
    perm[s:S - w] = s + r.permutation(S - w - s)
    sc2 = sc[..., perm]
    sp2, _ = oracle.select(sc2, s, w, budget)
    kept1 = sorted(sc[0, 0, sp[0, 0][sp[0, 0] >= 0]].tolist())
    kept2 = sorted(sc2[0, 0, sp2[0, 0][sp2[0, 0] >= 0]].tolist())
    assert kept1 == kept2


def test_gather_copies_rows_bytewise():
    B, Hkv, S, D, budget = 2, 3, 64, 8, 24
    r = np.random.default_rng(4)
    kb = r.integers(0, 65536, size=(B, Hkv, S, D), dtype=np.uint16)
    sc = synth.scores((B, Hkv, S), seed=9, kind="special").numpy()
    sp, _ = oracle.select(sc, 2, 5, budget)
    kc = oracle.gather(kb, sp)
    for b in range(B):
        for h in range(Hkv):
            for j in range(budget):
                if sp[b, h, j] < 0:
                    assert not kc[b, h, j].any()
                else:
                    assert kc[b, h, j].tobytes() == kb[b, h, sp[b, h, j]].tobytes()


def test_synth_scores_are_seeded():
    a = synth.scores((2, 100), seed=5, kind="special")
    b = synth.scores((2, 100), seed=5, kind="special")
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
