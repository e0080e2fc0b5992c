"""Pins of the oracle's draft-and-verify loop: a hand-worked example, the
target's greedy chain by brute force for any draft, and the two extremes
(the draft always agrees / never agrees) in closed form."""

import json
import math
import os

import numpy as np
import pytest

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
HAND = json.load(open(os.path.join(HERE, "golden", "speculation_hand_example.json")))


def test_hand_example():
    tgt, drf = HAND["target"], HAND["draft"]
    toks, st = O.speculative_decode(lambda t: drf[t], lambda t: tgt[t], HAND["first_token"], HAND["n_tokens"],
                                    HAND["k"])
    assert toks == HAND["tokens"]
    assert st == HAND["stats"]
    assert O.speculation_byte_ratio(st, HAND["n_tokens"]) == HAND["byte_ratio"]


def greedy_chain(next_fn, first, n):
    out, t = [], first
    for _ in range(n):
        t = next_fn(t)
        out.append(t)
    return out


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("k", [1, 2, 3, 7])
def test_emits_the_target_chain_for_any_draft(seed, k):
    rng = np.random.default_rng(seed)
    V = 40
    tgt = rng.integers(0, V, V)
    agree = rng.random(V) < rng.uniform(0.0, 1.0)
    drf = np.where(agree, tgt, rng.integers(0, V, V))
    n = 57
    toks, st = O.speculative_decode(lambda t: drf[t], lambda t: tgt[t], 3, n, k)
    assert toks == greedy_chain(lambda t: int(tgt[t]), 3, n)
    assert st["draft_steps"] == k * st["rounds"] and st["drafted"] == st["draft_steps"]
    assert st["emitted"] == st["accepted"] + st["rounds"] >= n
    assert st["emitted"] - n < k + 1          # only the last round overshoots


@pytest.mark.parametrize("k,n", [(1, 10), (3, 17), (4, 5), (7, 64)])
def test_a_perfect_draft_keeps_every_draft(k, n):
    nxt = lambda t: (3 * t + 1) % 11
    toks, st = O.speculative_decode(nxt, nxt, 2, n, k)
    assert toks == greedy_chain(nxt, 2, n)
    assert st["rounds"] == math.ceil(n / (k + 1))
    assert st["accepted"] == k * st["rounds"]
    # bytes per token: (k*4 + 8) / ((k + 1) * 8) when n is a multiple of k + 1
    if n % (k + 1) == 0:
        assert O.speculation_byte_ratio(st, n) == (4 * k + 8) / (8 * (k + 1))


@pytest.mark.parametrize("k", [1, 2, 5])
def test_a_draft_that_never_agrees_emits_one_token_per_round(k):
    tgt = lambda t: (t + 1) % 9
    drf = lambda t: (t + 2) % 9
    n = 12
    toks, st = O.speculative_decode(drf, tgt, 0, n, k)
    assert toks == greedy_chain(tgt, 0, n)
    assert st["rounds"] == n and st["accepted"] == 0 and st["emitted"] == n
    assert O.speculation_byte_ratio(st, n) == (4 * k + 8) / 8


def test_rejects_k_below_one():
    with pytest.raises(ValueError):
        O.speculative_decode(lambda t: t, lambda t: t, 0, 3, 0)
