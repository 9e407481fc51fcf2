"""Pins of the oracle's sampler and of its prompt-forcing, stop-token generation
loop to what the pages and the mathematics fix.

The sampler is the three-mode sample() of the "run.c 逐行解讀" page (§6): greedy
at temperature 0, else a draw from softmax(logits / temperature), over every
token, or with 0 < topp < 1 over the smallest most-likely set reaching topp.
The draw is the cumulative walk of sample() on the "run.c" page.  The checks
use closed forms on hand-sized distributions and an exact counting property of
the walk: on the coin grid (k + 1/2) / N, token i is drawn for N * p_i grid
points, give or take one, with p_i computed here by numpy in float64.
"""
import math

import numpy as np
import pytest

import oracle
import synth

LN = np.log(np.array([1.0, 2.0, 3.0, 4.0])).astype(np.float32)  # softmax -> [.1, .2, .3, .4]


@pytest.mark.parametrize("coin,tok", [(0.0, 0), (0.05, 0), (0.15, 1), (0.35, 2), (0.65, 3), (0.9999, 3)])
@pytest.mark.parametrize("topp", [0.0, 1.0, -0.5, 1.5])
def test_multinomial_closed_form(coin, tok, topp):
    # topp outside (0, 1): plain draw in index order, cumulative [.1, .3, .6, 1]
    assert oracle.sample(LN, 1.0, topp, coin) == tok


@pytest.mark.parametrize("coin,tok", [(0.0, 3), (0.5, 3), (0.57, 3), (0.58, 2), (0.99, 2)])
def test_top_p_closed_form(coin, tok):
    # topp 0.5: most likely first -> {3 (.4), 2 (.3)}, mass .7; walk .4/.7 = .5714 then 1
    assert oracle.sample(LN, 1.0, 0.5, coin) == tok


def test_top_p_walks_in_descending_probability():
    # topp 0.99 keeps all four tokens but walks them most likely first: a small coin draws token 3,
    # where the plain draw (topp 1) draws token 0
    assert oracle.sample(LN, 1.0, 0.99, 0.05) == 3
    assert oracle.sample(LN, 1.0, 1.0, 0.05) == 0


def test_top_p_set_is_the_smallest_that_reaches_p():
    # topp .75: .4 + .3 = .7 < .75, so token 1 (.2) joins; mass .9, walk .4/.9, .7/.9, 1
    assert oracle.sample(LN, 1.0, 0.75, 0.43) == 3
    assert oracle.sample(LN, 1.0, 0.75, 0.46) == 2
    assert oracle.sample(LN, 1.0, 0.75, 0.77) == 2
    assert oracle.sample(LN, 1.0, 0.75, 0.79) == 1
    # token 0 is never drawn
    assert all(oracle.sample(LN, 1.0, 0.75, c) != 0 for c in np.linspace(0, 0.9999, 101))


def test_top_p_ties_in_index_order():
    z = np.zeros(4, np.float32)  # uniform: the set for topp .5 is {0, 1}
    assert oracle.sample(z, 1.0, 0.5, 0.4) == 0
    assert oracle.sample(z, 1.0, 0.5, 0.6) == 1
    assert oracle.sample(z, 1.0, 0.3, 0.99) == 1  # .25 < .3: two tokens needed


@pytest.mark.parametrize("T,logits,cut", [(2.0, [0.0, math.log(4.0)], 1 / 3), (0.5, [0.0, math.log(2.0)], 0.2),
                                          (1.0, [0.0, math.log(4.0)], 0.2)])
def test_temperature_divides_the_logits(T, logits, cut):
    # softmax(l / T): T=2 on ln[1,4] -> [1/3, 2/3]; T=.5 on ln[1,2] -> [1/5, 4/5]
    l = np.array(logits, np.float32)
    assert oracle.sample(l, T, 0.0, cut - 1e-3) == 0
    assert oracle.sample(l, T, 0.0, cut + 1e-3) == 1


@pytest.mark.parametrize("T", [0.0, -1.0])
def test_temperature_zero_is_the_argmax(T):
    l = np.array([0.5, 3.0, -1.0, 3.0, 2.9], np.float32)
    for coin in (0.0, 0.3, 0.99):
        for topp in (0.0, 0.5, 1.0):
            assert oracle.sample(l, T, topp, coin) == 1  # first of the tied maxima


def _grid_counts(l, T, topp, N, page):
    coins = (np.arange(N) + 0.5) / N
    return np.bincount([oracle.sample(l, T, topp, c, page=page) for c in coins], minlength=l.size)


def _softmax64(l, T):
    z = l.astype(np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


@pytest.mark.parametrize("page", [False, True])
@pytest.mark.parametrize("T", [0.7, 1.0, 1.6])
def test_multinomial_grid_counts_are_the_softmax(T, page):
    l = np.random.default_rng(11).standard_normal(40).astype(np.float32) * 2
    N = 20000
    counts = _grid_counts(l, T, 0.0, N, page)
    assert np.all(np.abs(counts - N * _softmax64(l, T)) <= 1.01 + (4 if page else 0))


@pytest.mark.parametrize("page", [False, True])
@pytest.mark.parametrize("topp", [0.3, 0.6, 0.9])
def test_top_p_grid_counts_are_the_renormalised_nucleus(topp, page):
    l = np.random.default_rng(12).standard_normal(40).astype(np.float32) * 2
    T, N = 0.9, 8000
    p = _softmax64(l, T)
    order = np.lexsort((np.arange(p.size), -p))  # descending, ties to the lower index
    k = int(np.searchsorted(np.cumsum(p[order]), topp, side="left")) + 1
    keep = order[:k]
    want = np.zeros_like(p)
    want[keep] = p[keep] / p[keep].sum()
    counts = _grid_counts(l, T, topp, N, page)
    assert np.all(counts[want == 0] == 0)
    assert np.all(np.abs(counts - N * want) <= 1.01 + (4 if page else 0))


def test_sample_of_one_token():
    assert oracle.sample(np.array([3.0], np.float32), 1.0, 0.9, 0.7) == 0
    assert oracle.sample(np.array([3.0], np.float32), 1.0, 0.0, 0.7) == 0


# ----------------------------------------------------------------------------- generation loop

CFG = synth.CONFIGS["tiny"]


@pytest.fixture(scope="module")
def blob():
    return synth.make_blob(CFG)


def _coins(n, stream=5):
    return synth.coins(n, CFG.seed, stream)


def test_greedy_loop_is_the_special_case(blob):
    # temperature 0 with a one-token prompt is the greedy loop (the "run.c" page's main loop)
    n = 24
    toks, lg = oracle.generate_sampled(CFG, blob, oracle.KVCache(CFG), [1], 0, n, 0.0, 0.9, -1, _coins(n),
                                       keep_logits=True)
    ref, rlg = oracle.generate(CFG, blob, oracle.KVCache(CFG), 1, 0, n, keep_logits=True)
    assert np.array_equal(toks, ref) and np.array_equal(lg, rlg)


def test_prompt_tokens_are_forced_then_sampled(blob):
    prompt = np.array([1, 17, 200, 5, 99, 42], np.int32)
    n, T, topp = 20, 0.8, 0.9
    coins = _coins(n)
    toks, lg = oracle.generate_sampled(CFG, blob, oracle.KVCache(CFG), prompt, 0, n, T, topp, -1, coins,
                                       keep_logits=True)
    assert toks.size == n
    assert np.array_equal(toks[:prompt.size - 1], prompt[1:])
    # each step's logits are the teacher-forced ones on the token the loop fed in
    cache, fed = oracle.KVCache(CFG), np.concatenate([prompt[:1], toks[:-1]])
    for i in range(n):
        assert np.array_equal(lg[i], oracle.forward(CFG, blob, cache, int(fed[i]), i))
    # after the prompt, step i's token is the draw with coin i
    for i in range(prompt.size - 1, n):
        assert toks[i] == oracle.sample(lg[i], T, topp, float(coins[i]))
    # coins at forced steps are never used
    c2 = coins.copy()
    c2[:prompt.size - 1] = 0.999
    t2, _ = oracle.generate_sampled(CFG, blob, oracle.KVCache(CFG), prompt, 0, n, T, topp, -1, c2)
    assert np.array_equal(t2, toks)


def test_stop_token_ends_the_loop_and_is_returned(blob):
    n, T = 40, 1.2
    coins = _coins(n, 9)
    full, _ = oracle.generate_sampled(CFG, blob, oracle.KVCache(CFG), [1], 0, n, T, 0.0, -1, coins)
    j = next(i for i in range(1, n) if full[i] not in full[:i])  # first occurrence past step 0
    toks, _ = oracle.generate_sampled(CFG, blob, oracle.KVCache(CFG), [1], 0, n, T, 0.0, int(full[j]), coins)
    assert toks.size == j + 1 and np.array_equal(toks, full[:j + 1])
    # a forced prompt token equal to the stop token ends the loop too (the check follows the choice)
    toks, _ = oracle.generate_sampled(CFG, blob, oracle.KVCache(CFG), [1, 7, 9, 11], 0, n, T, 0.0, 9, coins)
    assert np.array_equal(toks, [7, 9])


def test_generation_from_a_later_position_continues_the_cache(blob):
    # two calls (positions 0..5 then 6..15) equal one call over 0..15
    prompt = np.array([1, 3, 4, 5], np.int32)
    coins = _coins(16, 3)
    whole, _ = oracle.generate_sampled(CFG, blob, oracle.KVCache(CFG), prompt, 0, 16, 0.9, 0.8, -1, coins)
    cache = oracle.KVCache(CFG)
    a, _ = oracle.generate_sampled(CFG, blob, cache, prompt, 0, 6, 0.9, 0.8, -1, coins[:6])
    b, _ = oracle.generate_sampled(CFG, blob, cache, [int(a[-1])], 6, 10, 0.9, 0.8, -1, coins[6:])
    assert np.array_equal(np.concatenate([a, b]), whole)


def test_generation_rejects_out_of_range_arguments(blob):
    c = oracle.KVCache(CFG)
    with pytest.raises(ValueError):
        oracle.generate_sampled(CFG, blob, c, [], 0, 4, 1.0, 0.0, -1, _coins(4))
    with pytest.raises(ValueError):
        oracle.generate_sampled(CFG, blob, c, [1], CFG.seq_len - 2, 3, 1.0, 0.0, -1, _coins(3))
