"""The device's next-token choice against the oracle: temperature and top-p
draws (ld_op_sample) and the prompt-forcing, stop-token generation loop
(ld_generate), through the C ABI.

A draw is a step function of the coin, so the device and the oracle agree
except where the coin sits within rounding of a step.  The bar:
  * on the same logits, the device's token equals the oracle's, or equals the
    oracle's for a coin (or topp) moved by at most 1e-5 (the device sums fp32
    numerators, 32 per thread in fp32 and across threads in double: a relative
    error near 1e-6);
  * in a generation, whose logits differ from the oracle's by up to the decode
    step's parity bar (1e-4 * max |logit|), the coin moves by at most
    2 * (that bar) / temperature + 1e-5, the most the move of the logits can
    shift a cumulative probability.  Tokens are compared up to the first step
    where the device's choice is only acceptable this way; from there the two
    continuations differ and both are right.
"""
import numpy as np
import pytest

import llama_transformer_decode_amd as pkg
import oracle
import synth
from gpu_util import dev, host, torch_or_skip
from llama_transformer_decode_amd import ld

pytestmark = pytest.mark.gpu

LN = np.log(np.array([1.0, 2.0, 3.0, 4.0])).astype(np.float32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch_or_skip()


def op_sample(logits, T, topp, coin):
    t = dev(np.asarray(logits, np.float32))
    return ld.ld_op_sample(t.data_ptr(), t.numel(), T, topp, coin)


def acceptable(tok, logits, T, topp, coin, delta):
    if tok == oracle.sample(logits, T, topp, coin):
        return True
    for dc in np.linspace(-delta, delta, 21):
        c = min(max(coin + dc, 0.0), 1.0 - 2.0 ** -24)
        for dp in ((0.0, -delta, delta) if 0 < topp < 1 else (0.0,)):
            if tok == oracle.sample(logits, T, topp + dp, c):
                return True
    return False


# ----------------------------------------------------------------------------- one draw

@pytest.mark.parametrize("coin,tok", [(0.0, 0), (0.05, 0), (0.15, 1), (0.35, 2), (0.65, 3), (0.9999, 3)])
@pytest.mark.parametrize("topp", [0.0, 1.0])
def test_multinomial_closed_form(coin, tok, topp):
    assert op_sample(LN, 1.0, topp, coin) == tok


@pytest.mark.parametrize("coin,tok", [(0.0, 3), (0.5, 3), (0.57, 3), (0.58, 2), (0.99, 2)])
def test_top_p_closed_form(coin, tok):
    assert op_sample(LN, 1.0, 0.5, coin) == tok


def test_top_p_set_order_and_ties():
    assert op_sample(LN, 1.0, 0.99, 0.05) == 3          # most likely first
    assert op_sample(LN, 1.0, 0.75, 0.79) == 1          # third token joins at topp .75
    z = np.zeros(4, np.float32)
    assert op_sample(z, 1.0, 0.5, 0.4) == 0              # equal probabilities in index order
    assert op_sample(z, 1.0, 0.5, 0.6) == 1
    assert op_sample(z, 1.0, 0.3, 0.99) == 1


def test_temperature_and_greedy():
    l = np.array([0.0, np.log(4.0)], np.float32)
    assert op_sample(l, 2.0, 0.0, 1 / 3 - 1e-3) == 0 and op_sample(l, 2.0, 0.0, 1 / 3 + 1e-3) == 1
    t = np.array([0.5, 3.0, -1.0, 3.0, 2.9], np.float32)
    for coin in (0.0, 0.5, 0.99):
        assert op_sample(t, 0.0, 0.9, coin) == 1         # temperature 0: first maximum
        assert op_sample(t, -1.0, 0.0, coin) == 1


@pytest.mark.parametrize("n", [1, 3, 256, 257, 1000, 1023, 1025, 4097, 8192, 8193, 32000, 32768])
@pytest.mark.parametrize("T,topp", [(1.0, 0.0), (0.6, 0.0), (1.0, 0.9), (0.8, 0.5), (1.5, 0.95)])
def test_random_logits_many_coins(n, T, topp):
    rng = np.random.default_rng(n * 7 + int(T * 10) + int(topp * 100))
    l = (rng.standard_normal(n) * 3).astype(np.float32)
    t = dev(l)
    coins = synth.coins(24, 4242, n)
    exact = 0
    for c in coins:
        got = ld.ld_op_sample(t.data_ptr(), n, T, topp, float(c))
        assert 0 <= got < n
        want = oracle.sample(l, T, topp, float(c))
        exact += got == want
        assert got == want or acceptable(got, l, T, topp, float(c), 1e-5), (n, T, topp, float(c), got, want)
    assert exact >= len(coins) - 1


def test_top_p_with_many_exact_ties():
    # integer logits: long runs of equal probabilities inside and at the edge of the set
    rng = np.random.default_rng(5)
    l = rng.integers(-3, 3, 5000).astype(np.float32)
    t = dev(l)
    for topp in (0.2, 0.5, 0.77):
        for c in synth.coins(16, 77, int(topp * 100)):
            got = ld.ld_op_sample(t.data_ptr(), l.size, 1.0, topp, float(c))
            assert acceptable(got, l, 1.0, topp, float(c), 1e-5)


def test_a_concentrated_distribution():
    l = np.full(32000, -50.0, np.float32)
    l[123] = 10.0
    l[77] = 9.0
    t = dev(l)
    for topp in (0.0, 0.5, 0.9, 0.99999):
        for c in (0.0, 0.3, 0.7310, 0.7312, 0.9999):
            got = ld.ld_op_sample(t.data_ptr(), l.size, 1.0, topp, c)
            assert acceptable(got, l, 1.0, topp, c, 1e-5)


# ----------------------------------------------------------------------------- generation loop

SMALL = ["tiny", "stories15m", "gqa_small"]
_blobs = {}


def blob_of(name):
    if name not in _blobs:
        cfg = synth.CONFIGS[name]
        b = synth.make_blob(cfg)
        _blobs[name] = (cfg, b, dev(b))
    return _blobs[name]


def compare_generation(cfg, blob, got, prompt, pos, T, topp, coins, cache=None):
    """Walk the device's tokens with the oracle, teacher-forced on them: every
    forced token must match, every drawn token must be the oracle's draw or
    within the generation bar of it.  Returns the number of steps that matched
    exactly before the first boundary case (or all of them) and the cache."""
    cache = cache if cache is not None else oracle.KVCache(cfg)
    tok = int(prompt[0])
    for i, g in enumerate(got):
        logits = oracle.forward(cfg, blob, cache, tok, pos + i)
        if i + 1 < len(prompt):
            assert g == prompt[i + 1]
        else:
            want = oracle.sample(logits, T, topp, float(coins[i]))
            if g != want:
                bar = 1e-4 * float(np.max(np.abs(logits)))
                delta = (2 * bar / T if T > 0 else 0) + 1e-5
                if T > 0:
                    assert acceptable(int(g), logits, T, topp, float(coins[i]), delta), (i, g, want)
                else:
                    assert logits[g] >= logits.max() - bar, (i, g, want)
                return i, cache
        tok = int(g)
    return len(got), cache


@pytest.mark.parametrize("graph", [True, False])
@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("T,topp", [(1.0, 0.0), (0.8, 0.9), (1.3, 0.5)])
def test_sampled_generation_matches_the_oracle(name, T, topp, graph):
    cfg, b, w = blob_of(name)
    prompt = synth.prefill_tokens(cfg, 9)
    prompt[0] = 1
    n = min(cfg.seq_len, 48)
    coins = synth.coins(n, cfg.seed, 11)
    with pkg.Model(cfg, w, graph=graph) as m:
        got = m.generate_sampled(prompt, 0, n, T, topp, -1, coins)
        assert got.size == n and np.all((got >= 0) & (got < cfg.vocab_size))
        matched, _ = compare_generation(cfg, b, got, prompt, 0, T, topp, coins)
        print(f"[{name} T={T} topp={topp}] {matched}/{n} steps equal to the oracle's before any boundary case")
        assert matched >= len(prompt) - 1


@pytest.mark.parametrize("name", SMALL)
def test_cache_rows_of_a_sampled_run(name):
    # cache rows 0..n-1 equal the oracle's within the decode bar; rows above untouched
    cfg, b, w = blob_of(name)
    prompt = np.array([1, 5, 9], np.int32)
    n = 20
    coins = synth.coins(n, cfg.seed, 12)
    with pkg.Model(cfg, w) as m:
        got = m.generate_sampled(prompt, 0, n, 0.9, 0.8, -1, coins)
        k, v = (host(t) for t in m.read_kv_cache())
    matched, cache = compare_generation(cfg, b, got, prompt, 0, 0.9, 0.8, coins)
    upto = matched  # rows the oracle computed on the same tokens
    for g, r in ((k, cache.k), (v, cache.v)):
        scale = np.max(np.abs(r[:, :upto]))
        assert np.max(np.abs(g[:, :upto] - r[:, :upto])) <= 1e-4 * scale
        assert np.all(g[:, n:] == 0)


def test_greedy_loop_through_generate_equals_generate_greedy():
    cfg, b, w = blob_of("stories15m")
    with pkg.Model(cfg, w) as m:
        a = m.generate(1, 0, 40)
        m.reset()
        g = m.generate_sampled([1], 0, 40, 0.0, 0.9, -1, None)
    assert np.array_equal(a, g)


@pytest.mark.parametrize("name", ["tiny", "gqa_small"])
def test_stop_token_ends_the_run_and_nothing_after_it_is_written(name):
    cfg, b, w = blob_of(name)
    n = min(cfg.seq_len, 60)
    coins = synth.coins(n, cfg.seed, 13)
    with pkg.Model(cfg, w) as m:
        full = m.generate_sampled([1], 0, n, 1.2, 0.0, -1, coins)
        # a stop token first drawn at step j >= 20 (so the stop lands past the first 16-step chunk)
        j = next((i for i in range(20, n) if full[i] not in full[:i]), None)
        if j is None:
            pytest.skip("no fresh token late in the run")
        m.reset()
        got = m.generate_sampled([1], 0, n, 1.2, 0.0, int(full[j]), coins)
        assert got.size == j + 1 and np.array_equal(got, full[:j + 1])
        k, v = (host(t) for t in m.read_kv_cache())
        assert np.all(k[:, j + 1:] == 0) and np.all(v[:, j + 1:] == 0)   # queued steps past the stop wrote nothing
        assert np.any(k[:, j] != 0)
        # the loop picks up after the stop: continuing from the stop token equals the unstopped run
        rest = m.generate_sampled([int(full[j])], j + 1, n - j - 1, 1.2, 0.0, -1, coins[j + 1:])
        assert np.array_equal(np.concatenate([got, rest]), full)


def test_forced_stop_token_inside_the_prompt():
    cfg, b, w = blob_of("tiny")
    with pkg.Model(cfg, w) as m:
        got = m.generate_sampled([1, 7, 9, 11], 0, 30, 1.0, 0.0, 9, synth.coins(30, 1, 2))
    assert np.array_equal(got, [7, 9])


def test_prompt_longer_than_the_run_and_resume_at_a_later_position():
    cfg, b, w = blob_of("gqa_small")
    prompt = synth.prefill_tokens(cfg, 40)
    with pkg.Model(cfg, w) as m:
        got = m.generate_sampled(prompt, 0, 25, 1.0, 0.9, -1, synth.coins(25, 3, 3))
        assert np.array_equal(got, prompt[1:26])
        # a second call continues the cache at position 25
        coins = synth.coins(10, 3, 4)
        more = m.generate_sampled([int(prompt[25])], 25, 10, 0.7, 0.0, -1, coins)
    cache = oracle.KVCache(cfg)
    for p in range(25):
        oracle.forward(cfg, b, cache, int(prompt[p]), p)
    matched, _ = compare_generation(cfg, b, more, [int(prompt[25])], 25, 0.7, 0.0, coins, cache=cache)
    assert matched >= 1


def test_generation_is_deterministic_and_graph_equals_direct():
    cfg, b, w = blob_of("stories15m")
    coins = synth.coins(64, 9, 9)
    with pkg.Model(cfg, w, graph=True) as g, pkg.Model(cfg, w, graph=False) as e:
        a = g.generate_sampled([1, 2, 3], 0, 64, 0.9, 0.9, -1, coins)
        g.reset()
        a2 = g.generate_sampled([1, 2, 3], 0, 64, 0.9, 0.9, -1, coins)
        c = e.generate_sampled([1, 2, 3], 0, 64, 0.9, 0.9, -1, coins)
    assert np.array_equal(a, a2) and np.array_equal(a, c)


@pytest.mark.parametrize("graph", [True, False])
@pytest.mark.parametrize("name", ["tiny", "gqa_small"])
def test_greedy_prompt_and_stop_token_match_the_oracle(name, graph):
    # at temperature 0: prompt forcing, the greedy steps after it and a stop
    # token must equal the oracle's loop, with and without graph replay
    cfg, b, w = blob_of(name)
    prompt = [int(t) for t in synth.prefill_tokens(cfg, 6)]
    n = 24
    with pkg.Model(cfg, w, graph=graph) as m:
        got = m.generate_sampled(prompt, 0, n, 0.0, 0.0, -1, None)
        assert got.size == n and np.array_equal(got[:len(prompt) - 1], prompt[1:])
        matched, _ = compare_generation(cfg, b, got, prompt, 0, 0.0, 0.0, np.zeros(n, np.float32))
        assert matched == n
        # stop at the first greedy token that is new to the run
        j = next((i for i in range(len(prompt), n) if got[i] not in got[:i]), None)
        if j is not None:
            m.reset()
            stopped = m.generate_sampled(prompt, 0, n, 0.0, 0.0, int(got[j]), None)
            assert np.array_equal(stopped, got[:j + 1])


def test_greedy_and_sampled_calls_alternate_on_one_model():
    # the control block changes call by call under one captured step:
    # switching between greedy and sampled calls changes no result
    cfg, b, w = blob_of("stories15m")
    coins = synth.coins(16, 5, 5)
    with pkg.Model(cfg, w) as m:
        g1 = m.generate(1, 0, 16)
        s1 = m.generate_sampled([int(g1[-1])], 16, 16, 0.9, 0.9, -1, coins)
        g2 = m.generate(int(s1[-1]), 32, 16)
    with pkg.Model(cfg, w) as a, pkg.Model(cfg, w) as c:
        assert np.array_equal(a.generate(1, 0, 16), g1)
        assert np.array_equal(a.generate_sampled([int(g1[-1])], 16, 16, 0.9, 0.9, -1, coins), s1)
        c.generate(1, 0, 16)
        c.generate_sampled([int(g1[-1])], 16, 16, 0.9, 0.9, -1, coins)
        assert np.array_equal(c.generate(int(s1[-1]), 32, 16), g2)
    matched, _ = compare_generation(cfg, b, g1, [1], 0, 0.0, 0.0, np.zeros(16, np.float32))
    assert matched == 16


def test_generate_range_errors():
    cfg, b, w = blob_of("tiny")
    with pkg.Model(cfg, w) as m:
        bad = [
            dict(prompt=[cfg.vocab_size], pos=0, n=4),
            dict(prompt=[1], pos=cfg.seq_len - 2, n=3),
            dict(prompt=[1], pos=-1, n=2),
            dict(prompt=[1], pos=0, n=4, stop_token=cfg.vocab_size),
            dict(prompt=[1], pos=0, n=4, stop_token=-2),
            dict(prompt=[1], pos=0, n=4, T=1.0, coins=[0.5, 0.5, 1.0, 0.5]),
            dict(prompt=[1], pos=0, n=4, T=float("nan"), coins=[0.5] * 4),
        ]
        for a in bad:
            with pytest.raises(ld.LdError) as e:
                m.generate_sampled(a["prompt"], a["pos"], a["n"], a.get("T", 0.0), 0.0, a.get("stop_token", -1),
                                   a.get("coins"))
            assert e.value.status == ld.LD_E_RANGE, a
        with pytest.raises(ld.LdError) as e:
            m.generate_sampled([1], 0, 4, 1.0, 0.0, -1, None)
        assert e.value.status == ld.LD_E_NULL
        with pytest.raises(ld.LdError) as e:
            m.generate_sampled([], 0, 4, 0.0, 0.0, -1, None)
        assert e.value.status in (ld.LD_E_NULL, ld.LD_E_RANGE)
        # the forced coins are not read: a prompt covering every step needs no valid coins
        got = m.generate_sampled([1, 2, 3, 4, 5], 0, 4, 1.0, 0.0, -1, [7.0, 7.0, 7.0, 7.0])
        assert np.array_equal(got, [2, 3, 4, 5])
        # the model still works after the rejected calls
        assert m.generate_sampled([1], 0, 3, 0.0, 0.0, -1, None).size == 3


def test_generation_up_to_the_last_position():
    # the loop runs to the end of the cache; the last step's draw is still made
    cfg, b, w = blob_of("tiny")
    coins = synth.coins(cfg.seq_len, cfg.seed, 21)
    with pkg.Model(cfg, w) as m:
        got = m.generate_sampled([1, 9], 0, cfg.seq_len, 1.1, 0.8, -1, coins)
    assert got.size == cfg.seq_len
    matched, _ = compare_generation(cfg, b, got, [1, 9], 0, 1.1, 0.8, coins)
    assert matched >= 1
