"""The whole decode step through the C ABI against the oracle.

Parity bar: at every step, max |logit_gpu - logit_oracle| <= 1e-4 * max |logit_oracle|
(fp32).  Runs are teacher-forced by the oracle's tokens (the GPU gets the
oracle's token at each step through ld_forward), so every step's logits are
compared.  A free-running greedy generation must reproduce the oracle's tokens
up to the first tie event, a step where the oracle's top two logits are within
that tolerance; from then on both continuations are correct.
"""
import numpy as np
import pytest

import llama_transformer_decode_amd as pkg
import oracle
import synth
from gpu_util import acceptable_token, dev, host, logits_close, tie_tolerance, top2_gap, torch_or_skip
from llama_transformer_decode_amd import ld

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "stories15m", "gqa_small"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch_or_skip()


_blobs = {}


def blob_of(name):
    if name not in _blobs:
        cfg = synth.CONFIGS[name]
        b = synth.make_blob(cfg)
        _blobs[name] = (cfg, b, dev(b))
    return _blobs[name]


_oracle_runs = {}


def oracle_run(name):
    """Oracle greedy run from token 1 at position 0 over the whole sequence."""
    if name not in _oracle_runs:
        cfg, b, _ = blob_of(name)
        toks, logits = oracle.generate(cfg, b, oracle.KVCache(cfg), 1, 0, cfg.seq_len, keep_logits=True)
        _oracle_runs[name] = (toks, logits)
    return _oracle_runs[name]


@pytest.mark.parametrize("graph", [True, False])
@pytest.mark.parametrize("name", SMALL)
def test_teacher_forced_logits_every_position(name, graph):
    cfg, b, w = blob_of(name)
    toks, ref = oracle_run(name)
    inputs = np.concatenate([[1], toks[:-1]])
    worst = 0.0
    with pkg.Model(cfg, w, graph=graph) as m:
        for p in range(cfg.seq_len):
            got = host(m.forward(int(inputs[p]), p))
            ok, err, tol = logits_close(got, ref[p])
            assert ok, f"{name} pos {p}: max |d logit| {err:.3g} > {tol:.3g}"
            worst = max(worst, err / tol)
            assert ld.ld_argmax_last(m.h) == oracle.argmax(got)
    print(f"{name}: worst error / tolerance = {worst:.3f}")


@pytest.mark.parametrize("name", SMALL)
def test_free_running_greedy_matches_up_to_first_tie(name):
    cfg, b, w = blob_of(name)
    toks, ref = oracle_run(name)
    with pkg.Model(cfg, w) as m:
        got = m.generate(1, 0, cfg.seq_len)
    ties = [p for p in range(cfg.seq_len) if top2_gap(ref[p]) <= tie_tolerance(ref[p])]
    first_tie = ties[0] if ties else cfg.seq_len
    assert np.array_equal(got[:first_tie], toks[:first_tie]), \
        f"{name}: first mismatch at {int(np.argmax(got[:first_tie] != toks[:first_tie]))}, first tie {first_tie}"
    if first_tie < cfg.seq_len:
        assert acceptable_token(int(got[first_tie]), ref[first_tie])
    print(f"{name}: {len(ties)} tie events, first at {first_tie}")


@pytest.mark.parametrize("name", SMALL)
def test_graph_and_direct_launches_are_bit_identical(name):
    cfg, b, w = blob_of(name)
    n = min(cfg.seq_len, 40)
    with pkg.Model(cfg, w, graph=True) as g, pkg.Model(cfg, w, graph=False) as e:
        tg, te = g.generate(1, 0, n), e.generate(1, 0, n)
        assert np.array_equal(tg, te)
        for p in (n - 1, n // 2):  # replays after a finished generation, then logits
            assert np.array_equal(host(g.forward(int(tg[p - 1]), p)), host(e.forward(int(te[p - 1]), p)))
        kg, vg = g.read_kv_cache()
        ke, ve = e.read_kv_cache()
        assert np.array_equal(host(kg), host(ke)) and np.array_equal(host(vg), host(ve))


def test_fused_and_separate_attention_launches_agree():
    # the tiny model runs q/k/v and attention as one launch at every position;
    # with LD_OPT_NO_FUSE it launches them apart: both within the bar of the
    # oracle, and of each other to the rounding of the attention's sums
    cfg, b, w = blob_of("tiny")
    toks, ref = oracle_run("tiny")
    inputs = np.concatenate([[1], toks[:-1]])
    with pkg.Model(cfg, w) as f, pkg.Model(cfg, w, fuse=False) as u:
        for p in range(cfg.seq_len):
            a, c = host(f.forward(int(inputs[p]), p)), host(u.forward(int(inputs[p]), p))
            assert logits_close(c, ref[p])[0], p
            assert np.max(np.abs(a - c)) <= 1e-5 * np.max(np.abs(ref[p])), p
        stats = {s["name"]: s["launches"] for s in u.profile(1, 0, 2)}
    assert stats["qkv_attention"] == 0 and stats["attention"] == 2 * cfg.n_layers


@pytest.mark.parametrize("name", ["tiny", "gqa_small"])
def test_kv_cache_rows_match_oracle(name):
    cfg, b, w = blob_of(name)
    n = 20
    cache = oracle.KVCache(cfg)
    oracle.generate(cfg, b, cache, 1, 0, n)
    with pkg.Model(cfg, w) as m:
        m.generate(1, 0, n)
        k, v = (host(t) for t in m.read_kv_cache())
    for got, ref in ((k, cache.k), (v, cache.v)):
        assert np.all(got[:, n:] == 0)  # never written above the last position
        scale = np.max(np.abs(ref[:, :n]))
        assert np.max(np.abs(got[:, :n] - ref[:, :n])) <= 1e-4 * scale


@pytest.mark.parametrize("name", ["tiny", "gqa_small"])
def test_rows_above_pos_are_never_read(name):
    cfg, b, w = blob_of(name)
    p = 9
    toks, _ = oracle_run(name)
    inputs = np.concatenate([[1], toks[:-1]])
    with pkg.Model(cfg, w) as m:
        for i in range(p):
            m.forward(int(inputs[i]), i)
        clean = host(m.forward(int(inputs[p]), p))
        k, v = m.read_kv_cache()
        k[:, p + 1:] = float("nan")
        v[:, p + 1:] = 1e30
        m.write_kv_cache(k, v)
        poisoned = host(m.forward(int(inputs[p]), p))
    assert np.array_equal(clean, poisoned)


def test_reset_restarts_from_a_zero_cache():
    cfg, b, w = blob_of("stories15m")
    with pkg.Model(cfg, w) as m:
        first = m.generate(1, 0, 30)
        k, _ = m.read_kv_cache()
        assert float(k.abs().max()) > 0
        m.reset()
        k, v = m.read_kv_cache()
        assert float(k.abs().max()) == 0 and float(v.abs().max()) == 0
        assert np.array_equal(m.generate(1, 0, 30), first)


def test_generate_resumes_after_forward_calls():
    # forward over a prefix, then generate from the next position: same tokens
    # as one generation over the whole range (the state is the cache)
    cfg, b, w = blob_of("gqa_small")
    with pkg.Model(cfg, w) as m:
        whole = m.generate(1, 0, 50)
        m.reset()
        tok = 1
        for p in range(20):
            m.forward(tok, p)
            tok = m.argmax_last()
            assert tok == whole[p]
        rest = m.generate(tok, 20, 30)
    assert np.array_equal(rest, whole[20:])


def test_range_and_argument_errors():
    cfg, b, w = blob_of("tiny")
    with pkg.Model(cfg, w) as m:
        for tok, pos in ((-1, 0), (cfg.vocab_size, 0), (0, -1), (0, cfg.seq_len)):
            with pytest.raises(ld.LdError) as e:
                m.forward(tok, pos)
            assert e.value.status == ld.LD_E_RANGE
        with pytest.raises(ld.LdError) as e:
            m.generate(1, cfg.seq_len - 3, 4)
        assert e.value.status == ld.LD_E_RANGE
        assert m.generate(1, cfg.seq_len - 3, 3).size == 3
        assert m.generate(1, 0, 0).size == 0
    with pytest.raises(ld.LdError) as e:
        pkg.Model(cfg, w[1:].clone()[:-1])  # wrong size
    assert e.value.status == ld.LD_E_SIZE


def test_tied_classifier_reads_the_embedding_table():
    # the stories15M-shaped model ties the classifier; untying it with a copy of
    # the embedding appended must give the same logits bit for bit
    import torch
    cfg, b, w = blob_of("stories15m")
    off, n = synth.offsets(cfg)["tok_embedding"]
    untied = torch.cat([w, w[off:off + n]])
    with pkg.Model(cfg, w) as t, pkg.Model(cfg, untied, shared_classifier=0) as u:
        for p, tok in enumerate([1, 5, 900]):
            assert np.array_equal(host(t.forward(tok, p)), host(u.forward(tok, p)))


def test_profile_counts_every_launch():
    cfg, b, w = blob_of("gqa_small")
    L = cfg.n_layers
    for fuse in (False, True):  # dim 288: the fused launch is not used either way
        with pkg.Model(cfg, w, fuse=fuse) as m:
            stats = {s["name"]: s for s in m.profile(1, 0, 4)}
        want = {"qkv_rope_append": L, "attention": L, "wo_residual": L, "w1w3_swiglu": L, "w2_residual": L,
                "classifier_argmax": 1}
        for k, per_step in want.items():
            assert stats[k]["launches"] == 4 * per_step and stats[k]["total_ms"] > 0
        assert stats["qkv_attention"]["launches"] == 0


def test_profile_counts_fused_launches():
    # the tiny shape (dim 64) takes the fused q/k/v + attention launch at every
    # position of its context (64 keys of 2 x 16 floats per kv head: 8 KB)
    cfg, b, w = blob_of("tiny")
    L = cfg.n_layers
    with pkg.Model(cfg, w) as m:
        stats = {s["name"]: s for s in m.profile(1, 60, 4)}
    want = {"qkv_attention": 4 * L, "qkv_rope_append": 0, "attention": 0, "wo_residual": 4 * L,
            "w1w3_swiglu": 4 * L, "w2_residual": 4 * L, "classifier_argmax": 4}
    for k, n in want.items():
        assert stats[k]["launches"] == n, k
