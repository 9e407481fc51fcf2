"""The stored full-size oracle runs (tests/golden/greedy_<workload>.npz) are
whole and were made by the current oracle.

They are written by oracle/make_goldens.py (hours of CPU time, so the GPU test
compares with them instead of rerunning the oracle).  Here, without a GPU and
without the 27 GB weights:
  * the recorded sha256 of the oracle and generator sources equals the sources
    in the tree (a change to the oracle's arithmetic means a new run);
  * the input tokens are the workload's: token 1 then the oracle's own greedy
    choices, after the seeded prompt where the workload has one;
  * each step's argmax is the first of its stored top 8, which run in
    descending order with equal values by index;
  * the sixteen full logit vectors agree with the per-step records of their
    positions (argmax, top 8, max |logit|);
  * the tie events are exactly the steps whose top-2 gap is within 1e-4 of max |logit|.
"""
import os

import numpy as np
import pytest

import synth
from oracle import make_goldens

NAMES = sorted(make_goldens.WORKLOADS)


@pytest.fixture(scope="module", params=NAMES)
def gold(request):
    name = request.param
    if not os.path.exists(make_goldens.golden_path(name)):
        pytest.skip(f"no stored oracle run for {name} yet")
    return name, make_goldens.load(name)


def test_made_by_the_current_oracle_sources(gold):
    name, g = gold
    assert g["meta"]["sources_sha256"] == make_goldens.source_digest()
    cfg = synth.CONFIGS[name]
    c = g["meta"]["config"]
    assert (c["dim"], c["hidden_dim"], c["n_layers"], c["n_heads"], c["n_kv_heads"], c["vocab_size"],
            c["seq_len"], c["seed"]) == cfg.fields() + (cfg.seed,)


def test_inputs_are_the_workload_and_the_oracle_chain(gold):
    name, g = gold
    forced, n = make_goldens.WORKLOADS[name][0], make_goldens.WORKLOADS[name][1]
    assert g["tok_in"].shape == (n,) and g["next"].shape == (n,)
    cfg = synth.CONFIGS[name]
    if forced:
        assert np.array_equal(g["tok_in"][:forced], synth.prefill_tokens(cfg, forced))
    else:
        assert g["tok_in"][0] == 1
    start = max(forced, 1)
    assert np.array_equal(g["tok_in"][start:], g["next"][start - 1:-1])
    assert np.all((g["next"] >= 0) & (g["next"] < cfg.vocab_size))


def test_top_lists_are_ordered(gold):
    _, g = gold
    idx, val = g["top_idx"], g["top_val"].astype(np.float64)
    assert np.array_equal(idx[:, 0], g["next"])
    assert np.all(np.diff(val, axis=1) <= 0)
    same = np.diff(val, axis=1) == 0
    assert np.all(np.diff(idx, axis=1)[same] > 0)
    assert np.all(g["maxabs"] >= np.abs(val).max(axis=1))


def test_full_logits_agree_with_the_step_records(gold):
    _, g = gold
    pos = g["logit_pos"]
    assert pos.size == 16 and np.all(np.diff(pos) > 0) and pos[-1] < g["next"].size
    for i, p in enumerate(pos):
        lg = g["logits"][i]
        assert np.all(np.isfinite(lg))
        assert int(np.argmax(lg)) == g["next"][p]
        ti, tv = make_goldens.top_k(lg)
        assert np.array_equal(ti, g["top_idx"][p]) and np.array_equal(tv, g["top_val"][p])
        assert np.float32(np.max(np.abs(lg))) == g["maxabs"][p]


def test_tie_events_follow_the_rule(gold):
    _, g = gold
    gap = g["top_val"][:, 0].astype(np.float64) - g["top_val"][:, 1]
    ties = np.flatnonzero(gap <= make_goldens.REL_TOL * g["maxabs"].astype(np.float64))
    assert g["meta"]["tie_steps"] == [int(t) for t in ties]
    assert g["meta"]["first_tie_step"] == (int(ties[0]) if ties.size else None)
