"""Pins of the CPU oracle to what the pages and the mathematics fix.

Every check compares the oracle with something other than itself: a closed
form, an invariant, a value a page prints, a second formulation taken from
another page, a library routine (numpy in float64), or a brute-force
recompute.  Each is chosen so that a plausible mistake (a dropped term, a
wrong sign or index, a transposed operand, an off-by-one range) fails it.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
U32 = 2.0 ** -24  # unit roundoff of fp32


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("c", [0.5, 1.0, 3.0, -2.0, 1e-3])
@pytest.mark.parametrize("page", [False, True])
def test_rmsnorm_constant_vector_closed_form(c, page):
    # x = c*1, g = 1  =>  each output is c / sqrt(c^2 + eps)   (eps inside the root, mean over n)
    n, eps = 96, 1e-5
    out = oracle.rmsnorm(np.full(n, c, np.float32), np.ones(n, np.float32), eps, page=page)
    c32 = float(np.float32(c))
    want = c32 / math.sqrt(c32 * c32 + eps)
    assert np.allclose(out, want, rtol=4 * U32, atol=0)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    x = rng(1).standard_normal(777).astype(np.float32)
    one = np.ones_like(x)
    y = oracle.rmsnorm(x, one, 0.0)
    assert abs(float(np.mean(y.astype(np.float64) ** 2)) - 1.0) < 1e-6
    # power-of-two scalings are exact: rmsnorm(a x) = sign(a) rmsnorm(x), rmsnorm(x, 2g) = 2 rmsnorm(x, g)
    assert np.array_equal(oracle.rmsnorm(4.0 * x, one, 0.0), y)
    assert np.array_equal(oracle.rmsnorm(-0.25 * x, one, 0.0), -y)
    g = rng(2).standard_normal(777).astype(np.float32)
    assert np.array_equal(oracle.rmsnorm(x, 2 * g, 0.0), 2 * oracle.rmsnorm(x, g, 0.0))


def test_rmsnorm_gain_is_elementwise():
    # a gain that is one-hot keeps only that coordinate: catches a gain applied at the wrong index
    x = rng(3).standard_normal(64).astype(np.float32)
    g = np.zeros(64, np.float32)
    g[17] = 1.0
    y = oracle.rmsnorm(x, g, 1e-5)
    assert np.count_nonzero(y) == 1 and y[17] != 0


# ----------------------------------------------------------------------------- matrix-vector product

def test_matvec_identity_and_one_hot_column():
    x = rng(4).standard_normal(50).astype(np.float32)
    assert np.array_equal(oracle.matvec(np.eye(50, dtype=np.float32), x), x)
    # non-square W (d=7 rows, n=13 columns): e_k selects column k, not row k
    w = rng(5).standard_normal((7, 13)).astype(np.float32)
    for k in (0, 6, 12):
        e = np.zeros(13, np.float32)
        e[k] = 1.0
        assert np.array_equal(oracle.matvec(w, e), w[:, k])


@pytest.mark.parametrize("d,n", [(1, 1), (3, 5), (64, 288), (31, 1000)])
def test_matvec_matches_float64_library_product(d, n):
    r = rng(d * 7919 + n)
    w = r.standard_normal((d, n)).astype(np.float32)
    x = r.standard_normal(n).astype(np.float32)
    ref = w.astype(np.float64) @ x.astype(np.float64)
    out = oracle.matvec(w, x).astype(np.float64)
    bound = U32 * np.abs(ref) + 1e-13 * (np.abs(w).astype(np.float64) @ np.abs(x).astype(np.float64))
    assert np.all(np.abs(out - ref) <= bound)


# ----------------------------------------------------------------------------- RoPE

@pytest.mark.parametrize("page", [False, True])
def test_rope_position_zero_is_identity(page):
    v = rng(6).standard_normal(6 * 48).astype(np.float32)
    assert np.array_equal(oracle.rope(v, 6, 48, 0, page=page), v)


def test_rope_preserves_pair_norms():
    v = rng(7).standard_normal(4 * 128).astype(np.float32)
    for pos in (1, 17, 511, 4095):
        r = oracle.rope(v, 4, 128, pos)
        n0 = np.hypot(v[0::2].astype(np.float64), v[1::2])
        n1 = np.hypot(r[0::2].astype(np.float64), r[1::2])
        assert np.allclose(n1, n0, rtol=4 * U32, atol=1e-30)


def test_rope_head_size_two_is_plain_rotation_by_pos_radians():
    # hs = 2: the only pair has frequency theta^0 = 1, so the angle is pos radians
    a, b = np.float32(0.75), np.float32(-1.25)
    for pos in (1, 2, 3, 100):
        r = oracle.rope(np.array([a, b], np.float32), 1, 2, pos)
        want = np.array([a * math.cos(pos) - b * math.sin(pos), a * math.sin(pos) + b * math.cos(pos)])
        assert np.allclose(r, want, rtol=2 * U32, atol=2 * U32)


def test_rope_second_pair_frequency_and_adjacent_pairing():
    # hs = 4: pair j = 1 (offsets 2,3) turns by pos * 10000^(-2/4) = pos / 100
    pos = 37
    v = np.array([0.0, 0.0, 1.0, 0.0], np.float32)
    r = oracle.rope(v, 1, 4, pos)
    assert r[0] == 0 and r[1] == 0  # pairs are adjacent: nothing leaks into offsets 0,1 (a half-split would)
    assert np.allclose(r[2:], [math.cos(pos / 100), math.sin(pos / 100)], rtol=2 * U32, atol=2 * U32)


def test_rope_relative_position_property():
    r = rng(8)
    q = r.standard_normal(64).astype(np.float32)
    k = r.standard_normal(64).astype(np.float32)
    for p, s, d in [(5, 2, 9), (100, 30, 250), (1000, 999, 3000)]:
        a = np.dot(oracle.rope(q, 1, 64, p).astype(np.float64), oracle.rope(k, 1, 64, s))
        b = np.dot(oracle.rope(q, 1, 64, p + d).astype(np.float64), oracle.rope(k, 1, 64, s + d))
        assert abs(a - b) <= 1e-5 * (np.linalg.norm(q) * np.linalg.norm(k))


def test_rope_matches_the_r_keras_formulation():
    # Second formulation (LLaMA.R precompute_rotarty_freqs / apply_rotary_embedding):
    # freqs_j = theta^-(j / (hs/2)), cos/sin repeated twice along the head axis,
    # out = x * cos + rotate_every_two(x) * sin, rotate_every_two(x) = interleave(-x[1::2], x[0::2]).
    hs, heads, theta = 48, 3, 10000.0
    x = rng(9).standard_normal(heads * hs).astype(np.float32)
    for pos in (0, 1, 63, 255, 2047):
        j = np.arange(hs // 2, dtype=np.float64) / (hs // 2)
        ang = pos * (1.0 / theta ** j)
        cos = np.repeat(np.cos(ang), 2)
        sin = np.repeat(np.sin(ang), 2)
        xs = x.reshape(heads, hs).astype(np.float64)
        rot = np.stack([-xs[:, 1::2], xs[:, 0::2]], axis=-1).reshape(heads, hs)
        want = (xs * cos + rot * sin).reshape(-1)
        got = oracle.rope(x, heads, hs, pos)
        assert np.allclose(got, want, rtol=0, atol=4 * U32 * np.abs(x).max())


def test_rope_rotates_only_the_requested_heads():
    v = rng(10).standard_normal(6 * 8).astype(np.float32)
    r = oracle.rope(v, 4, 8, 5)  # 4 of 6 heads, as for k with 4 kv heads
    assert np.array_equal(r[32:], v[32:]) and not np.array_equal(r[:32], v[:32])


# ----------------------------------------------------------------------------- GQA head map

def test_kv_head_map():
    g = GOLD["gqa_head_map_6_4"]
    assert [oracle.kv_head(h, g["n_heads"], g["n_kv_heads"]) for h in range(g["n_heads"])] == g["kv_head"]
    assert [oracle.kv_head(h, 32, 32) for h in range(32)] == list(range(32))  # MHA: identity
    assert [oracle.kv_head(h, 64, 8) for h in range(64)] == [h // 8 for h in range(64)]  # integer groups


# ----------------------------------------------------------------------------- attention

def _cache(r, pos, kv_dim, scale=1.0):
    kc = (scale * r.standard_normal((pos + 1, kv_dim))).astype(np.float32)
    vc = r.standard_normal((pos + 1, kv_dim)).astype(np.float32)
    return kc, vc


@pytest.mark.parametrize("H,KV,hs", [(4, 4, 16), (6, 4, 48), (8, 2, 8)])
def test_attention_single_position_returns_v_exactly(H, KV, hs):
    # pos = 0: one score, softmax weight exactly 1, output = the value row of the mapped kv head
    r = rng(H * 100 + KV)
    q = r.standard_normal(H * hs).astype(np.float32)
    kc, vc = _cache(r, 0, KV * hs)
    out = oracle.attention(q, kc, vc, H, KV, hs, 0)
    for h in range(H):
        g = oracle.kv_head(h, H, KV)
        assert np.array_equal(out[h * hs:(h + 1) * hs], vc[0, g * hs:(g + 1) * hs])


def test_attention_zero_query_is_mean_of_value_rows_0_to_pos():
    # q = 0: all scores equal, weights 1/(pos+1): catches an off-by-one in the causal range
    H, KV, hs, pos = 4, 2, 16, 9
    r = rng(11)
    kc, vc = _cache(r, pos + 5, KV * hs)
    out = oracle.attention(np.zeros(H * hs, np.float32), kc, vc, H, KV, hs, pos)
    for h in range(H):
        g = oracle.kv_head(h, H, KV)
        want = vc[:pos + 1, g * hs:(g + 1) * hs].astype(np.float64).mean(axis=0)
        assert np.allclose(out[h * hs:(h + 1) * hs], want, rtol=2 * U32, atol=2 * U32)


def test_attention_two_keys_closed_form_scale():
    # Two keys with q.k0 = a and q.k1 = 0: weight of key 0 is sigmoid(a / sqrt(hs)).
    hs = 16
    q = np.zeros(hs, np.float32)
    q[0] = 3.0
    kc = np.zeros((2, hs), np.float32)
    kc[0, 0] = 1.5  # q.k0 = 4.5
    vc = np.zeros((2, hs), np.float32)
    vc[0, :] = 1.0
    vc[1, :] = -2.0
    w0 = 1.0 / (1.0 + math.exp(-4.5 / math.sqrt(hs)))
    out = oracle.attention(q, kc, vc, 1, 1, hs, 1)
    assert np.allclose(out, w0 * 1.0 + (1 - w0) * -2.0, rtol=2 * U32, atol=2 * U32)


def test_attention_shift_invariance_and_convexity():
    H, KV, hs, pos = 2, 1, 32, 20
    r = rng(12)
    q = r.standard_normal(H * hs).astype(np.float32)
    kc, vc = _cache(r, pos, KV * hs)
    base = oracle.attention(q, kc, vc, H, KV, hs, pos)
    # shift the score of head 0 by adding a vector orthogonal to q_1 ... simpler: one head, one common key offset
    q1 = q[:hs].copy()
    u = np.zeros(hs, np.float32)
    u[3] = 0.5  # every key gets the same extra q.u
    out1 = oracle.attention(q1, kc + u, vc, 1, 1, hs, pos)
    out0 = oracle.attention(q1, kc, vc, 1, 1, hs, pos)
    assert np.allclose(out1, out0, rtol=1e-6, atol=1e-6)
    # output lies in the convex hull of the value rows (weights >= 0, sum 1)
    lo, hi = vc.min(axis=0), vc.max(axis=0)
    assert np.all(base[:hs] >= lo - 1e-6) and np.all(base[:hs] <= hi + 1e-6)
    # constant value rows: output is that constant
    vconst = np.tile(np.arange(hs, dtype=np.float32) * 0.25, (pos + 1, 1))
    assert np.allclose(oracle.attention(q1, kc, vconst, 1, 1, hs, pos), vconst[0], rtol=4 * U32, atol=0)


def test_attention_large_scores_stay_finite():
    # scores near 700 overflow exp() unless the maximum is subtracted first; the
    # dominant key then takes all the weight
    hs, pos = 16, 3
    q = np.full(hs, 10.0, np.float32)
    kc = np.zeros((pos + 1, hs), np.float32)
    kc[2, :] = 17.5  # q.k / 4 = 700
    kc[1, :] = 15.0  # 600: weight e^-100 relative to key 2
    vc = np.arange((pos + 1) * hs, dtype=np.float32).reshape(pos + 1, hs)
    out = oracle.attention(q, kc, vc, 1, 1, hs, pos)
    assert np.all(np.isfinite(out)) and np.array_equal(out, vc[2])


def test_attention_ignores_rows_after_pos():
    H, KV, hs, pos = 4, 2, 16, 6
    r = rng(13)
    q = r.standard_normal(H * hs).astype(np.float32)
    kc, vc = _cache(r, 12, KV * hs)
    a = oracle.attention(q, kc, vc, H, KV, hs, pos)
    kc[pos + 1:] = np.nan
    vc[pos + 1:] = 1e30
    assert np.array_equal(oracle.attention(q, kc, vc, H, KV, hs, pos), a)


# ----------------------------------------------------------------------------- SwiGLU, argmax

def test_swiglu_closed_forms():
    h1 = np.array([0.0, 1.0, 2.0, -1000.0, 50.0, 1.0], np.float32)
    h3 = np.array([5.0, 1.0, 1.0, 3.0, 1.0, 2.0], np.float32)
    out = oracle.swiglu(h1, h3)
    assert out[0] == 0.0
    assert out[1] == np.float32(1.0 / (1.0 + math.exp(-1.0)))          # silu(1) = 0.7310585786...
    assert out[2] == np.float32(2.0 / (1.0 + math.exp(-2.0)))          # silu(2) = 1.7615941559...
    assert out[3] == 0.0 and math.copysign(1.0, out[3]) == -1.0        # silu(-1000) = -0, no NaN
    assert out[4] == 50.0                                               # silu(u) -> u for large u
    # the gate goes on the w1 branch: silu(1) * 2, not silu(2) * 1
    assert out[5] == np.float32(2.0 / (1.0 + math.exp(-1.0)))
    assert not np.any(np.isnan(oracle.swiglu(np.float32([-1e4, -88.0, -100.0]), np.ones(3, np.float32))))


def test_argmax_first_maximum():
    g = GOLD["argmax_first_maximum"]
    assert oracle.argmax(np.array(g["values"], np.float32)) == g["index"]
    assert oracle.argmax(np.zeros(10, np.float32)) == 0
    v = np.arange(100, dtype=np.float32)
    assert oracle.argmax(v) == 99


# ----------------------------------------------------------------------------- configuration arithmetic

def test_page_printed_configuration_numbers():
    g = GOLD["kv_dim_example"]
    assert g["dim"] * g["n_kv_heads"] // g["n_heads"] == g["kv_dim"]
    c = synth.CONFIGS["gqa_small"]
    assert (c.dim, c.n_heads, c.n_kv_heads, c.kv_dim) == (g["dim"], g["n_heads"], g["n_kv_heads"], g["kv_dim"])
    f = GOLD["ffn_hidden_rule"]
    hidden = int(4 * f["dim"] * 2 / 3)
    hidden = (hidden + f["multiple_of"] - 1) // f["multiple_of"] * f["multiple_of"]
    assert hidden == f["hidden"] == synth.CONFIGS["llama7b"].hidden_dim
    s = GOLD["stories15m_parameters"]
    assert oracle.blob_floats(synth.CONFIGS["stories15m"]) == s["floats"]
    for c in synth.CONFIGS.values():
        assert oracle.blob_floats(c) == synth.blob_floats(c)


# ----------------------------------------------------------------------------- the whole step

def _tiny(**kw):
    base = dict(name="t", dim=48, hidden_dim=80, n_layers=2, n_heads=6, n_kv_heads=4, vocab_size=97,
                seq_len=24, shared_classifier=0, seed=77)
    base.update(kw)
    return synth.Config(**base)


def test_forward_residual_path_closed_form():
    # Wo = W2 = 0 in every layer: both branches add zero, x stays E[token], so
    # logits = Wcls (g_final * rmsnorm(E[token]))  -- catches a residual that overwrites instead of adding.
    c = _tiny()
    blob = synth.make_blob(c)
    off = synth.offsets(c)
    for name in ("wo", "w2"):
        o, n = off[name]
        blob[o:o + n] = 0
    E = blob[slice(*_span(off, "tok_embedding"))].reshape(c.vocab_size, c.dim).astype(np.float64)
    gf = blob[slice(*_span(off, "rms_final"))].astype(np.float64)
    W = blob[slice(*_span(off, "wcls"))].reshape(c.vocab_size, c.dim).astype(np.float64)
    kv = oracle.KVCache(c)
    for pos, tok in enumerate([3, 50, 96, 0]):
        e = E[tok]
        y = (gf * (e / math.sqrt(np.mean(e * e) + 1e-5))).astype(np.float32).astype(np.float64)
        want = W @ y
        got = oracle.forward(c, blob, kv, tok, pos)
        assert np.allclose(got, want, rtol=0, atol=4 * U32 * np.abs(want).max())


def _span(off, name):
    o, n = off[name]
    return o, o + n


@pytest.mark.parametrize("page", [False, True])
def test_forward_ignores_cache_rows_after_pos(page):
    c = _tiny()
    blob = synth.make_blob(c)
    kv = oracle.KVCache(c)
    toks = [1, 5, 9, 13, 2]
    for p, t in enumerate(toks):
        oracle.forward(c, blob, kv, t, p, page=page)
    clean = oracle.KVCache(c)
    clean.k[:] = kv.k
    clean.v[:] = kv.v
    a = oracle.forward(c, blob, clean, 7, 5, page=page)
    kv.k[:, 6:] = np.nan
    kv.v[:, 6:] = 1e30
    b = oracle.forward(c, blob, kv, 7, 5, page=page)
    assert np.array_equal(a, b)


def test_forward_gqa_equals_mha_with_replicated_kv_heads():
    # A GQA model equals the MHA model whose Wk/Wv head blocks are copied along the
    # head map (kv head floor(h*KV/H) serves query head h); pins the non-integer
    # group of 6 query heads on 4 kv heads.
    c = _tiny()
    blob = synth.make_blob(c)
    hs = c.head_size
    m = c.replace(n_kv_heads=c.n_heads)
    off, offm = synth.offsets(c), synth.offsets(m)
    mblob = np.empty(synth.blob_floats(m), np.float32)
    for name, (o, n) in off.items():
        om, nm = offm[name]
        if name in ("wk", "wv"):
            src = blob[o:o + n].reshape(c.n_layers, c.n_kv_heads, hs, c.dim)
            idx = [oracle.kv_head(h, c.n_heads, c.n_kv_heads) for h in range(c.n_heads)]
            mblob[om:om + nm] = src[:, idx].reshape(-1)
        else:
            mblob[om:om + nm] = blob[o:o + n]
    kg, km = oracle.KVCache(c), oracle.KVCache(m)
    for p, t in enumerate([1, 40, 7, 7, 90, 3, 12]):
        assert np.array_equal(oracle.forward(c, blob, kg, t, p), oracle.forward(m, mblob, km, t, p))


@pytest.mark.parametrize("name,positions", [("tiny", 64), ("stories15m", 16), ("gqa_small", 16)])
def test_forward_incremental_cache_equals_full_recompute(name, positions):
    c = synth.CONFIGS[name]
    blob = synth.make_blob(c)
    kv = oracle.KVCache(c)
    toks = [1] + list(synth.prefill_tokens(c, positions - 1))
    for p in range(positions):
        inc = oracle.forward(c, blob, kv, toks[p], p)
        if p in (0, 1, positions // 2, positions - 1) or name == "tiny":
            full = oracle.bruteforce(c, blob, toks[:p + 1], p)
            assert np.max(np.abs(inc - full)) <= 1e-6 * np.max(np.abs(full))


def test_forward_page_literal_build_agrees():
    for name, n in (("tiny", 64), ("stories15m", 12), ("gqa_small", 12)):
        c = synth.CONFIGS[name]
        blob = synth.make_blob(c)
        t0, l0 = oracle.generate(c, blob, oracle.KVCache(c), 1, 0, n, keep_logits=True)
        t1, l1 = oracle.generate(c, blob, oracle.KVCache(c), 1, 0, n, keep_logits=True, page=True)
        assert oracle.page_literal(True) and not oracle.page_literal(False)
        for i in range(n):
            assert np.max(np.abs(l0[i] - l1[i])) <= 1e-4 * np.max(np.abs(l0[i]))


def test_forward_rejects_out_of_range_arguments():
    c = _tiny()
    blob = synth.make_blob(c)
    kv = oracle.KVCache(c)
    for tok, pos in ((-1, 0), (c.vocab_size, 0), (0, -1), (0, c.seq_len)):
        with pytest.raises(ValueError):
            oracle.forward(c, blob, kv, tok, pos)


# ----------------------------------------------------------------------------- thread count

def test_thread_count_does_not_change_a_bit():
    # rows and heads shared out among threads: every output is the same sequential sum,
    # so a generation must be bit-identical for any thread count (the stored full-size
    # runs were made with several threads)
    cfg = synth.CONFIGS["gqa_small"].replace(seq_len=48)
    blob = synth.make_blob(cfg)
    runs = []
    try:
        for t in (1, 2, 5, 7):
            oracle.set_threads(t)
            runs.append(oracle.generate(cfg, blob, oracle.KVCache(cfg), 1, 0, 48, keep_logits=True))
    finally:
        oracle.set_threads(1)
    for toks, logits in runs[1:]:
        assert np.array_equal(toks, runs[0][0]) and np.array_equal(logits, runs[0][1])
