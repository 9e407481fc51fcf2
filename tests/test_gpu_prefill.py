"""Prompt prefill on the matrix cores against the oracle, through the C ABI.

* ld_op_gemm: bit-exact on small-integer operands (every product and partial
  sum is an integer below 2^24, so fp32 arithmetic is exact in any order and a
  wrong index or a dropped term shows as a mismatch), and within the fp32
  summation bound (K + 4) u sum |a w| on random operands, at the projection
  shapes of every workload.
* ld_op_attention_prefill: every query against oracle_attention at its own
  position, within max|V| (2 max_t ds_t + (n + 8) u), where ds_t bounds the
  fp32 error of score t (hs u sum |q k| / sqrt(hs) plus its rounding) and n is
  the number of keys.
* ld_prefill: the logits of the last prompt token within the decode step's
  bar (1e-4 max |logit|) of the oracle's, after the oracle ran the prompt one
  token at a time; every cache row written within 1e-4 of the oracle's rows;
  the greedy continuation equal to the oracle's up to the first tie.
"""
import numpy as np
import pytest

import llama_transformer_decode_amd as pkg
import oracle
import synth
from gpu_util import acceptable_token, dev, host, logits_close, tie_tolerance, top2_gap, torch_or_skip
from llama_transformer_decode_amd import ld

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch_or_skip()


def gemm(a, w):
    torch = torch_or_skip()
    m, k = a.shape
    n = w.shape[0]
    ta, tw = dev(a), dev(w)
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ld.ld_op_gemm(ta.data_ptr(), tw.data_ptr(), m, n, k, out.data_ptr())
    return host(out)


@pytest.mark.parametrize("m,n,k", [(1, 1, 4), (3, 5, 8), (128, 128, 16), (129, 130, 20), (200, 300, 100),
                                   (17, 1000, 36), (64, 1536, 288), (256, 1024, 4096), (5, 64, 176),
                                   # each row tile (16, 32, 64) with K split, ragged slabs and tails
                                   (16, 1000, 1028), (32, 520, 2052), (33, 300, 1000), (63, 260, 772),
                                   # 128-row tiles: ragged rows, columns and K (split), one-slab K
                                   (300, 1000, 1028), (2048, 256, 64), (129, 128, 4), (1000, 130, 292)])
def test_gemm_exact_on_small_integers(m, n, k):
    rng = np.random.default_rng(m * 1000 + n + k)
    a = rng.integers(-4, 5, (m, k)).astype(np.float32)
    w = rng.integers(-4, 5, (n, k)).astype(np.float32)
    want = (a.astype(np.int64) @ w.astype(np.int64).T).astype(np.float64)
    got = gemm(a, w)
    assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("m,n,k", [(64, 4096, 4096), (64, 11008, 4096), (33, 4096, 11008), (16, 8192, 8192),
                                   (16, 1024, 8192), (8, 8192, 28672), (100, 288, 288), (100, 768, 288),
                                   (100, 288, 768), (64, 176, 64), (64, 64, 176),
                                   (512, 4096, 4096), (2048, 1024, 4096), (200, 4096, 11008)])
def test_gemm_within_the_fp32_summation_bound(m, n, k):
    rng = np.random.default_rng(m + n + k)
    a = rng.standard_normal((m, k)).astype(np.float32)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    a64, w64 = a.astype(np.float64), w.astype(np.float64)
    want = a64 @ w64.T
    bound = (k + 4) * U * (np.abs(a64) @ np.abs(w64).T)
    got = gemm(a, w).astype(np.float64)
    err = np.abs(got - want)
    print(f"gemm {m}x{n}x{k}: max |err| / bound = {float(np.max(err / bound)):.3g}")
    assert np.all(err <= bound)


ATTN_CASES = [(4, 4, 16), (6, 4, 48), (6, 6, 48), (8, 2, 32), (4, 2, 64), (4, 4, 80), (3, 1, 96), (32, 32, 128),
              (64, 8, 128), (2, 1, 256)]


@pytest.mark.parametrize("H,KV,hs", ATTN_CASES)
@pytest.mark.parametrize("pos,T", [(0, 1), (0, 64), (7, 65), (100, 130), (31, 33)])
def test_attention_prefill_every_query(H, KV, hs, pos, T):
    torch = torch_or_skip()
    if H * hs > 4096 and T > 64:
        T = 64
    rng = np.random.default_rng(H * 100 + KV * 10 + hs + pos + T)
    kv = KV * hs
    n = pos + T
    q = rng.standard_normal((T, H * hs)).astype(np.float32)
    kc = rng.standard_normal((n, kv)).astype(np.float32)
    vc = rng.standard_normal((n, kv)).astype(np.float32)
    tq, tk, tv = dev(q), dev(kc), dev(vc)
    out = torch.empty((T, H * hs), dtype=torch.float32, device="cuda")
    ld.ld_op_attention_prefill(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), H, KV, hs, pos, T, out.data_ptr())
    got = host(out)
    vmax = float(np.max(np.abs(vc)))
    worst = 0.0
    for t in range(T):
        ref = oracle.attention(q[t], kc, vc, H, KV, hs, pos + t)
        for h in range(H):
            g = oracle.kv_head(h, H, KV)
            qa = np.abs(q[t, h * hs:(h + 1) * hs].astype(np.float64))
            ka = np.abs(kc[:pos + t + 1, g * hs:(g + 1) * hs].astype(np.float64))
            s = ka @ qa / np.sqrt(hs)
            ds = float(np.max((hs + 2) * U * s))
            bound = vmax * (2 * ds + (pos + t + 1 + 8) * U)
            e = float(np.max(np.abs(got[t, h * hs:(h + 1) * hs] - ref[h * hs:(h + 1) * hs])))
            worst = max(worst, e / bound)
            assert e <= bound, (t, h, e, bound)
    print(f"attention prefill H={H} KV={KV} hs={hs} pos={pos} T={T}: max err / bound = {worst:.3g}")


# ----------------------------------------------------------------------------- the whole prefill

SMALL = {"tiny": 64, "stories15m": 100, "gqa_small": 200}
_blobs = {}


def blob_of(name):
    if name not in _blobs:
        cfg = synth.CONFIGS[name]
        b = synth.make_blob(cfg)
        _blobs[name] = (cfg, b, dev(b))
    return _blobs[name]


def prompt_of(cfg, n):
    p = synth.prefill_tokens(cfg, n).copy()
    p[0] = 1
    return p


def oracle_prompt(cfg, blob, prompt, pos=0, cache=None):
    cache = cache if cache is not None else oracle.KVCache(cfg)
    logits = None
    for i, t in enumerate(prompt):
        logits = oracle.forward(cfg, blob, cache, int(t), pos + i)
    return logits, cache


@pytest.mark.parametrize("name", list(SMALL))
def test_prefill_logits_cache_and_continuation(name):
    cfg, b, w = blob_of(name)
    T = SMALL[name]
    prompt = prompt_of(cfg, T)
    ref, cache = oracle_prompt(cfg, b, prompt)
    with pkg.Model(cfg, w) as m:
        got = host(m.prefill(prompt, 0))
        ok, err, tol = logits_close(got, ref)
        print(f"[{name}] prefill of {T} tokens: max |d logit| {err:.3g} (tolerance {tol:.3g})")
        assert ok
        k, v = (host(t) for t in m.read_kv_cache())
        for g, r in ((k, cache.k), (v, cache.v)):
            scale = np.max(np.abs(r[:, :T]))
            assert np.max(np.abs(g[:, :T] - r[:, :T])) <= 1e-4 * scale
            assert np.all(g[:, T:] == 0)
        nxt = m.argmax_last()
        assert acceptable_token(nxt, ref)
        if T < cfg.seq_len and nxt == oracle.argmax(ref):
            # greedy continuation from the prefilled cache: the oracle's tokens up to the first tie
            n = min(16, cfg.seq_len - T)
            gen = m.generate(nxt, T, n)
            want, wl = oracle.generate(cfg, b, cache, nxt, T, n, keep_logits=True)
            for i in range(n):
                if gen[i] != want[i]:
                    assert acceptable_token(int(gen[i]), wl[i])
                    break


@pytest.mark.parametrize("name", list(SMALL))
def test_prefill_in_pieces_and_after_decode_steps(name):
    # decode 3 tokens, prefill 20 at position 3, prefill 1 more, then compare with the oracle
    cfg, b, w = blob_of(name)
    prompt = prompt_of(cfg, 24)
    ref, cache = oracle_prompt(cfg, b, prompt)
    with pkg.Model(cfg, w) as m:
        for p in range(3):
            m.forward(int(prompt[p]), p)
        m.prefill(prompt[3:23], 3)
        got = host(m.prefill(prompt[23:], 23))
        ok, err, tol = logits_close(got, ref)
        assert ok, (err, tol)
        k, _ = (host(t) for t in m.read_kv_cache())
        assert np.max(np.abs(k[:, :24] - cache.k[:, :24])) <= 1e-4 * np.max(np.abs(cache.k[:, :24]))


def test_prefill_graph_and_direct_models_agree_and_repeat_bit_identically():
    cfg, b, w = blob_of("stories15m")
    prompt = prompt_of(cfg, 77)
    with pkg.Model(cfg, w, graph=True) as g, pkg.Model(cfg, w, graph=False) as e:
        a = host(g.prefill(prompt, 0))
        g.reset()
        a2 = host(g.prefill(prompt, 0))
        c = host(e.prefill(prompt, 0))
    assert np.array_equal(a, a2) and np.array_equal(a, c)


def test_prefill_range_errors():
    cfg, b, w = blob_of("tiny")
    with pkg.Model(cfg, w) as m:
        for toks, pos in (([], 0), ([1, 2], cfg.seq_len - 1), ([cfg.vocab_size], 0), ([1], -1), ([-1], 0)):
            with pytest.raises(ld.LdError) as e:
                m.prefill_async(toks, pos)
            assert e.value.status in (ld.LD_E_RANGE, ld.LD_E_NULL)
        got = host(m.prefill([1, 2, 3], 0))  # still usable
        assert np.all(np.isfinite(got))
