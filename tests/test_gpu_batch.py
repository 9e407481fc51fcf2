"""Batch decode (several sequences per step, each with its own KV cache)
against the oracle, through the C ABI.

Every sequence of a batch is an independent decode: its row of the batch's
logits must be within the decode step's bar (1e-4 max |logit|) of
oracle_forward on that sequence's own cache, at its own position.  The
sequences start from seeded cache prefixes of different lengths (installed in
the GPU caches and in the oracle's), so one batched step mixes positions; the
appended cache rows must match the oracle's, and no other sequence's rows may
change.  Greedy generation in lockstep must reproduce each sequence's oracle
tokens up to its first tie.  Batches of up to 4 sequences take the batch
GEMV kernels, 5 to 64 the tiled matrix-core products (in planes of 16
sequences: one to four; products with no more row tiles than compute units and
no RMSNorm split K over blocks and merge in the last one), more the split-K
matrix-core products.
"""
import numpy as np
import pytest

import llama_transformer_decode_amd as pkg
import oracle
import synth
from gpu_util import acceptable_token, dev, host, logits_close, torch_or_skip
from llama_transformer_decode_amd import ld

pytestmark = pytest.mark.gpu

_blobs = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch_or_skip()


def blob_of(name):
    if name not in _blobs:
        cfg = synth.CONFIGS[name]
        b = synth.make_blob(cfg)
        _blobs[name] = (cfg, b, dev(b))
    return _blobs[name]


def prefixes(cfg, lengths, stream0):
    """A seeded cache prefix per sequence (rows 0..len-1 of every layer, N(0,1))."""
    kv = cfg.dim * cfg.n_kv_heads // cfg.n_heads
    caches = []
    for b, p in enumerate(lengths):
        c = oracle.KVCache(cfg)
        for l in range(cfg.n_layers):
            if p:
                c.k[l, :p] = synth.normal(p * kv, cfg.seed, stream0 + 40 * b + 2 * l, 0.0, 1.0).reshape(p, kv)
                c.v[l, :p] = synth.normal(p * kv, cfg.seed, stream0 + 40 * b + 2 * l + 1, 0.0, 1.0).reshape(p, kv)
        caches.append(c)
    return caches


def install(m, cfg, caches):
    import torch
    B = m.max_batch
    shape = (B, cfg.n_layers, cfg.seq_len, cfg.dim * cfg.n_kv_heads // cfg.n_heads)
    k = np.zeros(shape, np.float32)
    v = np.zeros(shape, np.float32)
    for b, c in enumerate(caches):
        k[b], v[b] = c.k, c.v
    m.write_kv_cache(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())


@pytest.mark.parametrize("graph", [True, False])
@pytest.mark.parametrize("name,lengths", [("tiny", [0, 5, 17, 40]), ("tiny", [60, 0, 59]),
                                          # one and two sequences: the batch GEMV's 1- and 2-vector instances
                                          ("stories15m", [37]), ("gqa_small", [5, 300]),
                                          ("stories15m", [3, 0, 100, 31, 64]), ("gqa_small", [200, 7, 0, 508]),
                                          # 5..16 sequences: the tiled matrix-core products
                                          ("tiny", [0, 1, 2, 3, 4, 5, 6, 7, 20, 30, 40, 59]),
                                          ("gqa_small", [0, 9, 18, 27, 36, 45, 54, 63, 100, 200, 300, 400, 450, 480,
                                                         500, 507]),
                                          # 17-32 sequences: two planes of 16 (gqa_small: wo and w2
                                          # with K split over blocks, 18 row tiles in groups of 4)
                                          ("tiny", [3 * i for i in range(20)]),
                                          ("gqa_small", [(41 * i) % 500 for i in range(24)]),
                                          # 33-48: three planes; 49-64: four
                                          ("stories15m", [(37 * i) % 250 for i in range(40)]),
                                          ("tiny", [(11 * i) % 60 for i in range(48)]),
                                          ("gqa_small", [(97 * i) % 500 for i in range(49)]),
                                          ("tiny", [(5 * i) % 60 for i in range(64)]),
                                          # more than 64: the split-K matrix-core products
                                          ("tiny", [(7 * i) % 60 for i in range(65)])])
def test_batch_steps_at_mixed_positions(name, lengths, graph):
    cfg, blob, w = blob_of(name)
    B = len(lengths)
    caches = prefixes(cfg, lengths, 700)
    toks = synth.prefill_tokens(cfg, 4 * B).reshape(4, B)
    with pkg.Model(cfg, w, graph=graph, max_batch=B) as m:
        install(m, cfg, caches)
        for s in range(4):
            pos = [p + s for p in lengths]
            got = host(m.forward_batch(toks[s], pos))
            assert got.shape == (B, cfg.vocab_size)
            for b in range(B):
                ref = oracle.forward(cfg, blob, caches[b], int(toks[s, b]), pos[b])
                ok, err, tol = logits_close(got[b], ref)
                assert ok, (s, b, err, tol)
        k, v = (host(t) for t in m.read_kv_cache())
    if B == 1:  # a one-sequence model's caches have no batch axis
        k, v = k[None], v[None]
    for b in range(B):
        n = lengths[b] + 4
        for g, r in ((k[b], caches[b].k), (v[b], caches[b].v)):
            assert np.array_equal(g[:, :lengths[b]], r[:, :lengths[b]])  # the prefix is untouched
            scale = np.max(np.abs(r[:, lengths[b]:n]))
            assert np.max(np.abs(g[:, lengths[b]:n] - r[:, lengths[b]:n])) <= 1e-4 * scale
            assert np.all(g[:, n:] == 0)


@pytest.mark.parametrize("dim,heads,hidden,B", [(256, 4, 5120, 24), (256, 4, 5120, 64), (256, 4, 11008, 20),
                                                (256, 4, 11008, 50), (3072, 24, 1024, 20), (3072, 24, 1024, 64)])
def test_batch_step_with_wide_products(dim, heads, hidden, B):
    # products with more row tiles than compute units take one block per CU of
    # ceil(row tiles / CUs) row tiles (the 7B shape's q/k/v, w1/w3 and
    # classifier); one-layer models put w1/w3 there with 3 (dim 256, hidden
    # 5120) and 6 (hidden 11008) row tiles per block, the q/k/v product with 3
    # (dim 3072: 576 row tiles), the classifier with 8, at two to four planes
    # of 16 sequences, beside the K split of wo and w2
    cfg = synth.Config(f"wide{dim}x{hidden}", dim, hidden, 1, heads, heads, 32000, 64, 0, 1011)
    blob = synth.make_blob(cfg)
    lengths = [(7 * b) % 60 for b in range(B)]
    caches = prefixes(cfg, lengths, 800)
    toks = synth.prefill_tokens(cfg, B)
    with pkg.Model(cfg, dev(blob), max_batch=B) as m:
        install(m, cfg, caches)
        got = host(m.forward_batch(toks, lengths))
    assert got.shape == (B, cfg.vocab_size)
    for b in range(B):
        ref = oracle.forward(cfg, blob, caches[b], int(toks[b]), lengths[b])
        ok, err, tol = logits_close(got[b], ref)
        assert ok, (b, err, tol)


@pytest.mark.parametrize("name,B", [("tiny", 2), ("stories15m", 8), ("gqa_small", 33)])
def test_greedy_generation_in_lockstep(name, B):
    cfg, blob, w = blob_of(name)
    n = min(24, cfg.seq_len)
    starts = synth.prefill_tokens(cfg, B)
    with pkg.Model(cfg, w, max_batch=B) as m:
        got = m.generate_batch(starts, [0] * B, n)
    assert got.shape == (B, n)
    for b in range(B):
        want, wl = oracle.generate(cfg, blob, oracle.KVCache(cfg), int(starts[b]), 0, n, keep_logits=True)
        for i in range(n):
            if got[b, i] != want[i]:
                assert acceptable_token(int(got[b, i]), wl[i]), (b, i)
                break


def test_a_batch_of_one_and_the_single_sequence_calls():
    cfg, blob, w = blob_of("stories15m")
    with pkg.Model(cfg, w, max_batch=3) as m:
        a = host(m.forward_batch([1], [0]))[0]
        m.reset()
        b = host(m.forward(1, 0))  # sequence 0 through the single-sequence path
    ref = oracle.forward(cfg, blob, oracle.KVCache(cfg), 1, 0)
    assert logits_close(a, ref)[0] and logits_close(b, ref)[0]


def test_batch_range_errors():
    cfg, blob, w = blob_of("tiny")
    with pkg.Model(cfg, w, max_batch=2) as m:
        for toks, pos in (([1, 2, 3], [0, 0, 0]), ([1], [cfg.seq_len]), ([cfg.vocab_size], [0]), ([1], [-1])):
            with pytest.raises(ld.LdError) as e:
                m.forward_batch(toks, pos)
            assert e.value.status == ld.LD_E_RANGE
        with pytest.raises(ld.LdError) as e:
            m.generate_batch([1, 1], [0, cfg.seq_len - 2], 3)
        assert e.value.status == ld.LD_E_RANGE
        assert np.all(np.isfinite(host(m.forward_batch([1, 2], [0, 0]))))
    with pkg.Model(cfg, w) as m:  # max_batch 1
        with pytest.raises(ld.LdError):
            m.forward_batch([1, 2], [0, 0])


@pytest.mark.parametrize("name", ["stories15m", "gqa_small"])
def test_prompts_prefilled_per_sequence_then_decoded_as_a_batch(name):
    # each sequence's prompt through ld_prefill_seq (lengths differ), then batched steps
    cfg, blob, w = blob_of(name)
    lengths = [37, 5, 64]
    B = len(lengths)
    prompts = [synth.prefill_tokens(cfg, 200)[10 * b:10 * b + n] for b, n in enumerate(lengths)]
    caches, nexts = [], []
    for pr in prompts:
        c = oracle.KVCache(cfg)
        for i, t in enumerate(pr):
            lg = oracle.forward(cfg, blob, c, int(t), i)
        caches.append(c)
        nexts.append(oracle.argmax(lg))
    with pkg.Model(cfg, w, max_batch=B) as m:
        for b, pr in enumerate(prompts):
            m.prefill(pr, 0, seq=b)
        got = host(m.forward_batch(nexts, lengths))
        k, _ = (host(t) for t in m.read_kv_cache())
    for b in range(B):
        ref = oracle.forward(cfg, blob, caches[b], nexts[b], lengths[b])
        ok, err, tol = logits_close(got[b], ref)
        assert ok, (b, err, tol)
        n = lengths[b] + 1
        scale = np.max(np.abs(caches[b].k[:, :n]))
        assert np.max(np.abs(k[b][:, :n] - caches[b].k[:, :n])) <= 1e-4 * scale
        assert np.all(k[b][:, n:] == 0)


def test_prefill_seq_range():
    cfg, blob, w = blob_of("tiny")
    with pkg.Model(cfg, w, max_batch=2) as m:
        for seq in (-1, 2):
            with pytest.raises(ld.LdError) as e:
                m.prefill([1, 2], 0, seq=seq)
            assert e.value.status == ld.LD_E_RANGE
