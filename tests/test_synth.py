"""The seeded input generator: published SplitMix64 outputs, determinism, layout."""
import numpy as np

import synth


def test_splitmix64_published_outputs():
    # SplitMix64 started from state 0 yields 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, ...
    # r(seed=0, stream=0, n) is the generator's n-th state, so n = 1, 2 give those outputs.
    assert synth.raw(0, 0, 1) == 0xE220A8397B1DCDAF
    assert synth.raw(0, 0, 2) == 0x6E789E6AA1B965F4


def test_independent_of_thread_count_and_offset():
    a = synth.normal(100_003, 5, 9, threads=1)
    for th in (2, 3, 8):
        assert np.array_equal(synth.normal(100_003, 5, 9, threads=th), a)
    part = np.empty(1001, np.float32)
    synth.fill_normal(part, 5, 9, 0.0, 1.0, first=777)
    assert np.array_equal(part, a[777:1778])


def test_distribution_moments():
    a = synth.normal(2_000_000, 11, 3, mean=1.0, std=0.01).astype(np.float64)
    assert abs(a.mean() - 1.0) < 1e-4 and abs(a.std() - 0.01) < 1e-4
    t = synth.uniform_int(200_000, 32000, 2005)
    assert t.min() >= 0 and t.max() < 32000 and abs(t.mean() - 16000) < 200


def test_blob_layout_and_streams():
    c = synth.CONFIGS["tiny"]
    blob = synth.make_blob(c)
    off = synth.offsets(c)
    assert blob.size == synth.blob_floats(c) == 133440
    o, n = off["rms_att"]
    assert abs(blob[o:o + n].mean() - 1.0) < 0.01
    o, n = off["wq"]
    assert abs(blob[o:o + n].std() - 0.02) < 0.002
    # tensor k of the blob is stream k
    assert np.array_equal(blob[o:o + 10], synth.normal(10, c.seed, 2, 0.0, 0.02))
    assert "wcls" in off and "wcls" not in synth.offsets(synth.CONFIGS["stories15m"])
