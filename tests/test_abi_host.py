"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/ld.h declares, sizes the weight blob as the oracle and the
generator do, and rejects bad arguments with the documented codes before any
device work."""
import ctypes
import os
import re

import pytest

import llama_transformer_decode_amd as pkg
from llama_transformer_decode_amd import ld
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "ld.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ld_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 17
    lib = pkg.library()
    for n in names:
        assert hasattr(lib, n), f"libld.so does not export {n}"
    assert sorted(ld.EXPORTS) == names


def test_status_texts():
    for code in (ld.LD_OK, ld.LD_E_NULL, ld.LD_E_CONFIG, ld.LD_E_SIZE, ld.LD_E_ALIGN, ld.LD_E_RANGE, ld.LD_E_OOM,
                 ld.LD_E_HIP, ld.LD_E_UNSUPPORTED):
        assert ld.ld_strerror(code)
    assert ld.ld_strerror(12345) == "unknown status"


@pytest.mark.parametrize("name", sorted(synth.CONFIGS))
def test_blob_size_agrees_with_oracle_and_generator(name):
    c = synth.CONFIGS[name]
    got = ld.ld_weights_size(ld.make_config(c), ld.make_options(shared_classifier=c.shared_classifier))
    assert got == 4 * synth.blob_floats(c) == 4 * oracle.blob_floats(c)


def test_blob_size_of_large_model_uses_64_bit_offsets():
    c = synth.CONFIGS["llama70b_8l"]
    assert ld.ld_weights_size(ld.make_config(c), ld.make_options()) == 4 * 7_369_531_392 > 2 ** 32


BAD = [
    dict(dim=0), dict(n_layers=-1), dict(vocab_size=0), dict(seq_len=0),
    dict(n_heads=5),                                   # 5 does not divide 64
    dict(dim=66, n_heads=6),                           # head size 11 is odd
    dict(n_kv_heads=8),                                # more kv heads than query heads
    dict(hidden_dim=178),                              # hidden not a multiple of 4
    dict(dim=8, n_heads=4, n_kv_heads=1, hidden_dim=16),  # kv_dim 2 not a multiple of 4
    dict(dim=18, n_heads=1, n_kv_heads=1),             # dim not a multiple of 4
]


@pytest.mark.parametrize("bad", BAD)
def test_invalid_config_rejected(bad):
    c = synth.CONFIGS["tiny"].replace(**bad)
    with pytest.raises(ld.LdError) as e:
        ld.ld_weights_size(ld.make_config(c), ld.make_options())
    assert e.value.status == ld.LD_E_CONFIG


@pytest.mark.parametrize("opt", [dict(norm_eps=-1.0), dict(rope_theta=0.0), dict(shared_classifier=2)])
def test_invalid_options_rejected(opt):
    with pytest.raises(ld.LdError) as e:
        ld.ld_weights_size(ld.make_config(synth.CONFIGS["tiny"]), ld.make_options(**opt))
    assert e.value.status == ld.LD_E_CONFIG


def test_null_arguments():
    lib = pkg.library()
    size = ctypes.c_size_t(0)
    assert lib.ld_weights_size(None, None, ctypes.byref(size)) == ld.LD_E_NULL
    c, o = ld.make_config(synth.CONFIGS["tiny"]), ld.make_options()
    assert lib.ld_weights_size(ctypes.byref(c), ctypes.byref(o), None) == ld.LD_E_NULL
    h = ctypes.c_void_p()
    assert lib.ld_create(ctypes.byref(c), ctypes.byref(o), None, 0, None, ctypes.byref(h)) == ld.LD_E_NULL
    for fn in ("ld_reset",):
        assert getattr(lib, fn)(None) == ld.LD_E_NULL
    out = ctypes.c_void_p()
    assert lib.ld_forward(None, 0, 0, ctypes.byref(out)) == ld.LD_E_NULL
    tok = ctypes.c_int32()
    assert lib.ld_argmax_last(None, ctypes.byref(tok)) == ld.LD_E_NULL
    lib.ld_destroy(None)  # accepted


def test_create_rejects_before_touching_the_device():
    lib = pkg.library()
    c0 = synth.CONFIGS["tiny"]
    c, o = ld.make_config(c0), ld.make_options()
    nbytes = 4 * synth.blob_floats(c0)
    h = ctypes.c_void_p()
    fake = 0x10000  # never dereferenced: each case fails validation first
    assert lib.ld_create(ctypes.byref(c), ctypes.byref(o), fake, nbytes - 4, None, ctypes.byref(h)) == ld.LD_E_SIZE
    assert lib.ld_create(ctypes.byref(c), ctypes.byref(o), fake + 4, nbytes, None, ctypes.byref(h)) == ld.LD_E_ALIGN
    odd = ld.make_config(c0.replace(dim=96, n_heads=4, n_kv_heads=4))  # head size 24 has no kernel
    assert lib.ld_create(ctypes.byref(odd), ctypes.byref(o), fake, nbytes, None, ctypes.byref(h)) == \
        ld.LD_E_UNSUPPORTED
    wide = ld.make_config(c0.replace(dim=64, n_heads=16, n_kv_heads=1))  # 16 query heads per kv head
    assert lib.ld_create(ctypes.byref(wide), ctypes.byref(o), fake, nbytes, None, ctypes.byref(h)) == \
        ld.LD_E_UNSUPPORTED
    assert h.value is None


def test_generate_and_sample_argument_checks_come_first():
    lib = pkg.library()
    smp = ld.ld_sampling(0.8, 0.9, -1, 0)
    toks = (ctypes.c_int32 * 4)()
    n_out = ctypes.c_int32(7)
    prompt = (ctypes.c_int32 * 1)(1)
    assert lib.ld_generate(None, prompt, 1, 0, 4, ctypes.byref(smp), None, toks, ctypes.byref(n_out)) == ld.LD_E_NULL
    fake = 0x10000  # never dereferenced: every case fails its argument check first
    tok = ctypes.c_int32()
    assert lib.ld_op_sample(None, 8, 1.0, 0.0, 0.5, ctypes.byref(tok), None) == ld.LD_E_NULL
    assert lib.ld_op_sample(fake, 8, 1.0, 0.0, 0.5, None, None) == ld.LD_E_NULL
    assert lib.ld_op_sample(fake, 0, 1.0, 0.0, 0.5, ctypes.byref(tok), None) == ld.LD_E_RANGE
    for coin in (-0.1, 1.0, float("nan")):
        assert lib.ld_op_sample(fake, 8, 1.0, 0.0, coin, ctypes.byref(tok), None) == ld.LD_E_RANGE
    for t in (float("nan"), float("inf")):
        assert lib.ld_op_sample(fake, 8, t, 0.0, 0.5, ctypes.byref(tok), None) == ld.LD_E_RANGE
    assert lib.ld_op_sample(fake, 8, 1.0, float("nan"), 0.5, ctypes.byref(tok), None) == ld.LD_E_RANGE
    assert lib.ld_op_sample(fake, 40000, 1.0, 0.9, 0.5, ctypes.byref(tok), None) == ld.LD_E_UNSUPPORTED


def test_prefill_and_gemm_argument_checks_come_first():
    lib = pkg.library()
    fake = 0x10000  # never dereferenced: every case fails its argument check first
    toks = (ctypes.c_int32 * 2)(1, 2)
    out = ctypes.c_void_p()
    assert lib.ld_prefill(None, toks, 2, 0, ctypes.byref(out)) == ld.LD_E_NULL
    assert lib.ld_op_gemm(None, fake, 4, 4, 4, fake, None) == ld.LD_E_NULL
    assert lib.ld_op_gemm(fake, fake, 0, 4, 4, fake, None) == ld.LD_E_RANGE
    assert lib.ld_op_gemm(fake, fake, 4, 4, 6, fake, None) == ld.LD_E_CONFIG
    assert lib.ld_op_gemm(fake + 4, fake, 4, 4, 4, fake, None) == ld.LD_E_ALIGN
    assert lib.ld_op_attention_prefill(fake, fake, fake, 4, 4, 24, 0, 2, fake, None) == ld.LD_E_UNSUPPORTED
    assert lib.ld_op_attention_prefill(fake, fake, fake, 4, 8, 16, 0, 2, fake, None) == ld.LD_E_CONFIG
    assert lib.ld_op_attention_prefill(fake, fake, fake, 4, 4, 16, 0, 0, fake, None) == ld.LD_E_RANGE
    assert lib.ld_op_attention_prefill(fake, fake, fake, 4, 4, 16, -1, 2, fake, None) == ld.LD_E_RANGE


def test_stream_read_argument_checks_come_first():
    lib = pkg.library()
    fake = 0x10000  # never dereferenced
    assert lib.ld_op_stream_read(None, 16, fake, None) == ld.LD_E_NULL
    assert lib.ld_op_stream_read(fake, 16, None, None) == ld.LD_E_NULL
    assert lib.ld_op_stream_read(fake, 0, fake, None) == ld.LD_E_SIZE
    assert lib.ld_op_stream_read(fake, 20, fake, None) == ld.LD_E_SIZE
    assert lib.ld_op_stream_read(fake + 4, 16, fake, None) == ld.LD_E_ALIGN
