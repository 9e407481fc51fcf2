"""ctypes wrapper of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
neither imports it nor shares any code with it.

Two builds of the same source exist: ``liboracle.so`` evaluates every
reduction and transcendental in double and rounds at the pages' fp32 store
points; ``liboracle_page.so`` (``page_literal=True``) uses the pages' own fp32
arithmetic.  Both are compiled by gcc with ``-O2 -fno-fast-math
-ffp-contract=off``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SOS = {False: os.path.join(_HERE, "liboracle.so"), True: os.path.join(_HERE, "liboracle_page.so")}
# A test that plants a mistake in a copy of oracle.c points this at the mutant build.
if os.environ.get("ORACLE_LIB"):
    _SOS[False] = os.environ["ORACLE_LIB"]
_libs: dict = {}

_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-fPIC", "-shared", "-pthread"]


def build(force: bool = True) -> None:
    src = os.path.join(_HERE, "oracle.c")
    for page, so in _SOS.items():
        if force or not os.path.exists(so):
            tmp = so + ".tmp"
            extra = ["-DORACLE_PAGE_LITERAL"] if page else []
            subprocess.run(["gcc", *_FLAGS, *extra, src, "-o", tmp, "-lm"], check=True)
            os.replace(tmp, so)


class OracleConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("dim", "hidden_dim", "n_layers", "n_heads", "n_kv_heads", "vocab_size", "seq_len")]


class OracleOptions(ctypes.Structure):
    _fields_ = [("norm_eps", ctypes.c_double), ("rope_theta", ctypes.c_double),
                ("shared_classifier", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int


def _load(page: bool = False):
    if page not in _libs:
        so = _SOS[page]
        if not os.path.exists(so):
            build(force=False)
        lib = ctypes.CDLL(so)
        sig = {
            "oracle_page_literal": ([], _I),
            "oracle_blob_floats": ([_P, _P], ctypes.c_int64),
            "oracle_rmsnorm": ([_P, _P, _P, _I, ctypes.c_double], None),
            "oracle_matvec": ([_P, _P, _P, _I, _I], None),
            "oracle_set_threads": ([_I], None),
            "oracle_rope": ([_P, _I, _I, _I, ctypes.c_double], None),
            "oracle_kv_head": ([_I, _I, _I], _I),
            "oracle_attention": ([_P, _P, _P, _P, _I, _I, _I, _I], None),
            "oracle_swiglu": ([_P, _P, _P, _I], None),
            "oracle_argmax": ([_P, _I], _I),
            "oracle_forward": ([_P, _P, _P, _P, _P, _I, _I, _P], _I),
            "oracle_generate": ([_P, _P, _P, _P, _P, _I, _I, _I, _P, _P], _I),
            "oracle_bruteforce": ([_P, _P, _P, _P, _I, _P], _I),
            "oracle_sample": ([_P, _I, ctypes.c_double, ctypes.c_double, ctypes.c_double], _I),
            "oracle_generate_sampled": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, ctypes.c_double, ctypes.c_double, _I,
                                         _P, _P, _P, _P], _I),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _libs[page] = lib
    return _libs[page]


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data


def _cfg(cfg):
    """cfg: any object with the seven Config fields (synth.Config works)."""
    return OracleConfig(cfg.dim, cfg.hidden_dim, cfg.n_layers, cfg.n_heads, cfg.n_kv_heads, cfg.vocab_size,
                        cfg.seq_len)


def _opt(cfg, shared=None, eps=None, theta=None):
    return OracleOptions(getattr(cfg, "norm_eps", 1e-5) if eps is None else eps,
                         getattr(cfg, "rope_theta", 10000.0) if theta is None else theta,
                         int(cfg.shared_classifier if shared is None else shared))


def page_literal(page: bool = False) -> bool:
    return bool(_load(page).oracle_page_literal())


def set_threads(n: int, page: bool = False) -> None:
    """Threads over which matrix rows and attention heads are shared out (default 1).
    Results are bit-identical for every count; only the wall time changes."""
    _load(page).oracle_set_threads(int(n))


def blob_floats(cfg, page: bool = False) -> int:
    return int(_load(page).oracle_blob_floats(ctypes.byref(_cfg(cfg)), ctypes.byref(_opt(cfg))))


def rmsnorm(x, g, eps=1e-5, page: bool = False) -> np.ndarray:
    x, g = _f32(x), _f32(g)
    out = np.empty_like(x)
    _load(page).oracle_rmsnorm(_ptr(out), _ptr(x), _ptr(g), x.size, eps)
    return out


def matvec(w, x, page: bool = False) -> np.ndarray:
    w, x = _f32(w), _f32(x)
    d, n = w.shape
    assert x.size == n
    out = np.empty(d, np.float32)
    _load(page).oracle_matvec(_ptr(out), _ptr(w), _ptr(x), d, n)
    return out


def rope(v, n_heads, head_size, pos, theta=10000.0, page: bool = False) -> np.ndarray:
    v = _f32(v).copy()
    assert v.size >= n_heads * head_size
    _load(page).oracle_rope(_ptr(v), n_heads, head_size, pos, theta)
    return v


def kv_head(h, n_heads, n_kv_heads) -> int:
    return int(_load().oracle_kv_head(h, n_heads, n_kv_heads))


def attention(q, kc, vc, n_heads, n_kv_heads, head_size, pos, page: bool = False) -> np.ndarray:
    q, kc, vc = _f32(q), _f32(kc), _f32(vc)
    kv_dim = n_kv_heads * head_size
    assert q.size == n_heads * head_size and kc.size >= (pos + 1) * kv_dim and vc.size >= (pos + 1) * kv_dim
    out = np.empty(n_heads * head_size, np.float32)
    _load(page).oracle_attention(_ptr(out), _ptr(q), _ptr(kc), _ptr(vc), n_heads, n_kv_heads, head_size, pos)
    return out


def swiglu(h1, h3, page: bool = False) -> np.ndarray:
    h1, h3 = _f32(h1), _f32(h3)
    out = np.empty_like(h1)
    _load(page).oracle_swiglu(_ptr(out), _ptr(h1), _ptr(h3), h1.size)
    return out


def argmax(v, page: bool = False) -> int:
    v = _f32(v)
    return int(_load(page).oracle_argmax(_ptr(v), v.size))


class KVCache:
    """A zero-filled (n_layers, seq_len, kv_dim) key cache and value cache."""

    def __init__(self, cfg):
        kv = cfg.dim * cfg.n_kv_heads // cfg.n_heads
        self.k = np.zeros((cfg.n_layers, cfg.seq_len, kv), np.float32)
        self.v = np.zeros((cfg.n_layers, cfg.seq_len, kv), np.float32)


def forward(cfg, blob, cache: KVCache, token: int, pos: int, page: bool = False, shared=None) -> np.ndarray:
    assert blob.dtype == np.float32 and blob.flags["C_CONTIGUOUS"]
    logits = np.empty(cfg.vocab_size, np.float32)
    rc = _load(page).oracle_forward(ctypes.byref(_cfg(cfg)), ctypes.byref(_opt(cfg, shared)), _ptr(blob),
                                    _ptr(cache.k), _ptr(cache.v), token, pos, _ptr(logits))
    if rc:
        raise ValueError(f"oracle_forward rejected token={token} pos={pos}")
    return logits


def generate(cfg, blob, cache: KVCache, token: int, pos: int, n: int, keep_logits: bool = False,
             page: bool = False):
    toks = np.empty(n, np.int32)
    logits = np.empty((n, cfg.vocab_size), np.float32) if keep_logits else None
    rc = _load(page).oracle_generate(ctypes.byref(_cfg(cfg)), ctypes.byref(_opt(cfg)), _ptr(blob), _ptr(cache.k),
                                     _ptr(cache.v), token, pos, n, _ptr(toks),
                                     _ptr(logits) if logits is not None else None)
    if rc:
        raise ValueError("oracle_generate rejected its arguments")
    return (toks, logits) if keep_logits else toks


def bruteforce(cfg, blob, tokens, p: int, page: bool = False, shared=None) -> np.ndarray:
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    logits = np.empty(cfg.vocab_size, np.float32)
    rc = _load(page).oracle_bruteforce(ctypes.byref(_cfg(cfg)), ctypes.byref(_opt(cfg, shared)), _ptr(blob),
                                       _ptr(tokens), p, _ptr(logits))
    if rc:
        raise ValueError("oracle_bruteforce rejected its arguments")
    return logits


def sample(logits, temperature, topp, coin, page: bool = False) -> int:
    v = _f32(logits)
    return int(_load(page).oracle_sample(_ptr(v), v.size, temperature, topp, coin))


def generate_sampled(cfg, blob, cache: KVCache, prompt, pos: int, n_steps: int, temperature: float, topp: float,
                     stop_token: int, coins, keep_logits: bool = False, page: bool = False):
    """Returns (tokens[:n_out], logits or None)."""
    prompt = np.ascontiguousarray(prompt, dtype=np.int32)
    coins = np.ascontiguousarray(coins, dtype=np.float32)
    assert coins.size >= n_steps
    toks = np.zeros(max(n_steps, 1), np.int32)
    n_out = ctypes.c_int(0)
    logits = np.empty((n_steps, cfg.vocab_size), np.float32) if keep_logits else None
    rc = _load(page).oracle_generate_sampled(ctypes.byref(_cfg(cfg)), ctypes.byref(_opt(cfg)), _ptr(blob),
                                             _ptr(cache.k), _ptr(cache.v), _ptr(prompt), prompt.size, pos, n_steps,
                                             temperature, topp, stop_token, _ptr(coins), _ptr(toks),
                                             ctypes.byref(n_out), _ptr(logits) if logits is not None else None)
    if rc:
        raise ValueError("oracle_generate_sampled rejected its arguments")
    return toks[:n_out.value], (logits[:n_out.value] if logits is not None else None)
