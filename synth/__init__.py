"""Seeded synthetic inputs for the decode step: weights, token streams, vectors.

This package draws random numbers and lays them out; it computes nothing of
the decode step itself.  The oracle and the GPU library both take their inputs
from here, so they see identical bits.  The stream definition (SplitMix64
finaliser over a counter, Box-Muller pairs) is documented in ``synth.c``.

Workloads
---------
``CONFIGS`` holds the five model shapes the decode step is exercised on.  The
pages' trained checkpoints (stories15M, LLaMA-7B) and their tokenizers are not
used: random weights of the same shapes stand in for them, since the cost of a
decode step does not depend on the weight values.

* matrices and the embedding table: N(0, 0.02^2) (std 0.02);
* RMSNorm gains: 1 + N(0, 0.01^2);
* classifier tied to the embedding only where the shape says so (the
  stories15M-shaped model), a separately drawn classifier otherwise.

Weight blob layout (fp32, contiguous, no padding) follows the checkpoint read
order of the "run.c" page (``checkpoint_init_weights``) with the grouped-query
shapes and the separate classifier of the "run.c 逐行解讀" page (§2, the
``TransformerWeights`` struct); the RoPE tables are not part of it:

  E (V,dim) | rms_att (L,dim) | wq (L,dim,dim) | wk (L,kv_dim,dim) |
  wv (L,kv_dim,dim) | wo (L,dim,dim) | rms_ffn (L,dim) | w1 (L,hidden,dim) |
  w2 (L,dim,hidden) | w3 (L,hidden,dim) | rms_final (dim) | [wcls (V,dim)]

Tensor number k in that order (0-based) is random stream k.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

GAIN_MEAN, GAIN_STD = 1.0, 0.01
WEIGHT_MEAN, WEIGHT_STD = 0.0, 0.02
TOKEN_STREAM = 255
COIN_STREAM = 254


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (plain C, pthreads)."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "synth.c")
        tmp = _SO + ".tmp"
        subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-pthread", src, "-o", tmp, "-lm"],
                       check=True)
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_double, ctypes.c_double, ctypes.c_int]
        lib.synth_fill_normal.restype = None
        lib.synth_fill_uniform_int.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                               ctypes.c_uint64, ctypes.c_int64, ctypes.c_int]
        lib.synth_fill_uniform_int.restype = None
        lib.synth_raw.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_raw.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, min(n, 16))


def raw(seed: int, stream: int, n: int) -> int:
    """The raw 64-bit draw r(seed, stream, n)."""
    return int(_load().synth_raw(seed, stream, n))


def fill_normal(out: np.ndarray, seed: int, stream: int, mean: float, std: float, first: int = 0,
                threads: int | None = None) -> np.ndarray:
    assert out.dtype == np.float32 and out.flags["C_CONTIGUOUS"]
    _load().synth_fill_normal(out.ctypes.data, first, out.size, seed, stream, mean, std,
                              threads or default_threads())
    return out


def normal(n: int, seed: int, stream: int, mean: float = 0.0, std: float = 1.0,
           threads: int | None = None) -> np.ndarray:
    return fill_normal(np.empty(n, np.float32), seed, stream, mean, std, threads=threads)


def uniform_int(n: int, bound: int, seed: int, stream: int = TOKEN_STREAM, first: int = 0) -> np.ndarray:
    out = np.empty(n, np.int32)
    _load().synth_fill_uniform_int(out.ctypes.data, first, n, seed, stream, bound, default_threads())
    return out


def coins(n: int, seed: int, stream: int = COIN_STREAM, first: int = 0) -> np.ndarray:
    """Seeded fp32 draws in [0, 1) on the 2^-24 grid (24 random bits over 2^24,
    the resolution of a float draw), one per sampled token."""
    return (uniform_int(n, 1 << 24, seed, stream, first).astype(np.float64) / float(1 << 24)).astype(np.float32)


@dataclass(frozen=True)
class Config:
    name: str
    dim: int
    hidden_dim: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    vocab_size: int
    seq_len: int
    shared_classifier: int
    seed: int
    norm_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def head_size(self) -> int:
        return self.dim // self.n_heads

    @property
    def kv_dim(self) -> int:
        return self.dim * self.n_kv_heads // self.n_heads

    def fields(self):
        return (self.dim, self.hidden_dim, self.n_layers, self.n_heads, self.n_kv_heads,
                self.vocab_size, self.seq_len)

    def replace(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


# The five workloads.  seed = 1000 + ordinal.
CONFIGS = {
    "tiny": Config("tiny", 64, 176, 2, 4, 4, 256, 64, 0, 1001),
    "stories15m": Config("stories15m", 288, 768, 6, 6, 6, 32000, 256, 1, 1002),
    "gqa_small": Config("gqa_small", 288, 768, 6, 6, 4, 32000, 512, 0, 1003),
    "llama7b": Config("llama7b", 4096, 11008, 32, 32, 32, 32000, 2048, 0, 1004),
    "llama70b_8l": Config("llama70b_8l", 8192, 28672, 8, 64, 8, 32000, 4096, 0, 1005),
}


def layout(cfg: Config):
    """[(name, n_floats, kind)] in blob order; kind is 'gain' or 'weight'."""
    d, h, L, V, kv = cfg.dim, cfg.hidden_dim, cfg.n_layers, cfg.vocab_size, cfg.kv_dim
    items = [
        ("tok_embedding", V * d, "weight"),
        ("rms_att", L * d, "gain"),
        ("wq", L * d * d, "weight"),
        ("wk", L * kv * d, "weight"),
        ("wv", L * kv * d, "weight"),
        ("wo", L * d * d, "weight"),
        ("rms_ffn", L * d, "gain"),
        ("w1", L * h * d, "weight"),
        ("w2", L * d * h, "weight"),
        ("w3", L * h * d, "weight"),
        ("rms_final", d, "gain"),
    ]
    if not cfg.shared_classifier:
        items.append(("wcls", V * d, "weight"))
    return items


def blob_floats(cfg: Config) -> int:
    return sum(n for _, n, _ in layout(cfg))


def offsets(cfg: Config):
    """{name: (offset, n_floats)} in floats."""
    out, off = {}, 0
    for name, n, _ in layout(cfg):
        out[name] = (off, n)
        off += n
    return out


def make_blob(cfg: Config, out: np.ndarray | None = None, threads: int | None = None) -> np.ndarray:
    """The seeded fp32 weight blob of ``cfg`` (see the module docstring)."""
    total = blob_floats(cfg)
    if out is None:
        out = np.empty(total, np.float32)
    assert out.dtype == np.float32 and out.size == total and out.flags["C_CONTIGUOUS"]
    off = 0
    for stream, (_, n, kind) in enumerate(layout(cfg)):
        mean, std = (GAIN_MEAN, GAIN_STD) if kind == "gain" else (WEIGHT_MEAN, WEIGHT_STD)
        fill_normal(out[off:off + n], cfg.seed, stream, mean, std, threads=threads)
        off += n
    return out


def prefill_tokens(cfg: Config, n: int) -> np.ndarray:
    """Seeded uniform token ids in [0, vocab) used to fill a KV cache by decoding."""
    return uniform_int(n, cfg.vocab_size, cfg.seed, TOKEN_STREAM)
