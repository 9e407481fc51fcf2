"""Thin ctypes binding of ``include/ld.h``: the same names, argument
marshalling only.  Every step of the decode path runs in the HIP kernels of
``libld.so``; nothing here computes.  The library is loaded on first use and a
missing build raises at once: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_SO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libld.so")
_lib = None

LD_OK = 0
LD_E_NULL = -1
LD_E_CONFIG = -2
LD_E_SIZE = -3
LD_E_ALIGN = -4
LD_E_RANGE = -5
LD_E_OOM = -6
LD_E_HIP = -7
LD_E_UNSUPPORTED = -8
LD_OPT_NO_GRAPH = 1
LD_OPT_NO_FUSE = 2
LD_NOALLOC_SCRATCH_BYTES = 4 << 20

# Every symbol include/ld.h declares.
EXPORTS = (
    "ld_weights_size", "ld_create", "ld_reset", "ld_forward", "ld_argmax_last", "ld_generate_greedy",
    "ld_generate", "ld_prefill", "ld_prefill_seq", "ld_forward_batch", "ld_generate_greedy_batch", "ld_kv_cache", "ld_destroy", "ld_strerror", "ld_last_error_detail",
    "ld_profile_steps", "ld_op_rmsnorm_gemv", "ld_op_gemv_residual", "ld_op_swiglu", "ld_op_qkv_rope",
    "ld_op_attention", "ld_op_gemm", "ld_op_attention_prefill", "ld_op_argmax", "ld_op_sample",
    "ld_op_stream_read", "ld_op_attention_noalloc", "ld_op_qkv_attention",
)


class LdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = ""
        if status in (LD_E_HIP, LD_E_OOM) and _lib is not None:
            detail = ": " + _lib.ld_last_error_detail().decode()
        super().__init__(f"{where} failed with {status} ({ld_strerror(status)}){detail}")


class ld_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("dim", "hidden_dim", "n_layers", "n_heads", "n_kv_heads", "vocab_size", "seq_len")]


class ld_options(ctypes.Structure):
    _fields_ = [("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("shared_classifier", ctypes.c_int32), ("flags", ctypes.c_int32), ("max_batch", ctypes.c_int32)]


class ld_sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("topp", ctypes.c_float), ("stop_token", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class ld_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float


def library():
    """Load libld.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # Load PyTorch's HIP runtime first when PyTorch is present: both it and
        # ROCm's carry the soname libamdhip64.so.7, so libld.so then binds to the
        # copy PyTorch already uses and the process holds a single runtime.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(_SO):
            raise RuntimeError(f"HIP library {_SO} is missing: build it with __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950); there is no CPU fallback")
        lib = ctypes.CDLL(_SO)
        sig = {
            "ld_weights_size": ([_P, _P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
            "ld_create": ([_P, _P, _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)], ctypes.c_int),
            "ld_reset": ([_P], ctypes.c_int),
            "ld_forward": ([_P, _I, _I, ctypes.POINTER(_P)], ctypes.c_int),
            "ld_argmax_last": ([_P, ctypes.POINTER(_I)], ctypes.c_int),
            "ld_generate_greedy": ([_P, _I, _I, _I, _P], ctypes.c_int),
            "ld_generate": ([_P, _P, _I, _I, _I, _P, _P, _P, ctypes.POINTER(_I)], ctypes.c_int),
            "ld_prefill": ([_P, _P, _I, _I, ctypes.POINTER(_P)], ctypes.c_int),
            "ld_prefill_seq": ([_P, _I, _P, _I, _I, ctypes.POINTER(_P)], ctypes.c_int),
            "ld_forward_batch": ([_P, _P, _P, _I, ctypes.POINTER(_P)], ctypes.c_int),
            "ld_generate_greedy_batch": ([_P, _P, _P, _I, _I, _P], ctypes.c_int),
            "ld_kv_cache": ([_P, ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_size_t)],
                            ctypes.c_int),
            "ld_destroy": ([_P], None),
            "ld_strerror": ([ctypes.c_int], ctypes.c_char_p),
            "ld_last_error_detail": ([], ctypes.c_char_p),
            "ld_profile_steps": ([_P, _I, _I, _I, _P, _I, ctypes.POINTER(_I)], ctypes.c_int),
            "ld_op_rmsnorm_gemv": ([_P, _P, _F, _P, _I, _I, _P, _P], ctypes.c_int),
            "ld_op_gemv_residual": ([_P, _P, _I, _I, _P, _P], ctypes.c_int),
            "ld_op_swiglu": ([_P, _P, _F, _P, _P, _I, _I, _P, _P], ctypes.c_int),
            "ld_op_qkv_rope": ([_P, _P, _F, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P], ctypes.c_int),
            "ld_op_qkv_attention": ([_P, _P, _F, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P], ctypes.c_int),
            "ld_op_attention": ([_P, _P, _P, _I, _I, _I, _I, _P, _P], ctypes.c_int),
            "ld_op_attention_noalloc": ([_P, _P, _P, _I, _I, _I, _I, _P, _P], ctypes.c_int),
            "ld_op_gemm": ([_P, _P, _I, _I, _I, _P, _P], ctypes.c_int),
            "ld_op_attention_prefill": ([_P, _P, _P, _I, _I, _I, _I, _I, _P, _P], ctypes.c_int),
            "ld_op_argmax": ([_P, _I, ctypes.POINTER(_I), _P], ctypes.c_int),
            "ld_op_sample": ([_P, _I, _F, _F, _F, ctypes.POINTER(_I), _P], ctypes.c_int),
            "ld_op_stream_read": ([_P, ctypes.c_size_t, _P, _P], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _check(status: int, where: str) -> None:
    if status != LD_OK:
        raise LdError(status, where)


def make_config(cfg) -> ld_config:
    """cfg: any object with the seven Config fields."""
    return ld_config(cfg.dim, cfg.hidden_dim, cfg.n_layers, cfg.n_heads, cfg.n_kv_heads, cfg.vocab_size,
                     cfg.seq_len)


def make_options(norm_eps: float = 1e-5, rope_theta: float = 10000.0, shared_classifier: int = 0,
                 flags: int = 0, max_batch: int = 1) -> ld_options:
    return ld_options(norm_eps, rope_theta, shared_classifier, flags, max_batch)


# --------------------------------------------------------------------------- entry points

def ld_strerror(status: int) -> str:
    return library().ld_strerror(status).decode()


def ld_weights_size(cfg: ld_config, opt: ld_options) -> int:
    out = ctypes.c_size_t(0)
    _check(library().ld_weights_size(ctypes.byref(cfg), ctypes.byref(opt), ctypes.byref(out)), "ld_weights_size")
    return out.value


def ld_create(cfg: ld_config, opt: ld_options, d_weights: int, nbytes: int, stream: int = 0) -> int:
    h = _P()
    _check(library().ld_create(ctypes.byref(cfg), ctypes.byref(opt), d_weights, nbytes, stream or None,
                               ctypes.byref(h)), "ld_create")
    return h.value


def ld_reset(h: int) -> None:
    _check(library().ld_reset(h), "ld_reset")


def ld_forward(h: int, token: int, pos: int) -> int:
    out = _P()
    _check(library().ld_forward(h, token, pos, ctypes.byref(out)), "ld_forward")
    return out.value


def ld_argmax_last(h: int) -> int:
    out = _I(0)
    _check(library().ld_argmax_last(h, ctypes.byref(out)), "ld_argmax_last")
    return out.value


def ld_generate_greedy(h: int, token: int, pos: int, n_steps: int) -> np.ndarray:
    out = np.zeros(max(n_steps, 1), np.int32)
    _check(library().ld_generate_greedy(h, token, pos, n_steps, out.ctypes.data), "ld_generate_greedy")
    return out[:n_steps]


def ld_generate(h: int, prompt, pos: int, n_steps: int, temperature: float = 0.0, topp: float = 0.0,
                stop_token: int = -1, coins=None) -> np.ndarray:
    """Returns the tokens of the steps run (fewer than n_steps after a stop)."""
    prompt = np.ascontiguousarray(prompt, dtype=np.int32)
    c = None
    if coins is not None:
        c = np.ascontiguousarray(coins, dtype=np.float32)
        if c.size < n_steps:
            raise ValueError("need one coin per step")
    out = np.zeros(max(n_steps, 1), np.int32)
    n_out = _I(0)
    smp = ld_sampling(temperature, topp, stop_token, 0)
    _check(library().ld_generate(h, prompt.ctypes.data if prompt.size else None, prompt.size, pos, n_steps,
                                 ctypes.byref(smp), c.ctypes.data if c is not None else None, out.ctypes.data,
                                 ctypes.byref(n_out)), "ld_generate")
    return out[:n_out.value]


def ld_prefill(h: int, tokens, pos: int) -> int:
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    out = _P()
    _check(library().ld_prefill(h, t.ctypes.data if t.size else None, t.size, pos, ctypes.byref(out)), "ld_prefill")
    return out.value


def ld_forward_batch(h: int, tokens, pos) -> int:
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    p = np.ascontiguousarray(pos, dtype=np.int32)
    if t.size != p.size:
        raise ValueError("one position per token")
    out = _P()
    _check(library().ld_forward_batch(h, t.ctypes.data if t.size else None, p.ctypes.data if p.size else None,
                                      t.size, ctypes.byref(out)), "ld_forward_batch")
    return out.value


def ld_generate_greedy_batch(h: int, tokens, pos, n_steps: int) -> np.ndarray:
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    p = np.ascontiguousarray(pos, dtype=np.int32)
    if t.size != p.size:
        raise ValueError("one position per token")
    out = np.zeros(max(t.size * n_steps, 1), np.int32)
    _check(library().ld_generate_greedy_batch(h, t.ctypes.data if t.size else None,
                                              p.ctypes.data if p.size else None, t.size, n_steps, out.ctypes.data),
           "ld_generate_greedy_batch")
    return out[:t.size * n_steps].reshape(t.size, n_steps)


def ld_prefill_seq(h: int, seq: int, tokens, pos: int) -> int:
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    out = _P()
    _check(library().ld_prefill_seq(h, seq, t.ctypes.data if t.size else None, t.size, pos, ctypes.byref(out)),
           "ld_prefill_seq")
    return out.value


def ld_kv_cache(h: int):
    k, v, n = _P(), _P(), ctypes.c_size_t(0)
    _check(library().ld_kv_cache(h, ctypes.byref(k), ctypes.byref(v), ctypes.byref(n)), "ld_kv_cache")
    return k.value, v.value, n.value


def ld_destroy(h: int) -> None:
    if h:
        library().ld_destroy(h)


def ld_profile_steps(h: int, token: int, pos: int, n_steps: int):
    stats = (ld_kernel_stat * 16)()
    n = _I(0)
    _check(library().ld_profile_steps(h, token, pos, n_steps, stats, 16, ctypes.byref(n)), "ld_profile_steps")
    return [{"name": stats[i].name.decode(), "launches": stats[i].launches, "total_ms": stats[i].total_ms}
            for i in range(n.value)]


def ld_op_rmsnorm_gemv(d_x, d_g, eps, d_w, rows, n, d_out, stream=0):
    _check(library().ld_op_rmsnorm_gemv(d_x, d_g or None, eps, d_w, rows, n, d_out, stream or None),
           "ld_op_rmsnorm_gemv")


def ld_op_gemv_residual(d_in, d_w, rows, n, d_x, stream=0):
    _check(library().ld_op_gemv_residual(d_in, d_w, rows, n, d_x, stream or None), "ld_op_gemv_residual")


def ld_op_swiglu(d_x, d_g, eps, d_w1, d_w3, hidden, n, d_hb, stream=0):
    _check(library().ld_op_swiglu(d_x, d_g or None, eps, d_w1, d_w3, hidden, n, d_hb, stream or None),
           "ld_op_swiglu")


def ld_op_qkv_rope(d_x, d_g, eps, d_wq, d_wk, d_wv, dim, n_heads, n_kv_heads, pos, theta, d_q, d_k, d_v,
                   stream=0):
    _check(library().ld_op_qkv_rope(d_x, d_g or None, eps, d_wq, d_wk, d_wv, dim, n_heads, n_kv_heads, pos, theta,
                                    d_q, d_k, d_v, stream or None), "ld_op_qkv_rope")


def ld_op_qkv_attention(d_x, d_g, eps, d_wq, d_wk, d_wv, dim, n_heads, n_kv_heads, pos, theta, d_kc, d_vc, d_out,
                        stream=0):
    _check(library().ld_op_qkv_attention(d_x, d_g or None, eps, d_wq, d_wk, d_wv, dim, n_heads, n_kv_heads, pos,
                                         theta, d_kc, d_vc, d_out, stream or None), "ld_op_qkv_attention")


def ld_op_attention(d_q, d_kc, d_vc, n_heads, n_kv_heads, head_size, pos, d_out, stream=0):
    _check(library().ld_op_attention(d_q, d_kc, d_vc, n_heads, n_kv_heads, head_size, pos, d_out, stream or None),
           "ld_op_attention")


def ld_op_attention_noalloc(d_q, d_kc, d_vc, n_heads, n_kv_heads, head_size, pos, d_out, stream=0):
    """Asynchronous on the stream (no allocation, no wait)."""
    _check(library().ld_op_attention_noalloc(d_q, d_kc, d_vc, n_heads, n_kv_heads, head_size, pos, d_out,
                                             stream or None), "ld_op_attention_noalloc")


def ld_op_argmax(d_v, n, stream=0) -> int:
    out = _I(0)
    _check(library().ld_op_argmax(d_v, n, ctypes.byref(out), stream or None), "ld_op_argmax")
    return out.value


def ld_op_sample(d_logits, n, temperature, topp, coin, stream=0) -> int:
    out = _I(0)
    _check(library().ld_op_sample(d_logits, n, temperature, topp, coin, ctypes.byref(out), stream or None),
           "ld_op_sample")
    return out.value


LD_STREAM_READ_BLOCKS = 2048


def ld_op_stream_read(d_src, nbytes, d_sums, stream=0):
    """Enqueue the plain streaming read of nbytes at d_src (asynchronous);
    d_sums (LD_STREAM_READ_BLOCKS floats) receives the per-share sums."""
    _check(library().ld_op_stream_read(d_src, nbytes, d_sums, stream or None), "ld_op_stream_read")


def ld_op_gemm(d_a, d_w, m, n, k, d_out, stream=0):
    _check(library().ld_op_gemm(d_a, d_w, m, n, k, d_out, stream or None), "ld_op_gemm")


def ld_op_attention_prefill(d_q, d_kc, d_vc, n_heads, n_kv_heads, head_size, pos, n_tokens, d_out, stream=0):
    _check(library().ld_op_attention_prefill(d_q, d_kc, d_vc, n_heads, n_kv_heads, head_size, pos, n_tokens, d_out,
                                             stream or None), "ld_op_attention_prefill")
