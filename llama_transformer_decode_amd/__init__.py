"""MI355X-native single-token Llama-2 decode step (fp32, batch 1, gfx950).

The decode step runs in the hand-written HIP kernels of ``libld.so`` behind
the C ABI of ``include/ld.h``; ``ld`` binds that ABI with ctypes under the
same names.  PyTorch only provides device memory and streams: ``Model`` takes
the weight blob as a CUDA (HIP) float32 tensor and hands its pointer and the
current stream to the library.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import ld
from .ld import (LD_E_ALIGN, LD_E_CONFIG, LD_E_HIP, LD_E_NULL, LD_E_OOM, LD_E_RANGE, LD_E_SIZE,
                 LD_E_UNSUPPORTED, LD_OK, LD_OPT_NO_FUSE, LD_OPT_NO_GRAPH, LdError, library)

__all__ = ["ld", "Model", "LdError", "library", "copy_from_device", "copy_to_device"]

_hip = None
_HIP_D2D, _HIP_H2D, _HIP_D2H = 3, 1, 2


def _hip_rt():
    global _hip
    if _hip is None:
        library()  # libld.so pulls in the HIP runtime it was linked with
        _hip = ctypes.CDLL("libamdhip64.so.7")  # by soname: the runtime already loaded
        _hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                        ctypes.c_void_p]
        _hip.hipMemcpyAsync.restype = ctypes.c_int
        _hip.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipStreamSynchronize.restype = ctypes.c_int
    return _hip


def copy_from_device(ptr: int, shape, dtype=None, stream=None):
    """A new torch CUDA tensor holding a copy of device memory at ``ptr``."""
    import torch
    dtype = dtype or torch.float32
    out = torch.empty(shape, dtype=dtype, device="cuda")
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rt = _hip_rt()
    rc = rt.hipMemcpyAsync(out.data_ptr(), ptr, out.numel() * out.element_size(), _HIP_D2D, s or None)
    if rc == 0:
        rc = rt.hipStreamSynchronize(s or None)
    if rc != 0:
        raise RuntimeError(f"hipMemcpyAsync failed with {rc}")
    return out


def copy_to_device(ptr: int, src, stream=None) -> None:
    """Copy a torch CUDA tensor into device memory at ``ptr``."""
    import torch
    src = src.contiguous()
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rt = _hip_rt()
    rc = rt.hipMemcpyAsync(ptr, src.data_ptr(), src.numel() * src.element_size(), _HIP_D2D, s or None)
    if rc == 0:
        rc = rt.hipStreamSynchronize(s or None)
    if rc != 0:
        raise RuntimeError(f"hipMemcpyAsync failed with {rc}")


class Model:
    """One model over a device weight blob (see ``ld_create`` in include/ld.h).

    cfg: any object with dim, hidden_dim, n_layers, n_heads, n_kv_heads,
    vocab_size, seq_len (and optionally shared_classifier, norm_eps,
    rope_theta).  weights: contiguous float32 CUDA tensor holding the blob.
    """

    def __init__(self, cfg, weights, *, graph: bool = True, shared_classifier=None, norm_eps=None,
                 rope_theta=None, stream=None, max_batch: int = 1, fuse: bool = True):
        import torch
        if not (weights.is_cuda and weights.dtype == torch.float32 and weights.is_contiguous()):
            raise ValueError("weights must be a contiguous float32 CUDA tensor")
        self.cfg = cfg
        self.weights = weights
        shared = getattr(cfg, "shared_classifier", 0) if shared_classifier is None else shared_classifier
        eps = getattr(cfg, "norm_eps", 1e-5) if norm_eps is None else norm_eps
        theta = getattr(cfg, "rope_theta", 10000.0) if rope_theta is None else rope_theta
        self.c = ld.make_config(cfg)
        flags = (0 if graph else LD_OPT_NO_GRAPH) | (0 if fuse else LD_OPT_NO_FUSE)
        self.o = ld.make_options(eps, theta, int(shared), flags, int(max_batch))
        self.max_batch = max(1, int(max_batch))
        self.stream = stream or torch.cuda.current_stream()
        self.kv_dim = cfg.dim * cfg.n_kv_heads // cfg.n_heads
        self.h = 0
        self.h = ld.ld_create(self.c, self.o, weights.data_ptr(), weights.numel() * 4, self.stream.cuda_stream)

    def forward(self, token: int, pos: int):
        """Logits of one decode step, copied into a new torch CUDA tensor."""
        ptr = ld.ld_forward(self.h, int(token), int(pos))
        return copy_from_device(ptr, (self.cfg.vocab_size,), stream=self.stream)

    def prefill(self, tokens, pos: int, seq: int = 0):
        """All prompt tokens at positions pos.. at once; returns the last token's logits (a copy)."""
        ptr = self.prefill_async(tokens, pos, seq)
        return copy_from_device(ptr, (self.cfg.vocab_size,), stream=self.stream)

    def prefill_async(self, tokens, pos: int, seq: int = 0) -> int:
        """Queue a prompt prefill (into sequence seq of a batch model); returns the
        library-owned device logits pointer."""
        return ld.ld_prefill_seq(self.h, int(seq), tokens, int(pos))

    def forward_async(self, token: int, pos: int) -> int:
        """Queue one decode step; returns the library-owned device logits pointer."""
        return ld.ld_forward(self.h, int(token), int(pos))

    def argmax_last(self) -> int:
        return ld.ld_argmax_last(self.h)

    def generate(self, token: int, pos: int, n: int) -> np.ndarray:
        return ld.ld_generate_greedy(self.h, int(token), int(pos), int(n))

    def generate_sampled(self, prompt, pos: int, n: int, temperature: float = 0.0, topp: float = 0.0,
                         stop_token: int = -1, coins=None) -> np.ndarray:
        """The prompt-forcing, sampling generation loop (ld_generate)."""
        return ld.ld_generate(self.h, prompt, int(pos), int(n), float(temperature), float(topp), int(stop_token),
                              coins)

    def forward_batch(self, tokens, pos):
        """One decode step for sequences 0..n-1 (token b at position pos[b]); (n, vocab) logits, a copy."""
        ptr = ld.ld_forward_batch(self.h, tokens, pos)
        return copy_from_device(ptr, (len(tokens), self.cfg.vocab_size), stream=self.stream)

    def generate_batch(self, tokens, pos, n: int) -> np.ndarray:
        """Greedy generation of n steps for each sequence in lockstep; (batch, n) tokens."""
        return ld.ld_generate_greedy_batch(self.h, tokens, pos, int(n))

    def reset(self) -> None:
        ld.ld_reset(self.h)

    def kv_cache_pointers(self):
        return ld.ld_kv_cache(self.h)

    def read_kv_cache(self):
        import torch
        k, v, n = ld.ld_kv_cache(self.h)
        shape = (self.cfg.n_layers, self.cfg.seq_len, self.kv_dim)
        if self.max_batch > 1:
            shape = (self.max_batch,) + shape
        return (copy_from_device(k, shape, torch.float32, self.stream),
                copy_from_device(v, shape, torch.float32, self.stream))

    def write_kv_cache(self, k, v) -> None:
        kp, vp, n = ld.ld_kv_cache(self.h)
        assert k.numel() == n and v.numel() == n
        copy_to_device(kp, k, self.stream)
        copy_to_device(vp, v, self.stream)

    def profile(self, token: int, pos: int, n: int):
        return ld.ld_profile_steps(self.h, int(token), int(pos), int(n))

    def close(self) -> None:
        if self.h:
            ld.ld_destroy(self.h)
            self.h = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
