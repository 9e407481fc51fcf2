"""The no-allocation attention entry point against the allocating one.

ld_op_attention_noalloc keeps its split partials, arrival counts and position
in a device array the library holds per GPU; it must give ld_op_attention's
result bit for bit (same kernels, same splits), on consecutive calls whose
shapes shrink (the second and third reuse the array the first filled), and
stay within the attention bar of the oracle.  A shape whose partials exceed
the array is rejected before anything runs.
"""
import numpy as np
import pytest

from llama_transformer_decode_amd import ld
import oracle
import synth
from gpu_util import dev, host, torch_or_skip

pytestmark = pytest.mark.gpu

CALLS = [  # (n_heads, n_kv_heads, head_size, pos): each smaller than the one before
    (64, 8, 128, 4095),   # eight heads per kv head, 64 splits merged by the merge kernel
    (32, 32, 128, 700),   # splits merged by the last block of each kv head
    (6, 4, 48, 100),      # one split, non-integer head map
]


def _inputs(H, KV, hs, pos, seed):
    kv = KV * hs
    q = synth.normal(H * hs, seed, 1)
    kc = synth.normal((pos + 1) * kv, seed, 2).reshape(pos + 1, kv)
    vc = synth.normal((pos + 1) * kv, seed, 3).reshape(pos + 1, kv)
    return q, kc, vc


def test_noalloc_attention_equals_the_allocating_entry_point():
    torch = torch_or_skip()
    stream = torch.cuda.current_stream().cuda_stream
    for i, (H, KV, hs, pos) in enumerate(CALLS):
        q, kc, vc = _inputs(H, KV, hs, pos, 7100 + i)
        dq, dk, dv = dev(q), dev(kc), dev(vc)
        ref = dev(np.zeros(H * hs, np.float32))
        got = dev(np.full(H * hs, np.nan, np.float32))
        ld.ld_op_attention(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), H, KV, hs, pos, ref.data_ptr(), stream)
        ld.ld_op_attention_noalloc(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), H, KV, hs, pos, got.data_ptr(),
                                   stream)
        torch.cuda.synchronize()
        g, r = host(got), host(ref)
        print(f"call {i}: heads {H}/{KV}, head size {hs}, pos {pos}: max |d| against ld_op_attention "
              f"{float(np.max(np.abs(g - r))):.3g}", flush=True)
        assert np.array_equal(g, r)
        want = oracle.attention(q, kc, vc, H, KV, hs, pos)
        assert np.max(np.abs(g - want)) <= 2e-5 * np.max(np.abs(vc))


def test_noalloc_attention_rejects_partials_beyond_the_array():
    torch = torch_or_skip()
    # eight heads on one kv head, head size 256, 16384 positions: 512 splits of
    # 258 floats per head, 4.2 MB of partials
    H, KV, hs, pos = 8, 1, 256, 16383
    q = dev(np.zeros(H * hs, np.float32))
    kc = torch.zeros((pos + 1) * KV * hs, dtype=torch.float32, device="cuda")
    out = dev(np.zeros(H * hs, np.float32))
    with pytest.raises(ld.LdError) as e:
        ld.ld_op_attention_noalloc(q.data_ptr(), kc.data_ptr(), kc.data_ptr(), H, KV, hs, pos, out.data_ptr())
    assert e.value.status == ld.LD_E_SIZE
    assert b"scratch" in ld.library().ld_last_error_detail()
