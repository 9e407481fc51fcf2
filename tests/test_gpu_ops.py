"""Each kernel of the decode step against the oracle's definition of that step,
through the single-kernel entry points of the C ABI (ld_op_*), on seeded
inputs at every workload's shapes, including tails that are not a multiple of
the block or row-group size.

Floating-point tolerances are error bounds of the fp32 evaluation order used
by the kernels: a matrix-vector sum of n terms is a sequential sum of at most
64 products per thread, a 6-level wave tree and at most 8 wave partials, so
|error| <= 80 u sum_j |w_j x_j| (u = 2^-24), plus the rounding of x' by the
fused RMSNorm and of the result.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import U32, dev, host, torch_or_skip
from llama_transformer_decode_amd import ld

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch_or_skip()


def _normal(n, seed, stream, mean=0.0, std=1.0):
    return synth.normal(n, seed, stream, mean, std)


def gemv_bound(w, xp, y):
    a = np.abs(w.astype(np.float64)) @ np.abs(xp.astype(np.float64))
    return 80 * U32 * a + 4 * U32 * np.abs(y.astype(np.float64)) + 1e-30


# (rows, n): every matrix shape of the five workloads, plus ragged tails
GEMV_SHAPES = [
    (4, 4), (12, 64), (176, 64), (64, 176), (288, 288), (768, 288), (288, 768), (192, 288), (100, 1000),
    (1020, 4096), (12288, 4096), (11008, 4096), (4096, 11008), (32000, 4096), (10240, 8192), (8192, 8192),
    (28672, 8192), (8192, 28672), (32000, 8192), (8, 12288), (36, 32768),
]


@pytest.mark.parametrize("rows,n", GEMV_SHAPES)
@pytest.mark.parametrize("norm", [False, True])
def test_gemv_matches_oracle(rows, n, norm):
    seed = 10_000 + rows * 7 + n
    w = _normal(rows * n, seed, 1, std=0.02).reshape(rows, n)
    x = _normal(n, seed, 2)
    g = _normal(n, seed, 3, 1.0, 0.01)
    out = dev(np.zeros(rows, np.float32))
    dw, dx, dg = dev(w), dev(x), dev(g)
    ld.ld_op_rmsnorm_gemv(dx.data_ptr(), dg.data_ptr() if norm else 0, 1e-5, dw.data_ptr(), rows, n, out.data_ptr())
    xp = oracle.rmsnorm(x, g, 1e-5) if norm else x
    ref = oracle.matvec(w, xp)
    got = host(out)
    bound = gemv_bound(w, xp, ref)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= bound), float(np.max(np.abs(got - ref) / bound))


@pytest.mark.parametrize("n", [64, 288, 768, 4096, 8192])
def test_fused_rmsnorm_alone(n):
    # W = I turns the kernel into RMSNorm: x' = g * x / sqrt(mean(x^2) + eps)
    x = _normal(n, 77, 1, std=3.0)
    g = _normal(n, 77, 2, 1.0, 0.01)
    eye = np.eye(n, dtype=np.float32)
    out = dev(np.zeros(n, np.float32))
    dx, dg, dw = dev(x), dev(g), dev(eye)
    ld.ld_op_rmsnorm_gemv(dx.data_ptr(), dg.data_ptr(), 1e-5, dw.data_ptr(), n, n, out.data_ptr())
    ref = oracle.rmsnorm(x, g, 1e-5)
    assert np.allclose(host(out), ref, rtol=8 * U32, atol=0)


@pytest.mark.parametrize("rows,n", [(64, 64), (64, 176), (288, 768), (4096, 4096), (4096, 11008), (8192, 28672)])
def test_gemv_residual(rows, n):
    w = _normal(rows * n, 31 + n, 1, std=0.02).reshape(rows, n)
    xin = _normal(n, 31 + n, 2)
    x0 = _normal(rows, 31 + n, 3)
    dx, din, dw = dev(x0), dev(xin), dev(w)
    ld.ld_op_gemv_residual(din.data_ptr(), dw.data_ptr(), rows, n, dx.data_ptr())
    y = oracle.matvec(w, xin)
    ref = x0.astype(np.float64) + y
    bound = gemv_bound(w, xin, y) + 2 * U32 * np.abs(ref)
    assert np.all(np.abs(host(dx) - ref) <= bound)


@pytest.mark.parametrize("hidden,n", [(176, 64), (768, 288), (11008, 4096), (28672, 8192), (6, 8)])
def test_swiglu(hidden, n):
    w1 = _normal(hidden * n, 500 + n, 1, std=0.02).reshape(hidden, n)
    w3 = _normal(hidden * n, 500 + n, 2, std=0.02).reshape(hidden, n)
    x = _normal(n, 500 + n, 3)
    g = _normal(n, 500 + n, 4, 1.0, 0.01)
    hb = dev(np.zeros(hidden, np.float32))
    dx, dg, dw1, dw3 = dev(x), dev(g), dev(w1), dev(w3)
    ld.ld_op_swiglu(dx.data_ptr(), dg.data_ptr(), 1e-5, dw1.data_ptr(), dw3.data_ptr(), hidden, n, hb.data_ptr())
    xp = oracle.rmsnorm(x, g, 1e-5)
    a, b = oracle.matvec(w1, xp), oracle.matvec(w3, xp)
    ref = oracle.swiglu(a, b).astype(np.float64)
    # silu(a) b: propagate the bounds of a and b, plus a few roundings of the gate
    ea, eb = gemv_bound(w1, xp, a), gemv_bound(w3, xp, b)
    sig = 1 / (1 + np.exp(-a.astype(np.float64)))
    dsilu = np.abs(sig * (1 + a * (1 - sig)))
    bound = dsilu * np.abs(b) * ea + np.abs(a * sig) * eb + 8 * U32 * np.abs(ref) + 1e-30
    assert np.all(np.abs(host(hb) - ref) <= bound)


QKV_CASES = [  # (dim, n_heads, n_kv_heads, pos)
    (64, 4, 4, 0), (64, 4, 4, 63), (288, 6, 6, 1), (288, 6, 6, 255), (288, 6, 4, 17), (288, 6, 4, 511),
    (4096, 32, 32, 0), (4096, 32, 32, 2047), (8192, 64, 8, 3584), (8192, 64, 8, 4095), (256, 2, 1, 1000),
]


@pytest.mark.parametrize("dim,H,KV,pos", QKV_CASES)
def test_qkv_rope(dim, H, KV, pos):
    hs, kv = dim // H, dim // H * KV
    s = 900 + dim + pos
    wq = _normal(dim * dim, s, 1, std=0.02).reshape(dim, dim)
    wk = _normal(kv * dim, s, 2, std=0.02).reshape(kv, dim)
    wv = _normal(kv * dim, s, 3, std=0.02).reshape(kv, dim)
    x = _normal(dim, s, 4)
    g = _normal(dim, s, 5, 1.0, 0.01)
    q, k, v = (dev(np.zeros(m, np.float32)) for m in (dim, kv, kv))
    dx, dg, dq, dk, dv = dev(x), dev(g), dev(wq), dev(wk), dev(wv)
    ld.ld_op_qkv_rope(dx.data_ptr(), dg.data_ptr(), 1e-5, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dim, H, KV,
                      pos, 10000.0, q.data_ptr(), k.data_ptr(), v.data_ptr())
    xp = oracle.rmsnorm(x, g, 1e-5)
    q0, k0, v0 = oracle.matvec(wq, xp), oracle.matvec(wk, xp), oracle.matvec(wv, xp)
    qr, kr = oracle.rope(q0, H, hs, pos), oracle.rope(k0, KV, hs, pos)
    # a rotation mixes the two bounds of a pair; the table's cos/sin are rounded once
    for got, base, rot, w in ((host(q), q0, qr, wq), (host(k), k0, kr, wk)):
        e = gemv_bound(w, xp, base)
        pair = np.maximum(e[0::2], e[1::2]).repeat(2) * 2
        mag = np.hypot(base[0::2].astype(np.float64), base[1::2]).repeat(2)
        assert np.all(np.abs(got - rot) <= pair + 4 * U32 * mag + 1e-30)
    assert np.all(np.abs(host(v) - v0) <= gemv_bound(wv, xp, v0))


QKV_ATT_CASES = [  # (dim, n_heads, n_kv_heads, pos): the fused shapes of the workloads, and every
    # head size and group width the fused kernel covers, at position 0 (no cached key), a few keys, and
    # contexts of several key rounds of the block
    (64, 4, 4, 0), (64, 4, 4, 1), (64, 4, 4, 63), (288, 6, 6, 0), (288, 6, 6, 100), (288, 6, 6, 255),
    (288, 6, 4, 0), (288, 6, 4, 17), (288, 6, 4, 511), (4096, 32, 32, 0), (4096, 32, 32, 1), (4096, 32, 32, 63),
    (4096, 32, 32, 200), (128, 4, 2, 9), (256, 4, 4, 30), (512, 8, 4, 40), (1024, 8, 8, 70), (96, 6, 3, 5),
    (2048, 16, 16, 130),
]


@pytest.mark.parametrize("dim,H,KV,pos", QKV_ATT_CASES)
def test_qkv_attention(dim, H, KV, pos):
    """The fused q/k/v + attention launch against the oracle's q/k/v, RoPE and
    attention (steps 2a-2e), with rows above pos poisoned and row pos poisoned
    before the call (the kernel must write it, and take the current key and
    value from its own hand-off).  Bound: the attention of exact inputs (as in
    test_attention) plus the effect of the q/k/v products' rounding on the
    scores, taken from the worst pair error seen over the key rows."""
    hs, kv = dim // H, dim // H * KV
    s = 7100 + dim + 3 * pos + KV
    wq = _normal(dim * dim, s, 1, std=0.02).reshape(dim, dim)
    wk = _normal(kv * dim, s, 2, std=0.02).reshape(kv, dim)
    wv = _normal(kv * dim, s, 3, std=0.02).reshape(kv, dim)
    x = _normal(dim, s, 4)
    g = _normal(dim, s, 5, 1.0, 0.01)
    rows = pos + 3
    kc = _normal(rows * kv, s, 6).reshape(rows, kv)
    vc = _normal(rows * kv, s, 7).reshape(rows, kv)
    kc[pos:] = np.nan
    vc[pos:] = np.nan
    out = dev(np.full(dim, np.nan, np.float32))
    dx, dg, dwq, dwk, dwv, dk, dv = dev(x), dev(g), dev(wq), dev(wk), dev(wv), dev(kc), dev(vc)
    ld.ld_op_qkv_attention(dx.data_ptr(), dg.data_ptr(), 1e-5, dwq.data_ptr(), dwk.data_ptr(), dwv.data_ptr(), dim, H,
                           KV, pos, 10000.0, dk.data_ptr(), dv.data_ptr(), out.data_ptr())
    xp = oracle.rmsnorm(x, g, 1e-5)
    q0, k0, v = oracle.matvec(wq, xp), oracle.matvec(wk, xp), oracle.matvec(wv, xp)
    q, k = oracle.rope(q0, H, hs, pos), oracle.rope(k0, KV, hs, pos)

    def rotated_bound(w, base):  # as in test_qkv_rope: a rotation mixes the bounds of a pair
        e = gemv_bound(w, xp, base)
        mag = np.hypot(base[0::2].astype(np.float64), base[1::2]).repeat(2)
        return np.maximum(e[0::2], e[1::2]).repeat(2) * 2 + 4 * U32 * mag + 1e-30

    kc_got, vc_got = host(dk), host(dv)
    # row pos of the caches: the rotated k and the v of this position
    kbound = rotated_bound(wk, k0)
    assert np.all(np.abs(kc_got[pos] - k) <= kbound)
    assert np.all(np.abs(vc_got[pos] - v) <= gemv_bound(wv, xp, v))
    assert np.all(np.isnan(kc_got[pos + 1:])) and np.all(np.isnan(vc_got[pos + 1:]))
    kc[pos], vc[pos] = k, v
    ref = oracle.attention(q, kc[: pos + 1], vc[: pos + 1], H, KV, hs, pos)
    got = host(out)
    assert np.all(np.isfinite(got))
    # scores move by at most |dq|.|k| + |q|.|dk| (scaled); softmax weights by a
    # factor within exp(+-2 max shift)
    qb = rotated_bound(wq, q0)
    kk = np.abs(kc[: pos + 1].astype(np.float64))
    shift = 0.0
    for h in range(H):
        gk = h * KV // H
        sl, kl = slice(h * hs, (h + 1) * hs), slice(gk * hs, (gk + 1) * hs)
        ds = kk[:, kl] @ qb[sl] + np.abs(q[sl]) @ kbound[kl]
        shift = max(shift, float(np.max(ds)) / np.sqrt(hs))
    vmax = float(np.max(np.abs(vc[: pos + 1])))
    bound = 2e-5 * vmax + 2 * np.expm1(2 * shift) * vmax + float(np.max(gemv_bound(wv, xp, v)))
    assert np.max(np.abs(got - ref)) <= bound, (float(np.max(np.abs(got - ref))), bound)


def test_qkv_attention_matches_the_separate_kernels():
    """Fused and separate launches compute the same q/k/v rows and attention:
    the cache rows agree bit for bit, the attention to rounding."""
    dim, H, KV, pos = 288, 6, 4, 40
    hs, kv = dim // H, dim // H * KV
    s = 7300
    wq = _normal(dim * dim, s, 1, std=0.02).reshape(dim, dim)
    wk = _normal(kv * dim, s, 2, std=0.02).reshape(kv, dim)
    wv = _normal(kv * dim, s, 3, std=0.02).reshape(kv, dim)
    x = _normal(dim, s, 4)
    g = _normal(dim, s, 5, 1.0, 0.01)
    kc = _normal((pos + 1) * kv, s, 6).reshape(pos + 1, kv)
    vc = _normal((pos + 1) * kv, s, 7).reshape(pos + 1, kv)
    dx, dg, dwq, dwk, dwv = dev(x), dev(g), dev(wq), dev(wk), dev(wv)
    dk1, dv1, out1 = dev(kc), dev(vc), dev(np.zeros(dim, np.float32))
    ld.ld_op_qkv_attention(dx.data_ptr(), dg.data_ptr(), 1e-5, dwq.data_ptr(), dwk.data_ptr(), dwv.data_ptr(), dim, H,
                           KV, pos, 10000.0, dk1.data_ptr(), dv1.data_ptr(), out1.data_ptr())
    q, k, v = (dev(np.zeros(m, np.float32)) for m in (dim, kv, kv))
    ld.ld_op_qkv_rope(dx.data_ptr(), dg.data_ptr(), 1e-5, dwq.data_ptr(), dwk.data_ptr(), dwv.data_ptr(), dim, H, KV,
                      pos, 10000.0, q.data_ptr(), k.data_ptr(), v.data_ptr())
    kc[pos], vc[pos] = host(k), host(v)
    assert np.array_equal(host(dk1), kc) and np.array_equal(host(dv1), vc)
    dk2, dv2, out2 = dev(kc), dev(vc), dev(np.zeros(dim, np.float32))
    ld.ld_op_attention(q.data_ptr(), dk2.data_ptr(), dv2.data_ptr(), H, KV, hs, pos, out2.data_ptr())
    assert np.max(np.abs(host(out1) - host(out2))) <= 2e-6 * np.max(np.abs(vc))


def test_qkv_attention_unsupported_shapes():
    x = dev(np.zeros(8192, np.float32))
    p = x.data_ptr()
    for dim, H, KV in ((8192, 64, 8), (240, 3, 3), (512, 16, 2)):  # dim > 4096; head size 80; 8 heads per kv head
        with pytest.raises(ld.LdError) as e:
            ld.ld_op_qkv_attention(p, p, 1e-5, p, p, p, dim, H, KV, 0, 10000.0, p, p, p)
        assert e.value.status == ld.LD_E_UNSUPPORTED


ATTN_CASES = [  # (n_heads, n_kv_heads, head_size, pos)
    (4, 4, 16, 0), (4, 4, 16, 1), (4, 4, 16, 63), (6, 6, 48, 64), (6, 6, 48, 255), (6, 4, 48, 0), (6, 4, 48, 65),
    (6, 4, 48, 511), (32, 32, 128, 0), (32, 32, 128, 31), (32, 32, 128, 32), (32, 32, 128, 33),
    (32, 32, 128, 511), (32, 32, 128, 2047), (64, 8, 128, 0), (64, 8, 128, 3583), (64, 8, 128, 4095),
    (8, 1, 64, 700), (3, 2, 32, 5), (4, 2, 256, 100), (2, 2, 80, 70), (4, 2, 96, 129),
    # split partials merged by the last block of each kv group: 256 and 512
    # float4 outputs per group (one and two passes of the block), four splits
    (8, 2, 256, 90), (16, 2, 256, 70), (64, 8, 128, 200),
    # the register kernel at every head size and group width, with several
    # splits merged by the last block (hs 48, 16, 32, 96, 80, 64) or by the
    # merge kernel (eight heads per kv head, many splits), ragged in every tile
    (6, 6, 48, 1500), (4, 4, 16, 3000), (3, 2, 32, 2500), (4, 1, 96, 1000), (2, 1, 80, 300),
    (16, 2, 64, 777), (32, 4, 128, 1234), (6, 4, 48, 2047), (32, 32, 128, 255), (32, 32, 128, 256),
    (32, 32, 128, 1025),
]


@pytest.mark.parametrize("H,KV,hs,pos", ATTN_CASES)
def test_attention(H, KV, hs, pos):
    kv = KV * hs
    s = 4000 + H * 31 + pos
    q = _normal(H * hs, s, 1)
    kc = _normal((pos + 1) * kv, s, 2).reshape(pos + 1, kv)
    vc = _normal((pos + 1) * kv, s, 3).reshape(pos + 1, kv)
    out = dev(np.zeros(H * hs, np.float32))
    dq, dk, dv = dev(q), dev(kc), dev(vc)
    ld.ld_op_attention(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), H, KV, hs, pos, out.data_ptr())
    ref = oracle.attention(q, kc, vc, H, KV, hs, pos)
    got = host(out)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref)) <= 2e-5 * np.max(np.abs(vc))


def test_attention_never_reads_rows_after_pos():
    H, KV, hs, pos = 8, 2, 128, 77
    kv = KV * hs
    q = _normal(H * hs, 5, 1)
    kc = _normal(200 * kv, 5, 2).reshape(200, kv)
    vc = _normal(200 * kv, 5, 3).reshape(200, kv)
    a = dev(np.zeros(H * hs, np.float32))
    dq, dk, dv = dev(q), dev(kc), dev(vc)
    ld.ld_op_attention(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), H, KV, hs, pos, a.data_ptr())
    kc[pos + 1:] = np.nan
    vc[pos + 1:] = 1e30
    b = dev(np.zeros(H * hs, np.float32))
    dk2, dv2 = dev(kc), dev(vc)
    ld.ld_op_attention(dq.data_ptr(), dk2.data_ptr(), dv2.data_ptr(), H, KV, hs, pos, b.data_ptr())
    assert np.array_equal(host(a), host(b))


@pytest.mark.parametrize("n", [1, 2, 255, 256, 257, 32000, 100_003])
def test_argmax_matches_oracle(n):
    v = _normal(n, 60 + n, 1)
    dv = dev(v)
    assert ld.ld_op_argmax(dv.data_ptr(), n) == oracle.argmax(v)


def test_argmax_ties_take_the_lowest_index():
    v = np.zeros(32000, np.float32)
    v[[31999, 7, 20000, 12345]] = 3.0
    dv = dev(v)
    assert ld.ld_op_argmax(dv.data_ptr(), v.size) == 7 == oracle.argmax(v)
    dz = dev(np.zeros(1000, np.float32))
    assert ld.ld_op_argmax(dz.data_ptr(), 1000) == 0
    v = np.full(5000, -np.inf, np.float32)
    v[4999] = -1e38
    dv = dev(v)
    assert ld.ld_op_argmax(dv.data_ptr(), v.size) == 4999


def test_op_argument_errors():
    with pytest.raises(ld.LdError) as e:
        ld.ld_op_rmsnorm_gemv(0, 0, 1e-5, 0, 4, 4, 0)
    assert e.value.status == ld.LD_E_NULL
    x = dev(np.zeros(8, np.float32))
    with pytest.raises(ld.LdError) as e:
        ld.ld_op_rmsnorm_gemv(x.data_ptr(), 0, 1e-5, x.data_ptr(), 2, 6, x.data_ptr())
    assert e.value.status == ld.LD_E_CONFIG
    with pytest.raises(ld.LdError) as e:
        ld.ld_op_rmsnorm_gemv(x.data_ptr() + 4, 0, 1e-5, x.data_ptr(), 1, 4, x.data_ptr())
    assert e.value.status == ld.LD_E_ALIGN
    with pytest.raises(ld.LdError) as e:
        ld.ld_op_attention(x.data_ptr(), x.data_ptr(), x.data_ptr(), 1, 1, 24, 0, x.data_ptr())
    assert e.value.status == ld.LD_E_UNSUPPORTED


@pytest.mark.parametrize("n4", [1, 7, 2048, 2049, 100_003, 2_000_000])
def test_stream_read_sums_every_share(n4):
    # small integers: every partial sum is exact in fp32, in any order
    import torch
    rng = np.random.default_rng(n4)
    v = rng.integers(-2, 3, 4 * n4).astype(np.float32)
    dv = dev(v)
    sums = torch.full((ld.LD_STREAM_READ_BLOCKS,), float("nan"), dtype=torch.float32, device="cuda")
    ld.ld_op_stream_read(dv.data_ptr(), 16 * n4, sums.data_ptr())
    torch.cuda.synchronize()
    got = host(sums).astype(np.float64)
    per = -(-n4 // ld.LD_STREAM_READ_BLOCKS)
    want = np.zeros(ld.LD_STREAM_READ_BLOCKS)
    for b in range(ld.LD_STREAM_READ_BLOCKS):
        lo, hi = min(n4, b * per), min(n4, (b + 1) * per)
        want[b] = v[4 * lo:4 * hi].astype(np.float64).sum()
    assert np.array_equal(got, want)
