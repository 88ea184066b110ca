"""Pins of the CPU oracle to things other than itself.

Each test checks an oracle routine against a closed form, an invariant of the
mathematics, a brute-force computation with a library routine, or a special
case that reduces to a textbook definition -- never against a retyped copy of
the oracle's own formula.  Together they are chosen so that a plausible slip
(a dropped term, a wrong sign, index or pairing, a transposed operand, eps in
the wrong place, a wrong head-to-group map) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from persistent_resident_execution_amd import synth


# ----------------------------------------------------------------- codecs

def test_bf16_decode_known_values(oracle_lib):
    o = oracle_lib
    bits = [0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x7F80, 0x0001, 0x3F81]
    want = [1.0, -1.0, 2.0, 0.0, -0.0, math.inf, 2.0 ** -133, 1.0 + 2.0 ** -7]
    assert list(o.bf16_to_f64(bits)) == want


def test_bf16_round_to_nearest_even(oracle_lib):
    o = oracle_lib
    as_f = lambda u: np.array([u], dtype=np.uint32).view(np.float32)[0]  # noqa: E731
    # exact halfway cases go to the even neighbour
    assert o.f32_to_bf16([as_f(0x3F808000)])[0] == 0x3F80
    assert o.f32_to_bf16([as_f(0x3F818000)])[0] == 0x3F82
    # just above / below halfway
    assert o.f32_to_bf16([as_f(0x3F808001)])[0] == 0x3F81
    assert o.f32_to_bf16([as_f(0x3F807FFF)])[0] == 0x3F80
    # overflow past the largest bf16 rounds to infinity; the largest stays
    assert o.f32_to_bf16([as_f(0x7F7FFFFF)])[0] == 0x7F80
    assert o.f32_to_bf16([as_f(0x7F7F0000)])[0] == 0x7F7F
    # subnormal and negative values
    assert o.f32_to_bf16([as_f(0x00018000)])[0] == 0x0002
    assert o.f32_to_bf16([-1.0])[0] == 0xBF80
    # NaN stays NaN
    r = o.f32_to_bf16([float("nan")])[0]
    assert (r & 0x7F80) == 0x7F80 and (r & 0x7F) != 0


def test_bf16_matches_torch_cast(oracle_lib):
    g = torch.Generator().manual_seed(7)
    x = torch.randn(4000, generator=g) * torch.exp(torch.randn(4000, generator=g) * 8)
    ours = oracle_lib.f32_to_bf16(x.numpy())
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_fp8_e4m3_all_codes(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_lib.fp8_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


# ----------------------------------------------------------------- norms

@pytest.mark.parametrize("c", [0.01, 1.0, -3.5])
def test_rmsnorm_constant_vector(oracle_lib, c):
    n, eps = 64, 1e-5
    g = synth.to_bits(torch.ones(n, dtype=torch.bfloat16))
    out = oracle_lib.rmsnorm(np.full(n, c), g, eps)
    np.testing.assert_allclose(out, c / math.sqrt(c * c + eps), rtol=1e-14)


def test_rmsnorm_zero_vector_and_gains(oracle_lib):
    n = 32
    g = torch.linspace(-2, 2, n).to(torch.bfloat16)
    out = oracle_lib.rmsnorm(np.zeros(n), synth.to_bits(g), 1e-5)
    assert np.all(out == 0.0)
    ones = synth.to_bits(torch.ones(n, dtype=torch.bfloat16))
    x = np.random.default_rng(0).normal(size=n)
    base = oracle_lib.rmsnorm(x, ones, 1e-5)
    scaled = oracle_lib.rmsnorm(x, synth.to_bits(g), 1e-5)
    np.testing.assert_allclose(scaled, base * g.double().numpy(), rtol=1e-14, atol=1e-300)
    # against the library's definition
    ref = F.rms_norm(torch.from_numpy(x)[None], (n,), weight=g.double(), eps=1e-5)[0].numpy()
    np.testing.assert_allclose(scaled, ref, rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------- GEMV

def test_gemv_bf16_bruteforce(oracle_lib):
    g = torch.Generator().manual_seed(1)
    for m, k in [(1, 1), (3, 5), (17, 64), (40, 129)]:
        W = torch.randn(m, k, generator=g).to(torch.bfloat16)
        x = np.random.default_rng(m * 1000 + k).normal(size=k)
        y = oracle_lib.gemv_bf16(synth.to_bits(W), x)
        ref = W.double().numpy() @ x
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_gemv_bf16_one_hot_rows_select_input(oracle_lib):
    k = 50
    W = torch.zeros(k, k, dtype=torch.bfloat16)
    perm = torch.randperm(k, generator=torch.Generator().manual_seed(3))
    W[torch.arange(k), perm] = 1.0
    x = np.random.default_rng(5).normal(size=k)
    y = oracle_lib.gemv_bf16(synth.to_bits(W), x)
    assert np.array_equal(y, x[perm.numpy()])  # exact: no transposition


def test_gemv_fp8_bruteforce(oracle_lib):
    g = torch.Generator().manual_seed(2)
    for m, k in [(5, 7), (130, 200), (256, 384)]:
        w = torch.randn(m, k, generator=g) * 0.02
        q, s = synth.quantize_fp8_blocks(w)
        x = np.random.default_rng(k).normal(size=k)
        y = oracle_lib.gemv_fp8(synth.to_bits(q), synth.to_bits(s), x)
        deq = q.to(torch.float64) * s.double().repeat_interleave(128, 0).repeat_interleave(128, 1)[:m, :k]
        ref = deq.numpy() @ x
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
        # quantisation error is what the e4m3 format allows (3 mantissa bits)
        assert torch.allclose(deq.float(), w, rtol=2 ** -4, atol=float(s.float().max()) * 2 ** -9)


# ----------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity(oracle_lib):
    v = np.random.default_rng(0).normal(size=128)
    assert np.array_equal(oracle_lib.rope(v, 0, 10000.0), v)


def test_rope_rotate_half_pairs_and_direction(oracle_lib):
    # d = 4: pair 0 is (0, 2) with inv_freq 1, pair 1 is (1, 3) with
    # inv_freq theta^(-1/2).  A unit vector on element 0 at position p turns
    # counter-clockwise by p radians into element 2 (not into element 1, as
    # interleaved pairs would).
    p, theta = 3, 10000.0
    out = oracle_lib.rope([1.0, 0, 0, 0], p, theta)
    np.testing.assert_allclose(out, [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    out = oracle_lib.rope([0, 1.0, 0, 0], p, theta)
    a = p * theta ** -0.5
    np.testing.assert_allclose(out, [0, math.cos(a), 0, math.sin(a)], atol=1e-15)
    # the second element of a pair turns the same way: (0, 1) -> (-sin, cos)
    out = oracle_lib.rope([0, 0, 1.0, 0], p, theta)
    np.testing.assert_allclose(out, [-math.sin(p), 0, math.cos(p), 0], atol=1e-15)


def test_rope_preserves_pair_norms_and_relative_positions(oracle_lib):
    rng = np.random.default_rng(1)
    d = 64
    q, k = rng.normal(size=d), rng.normal(size=d)
    for p in (1, 17, 1000):
        r = oracle_lib.rope(q, p, 10000.0)
        np.testing.assert_allclose(r[:32] ** 2 + r[32:] ** 2, q[:32] ** 2 + q[32:] ** 2, rtol=1e-12)
    # <R_p q, R_p' k> depends on p - p' only
    base = np.dot(oracle_lib.rope(q, 9, 10000.0), oracle_lib.rope(k, 4, 10000.0))
    for s in (1, 50, 700):
        sh = np.dot(oracle_lib.rope(q, 9 + s, 10000.0), oracle_lib.rope(k, 4 + s, 10000.0))
        assert abs(sh - base) < 1e-10


# ----------------------------------------------------------------- softmax / attention

def test_softmax_properties(oracle_lib):
    rng = np.random.default_rng(2)
    for n in (1, 2, 7, 1000):
        s = rng.normal(size=n) * 10
        p = oracle_lib.softmax(s)
        assert abs(p.sum() - 1.0) < 1e-12 and np.all(p >= 0)
        np.testing.assert_allclose(oracle_lib.softmax(s + 123.0), p, rtol=1e-12)
    np.testing.assert_allclose(oracle_lib.softmax([0.0, math.log(2.0)]), [1 / 3, 2 / 3], rtol=1e-15)
    p = oracle_lib.softmax([1000.0, 0.0])
    assert p[0] == 1.0 and p[1] < 1e-300


def _bf(a):
    return synth.to_bits(torch.as_tensor(np.asarray(a), dtype=torch.float32).to(torch.bfloat16))


def test_attention_single_key_returns_v(oracle_lib):
    rng = np.random.default_rng(3)
    d = 128
    K, V = _bf(rng.normal(size=(1, d))), _bf(rng.normal(size=(1, d)))
    o = oracle_lib.attend(rng.normal(size=d) * 50, K, V)
    assert np.array_equal(o, oracle_lib.bf16_to_f64(V))


def test_attention_identical_keys_mean_and_dominant_key(oracle_lib):
    rng = np.random.default_rng(4)
    d, n = 64, 9
    krow = rng.normal(size=d)
    K = _bf(np.tile(krow, (n, 1)))
    V = _bf(rng.normal(size=(n, d)))
    Vd = oracle_lib.bf16_to_f64(V).reshape(n, d)
    o = oracle_lib.attend(rng.normal(size=d), K, V)
    np.testing.assert_allclose(o, Vd.mean(0), rtol=1e-12, atol=1e-14)
    # one key aligned with a large query dominates
    K2 = np.zeros((n, d))
    K2[5, 0] = 1.0
    o = oracle_lib.attend(np.eye(d)[0] * 4000.0, _bf(K2), V)
    np.testing.assert_allclose(o, Vd[5], rtol=1e-12)


def test_attention_scale_is_inverse_sqrt_d(oracle_lib):
    # two keys whose scores differ by delta: weight of the first = sigmoid(delta / sqrt(d))
    d = 64
    K = np.zeros((2, d))
    K[0, 0] = 1.0
    V = np.zeros((2, d))
    V[0, 0] = 1.0
    q = np.zeros(d)
    q[0] = 3.0
    o = oracle_lib.attend(q, _bf(K), _bf(V))
    assert abs(o[0] - 1.0 / (1.0 + math.exp(-3.0 / 8.0))) < 1e-14


def test_attention_matches_library_sdpa(oracle_lib):
    rng = np.random.default_rng(5)
    n, d = 37, 64
    K, V = _bf(rng.normal(size=(n, d))), _bf(rng.normal(size=(n, d)))
    q = rng.normal(size=d)
    o = oracle_lib.attend(q, K, V)
    Kd = torch.from_numpy(oracle_lib.bf16_to_f64(K).reshape(n, d))
    Vd = torch.from_numpy(oracle_lib.bf16_to_f64(V).reshape(n, d))
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None], Kd[None], Vd[None])[0, 0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------- argmax / top-k / silu

def test_argmax_ties_and_nan(oracle_lib):
    assert oracle_lib.argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert oracle_lib.argmax([5.0, 5.0]) == 0
    assert oracle_lib.argmax([-1.0]) == 0
    assert oracle_lib.argmax([0.0, float("nan"), 1.0]) == -1
    v = np.random.default_rng(6).normal(size=5000)
    assert oracle_lib.argmax(v) == int(np.argmax(v))


def test_topk_bruteforce_and_ties(oracle_lib):
    rng = np.random.default_rng(7)
    for n, k in [(8, 8), (128, 8), (16, 4)]:
        p = rng.random(n)
        assert list(oracle_lib.topk(p, k)) == list(np.argsort(-p, kind="stable")[:k])
    p = np.array([0.1, 0.3, 0.3, 0.2, 0.3])
    assert list(oracle_lib.topk(p, 3)) == [1, 2, 4]


def test_silu_closed_forms(oracle_lib):
    assert oracle_lib.silu(0.0) == 0.0
    assert abs(oracle_lib.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(oracle_lib.silu(40.0) - 40.0) < 1e-14
    assert abs(oracle_lib.silu(-40.0)) < 1e-15
    for z in (-3.0, -0.5, 0.25, 2.0):
        assert abs(oracle_lib.silu(z) - float(F.silu(torch.tensor(z, dtype=torch.float64)))) < 1e-15


# ----------------------------------------------------------------- fp8 K/V cache

def _torch_fp8_sat(x):
    """torch's float8_e4m3fn cast (round to nearest even) after clamping to
    the largest finite magnitude, as bit patterns."""
    t = torch.as_tensor(np.asarray(x, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_encode_matches_library_saturating_cast(oracle_lib):
    g = torch.Generator().manual_seed(11)
    x = (torch.randn(6000, generator=g) * torch.exp2(torch.randint(-14, 12, (6000,), generator=g).float()))
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle_lib.fp8_to_f64(codes)
    finite = np.sort(np.unique(vals[~np.isnan(vals)]))
    mids = (finite[1:] + finite[:-1]) / 2  # exact halfway points: ties to the even code
    probe = np.concatenate([x.numpy(), finite, mids, mids * (1 + 2 ** -20), mids * (1 - 2 ** -20),
                            [447.0, 448.0, 455.0, 464.0, 479.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -10]])
    probe = np.concatenate([probe, -probe]).astype(np.float32)
    ours = oracle_lib.f32_to_fp8(probe)
    assert np.array_equal(ours, _torch_fp8_sat(probe))


def test_fp8_encode_round_trips_every_finite_code(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle_lib.fp8_to_f64(codes)
    keep = ~np.isnan(vals) & (codes != 0x80)  # (-0 encodes back as 0x80 too: checked on its own)
    assert np.array_equal(oracle_lib.f32_to_fp8(vals[keep]), codes[keep])
    assert oracle_lib.f32_to_fp8([-0.0])[0] == 0x80
    assert oracle_lib.f32_to_fp8([float("nan")])[0] == 0x7F


def test_fp8_row_quantizer(oracle_lib):
    g = torch.Generator().manual_seed(12)
    for n, mag in ((128, 1.0), (64, 1e-3), (128, 300.0)):
        x = (torch.randn(n, generator=g) * mag).numpy().astype(np.float32)
        codes, sc = oracle_lib.quantize_row_fp8(x)
        amax = np.float32(np.abs(x).max())
        assert sc == np.float32(amax / np.float32(448.0))  # the fp32 quotient
        i = int(np.argmax(np.abs(x)))
        assert codes[i] in (0x7E, 0xFE)  # the largest element lands on +-448
        deq = oracle_lib.fp8_to_f64(codes) * sc
        # within half a step of the 3-bit mantissa (or of the subnormal step)
        bound = np.maximum(np.abs(x) * 2.0 ** -4, sc * 2.0 ** -10)
        assert np.all(np.abs(deq - x) <= bound * (1 + 1e-6))
    codes, sc = oracle_lib.quantize_row_fp8(np.zeros(16, np.float32))
    assert sc == 1.0 and not codes.any()


def test_fp8_attention_matches_dequantized_bf16_free_path(oracle_lib):
    """Attention over fp8 rows equals the plain attention over the rows'
    dequantized values (computed here with the library)."""
    g = torch.Generator().manual_seed(13)
    n, d = 37, 64
    Kc = torch.randint(0, 256, (n, d), generator=g, dtype=torch.int64).numpy().astype(np.uint8)
    Vc = torch.randint(0, 256, (n, d), generator=g, dtype=torch.int64).numpy().astype(np.uint8)
    Kc[(Kc & 0x7F) == 0x7F] = 0  # no NaN codes
    Vc[(Vc & 0x7F) == 0x7F] = 0
    Ks = (torch.rand(n, generator=g) * 0.01 + 1e-3).numpy().astype(np.float32)
    Vs = (torch.rand(n, generator=g) * 0.01 + 1e-3).numpy().astype(np.float32)
    q = torch.randn(d, generator=g, dtype=torch.float64).numpy() * 40
    o = oracle_lib.attend_fp8(q, Kc, Ks, Vc, Vs)
    K = torch.from_numpy(Kc).view(torch.float8_e4m3fn).double() * torch.from_numpy(Ks).double()[:, None]
    V = torch.from_numpy(Vc).view(torch.float8_e4m3fn).double() * torch.from_numpy(Vs).double()[:, None]
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None, None], K[None, None], V[None, None])
    np.testing.assert_allclose(o, ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-14)
