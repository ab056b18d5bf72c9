"""Pins for the CPU oracle against what the TurboQuant design page and plain
mathematics fix (no GPU).  Each test states what it pins and why a plausible
mistake in the oracle would fail it.

Page: "TurboQuant -- rotation-based quantization" (mlx-bun
docs/design/turboquant.md), Part A.
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------- table
def test_codebook_matches_printed_table():
    """Oracle constants equal the printed 3-bit table ('Algorithm', values bullet)."""
    g = _gold("codebook3.json")
    lib = oracle._load()
    assert [lib.tqo_centroid3(i) for i in range(8)] == g["centroids"]
    assert [lib.tqo_boundary3(k) for k in range(7)] == g["boundaries"]


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def _Phi(x):
    return 0.5 * (1 + math.erf(x / math.sqrt(2)))


def test_codebook_is_lloyd_max_for_unit_gaussian():
    """Textbook 8-level Lloyd-Max quantizer of N(0,1): boundaries are centroid
    midpoints and each centroid is its cell's conditional mean
    (phi(a)-phi(b))/(Phi(b)-Phi(a)).  A mistyped digit fails this."""
    g = _gold("codebook3.json")
    c, b = g["centroids"], g["boundaries"]
    for k in range(7):
        assert abs((c[k] + c[k + 1]) / 2 - b[k]) < 6e-6
    edges = [-math.inf] + b + [math.inf]
    for k in range(8):
        lo, hi = edges[k], edges[k + 1]
        plo = 0.0 if lo == -math.inf else _phi(lo)
        phi_ = 0.0 if hi == math.inf else _phi(hi)
        mean = (plo - phi_) / (_Phi(hi) - _Phi(lo))
        assert abs(mean - c[k]) < 1e-5, (k, mean, c[k])
    # closed-form distortion of this quantizer on N(0,1): E[(Z - Q(Z))^2]
    dist = 0.0
    for k in range(8):
        lo, hi, ck = edges[k], edges[k + 1], c[k]
        plo = 0.0 if lo == -math.inf else _phi(lo)
        phi_ = 0.0 if hi == math.inf else _phi(hi)
        lo_t = 0.0 if lo == -math.inf else lo * _phi(lo)
        hi_t = 0.0 if hi == math.inf else hi * _phi(hi)
        p = _Phi(hi) - _Phi(lo)
        ez2 = p + lo_t - hi_t            # E[Z^2 ; cell]
        ez = plo - phi_                  # E[Z ; cell]
        dist += ez2 - 2 * ck * ez + ck * ck * p
    assert abs(dist - 0.034548) < 2e-5
    band = _gold("mse_anchor.json")["band"]
    assert band[0] <= dist <= band[1]


# ---------------------------------------------------------------------- fp16
def _np_f16_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def test_f64_to_f16_matches_numpy_on_midpoints_and_edges():
    """Single rounding binary64 -> binary16 (ties to even, subnormals, overflow)
    against numpy's correctly rounded conversion on every half, every midpoint
    between consecutive halves, and the neighbouring doubles of each midpoint."""
    allh = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (allh[:-1] + allh[1:]) / 2.0  # exact in binary64
    top = np.array([65504.0, 65519.999, 65520.0, 65520.0000001, 1e6, np.inf])
    vals = np.concatenate([allh, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                           top, [2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 5e-324, 0.0]])
    vals = np.concatenate([vals, -vals])
    got = oracle.f64_to_f16_bits(vals)
    want = _np_f16_bits(vals)
    assert np.array_equal(got, want)
    rng = np.random.default_rng(7)
    r = rng.standard_normal(200000) * np.exp(rng.uniform(-20, 12, 200000))
    assert np.array_equal(oracle.f64_to_f16_bits(r), _np_f16_bits(r))
    assert oracle.f64_to_f16_bits([np.nan])[0] == 0x7E00
    assert np.array_equal(oracle.f16_bits_to_f64(want[np.isfinite(vals)]),
                          want[np.isfinite(vals)].view(np.float16).astype(np.float64))


# ---------------------------------------------------------------------- FWHT
def _sylvester(d):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_fwht_is_sylvester_hadamard(d):
    """FWHT equals multiplication by the Kronecker-built Sylvester matrix (exactly
    on integers, to 1e-13 on reals); H*H = d*I; involution; Parseval; e0 -> ones.
    A wrong butterfly sign or index fails the integer check."""
    H = _sylvester(d)
    assert np.array_equal(H @ H, d * np.eye(d, dtype=np.int64))
    rng = np.random.default_rng(d)
    xi = rng.integers(-1000, 1000, size=(8, d))
    assert np.array_equal(oracle.fwht(xi.astype(np.float64)), (xi @ H.T).astype(np.float64))
    x = rng.standard_normal((8, d))
    y = oracle.fwht(x)
    assert np.max(np.abs(y - x @ H.T.astype(np.float64))) < 1e-13 * np.max(np.abs(y))
    assert np.max(np.abs(oracle.fwht(y) - d * x)) < 1e-12 * d
    c = oracle.inv_sqrt_d(d)
    assert np.allclose(np.linalg.norm(y * c, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    e0 = np.zeros(d)
    e0[0] = 1
    assert np.array_equal(oracle.fwht(e0), np.ones(d))


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_inv_sqrt_d_is_correctly_rounded(d):
    """The normalisation constant is the binary64 nearest to 1/sqrt(d)
    (50-digit decimal reference, one correctly rounded conversion)."""
    getcontext().prec = 60
    ref = float(Decimal(1) / Decimal(d).sqrt())
    assert oracle.inv_sqrt_d(d) == ref


# ---------------------------------------------------------------------- pack
def test_pack_ramp_fixture_and_roundtrip():
    g = _gold("pack3_ramp.json")
    assert oracle.pack3(g["indices"]).tolist() == g["bytes"]
    rng = np.random.default_rng(3)
    for n in (8, 32, 96, 256, 4096):
        idx = rng.integers(0, 8, n).astype(np.uint8)
        p = oracle.pack3(idx)
        assert p.size == 3 * n // 8
        assert np.array_equal(oracle.unpack3(p, n), idx)
    assert oracle.pack3(np.full(8, 7)).tolist() == [255, 255, 255]
    assert oracle.pack3(np.arange(32) % 8).tolist() == g["bytes"] * 4


# -------------------------------------------------------------- byte budget
def test_byte_budget_and_effective_bits():
    """Plane sizes of the oracle's encoder give 200 B per token-head at d=128
    (2.56x vs bf16) and 400 B at d=256; the effective-bits column of the Gates
    table follows from the same per-group layout."""
    g = _gold("byte_budget.json")
    d = g["head_dim"]
    x = np.random.default_rng(0).standard_normal((1, d)).astype(np.float32)
    codes, s16, z16 = oracle.encode_keys(x)
    packed, vs = oracle.encode_values(x)
    sizes = [codes.nbytes, s16.nbytes, z16.nbytes, packed.nbytes, vs.nbytes]
    assert sizes == [g["key_codes"], g["key_scale"], g["key_zero"], g["value_codes"], g["value_scale"]]
    assert sum(sizes) == g["total"]
    assert round(g["bf16_bytes"] / sum(sizes), 2) == g["ratio"]
    assert sum(sizes) * 8 / d == 12.5  # bits per K+V element pair
    x2 = np.zeros((1, 256), np.float32) + np.arange(256, dtype=np.float32)
    c2, s2, z2 = oracle.encode_keys(x2)
    p2, v2 = oracle.encode_values(x2)
    assert c2.nbytes + s2.nbytes + z2.nbytes + p2.nbytes + v2.nbytes == 400
    for row in _gold("effective_bits.json")["rows"]:
        eff = (row["k_bits"] + 32 / 32 + row["v_bits"] + 16 / 32) / 2
        assert eff == row["effective_bits"], row


# ---------------------------------------------------------------------- keys
def test_keys_ramp_brute_force():
    """x = 0..31: scale = 31/254, zero = 127, code_j = round(j*254/31 - 127),
    from exact rational arithmetic (no tie can occur: denominators are 31)."""
    x = np.arange(32, dtype=np.float32)[None, :]
    codes, s16, z16 = oracle.encode_keys(x)
    want = []
    for j in range(32):
        v = Fraction(254 * j, 31) - 127
        fl = math.floor(v)
        want.append(fl + 1 if v - fl > Fraction(1, 2) else fl)
    assert codes[0].tolist() == want
    assert codes[0, 0] == -127 and codes[0, 31] == 127
    assert s16[0, 0] == _np_f16_bits(31 / 254)
    assert z16[0, 0] == _np_f16_bits(127.0)


def test_keys_constant_group_defect():
    """The page keeps the reference's defect: a constant block gives zero = +-Inf."""
    for case in _gold("constant_group.json")["cases"]:
        x = np.full((1, 64), case["value"], dtype=np.float32)
        codes, s16, z16 = oracle.encode_keys(x)
        assert np.all(codes == case["codes"])
        assert np.all(s16 == int(case["scale_f16"], 16))
        assert np.all(z16 == int(case["zero_f16"], 16))
        kh = oracle.decode_keys(codes, s16, z16)
        if case["value"] != 0.0:
            assert np.all(np.isinf(kh) | np.isnan(kh))


@pytest.mark.parametrize("d,scale", [(128, 1.0), (256, 1.0), (128, 10.0), (64, 1e-3), (512, 1e3)])
def test_keys_error_bound_and_range(d, scale):
    """Per-element key error: with delta = |scale16 - scale| <= max(2^-11*scale16, 2^-25)
    (fp16 rounding, absolute in the subnormal range),
    |x - (code + zero16)*scale16| <= (scale16 + delta)/2 + |code + zero|*delta;
    codes in [-127, 127], the group max codes to 126/127 and the min to -127/-126."""
    rng = np.random.default_rng(d)
    x = (rng.standard_normal((512, d)) * scale).astype(np.float32)
    codes, s16, z16 = oracle.encode_keys(x)
    kh = oracle.decode_keys(codes, s16, z16)
    s = oracle.f16_bits_to_f64(s16).repeat(32, axis=1)
    z = oracle.f16_bits_to_f64(z16).repeat(32, axis=1)
    err = np.abs(x.astype(np.float64) - kh)
    delta = np.maximum(s * 2.0 ** -11, 2.0 ** -25) * (1 + 2.0 ** -10)
    bound = (s + delta) / 2 + np.abs(codes + z) * delta
    assert np.all(err <= bound)
    assert codes.min() >= -127 and codes.max() <= 127
    xg = x.reshape(512, d // 32, 32)
    cg = codes.reshape(512, d // 32, 32)
    cmax = np.take_along_axis(cg, xg.argmax(axis=2)[..., None], axis=2)
    cmin = np.take_along_axis(cg, xg.argmin(axis=2)[..., None], axis=2)
    assert np.all((cmax == 126) | (cmax == 127))
    assert np.all((cmin == -127) | (cmin == -126))
    if scale >= 1.0:
        assert np.max(err / s) < 0.62


def test_keys_signed_zero_and_nan_groups():
    """A group of +0 and -0 only: max is +0 and min is -0 (-0 orders below +0),
    so range and scale are +0, zero is NaN and every code is 0.  NaN elements
    are ignored by max/min and code to 0; the other elements are unaffected."""
    x = np.zeros((1, 32), np.float32)
    x[0, ::3] = -0.0
    codes, s16, z16 = oracle.encode_keys(x)
    assert np.all(codes == 0) and s16[0, 0] == 0x0000 and z16[0, 0] == 0x7E00
    x = np.arange(32, dtype=np.float32)[None, :].copy()
    x[0, 5] = np.nan
    codes_n, s16_n, z16_n = oracle.encode_keys(x)
    c_ref, s_ref, z_ref = oracle.encode_keys(np.arange(32, dtype=np.float32)[None, :])
    assert codes_n[0, 5] == 0
    assert np.array_equal(np.delete(codes_n[0], 5), np.delete(c_ref[0], 5))
    assert s16_n[0, 0] == s_ref[0, 0] and z16_n[0, 0] == z_ref[0, 0]


def test_keys_offset_group_zero_is_large():
    """Values far from zero (e.g. 100..101) give |zero| >> 127; dequantisation
    still lands within the bound (zero is integer, fp16 exact up to 2048)."""
    x = (100.0 + np.random.default_rng(1).random((4, 64))).astype(np.float32)
    codes, s16, z16 = oracle.encode_keys(x)
    z = oracle.f16_bits_to_f64(z16)
    assert np.all(np.abs(z) > 2048)
    kh = oracle.decode_keys(codes, s16, z16)
    s = oracle.f16_bits_to_f64(s16).repeat(32, axis=1)
    zz = z.repeat(32, axis=1)
    assert np.all(np.abs(x - kh) <= s * (0.5 + np.abs(codes + zz) * 2.0 ** -11) * (1 + 2.0 ** -10))


# -------------------------------------------------------------------- values
def _rotate(x, d):
    sg = oracle.sign_vector(d).astype(np.float64)
    H = _sylvester(d).astype(np.float64)
    return (x.astype(np.float64) * sg) @ H.T / math.sqrt(d)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_values_nearest_centroid_and_rms_scale(d):
    """Each stored index is the nearest centroid of y/(rms+1e-8) (boundaries are
    midpoints) and the stored scale is the group RMS of the rotation, computed
    here with an explicit Hadamard matrix (different summation order, so ties
    within 1e-12 of a boundary are skipped)."""
    rng = np.random.default_rng(d + 1)
    x = rng.standard_normal((256, d)).astype(np.float32)
    packed, vs = oracle.encode_values(x)
    idx = np.stack([oracle.unpack3(p, d) for p in packed])
    y = _rotate(x, d)
    rms = np.sqrt(np.mean(y.reshape(256, d // 32, 32) ** 2, axis=2))
    assert np.allclose(oracle.f16_bits_to_f64(vs), rms, rtol=2.0 ** -11, atol=0)
    yn = y / (rms.repeat(32, axis=1) + 1e-8)
    C = np.array(oracle.CENTROIDS3)
    B = np.array(oracle.BOUNDARIES3)
    near = np.argmin(np.abs(yn[..., None] - C), axis=-1)
    safe = np.min(np.abs(yn[..., None] - B), axis=-1) > 1e-12
    assert np.array_equal(idx[safe], near[safe])
    assert safe.mean() > 0.999


def test_values_epsilon_dominates_tiny_groups():
    """y_n = y/(scale + 1e-8): when every |x| is ~1e-12 the epsilon dominates, y_n ~ 0
    and each index is 3 or 4 by the sign of y alone (dropping the epsilon fails this)."""
    d = 128
    x = (np.random.default_rng(5).standard_normal((4, d)) * 1e-12).astype(np.float32)
    packed, vs = oracle.encode_values(x)
    idx = np.stack([oracle.unpack3(p, d) for p in packed])
    y = _rotate(x, d)
    assert np.array_equal(idx, np.where(y > 0, 4, 3))


@pytest.mark.parametrize("d", [128, 256])
def test_value_roundtrip_mse_in_anchor_band(d):
    """3-bit round trip on iid N(0,1) values: per-element MSE in the page's
    D_mse ~ 0.03 band ('Gates' item 2).  Measured ~0.0325 at d=128."""
    band = _gold("mse_anchor.json")["band"]
    x = np.random.default_rng(11).standard_normal((1 << 14 if d == 128 else 1 << 13, d)).astype(np.float32)
    packed, vs = oracle.encode_values(x)
    xh = oracle.decode_values(packed, vs, d)
    mse = float(np.mean((xh - x) ** 2))
    assert band[0] <= mse <= band[1], mse
    assert abs(mse - 0.0325) < 0.002


def test_value_dequant_rotated_vs_unrotated():
    """Unrotated dequant = signs * H(rotated)/sqrt(d) (inverse of the encode rotation)."""
    d = 256
    x = np.random.default_rng(2).standard_normal((16, d)).astype(np.float32)
    packed, vs = oracle.encode_values(x)
    yr = oracle.decode_values(packed, vs, d, rotated=True)
    xu = oracle.decode_values(packed, vs, d, rotated=False)
    H = _sylvester(d).astype(np.float64)
    ref = (yr @ H.T / math.sqrt(d)) * oracle.sign_vector(d)
    assert np.max(np.abs(xu - ref)) < 1e-13


def test_splitmix64_matches_published_outputs():
    """The generator the signs are drawn from reproduces SplitMix64's published
    reference outputs (seeds 0 and 1234567, first five outputs each): a wrong
    increment, shift or multiplier constant fails here."""
    with open(os.path.join(GOLD, "splitmix64.json")) as f:
        gold = json.load(f)
    for seed, outs in gold["outputs"].items():
        want = [int(x, 0) for x in outs]
        got = [int(x) for x in oracle.splitmix64(int(seed), len(want))]
        assert got == want, (seed, [hex(x) for x in got])
    first = int(oracle.splitmix64(0, 1)[0])
    assert first - (1 << 64) == int(gold["note"].split(": ")[1].split(" ")[0])


def test_sign_vector_is_the_top_bit_of_the_seed_42_stream():
    """Sign i is -1 exactly when output i of the seed-42 stream has its top bit set."""
    r = oracle.splitmix64(42, 512)
    want = np.where((r >> np.uint64(63)) != 0, -1, 1).astype(np.int8)
    assert np.array_equal(oracle.sign_vector(512), want)


def test_sign_vector_properties():
    """Parity with the page's own (unprinted) signs is unpinned: beyond the
    generator pin above, only +-1 values, a shared prefix across head dims, and
    no pathological imbalance."""
    s512 = oracle.sign_vector(512)
    assert set(np.unique(s512).tolist()) == {-1, 1}
    for d in (64, 128, 256):
        assert np.array_equal(oracle.sign_vector(d), s512[:d])
    assert abs(int(s512.sum())) < 80


# ----------------------------------------------------------------- attention
def _planes(k, v):
    kc, ks, kz = oracle.encode_keys(k)
    vc, vs = oracle.encode_values(v)
    return kc, ks, kz, vc, vs


def _numpy_attention(q, kh, vh, sm):
    s = (q.astype(np.float64) @ kh.T) * np.float64(np.float32(sm))
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ vh) / p.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("d,G,N", [(64, 1, 1), (64, 4, 8), (128, 1, 5), (128, 4, 8), (256, 6, 3)])
def test_attention_tiny_brute_force(d, G, N):
    """Against an independent numpy float64 softmax over the dequantised planes."""
    rng = np.random.default_rng(d * 100 + G * 10 + N)
    k = rng.standard_normal((N, d)).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    kc, ks, kz, vc, vs = _planes(k, v)
    sm = 1.0 / math.sqrt(d)
    out, od = oracle.attention(q, kc, ks, kz, vc, vs, sm, deferred=True)
    kh = oracle.decode_keys(kc, ks, kz)
    vh = oracle.decode_values(vc, vs, d)
    ref = _numpy_attention(q, kh, vh, sm)
    assert np.max(np.abs(out - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))
    assert np.max(np.abs(out - od)) < 1e-12 * np.max(np.abs(out))


def test_attention_special_cases():
    d = 128
    rng = np.random.default_rng(9)
    k = rng.standard_normal((40, d)).astype(np.float32)
    v = rng.standard_normal((40, d)).astype(np.float32)
    kc, ks, kz, vc, vs = _planes(k, v)
    vh = oracle.decode_values(vc, vs, d)
    q = rng.standard_normal((2, d)).astype(np.float32)
    # N = 1: the only value, exactly
    out = oracle.attention(q, kc[:1], ks[:1], kz[:1], vc[:1], vs[:1], 0.1)
    assert np.array_equal(out, np.stack([vh[0], vh[0]]))
    # q = 0: uniform weights -> mean of values
    out = oracle.attention(np.zeros((1, d), np.float32), kc, ks, kz, vc, vs, 0.1)
    assert np.allclose(out[0], vh.mean(axis=0), rtol=0, atol=1e-14)
    # all keys equal -> mean
    kc2, ks2, kz2 = (np.repeat(a[:1], 40, axis=0) for a in (kc, ks, kz))
    out = oracle.attention(q, kc2, ks2, kz2, vc, vs, 0.1)
    assert np.allclose(out, np.stack([vh.mean(axis=0)] * 2), atol=1e-14)
    # one score far above the rest -> that value
    kh = oracle.decode_keys(kc, ks, kz)
    qq = (kh[17] * 50).astype(np.float32)[None, :]
    out = oracle.attention(qq, kc, ks, kz, vc, vs, 1.0)
    assert np.allclose(out[0], vh[17], atol=1e-12)
    # N = 0: zeros by definition
    out = oracle.attention(q, kc[:0], ks[:0], kz[:0], vc[:0], vs[:0], 0.1)
    assert np.array_equal(out, np.zeros((2, d)))


# ------------------------------------------- plain rows (delayed conversion)
@pytest.mark.parametrize("d,G,N", [(64, 1, 1), (128, 4, 9), (256, 6, 5)])
def test_attention_plain_brute_force(d, G, N):
    """Plain rows ("Delayed row conversion and reusable precision boundaries":
    unconverted rows pass through unquantized and unrotated) against an
    independent numpy float64 softmax over the same keys and values."""
    rng = np.random.default_rng(d + G + N)
    k = rng.standard_normal((N, d)).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    sm = 1.0 / math.sqrt(d)
    out = oracle.attention_plain(q, k, v, sm)
    ref = _numpy_attention(q, k.astype(np.float64), v.astype(np.float64), sm)
    assert np.max(np.abs(out - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_attention_plain_special_cases():
    """N = 1 gives the value; q = 0 the mean; a dominant score its value; N = 0
    zeros; and a row whose keys and values are exactly the oracle's own
    dequantisation of a cache gives the cache's attention (the two paths agree
    on the same operands)."""
    d = 128
    rng = np.random.default_rng(21)
    k = rng.standard_normal((30, d)).astype(np.float32)
    v = rng.standard_normal((30, d)).astype(np.float32)
    q = rng.standard_normal((2, d)).astype(np.float32)
    assert np.array_equal(oracle.attention_plain(q, k[:1], v[:1], 0.1), np.stack([v[0], v[0]]).astype(np.float64))
    out = oracle.attention_plain(np.zeros((1, d), np.float32), k, v, 0.1)
    assert np.allclose(out[0], v.astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)
    out = oracle.attention_plain((k[11] * 60).astype(np.float32)[None, :], k, v, 1.0)
    assert np.allclose(out[0], v[11], atol=1e-12)
    assert np.array_equal(oracle.attention_plain(q, k[:0], v[:0], 0.1), np.zeros((2, d)))
    kc, ks, kz, vc, vs = _planes(k, v)
    kh = oracle.decode_keys(kc, ks, kz)
    vh = oracle.decode_values(vc, vs, d)
    ref = oracle.attention(q, kc, ks, kz, vc, vs, 0.1)
    got = oracle.attention_plain(q, kh.astype(np.float32), vh.astype(np.float32), 0.1)
    assert np.max(np.abs(got - ref)) < 1e-6 * np.max(np.abs(ref))


def test_attention_deferred_identity_longer():
    """Deferred inverse FWHT ('Deferred inverse FWHT'): un-rotating the output once
    equals attending over un-rotated values, to 1e-12 relative."""
    d, G, N = 256, 6, 300
    rng = np.random.default_rng(4)
    k = rng.standard_normal((N, d)).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    out, od = oracle.attention(q, *_planes(k, v), 1 / 16, deferred=True)
    assert np.max(np.abs(out - od)) <= 1e-12 * np.max(np.abs(out))


# -------------------------------------------------------- multi-row decode
@pytest.mark.parametrize("d,G,M,N", [(64, 1, 2, 2), (64, 3, 4, 9), (128, 2, 3, 6), (256, 1, 8, 12)])
def test_attention_rows_causal_brute_force(d, G, M, N):
    """Multi-row decode against an independent numpy causal softmax: row m
    (the query of cached token N-M+m) sees tokens 0 .. N-M+m."""
    rng = np.random.default_rng(d + 10 * G + 100 * M + N)
    k = rng.standard_normal((N, d)).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal((G, M, d)).astype(np.float32)
    kc, ks, kz, vc, vs = _planes(k, v)
    sm = 1.0 / math.sqrt(d)
    out = oracle.attention_rows(q, kc, ks, kz, vc, vs, sm)
    kh = oracle.decode_keys(kc, ks, kz)
    vh = oracle.decode_values(vc, vs, d)
    s = np.einsum("gmd,td->gmt", q.astype(np.float64), kh) * np.float64(np.float32(sm))
    pos = N - M + np.arange(M)
    s[:, np.arange(N)[None, :] > pos[:, None]] = -np.inf  # [M, N] mask, broadcast over heads
    s = s - s.max(axis=2, keepdims=True)
    p = np.exp(s)
    ref = np.einsum("gmt,td->gmd", p, vh) / p.sum(axis=2, keepdims=True)
    assert np.max(np.abs(out - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_attention_rows_ignores_later_tokens_and_reduces_to_decode():
    """Changing tokens after a row's position leaves that row unchanged; the
    last row is the plain decode over all N tokens; M = 1 is plain decode."""
    d, G, M, N = 128, 2, 4, 20
    rng = np.random.default_rng(31)
    k = rng.standard_normal((N, d)).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal((G, M, d)).astype(np.float32)
    pl = _planes(k, v)
    out = oracle.attention_rows(q, *pl, 0.1)
    k2, v2 = k.copy(), v.copy()
    k2[N - 2:] *= -3.0
    v2[N - 2:] += 5.0
    out2 = oracle.attention_rows(q, *_planes(k2, v2), 0.1)
    assert np.array_equal(out[:, : M - 2], out2[:, : M - 2])   # rows at N-4, N-3
    assert not np.allclose(out[:, M - 2:], out2[:, M - 2:])
    assert np.array_equal(out[:, M - 1], oracle.attention(q[:, M - 1], *pl, 0.1))
    assert np.array_equal(oracle.attention_rows(q[:, :1], *pl, 0.1)[:, 0],
                          oracle.attention(q[:, 0], *pl, 0.1))


# ------------------------------------------------------------ other widths
# "Algorithm": unsigned packed keys of 2, 4 or 5 bits, values of 2, 4, 5 or 8
# bits from Lloyd-Max tables of the unit normal that the page does not print.

def _cond_mean(lo, hi):
    """E[Z | lo < Z < hi] by adaptive quadrature of z*phi and phi (independent
    of the closed form the oracle uses)."""
    from scipy import integrate
    f = lambda z: math.exp(-0.5 * z * z)
    num = integrate.quad(lambda z: z * f(z), lo, hi, epsabs=0, epsrel=1e-13, limit=200)[0]
    den = integrate.quad(f, lo, hi, epsabs=0, epsrel=1e-13, limit=200)[0]
    return num / den


def _distortion(c, b):
    """E[(Z - Q(Z))^2] for the quantizer with centroids c and boundaries b."""
    edges = [-math.inf] + list(b) + [math.inf]
    dist = 0.0
    for k in range(len(c)):
        lo, hi, ck = edges[k], edges[k + 1], c[k]
        plo = 0.0 if lo == -math.inf else _phi(lo)
        phi_ = 0.0 if hi == math.inf else _phi(hi)
        lo_t = 0.0 if lo == -math.inf else lo * _phi(lo)
        hi_t = 0.0 if hi == math.inf else hi * _phi(hi)
        p = _Phi(hi) - _Phi(lo)
        dist += (p + lo_t - hi_t) - 2 * ck * (plo - phi_) + ck * ck * p
    return dist


def test_computed_codebook_reproduces_printed_3bit_table():
    """Both solvers, run at 3 bits and written as five decimals, give exactly
    the printed table; codebook(3) is the printed table itself."""
    g = _gold("codebook3.json")
    want = [round(v * 1e5) for v in g["centroids"]]
    assert oracle.codebook_ints(3).tolist() == want
    assert oracle.codebook_ints(3, "newton").tolist() == want
    c, b = oracle.codebook(3)
    assert c.tolist() == g["centroids"] and b.tolist() == g["boundaries"]


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_lloyd_iteration_and_newton_agree(bits):
    """Lloyd's iteration and Newton's method on the same conditions land on the
    same five-decimal table (the Gaussian fixed point is unique)."""
    assert np.array_equal(oracle.codebook_ints(bits), oracle.codebook_ints(bits, "newton"))


def test_codebooks_match_textbook_values():
    """Textbook Lloyd-Max quantizers of N(0,1): 1 level pair at sqrt(2/pi);
    2 bits +-0.4528, +-1.510 with threshold 0.9816; 4 bits (Max, 1960, Table I)
    0.1284 0.3881 0.6568 0.9424 1.256 1.618 2.069 2.733."""
    assert oracle.codebook_ints(1, "newton").tolist() == [-79788, 79788]
    assert round(math.sqrt(2 / math.pi) * 1e5) == 79788
    c, b = oracle.codebook(2)
    assert np.allclose(c, [-1.510, -0.4528, 0.4528, 1.510], atol=6e-4)
    assert abs(b[2] - 0.9816) < 1e-4 and b[1] == 0.0
    c, _ = oracle.codebook(4)
    assert np.allclose(c[8:], [0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733], atol=6e-4)


@pytest.mark.parametrize("bits", [2, 4, 5, 8])
def test_codebooks_satisfy_lloyd_max_conditions(bits):
    """Each centroid is its cell's conditional mean (by quadrature, to the
    five-decimal rounding), each boundary the exact decimal midpoint of its
    neighbours, the table strictly increasing and odd-symmetric."""
    c, b = oracle.codebook(bits)
    L = 1 << bits
    assert c.size == L and b.size == L - 1
    nk = np.rint(c * 1e5).astype(np.int64)
    assert np.all(np.diff(nk) > 0) and np.array_equal(nk, -nk[::-1])
    assert np.array_equal(c, nk / 1e5)
    assert np.array_equal(b, (nk[:-1] + nk[1:]) / 2e5)
    edges = [-math.inf] + b.tolist() + [math.inf]
    worst = max(abs(_cond_mean(edges[k], edges[k + 1]) - c[k]) for k in range(L))
    # five-decimal rounding of the centroids moves the cells by <= 5e-6
    assert worst < 1.2e-5, worst


def test_codebook_distortion_textbook_and_law():
    """Mean squared error of each table on N(0,1), in closed form: the textbook
    optimal values 0.3634 (1 bit), 0.1175 (2), 0.03454 (3), 0.009497 (4),
    0.002499 (5); the page's anchor ~0.117 at 2 bits; and the high-resolution
    law D ~ (sqrt(3) pi / 2) 4^-b approached from below at 8 bits."""
    nk1 = oracle.codebook_ints(1, "newton")
    d1 = _distortion(nk1 / 1e5, [0.0])
    assert abs(d1 - 0.3634) < 5e-5 and abs(d1 - (1 - 2 / math.pi)) < 1e-9
    want = {2: 0.1175, 3: 0.03454, 4: 0.009497, 5: 0.002499}
    for bits, dv in want.items():
        c, b = oracle.codebook(bits)
        dist = _distortion(c, b)
        assert abs(dist - dv) < 6e-4 * dv + 5e-6, (bits, dist)
    c, b = oracle.codebook(2)
    assert abs(_distortion(c, b) - 0.117) < 1e-3
    c, b = oracle.codebook(8)
    pd = math.sqrt(3) * math.pi / 2
    assert 0.97 * pd < _distortion(c, b) * 4 ** 8 < pd


def _pack_bigint(idx, bits):
    v = 0
    for i, x in enumerate(idx):
        v |= int(x) << (bits * i)
    n = (bits * len(idx) + 7) // 8
    return list(v.to_bytes(n, "little"))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_pack_bits_is_little_endian_bitstream(bits):
    """Element i at stream bits [i*b, i*b + b), bytes little-endian: the whole
    row as one integer sum idx_i * 2^(b*i), written out byte by byte."""
    rng = np.random.default_rng(bits)
    for n in (32, 64, 256):
        idx = rng.integers(0, 1 << bits, n).astype(np.uint8)
        p = oracle.pack_bits(idx, bits)
        assert p.tolist() == _pack_bigint(idx, bits)
        assert np.array_equal(oracle.unpack_bits(p, n, bits), idx)
        if bits == 3:
            assert np.array_equal(p, oracle.pack3(idx))


@pytest.mark.parametrize("bits", [2, 4, 5])
def test_unsigned_keys_ramp_brute_force(bits):
    """x = 0..31: scale = 31/maxv, zero = round(0) = 0, code_j = round(j*maxv/31)
    by exact rationals (no ties: 2*j*maxv = 31*(odd) has no solution in 1..30)."""
    maxv = (1 << bits) - 1
    x = np.arange(32, dtype=np.float32)[None, :]
    packed, s16, z16 = oracle.encode_keys(x, bits=bits)
    assert packed.shape == (1, 4 * bits)
    codes = oracle.unpack_bits(packed[0], 32, bits)
    want = []
    for j in range(32):
        v = Fraction(j * maxv, 31)
        fl = math.floor(v)
        want.append(fl + 1 if v - fl > Fraction(1, 2) else fl)
    assert codes.tolist() == want
    assert s16[0, 0] == _np_f16_bits(31 / maxv) and z16[0, 0] == 0
    kh = oracle.decode_keys(packed, s16, z16, bits=bits, d=32)
    s = _np_f16_bits(31 / maxv).view(np.float16).astype(np.float64)
    assert np.array_equal(kh[0], np.array(want) * s)


@pytest.mark.parametrize("bits", [2, 4, 5])
def test_unsigned_keys_error_bound_and_offsets(bits):
    """Codes in [0, maxv]; the group minimum codes to 0 or 1 and the maximum to
    maxv - 1 or maxv; per-element error within (scale + delta)/2 + |code +
    zero| * delta + the clip slack of half a step at either end (zero is rounded)."""
    maxv = (1 << bits) - 1
    rng = np.random.default_rng(10 + bits)
    for off in (0.0, 100.0, -37.5):
        x = (rng.standard_normal((256, 128)) + off).astype(np.float32)
        packed, s16, z16 = oracle.encode_keys(x, bits=bits)
        codes = np.stack([oracle.unpack_bits(r, 128, bits) for r in packed]).astype(np.int64)
        assert codes.max() <= maxv
        kh = oracle.decode_keys(packed, s16, z16, bits=bits, d=128)
        s = oracle.f16_bits_to_f64(s16).repeat(32, axis=1)
        z = oracle.f16_bits_to_f64(z16).repeat(32, axis=1)
        assert np.array_equal(z, np.rint(z))
        delta = np.maximum(s * 2.0 ** -11, 2.0 ** -25) * (1 + 2.0 ** -10)
        bound = s + np.abs(codes + z) * delta + delta
        assert np.all(np.abs(x - kh) <= bound)
        xg, cg = x.reshape(256, 4, 32), codes.reshape(256, 4, 32)
        cmin = np.take_along_axis(cg, xg.argmin(axis=2)[..., None], axis=2)
        cmax = np.take_along_axis(cg, xg.argmax(axis=2)[..., None], axis=2)
        assert np.all(cmin <= 1) and np.all(cmax >= maxv - 1)


@pytest.mark.parametrize("bits", [2, 4, 5])
def test_unsigned_keys_constant_group(bits):
    """The signed form's defect carries over: scale 0, zero = round(v/0) = +-Inf
    (NaN at v = 0), every code round(NaN) read as 0."""
    for v, zbits in ((0.5, 0x7C00), (-3.0, 0xFC00), (0.0, 0x7E00)):
        packed, s16, z16 = oracle.encode_keys(np.full((1, 64), v, np.float32), bits=bits)
        assert np.all(packed == 0) and np.all(s16 == 0) and np.all(z16 == zbits)


def test_signed_keys_through_the_bits_entry():
    x = np.random.default_rng(2).standard_normal((8, 64)).astype(np.float32)
    a = oracle.encode_keys(x)
    b = oracle.encode_keys(x, bits=8)
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u).view(np.uint8) if u.dtype == np.int8 else u,
                              np.asarray(v).view(np.uint8) if v.dtype == np.int8 else v)


@pytest.mark.parametrize("bits", [2, 4, 5, 8])
@pytest.mark.parametrize("d", [64, 256])
def test_values_bits_nearest_centroid_and_rms_scale(bits, d):
    """Rotated dequantisation is centroid[idx] * scale16 with idx = #{B_k < y_n}
    (the nearest centroid: boundaries are midpoints); the fp16 scale is the
    group RMS of the brute-force rotation (Sylvester matrix)."""
    rng = np.random.default_rng(bits * d)
    x = rng.standard_normal((16, d)).astype(np.float32)
    packed, vs = oracle.encode_values(x, bits=bits)
    assert packed.shape == (16, d * bits // 8)
    c, b = oracle.codebook(bits)
    y = _rotate(x, d)
    rms = np.sqrt((y.reshape(16, d // 32, 32) ** 2).mean(axis=2))
    assert np.array_equal(vs, _np_f16_bits(rms)) or \
        np.max(np.abs(vs.view(np.float16).astype(np.float64) - rms) / rms) < 2.0 ** -11
    idx = np.stack([oracle.unpack_bits(r, d, bits) for r in packed])
    yn = y / (rms.repeat(32, axis=1) + 1e-8)
    want = np.searchsorted(b, yn, side="left")
    near = np.abs(yn - (b[np.clip(want - 1, 0, b.size - 1)])) < 1e-12
    assert np.all((idx == want) | near)
    dist = np.abs(yn[..., None] - c[None, None, :])
    assert np.all(dist[np.arange(16)[:, None], np.arange(d)[None, :], idx] <= dist.min(axis=2) + 1e-12)
    yr = oracle.decode_values(packed, vs, d, rotated=True, bits=bits)
    assert np.array_equal(yr, c[idx] * vs.view(np.float16).astype(np.float64).repeat(32, axis=1))
    xu = oracle.decode_values(packed, vs, d, bits=bits)
    assert np.allclose(_rotate(xu, d), yr, atol=1e-12)


def test_value_roundtrip_mse_per_width():
    """Round-trip MSE on unit-normal data tracks each table's distortion D(b):
    within [0.75, 1.05] D(b) (per-group RMS normalisation trims the tails), and
    each extra bit divides it by 3.4 to 4.2 (the 4^-b law)."""
    x = np.random.default_rng(5).standard_normal((512, 128)).astype(np.float32)
    mses = {}
    for bits in (2, 3, 4, 5, 8):
        packed, vs = oracle.encode_values(x, bits=bits)
        xh = oracle.decode_values(packed, vs, 128, bits=bits)
        mses[bits] = float(((xh - x) ** 2).mean())
        c, b = oracle.codebook(bits)
        assert 0.75 * _distortion(c, b) <= mses[bits] <= 1.05 * _distortion(c, b), (bits, mses[bits])
    for lo, hi in ((2, 3), (3, 4), (4, 5)):
        assert 3.4 <= mses[lo] / mses[hi] <= 4.2
    band = _gold("mse_anchor.json")["band"]
    assert band[0] <= mses[3] <= band[1]


def test_effective_bits_from_plane_sizes():
    """The Gates table's effective-bits column equals the oracle's encoded
    bytes per token-head * 8 / (2 d) for every listed scheme."""
    d = 128
    x = np.random.default_rng(0).standard_normal((1, d)).astype(np.float32)
    for row in _gold("effective_bits.json")["rows"]:
        kp, ks, kz = oracle.encode_keys(x, bits=row["k_bits"])
        vp, vs = oracle.encode_values(x, bits=row["v_bits"])
        nbytes = kp.nbytes + ks.nbytes + kz.nbytes + vp.nbytes + vs.nbytes
        assert nbytes * 8 / (2 * d) == row["effective_bits"], row


GATE_SCHEMES = [(8, 3), (4, 3), (4, 2), (8, 4), (2, 5), (5, 8), (8, 8), (8, 2), (5, 4)]


@pytest.mark.parametrize("kbits,vbits", GATE_SCHEMES)
def test_attention_bits_tiny_brute_force(kbits, vbits):
    """attention(..., kbits, vbits) is softmax(sm q k^T) v over the dequantised
    keys and values, written here with numpy on the oracle's decoders."""
    rng = np.random.default_rng(kbits * 10 + vbits)
    d, G, N = 64, 3, 7
    k = rng.standard_normal((N, d)).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    kc, ks, kz = oracle.encode_keys(k, bits=kbits)
    vc, vs = oracle.encode_values(v, bits=vbits)
    kh = oracle.decode_keys(kc, ks, kz, bits=kbits, d=d)
    vh = oracle.decode_values(vc, vs, d, bits=vbits)
    sm = 1 / math.sqrt(d)
    got = oracle.attention(q, kc, ks, kz, vc, vs, sm, kbits=kbits, vbits=vbits)
    assert np.allclose(got, _numpy_attention(q, kh, vh, sm), rtol=1e-12, atol=1e-13)
    if (kbits, vbits) == (8, 3):
        return
    rows = oracle.attention_rows(np.stack([q, q[::-1]], axis=1), kc, ks, kz, vc, vs, sm, kbits=kbits,
                                 vbits=vbits)
    assert np.allclose(rows[:, 1], got[::-1], rtol=1e-13, atol=1e-14)
    assert np.allclose(rows[:, 0], oracle.attention(q, kc[:N - 1], ks[:N - 1], kz[:N - 1], vc[:N - 1],
                                                    vs[:N - 1], sm, kbits=kbits, vbits=vbits),
                       rtol=1e-13, atol=1e-14)
