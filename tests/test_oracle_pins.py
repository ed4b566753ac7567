"""Pins for the CPU oracle: it is checked against things other than itself.

Each test names what fixes the expected value: a number printed on the pages
(tests/golden/pages_numbers.txt), a textbook table or routine, a closed form,
an invariant, or brute force on tiny inputs.  They are chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a wrong normalisation) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.linalg
from scipy import integrate, stats

from oracle import tq_oracle as o


def _golden(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([p.strip() for p in line.split("|")])
    return rows


def _pages(golden_dir):
    return {r[0]: r[1] for r in _golden(golden_dir, "pages_numbers.txt")}


# ---------------------------------------------------------------- Hadamard ----
@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_matches_scipy_sylvester(d):
    # scipy.linalg.hadamard builds the Sylvester matrix by Kronecker doubling,
    # a different construction from the popcount definition in the oracle.
    assert np.array_equal(o.hadamard(d), scipy.linalg.hadamard(d).astype(np.float64))


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_hadamard_orthogonality_exact(d):
    H = o.hadamard(d)
    assert np.array_equal(H @ H.T, d * np.eye(d))  # integers: exact
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_preserves_norm_and_cancels(d):
    rng = np.random.default_rng(5)
    c = o.Codec(3, d, seed=11)
    x = rng.standard_normal((16, d))
    y = o.rotate(x, c)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), math.sqrt(d) * np.linalg.norm(x, axis=1), rtol=1e-13)
    # <H D q, H D k> = d <q, k>: the rotation cancels between Q and K
    # (llama.cpp README, v1.7.0 "핵심 설계 결정" item 4: Parseval).
    q = rng.standard_normal((4, d))
    np.testing.assert_allclose(o.rotate(q, c) @ y.T, d * (q @ x.T), rtol=1e-12, atol=1e-10)


# ----------------------------------------------------------------- Signs ----
def test_splitmix64_reference_vector(golden_dir):
    want = [int(r[0], 16) for r in _golden(golden_dir, "splitmix64_seed0.txt")]
    assert o.splitmix64(0, 3) == want


def test_sign_vector_reads_bit63():
    outs = o.splitmix64(12345, 256)
    s = o.sign_vector(12345, 256)
    for i in range(256):
        assert s[i] == (-1.0 if outs[i] >= (1 << 63) else 1.0)
    # roughly balanced
    assert 80 < np.sum(s < 0) < 176


# -------------------------------------------------------------- Lloyd-Max ----
def test_lloyd_max_textbook_levels(golden_dir):
    for bits_s, tol_s, levels_s, mse_s in _golden(golden_dir, "lloyd_max_gaussian.txt"):
        bits = int(bits_s)
        c, t = o.lloyd_max_gaussian(bits)
        pos = c[len(c) // 2:]
        want = np.array([float(v) for v in levels_s.split()])
        np.testing.assert_allclose(pos, want, atol=float(tol_s))
        # Max printed 4 significant digits and his last digits are off by a few
        # units; the quadrature test below pins the MSE to 1e-12
        assert abs(o.lloyd_max_mse(c, t) / float(mse_s) - 1) < 5e-4


def test_lloyd_max_one_bit_closed_form():
    c, t = o.lloyd_max_gaussian(1)
    assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-15 and c[0] == -c[1] and t[0] == 0.0
    assert abs(o.lloyd_max_mse(c, t) - (1 - 2 / math.pi)) < 1e-15


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_fixed_point_by_quadrature(bits):
    """Centroid = conditional mean (numerical quadrature, scipy), threshold = midpoint."""
    c, t = o.lloyd_max_gaussian(bits)
    assert np.all(np.diff(c) > 0) and np.array_equal(c, -c[::-1]) and t[len(t) // 2] == 0.0
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    for k in range(len(c)):
        num = integrate.quad(lambda x: x * stats.norm.pdf(x), edges[k], edges[k + 1],
                             epsabs=1e-14, epsrel=1e-13)[0]
        den = stats.norm.cdf(edges[k + 1]) - stats.norm.cdf(edges[k])
        assert abs(num / den - c[k]) < 1e-10
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)
    mse_q = sum(integrate.quad(lambda x: (x - c[k]) ** 2 * stats.norm.pdf(x), edges[k], edges[k + 1],
                               epsabs=1e-15, epsrel=1e-12)[0] for k in range(len(c)))
    assert abs(mse_q - o.lloyd_max_mse(c, t)) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codec_rounds_to_float32_symmetrically(bits):
    c = o.Codec(bits, 128, 0)
    assert c.centroid.dtype == np.float32 and c.threshold.dtype == np.float32
    assert np.array_equal(c.centroid, -c.centroid[::-1])
    assert c.threshold[len(c.threshold) // 2] == 0.0
    assert len(c.centroid) == 1 << bits and len(c.threshold) == (1 << bits) - 1


# --------------------------------------------------------------- Quantize ----
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_threshold_count_is_nearest_centroid(bits):
    c = o.Codec(bits, 128, 0)
    rng = np.random.default_rng(bits)
    z = np.concatenate([rng.standard_normal(200000) * 1.5, c.centroid.astype(np.float64),
                        [0.0, -0.0, 1e-30, -1e-30, 50.0, -50.0]])
    idx = o.quantize(z, c)
    cent = c.centroid.astype(np.float64)
    brute = np.argmin(np.abs(z[:, None] - cent[None, :]), axis=1)  # ties -> lower index
    mid = 0.5 * (cent[:-1] + cent[1:])
    near = np.min(np.abs(z[:, None] - mid[None, :]), axis=1) < 1e-6  # fp32 thresholds vs fp64 midpoints
    assert np.array_equal(idx[~near], brute[~near])
    # a value exactly on a threshold goes to the lower cell; z = 0 -> L/2 - 1
    L = 1 << bits
    assert o.quantize(np.array([0.0]), c)[0] == L // 2 - 1
    t = c.threshold.astype(np.float64)
    assert np.array_equal(o.quantize(t, c), np.arange(L - 1))


# ------------------------------------------------------------------- Pack ----
def _naive_pack(idx, bits):
    n, d = idx.shape
    out = np.zeros((n, (d * bits + 7) // 8), dtype=np.uint8)
    for r in range(n):
        pos = 0
        for i in range(d):
            for b in range(bits):
                if (int(idx[r, i]) >> b) & 1:
                    out[r, pos // 8] |= 1 << (pos % 8)
                pos += 1
    return out


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_pack_matches_naive_bit_loop_and_round_trips(bits, d):
    rng = np.random.default_rng(bits * 1000 + d)
    idx = rng.integers(0, 1 << bits, size=(7, d))
    packed = o.pack_indices(idx, bits)
    assert packed.shape == (7, d * bits // 8)
    assert np.array_equal(packed, _naive_pack(idx, bits))
    assert np.array_equal(o.unpack_indices(packed, d, bits), idx)


def test_first_index_is_lowest_bits():
    idx = np.zeros((1, 128), dtype=np.int64)
    idx[0, 0] = 5  # 3-bit 101
    idx[0, 1] = 3  # 011 at bits 3..5
    p = o.pack_indices(idx, 3)
    assert p[0, 0] == 0b00011101


def test_byte_counts_match_pages(golden_dir):
    pages = _pages(golden_dir)
    # 3-bit, d=128: 48 B of codes + 2 B norm = 50 B per block
    assert o.Codec(3, 128, 0).code_bytes == 48
    assert o.packed_bytes(128, 3) == int(pages["block_bytes_d128_b3"])
    assert o.Codec(4, 128, 0).code_bytes == 64 and o.Codec(2, 128, 0).code_bytes == 32
    # K4/V2 at d=128: (64+2)+(32+2) = 100 B per token-head vs 2*256 B fp16 -> 5.12x
    fp16 = 2 * 128 * 2
    assert round(fp16 / (o.packed_bytes(128, 4) + o.packed_bytes(128, 2)), 2) == float(pages["ratio_k4v2_d128"])
    # the page's 3-bit-stored-as-4-bit packing gives 3.88x for K3/V3, ours gives 5.12x
    assert round(fp16 / (2 * o.packed_bytes(128, 4)), 2) == float(pages["ratio_k3v3_as_4bit_d128"])
    assert round(fp16 / (2 * o.packed_bytes(128, 3)), 2) == 5.12
    # 52 B per 3-bit vector -> 4.9x against 256 B of fp16 (48 B codes + a 4 B norm)
    assert round(256 / int(pages["bytes_3bit_v3_d128"]), 1) == float(pages["ratio_3bit_v3"])
    # QJL payload: m/8 B of signs + 2 B gamma
    assert o.packed_bytes(128, 3, 128) == 50 + 16 + 2
    assert o.packed_bytes(256, 3, 256) == 96 + 2 + 32 + 2


# ------------------------------------------------------------- Encode/decode ----
def test_half_norm_rounding():
    assert o.to_half(np.array([1 + 2 ** -11 + 2 ** -40]))[0] == np.float16(1 + 2 ** -10)  # round up past the tie
    assert o.to_half(np.array([1 + 2 ** -11]))[0] == np.float16(1.0)  # tie -> even
    assert o.to_half(np.array([1e9]))[0] == np.float16(65504.0)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_reconstruction_error_matches_lloyd_mse(bits):
    """Relative squared error of decode(encode(x)) for Gaussian x is the
    quantiser's MSE per unit-variance coordinate (up to finite-d effects)."""
    d = 128
    c = o.Codec(bits, d, seed=3)
    rng = np.random.default_rng(100 + bits)
    x = rng.standard_normal((4096, d))
    e = o.encode(x, c)
    xh = o.decode(e["codes"], e["norms"], c)
    rel = np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1)
    cc, tt = o.lloyd_max_gaussian(bits)
    assert abs(rel.mean() / o.lloyd_max_mse(cc, tt) - 1) < 0.03
    # the error also equals the rotated-domain residual ||z - c[idx]||^2 / d (Parseval),
    # up to the half rounding of the norm
    res = np.sum((e["z"] - c.centroid.astype(np.float64)[e["idx"]]) ** 2, axis=1) / d
    np.testing.assert_allclose(rel, res, rtol=2e-3, atol=2e-5)


def test_encode_scale_and_sign_invariance():
    d, bits = 128, 4
    c = o.Codec(bits, d, seed=9)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((256, d))
    e1 = o.encode(x, c)
    e2 = o.encode(4.0 * x, c)  # power-of-two scale: exact
    assert np.array_equal(e1["codes"], e2["codes"])
    assert np.array_equal(e1["norms"].astype(np.float64) * 4, e2["norms"].astype(np.float64))
    e3 = o.encode(-x, c)  # symmetric codebook: idx -> L-1-idx
    assert np.array_equal(e3["idx"], (1 << bits) - 1 - e1["idx"])


def test_zero_vector():
    c = o.Codec(3, 128, 0)
    e = o.encode(np.zeros((2, 128)), c)
    assert np.all(e["idx"] == 3) and np.all(e["norms"] == 0)
    assert np.array_equal(o.decode(e["codes"], e["norms"], c), np.zeros((2, 128)))


def test_decode_inverts_exact_rotation():
    """With centroid-valued rotated coordinates, decode returns x exactly
    (H H = d I, D D = I): build x = n D H c / d and check decode reproduces it."""
    d, bits = 128, 3
    c = o.Codec(bits, d, seed=4)
    rng = np.random.default_rng(2)
    idx = rng.integers(0, 8, size=(5, d))
    codes = o.pack_indices(idx, bits)
    n16 = np.array([1.0, 2.0, 0.5, 3.0, 1.5], dtype=np.float16)
    xh = o.decode(codes, n16, c)
    cent = c.centroid.astype(np.float64)[idx]
    # applying the forward rotation gives back n16 * c[idx]
    np.testing.assert_allclose(o.rotate(xh, c), n16.astype(np.float64)[:, None] * cent, rtol=0, atol=1e-12)


# -------------------------------------------------------------- Attention ----
def _craft_query(K, target, scale):
    """q with scale*<q, K_t> = target_t (least squares, exact for full-rank K)."""
    return np.linalg.lstsq(scale * K, target, rcond=None)[0]


def test_softmax_worked_example(golden_dir):
    pages = _pages(golden_dir)
    d = 128
    kc, vc = o.Codec(4, d, 1), o.Codec(2, d, 1)
    rng = np.random.default_rng(8)
    ek = o.encode(rng.standard_normal((3, d)), kc)
    ev = o.encode(rng.standard_normal((3, d)), vc)
    K = o.decode(ek["codes"], ek["norms"], kc)
    V = o.decode(ev["codes"], ev["norms"], vc)
    scale = 1 / math.sqrt(d)
    for key_in, key_out, exact in (("softmax_in_a", "softmax_out_a_percent", True),
                                   ("softmax_in_b", "softmax_out_b_percent_printed", False)):
        s = np.array([float(v) for v in pages[key_in].split()])
        q = _craft_query(K, s, scale)
        out = o.attention(q[None], ek["codes"], ek["norms"], ev["codes"], ev["norms"], kc, vc, scale)[0]
        p = np.linalg.lstsq(V.T, out, rcond=None)[0]  # recover the weights
        printed = np.array([float(v) for v in pages[key_out].split()]) / 100
        if exact:
            np.testing.assert_allclose(p, printed, atol=0.005)  # printed to whole percent
            np.testing.assert_allclose(p, [0.332, 0.367, 0.301], atol=5e-4)
        else:
            # the second printed triple is garbled (sums to 0.79); the true softmax:
            assert abs(printed.sum() - 1) > 0.2
            np.testing.assert_allclose(p, [0.307, 0.506, 0.186], atol=5e-4)


def test_attention_special_cases():
    d = 128
    kc, vc = o.Codec(3, d, 2), o.Codec(3, d, 2)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, d))
    ek, ev = o.encode(x, kc), o.encode(rng.standard_normal((6, d)), vc)
    V = o.decode(ev["codes"], ev["norms"], vc)
    q = rng.standard_normal((3, d))
    # one-token context: output is the reconstructed value
    out1 = o.attention(q, ek["codes"][:1], ek["norms"][:1], ev["codes"][:1], ev["norms"][:1], kc, vc, 0.1)
    np.testing.assert_allclose(out1, np.repeat(V[:1], 3, axis=0), rtol=1e-13)
    # identical keys: uniform weights, output is the mean of the values
    kk = np.repeat(ek["codes"][:1], 6, axis=0)
    kn = np.repeat(ek["norms"][:1], 6, axis=0)
    out2 = o.attention(q, kk, kn, ev["codes"], ev["norms"], kc, vc, 0.1)
    np.testing.assert_allclose(out2, np.repeat(V.mean(0, keepdims=True), 3, axis=0), rtol=1e-12, atol=1e-14)
    # empty context -> zeros
    assert np.array_equal(o.attention(q, ek["codes"][:0], ek["norms"][:0], ev["codes"][:0], ev["norms"][:0],
                                      kc, vc, 0.1), np.zeros((3, d)))


def test_attention_rotated_domain_equals_decoded():
    """Scores computed in the rotated domain, n/d <H(Dq), c[idx]>, equal <q, K_hat>."""
    d = 128
    kc = o.Codec(4, d, 5)
    rng = np.random.default_rng(10)
    ek = o.encode(rng.standard_normal((50, d)) * 30, kc)
    q = rng.standard_normal((4, d))
    K = o.decode(ek["codes"], ek["norms"], kc)
    a = o.rotate(q, kc)
    rot = (a @ kc.centroid.astype(np.float64)[ek["idx"]].T) * ek["norms"].astype(np.float64)[None, :] / d
    np.testing.assert_allclose(q @ K.T, rot, rtol=1e-11, atol=1e-9)


def test_gqa_head_mapping():
    d, B, Hq, Hkv, ctx = 64, 2, 6, 2, 9
    kc, vc = o.Codec(2, d, 1), o.Codec(2, d, 1)
    rng = np.random.default_rng(11)
    ek = o.encode(rng.standard_normal((B * Hkv * ctx, d)), kc)
    ev = o.encode(rng.standard_normal((B * Hkv * ctx, d)), vc)
    kcodes = ek["codes"].reshape(B, Hkv, ctx, -1)
    kn = ek["norms"].reshape(B, Hkv, ctx)
    vcodes = ev["codes"].reshape(B, Hkv, ctx, -1)
    vn = ev["norms"].reshape(B, Hkv, ctx)
    q = rng.standard_normal((B, Hq, d))
    ctx_len = np.array([9, 4])
    out = o.gqa_attention(q, ctx_len, kcodes, kn, vcodes, vn, kc, vc, 0.125)
    for row, (b, h) in enumerate([(b, h) for b in range(B) for h in range(Hq)]):
        kh = h // 3  # g = 3
        n = ctx_len[b]
        want = o.attention(q[b, h][None], kcodes[b, kh, :n], kn[b, kh, :n], vcodes[b, kh, :n], vn[b, kh, :n],
                           kc, vc, 0.125)[0]
        np.testing.assert_allclose(out[row], want, rtol=1e-14)


def _mq_cache(rng, B, Hkv, cap, d, kc, vc, keys=None):
    K = keys if keys is not None else rng.standard_normal((B * Hkv * cap, d)) * 3
    ek = o.encode(K, kc)
    ev = o.encode(rng.standard_normal((B * Hkv * cap, d)), vc)
    return (ek["codes"].reshape(B, Hkv, cap, -1), ek["norms"].reshape(B, Hkv, cap),
            ev["codes"].reshape(B, Hkv, cap, -1), ev["norms"].reshape(B, Hkv, cap))


def test_mq_causal_closed_forms():
    """Multi-query decode, closed forms: with ctx_len = C, column c sees tokens
    0..c, so column 0 returns V_hat_0 exactly; with identical keys column c
    returns the mean of V_hat_0..V_hat_c; the last column equals single-query
    decode over the whole context."""
    d, C, cap = 64, 4, 4
    kc, vc = o.Codec(3, d, 3), o.Codec(2, d, 3)
    rng = np.random.default_rng(21)
    kcodes, kn, vcodes, vn = _mq_cache(rng, 1, 1, cap, d, kc, vc)
    V = o.decode(vcodes[0, 0], vn[0, 0], vc)
    q = rng.standard_normal((1, C, 2, d))
    out = o.mq_attention(q, [C], kcodes, kn, vcodes, vn, kc, vc, 0.3).reshape(C, 2, d)
    np.testing.assert_allclose(out[0], np.repeat(V[:1], 2, axis=0), rtol=1e-13)
    # identical keys: uniform weights over the visible prefix
    same = np.repeat(rng.standard_normal((1, d)), cap, axis=0) * 5
    kcodes2, kn2, _, _ = _mq_cache(rng, 1, 1, cap, d, kc, vc, keys=same)
    out2 = o.mq_attention(q, [C], kcodes2, kn2, vcodes, vn, kc, vc, 0.3).reshape(C, 2, d)
    for c in range(C):
        np.testing.assert_allclose(out2[c], np.repeat(V[:c + 1].mean(0, keepdims=True), 2, axis=0),
                                   rtol=1e-12, atol=1e-14)
    # last column = plain decode over everything
    full = o.gqa_attention(q[:, C - 1], [C], kcodes, kn, vcodes, vn, kc, vc, 0.3)
    np.testing.assert_allclose(out[C - 1], full, rtol=1e-14)


def test_mq_is_causal():
    """Column c ignores every token at or after its own position + 1: changing
    those keys and values leaves it unchanged and changes the later columns."""
    d, B, Hkv, g, C, cap = 64, 2, 2, 3, 3, 20
    kc, vc = o.Codec(4, d, 5), o.Codec(3, d, 5)
    rng = np.random.default_rng(22)
    kcodes, kn, vcodes, vn = _mq_cache(rng, B, Hkv, cap, d, kc, vc)
    ctx = np.array([20, 9])
    q = rng.standard_normal((B, C, Hkv * g, d))
    base = o.mq_attention(q, ctx, kcodes, kn, vcodes, vn, kc, vc, 0.2).reshape(B, C, Hkv * g, d)
    # overwrite the last token of sequence 1 (position ctx-1, seen only by column C-1)
    k2, n2, v2, vn2 = kcodes.copy(), kn.copy(), vcodes.copy(), vn.copy()
    k2[1, :, ctx[1] - 1] = kcodes[0, :, 0]
    v2[1, :, ctx[1] - 1] = vcodes[0, :, 0]
    n2[1, :, ctx[1] - 1] = kn[0, :, 0]
    vn2[1, :, ctx[1] - 1] = vn[0, :, 0]
    moved = o.mq_attention(q, ctx, k2, n2, v2, vn2, kc, vc, 0.2).reshape(B, C, Hkv * g, d)
    assert np.array_equal(moved[0], base[0])
    assert np.array_equal(moved[1, :C - 1], base[1, :C - 1])
    assert np.abs(moved[1, C - 1] - base[1, C - 1]).max() > 1e-6
    # a context shorter than the columns: early columns see no token -> zero
    short = o.mq_attention(q, [2, 1], kcodes, kn, vcodes, vn, kc, vc, 0.2).reshape(B, C, Hkv * g, d)
    assert np.all(short[0, 0] == 0) and np.all(short[1, :2] == 0)
    assert np.all(np.linalg.norm(short[0, 1:], axis=-1) > 0)


def test_mq_single_column_is_decode():
    d, B, Hkv, g, cap = 128, 2, 2, 4, 30
    kc, vc = o.Codec(4, d, 6), o.Codec(2, d, 6)
    rng = np.random.default_rng(23)
    kcodes, kn, vcodes, vn = _mq_cache(rng, B, Hkv, cap, d, kc, vc)
    q = rng.standard_normal((B, 1, Hkv * g, d))
    ctx = [30, 17]
    np.testing.assert_array_equal(o.mq_attention(q, ctx, kcodes, kn, vcodes, vn, kc, vc, 0.1),
                                  o.gqa_attention(q[:, 0], ctx, kcodes, kn, vcodes, vn, kc, vc, 0.1))


def test_score_factor_closed_forms(golden_dir):
    """alpha(N): sharpening gives 1 + 1/(2 SQNR) at N = N0 and grows as
    sqrt(ln N / ln N0) above 1; softening gives SQNR/(SQNR + 1) at N0 and
    shrinks; both are 1 for N <= 1 and tend to 1 as SQNR grows."""
    n0 = int(_pages(golden_dir)["sharpen_n0"])
    for sq in (2.0, 11.6, 30.0):
        assert o.score_factor(o.SCORE_SHARPEN, n0, sq) == pytest.approx(1 + 1 / (2 * sq), rel=1e-15)
        assert o.score_factor(o.SCORE_SOFTEN, n0, sq) == pytest.approx(sq / (sq + 1), rel=1e-15)
        for n in (3, 100, 262144, 1 << 20):
            ratio = (o.score_factor(o.SCORE_SHARPEN, n, sq) - 1) / (1 / (2 * sq))
            assert ratio == pytest.approx(math.sqrt(math.log(n) / math.log(n0)), rel=1e-13)
        for n in (0, 1):
            assert o.score_factor(o.SCORE_SHARPEN, n, sq) == 1.0 == o.score_factor(o.SCORE_SOFTEN, n, sq)
        ns = [2, 64, 2048, 65536, 1 << 20]
        sh = [o.score_factor(o.SCORE_SHARPEN, n, sq) for n in ns]
        so = [o.score_factor(o.SCORE_SOFTEN, n, sq) for n in ns]
        assert all(a < b for a, b in zip(sh, sh[1:])) and all(a > b for a, b in zip(so, so[1:]))
    assert o.score_factor(o.SCORE_SHARPEN, 5000, 1e12) == pytest.approx(1.0, abs=1e-11)
    assert o.score_factor(o.SCORE_PLAIN, 5000, 3.0) == 1.0


def test_sharpening_matches_the_pages_range(golden_dir):
    """The page's figures: over 2048 -> 262144 tokens the factor moves by about
    0.012 while staying in 1.007-1.048.  With the top of that range reached at
    262144 tokens, the sqrt(ln N) law gives a move of 0.0105; a law linear in
    ln N would give 0.019, outside 'about 0.012'."""
    pages = _pages(golden_dir)
    lo, hi = (float(v) for v in pages["sharpen_alpha_range"].split())
    delta = float(pages["sharpen_delta_2048_262144"])
    growth = math.sqrt(math.log(262144) / math.log(2048))
    sq = growth / (2 * (hi - 1))  # SQNR_eff with alpha(262144) = 1.048
    a0, a1 = o.score_factor(o.SCORE_SHARPEN, 2048, sq), o.score_factor(o.SCORE_SHARPEN, 262144, sq)
    assert a1 == pytest.approx(hi, rel=1e-12)
    assert lo <= a0 < a1 <= hi
    assert abs((a1 - a0) - delta) < 0.003
    linear = (hi - 1) * (1 - math.log(2048) / math.log(262144))
    assert abs(linear - delta) > 0.005


def _sharpen_case(seed=24, d=64, n=30):
    kc, vc = o.Codec(3, d, 9), o.Codec(3, d, 9)
    rng = np.random.default_rng(seed)
    ek, ev = o.encode(rng.standard_normal((n, d)) * 4, kc), o.encode(rng.standard_normal((n, d)), vc)
    q = rng.standard_normal((2, d))
    return kc, vc, ek, ev, q


def test_score_factor_enters_as_a_scale():
    """attention(alpha = a) is plain attention at scale a * scale; in
    mq_attention every column uses alpha of the tokens it sees."""
    kc, vc, ek, ev, q = _sharpen_case()
    a = 1.37
    np.testing.assert_allclose(
        o.attention(q, ek["codes"], ek["norms"], ev["codes"], ev["norms"], kc, vc, 0.2, alpha=a),
        o.attention(q, ek["codes"], ek["norms"], ev["codes"], ev["norms"], kc, vc, 0.2 * a), rtol=1e-13)
    C, n, sq = 3, 30, 4.0
    qq = np.random.default_rng(25).standard_normal((1, C, 2, kc.d))
    kcodes, kn = ek["codes"][None, None], ek["norms"][None, None]
    vcodes, vn = ev["codes"][None, None], ev["norms"][None, None]
    got = o.mq_attention(qq, [n], kcodes, kn, vcodes, vn, kc, vc, 0.2, score_mode=o.SCORE_SHARPEN,
                         sqnr=sq).reshape(C, 2, -1)
    for c in range(C):
        nc = n - (C - 1 - c)
        want = o.attention(qq[0, c], ek["codes"][:nc], ek["norms"][:nc], ev["codes"][:nc], ev["norms"][:nc], kc,
                           vc, 0.2 * (1 + math.sqrt(math.log(nc)) / (2 * sq * math.sqrt(math.log(2048)))))
        np.testing.assert_allclose(got[c], want, rtol=1e-12)
    # sharpening concentrates the weights: the output moves toward the top value
    plain = o.mq_attention(qq, [n], kcodes, kn, vcodes, vn, kc, vc, 0.2).reshape(C, 2, -1)
    assert np.abs(got - plain).max() > 1e-4


def test_sparse_v_closed_forms(golden_dir):
    """Sparse V: tau = 0 is plain attention; tau = 1 keeps only the top token
    (o = V_top / sum_t exp(s_t - s_top)); in general the output moves by at
    most the dropped weight times the dropped values' norms."""
    kc, vc, ek, ev, q = _sharpen_case(seed=26, n=40)
    args = (ek["codes"], ek["norms"], ev["codes"], ev["norms"], kc, vc, 0.5)
    plain = o.attention(q, *args)
    np.testing.assert_array_equal(o.attention(q, *args, sparse_v=0.0), plain)
    K, V = o.decode(ek["codes"], ek["norms"], kc), o.decode(ev["codes"], ev["norms"], vc)
    s = 0.5 * q @ K.T
    top = np.argmax(s, axis=1)
    want = V[top] / np.exp(s - s.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(o.attention(q, *args, sparse_v=1.0), want, rtol=1e-13)
    tau = float(_pages(golden_dir)["sparse_v_threshold"])
    for t in (tau, 1e-3, 0.05):
        got = o.attention(q, *args, sparse_v=t)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        bound = np.where(e < t, p, 0.0) @ np.linalg.norm(V, axis=1)
        assert np.all(np.linalg.norm(got - plain, axis=1) <= bound + 1e-15)
    assert np.abs(o.attention(q, *args, sparse_v=0.05) - plain).max() > 1e-6


def test_window_is_concatenation():
    """Tokens moved from the packed cache into the residual window (as their
    decoded values) leave the output unchanged: the window joins the same softmax."""
    d = 128
    kc, vc = o.Codec(4, d, 3), o.Codec(2, d, 3)
    rng = np.random.default_rng(21)
    ek = o.encode(rng.standard_normal((40, d)) * 20, kc)
    ev = o.encode(rng.standard_normal((40, d)), vc)
    K = o.decode(ek["codes"], ek["norms"], kc)
    V = o.decode(ev["codes"], ev["norms"], vc)
    q = rng.standard_normal((3, d))
    full = o.attention(q, ek["codes"], ek["norms"], ev["codes"], ev["norms"], kc, vc, 0.09)
    for j in (1, 7, 40):
        split = o.attention(q, ek["codes"][:40 - j], ek["norms"][:40 - j], ev["codes"][:40 - j],
                            ev["norms"][:40 - j], kc, vc, 0.09, k_win=K[40 - j:], v_win=V[40 - j:])
        np.testing.assert_allclose(split, full, rtol=1e-12, atol=1e-14)


def test_window_closed_forms():
    """Window-only attention: two tokens give the logistic weight in closed form,
    one token gives its value, and a dominating key selects its value."""
    d = 64
    kc, vc = o.Codec(3, d, 1), o.Codec(3, d, 1)
    empty_k = np.zeros((0, d * 3 // 8), np.uint8)
    empty_n = np.zeros(0, np.float16)
    rng = np.random.default_rng(22)
    q = np.zeros((1, d)); q[0, 5] = 2.0
    kw = np.zeros((2, d)); kw[0, 5] = 1.5; kw[1, 5] = -0.5; kw[1, 7] = 9.0
    vw = rng.standard_normal((2, d))
    scale = 0.3
    out = o.attention(q, empty_k, empty_n, empty_k, empty_n, kc, vc, scale, k_win=kw, v_win=vw)
    # s = scale * (3.0, -1.0): p_0 = 1 / (1 + e^{-scale * 4})
    p0 = 1.0 / (1.0 + math.exp(-scale * 4.0))
    np.testing.assert_allclose(out[0], p0 * vw[0] + (1 - p0) * vw[1], rtol=1e-13)
    one = o.attention(q, empty_k, empty_n, empty_k, empty_n, kc, vc, scale, k_win=kw[1:], v_win=vw[1:])
    np.testing.assert_allclose(one[0], vw[1], rtol=1e-14)
    # a window key 200 score units above every decoded key takes all the weight
    ek = o.encode(rng.standard_normal((16, d)), kc)
    ev = o.encode(rng.standard_normal((16, d)), vc)
    kbig = np.zeros((1, d)); kbig[0, 5] = 200.0 / (scale * 2.0)
    dom = o.attention(q, ek["codes"], ek["norms"], ev["codes"], ev["norms"], kc, vc, scale, k_win=kbig, v_win=vw[:1])
    np.testing.assert_allclose(dom[0], vw[0], rtol=1e-12)


def test_gqa_window_mapping():
    d, B, Hq, Hkv, ctx, wcap = 64, 2, 4, 2, 5, 3
    kc, vc = o.Codec(2, d, 1), o.Codec(2, d, 1)
    rng = np.random.default_rng(23)
    ek = o.encode(rng.standard_normal((B * Hkv * ctx, d)), kc)
    ev = o.encode(rng.standard_normal((B * Hkv * ctx, d)), vc)
    kcodes, kn = ek["codes"].reshape(B, Hkv, ctx, -1), ek["norms"].reshape(B, Hkv, ctx)
    vcodes, vn = ev["codes"].reshape(B, Hkv, ctx, -1), ev["norms"].reshape(B, Hkv, ctx)
    kw, vw = rng.standard_normal((B, Hkv, wcap, d)), rng.standard_normal((B, Hkv, wcap, d))
    q = rng.standard_normal((B, Hq, d))
    ctx_len, win_len = np.array([5, 0]), np.array([2, 3])
    out = o.gqa_attention(q, ctx_len, kcodes, kn, vcodes, vn, kc, vc, 0.2, k_win=kw, v_win=vw, win_len=win_len)
    for row, (b, h) in enumerate([(b, h) for b in range(B) for h in range(Hq)]):
        kh, n, w = h // 2, ctx_len[b], win_len[b]
        want = o.attention(q[b, h][None], kcodes[b, kh, :n], kn[b, kh, :n], vcodes[b, kh, :n], vn[b, kh, :n],
                           kc, vc, 0.2, k_win=kw[b, kh, :w], v_win=vw[b, kh, :w])[0]
        np.testing.assert_allclose(out[row], want, rtol=1e-14)


def test_append_token_by_token_equals_whole_encode():
    """Appending a sequence one token per step (each sequence at its own
    position) gives the bytes of encoding every token at once; positions
    outside the cache write nothing."""
    d, B, H, cap, steps = 64, 3, 2, 6, 4
    rng = np.random.default_rng(24)
    for m in (0, 32):
        codec = o.Codec(3, d, 4, m)
        S = rng.standard_normal((m, d)) if m else None
        X = rng.standard_normal((B, H, steps, d)) * 5
        start = np.array([0, 2, 4])  # sequence 2 runs past the end at step 2
        rowb = d * 3 // 8
        codes = np.full((B, H, cap, rowb), 0xAB, np.uint8)
        norms = np.full((B, H, cap), 0x1234, np.uint16).view(np.float16)
        qjl = np.full((B, H, cap, max(m // 8, 1)), 0xCD, np.uint8)
        gamma = np.full((B, H, cap), 0x4321, np.uint16).view(np.float16)
        for t in range(steps):
            o.append(codes, norms, X[:, :, t], start + t, codec, S, qjl, gamma)
        whole = o.encode(X.reshape(-1, d), codec, S)
        for b in range(B):
            for h in range(H):
                for t in range(steps):
                    p = start[b] + t
                    r = (b * H + h) * steps + t
                    if p < cap:
                        assert np.array_equal(codes[b, h, p], whole["codes"][r])
                        assert norms[b, h, p] == whole["norms"][r]
                        if m:
                            assert np.array_equal(qjl[b, h, p], whole["qjl"][r])
                            assert gamma[b, h, p] == whole["gamma"][r]
                untouched = [p for p in range(cap) if not start[b] <= p < start[b] + steps]
                assert np.all(codes[b, h, untouched] == 0xAB)
                assert np.all(norms[b, h, untouched].view(np.uint16) == 0x1234)


def test_prefill_chunks_equal_whole_encode():
    """Prefilling a sequence chunk by chunk gives the bytes of encoding every
    token at once, at the right slots; slots past the prefill stay untouched
    and a chunk outside the cache is rejected."""
    d, H, cap, T = 64, 3, 20, 4
    rng = np.random.default_rng(25)
    codec = o.Codec(3, d, 6)
    X = rng.standard_normal((H, 3 * T, d)) * 3
    codes = np.full((H, cap, d * 3 // 8), 0xAB, np.uint8)
    norms = np.full((H, cap), 0x1234, np.uint16).view(np.float16)
    for c in range(3):
        o.prefill(codes, norms, X[:, c * T:(c + 1) * T], 2 + c * T, codec)
    whole = o.encode(X.reshape(-1, d), codec)
    for h in range(H):
        for t in range(3 * T):
            r = h * 3 * T + t
            assert np.array_equal(codes[h, 2 + t], whole["codes"][r]) and norms[h, 2 + t] == whole["norms"][r]
        assert np.all(codes[h, :2] == 0xAB) and np.all(codes[h, 2 + 3 * T:] == 0xAB)
    with pytest.raises(ValueError):
        o.prefill(codes, norms, X[:, :T], cap - T + 1, codec)


# -------------------------------------------------------------------- QJL ----
def test_qjl_sign_projection_closed_form():
    """E[sign(s.r) (s.a)] = sqrt(2/pi) <a, r>/||r|| for s ~ N(0, I)."""
    rng = np.random.default_rng(12)
    d, n = 16, 1_000_000
    a, r = rng.standard_normal(d), rng.standard_normal(d)
    s = rng.standard_normal((n, d))
    x = np.sign(s @ r) * (s @ a)
    mean, se = x.mean(), x.std() / math.sqrt(n)
    want = math.sqrt(2 / math.pi) * (a @ r) / np.linalg.norm(r)
    assert abs(mean - want) < 4 * se


def test_qjl_estimator_unbiased():
    """The oracle's inner-product estimate (MSE part + QJL term), with exact
    float64 norm and gamma, converges to <q, x> as the projection count grows;
    the error stays within 4 standard deviations of the closed-form spread."""
    d, m = 32, 1 << 17
    rng = np.random.default_rng(13)
    S = rng.standard_normal((m, d))
    c = o.Codec(2, d, seed=21, qjl_m=m)
    zs = []
    for trial in range(12):
        x = rng.standard_normal((1, d))
        q = rng.standard_normal((1, d))
        e = o.encode(x, c, S)
        n64, g64 = e["norm"], e["gamma64"]
        est = o.ip_scores(q, e["codes"], n64, e["qjl"], g64, S, c)[0, 0]
        # MSE part uses n (not n16) here too, so the only error is the QJL sampling
        truth = float(q[0] @ x[0])
        a = o.rotate(q, c)[0]
        r = e["r"][0]
        rhat = r / np.linalg.norm(r)
        var1 = (a @ a) / d - (2 / math.pi) * ((a @ rhat) ** 2) / d  # one projection of a/sqrt(d)
        sd = n64[0] * g64[0] * math.sqrt(math.pi / 2) * math.sqrt(var1 / m)
        zs.append((est - truth) / sd)
    zs = np.array(zs)
    assert np.all(np.abs(zs) < 4), zs
    assert abs(zs.mean()) < 4 / math.sqrt(len(zs))


def test_pack_signs_bit_order():
    """QJL sign bits use the same LSB-first stream as 1-bit indices: projection
    j sits in bit j % 8 of byte j // 8 (the layout the library documents)."""
    rng = np.random.default_rng(16)
    bits = rng.integers(0, 2, size=(5, 64)).astype(np.uint8)
    packed = o.pack_signs(bits)
    assert np.array_equal(packed, o.pack_indices(bits, 1))
    assert np.array_equal(packed, _naive_pack(bits, 1))
    assert np.array_equal(o.unpack_signs(packed, 64), bits)
    one = np.zeros((1, 16), dtype=np.uint8)
    one[0, 0] = 1
    one[0, 9] = 1
    assert o.pack_signs(one).tolist() == [[0x01, 0x02]]


def _qjl_case(seed, d=64, m=64, n=40, kscale=3.0):
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((m, d))
    kc, vc = o.Codec(3, d, seed=5, qjl_m=m), o.Codec(2, d, seed=6)
    ek = o.encode(kscale * rng.standard_normal((n, d)), kc, S)
    ev = o.encode(rng.standard_normal((n, d)), vc)
    q = rng.standard_normal((3, d))
    return S, kc, vc, ek, ev, q


def test_qjl_attention_is_softmax_of_scaled_estimates():
    """With QJL keys, attention() is softmax(scale * est) V_hat where est is the
    inner-product estimator ip_scores() (pinned by its unbiasedness): the whole
    estimate, QJL term included, carries the softmax scale."""
    from scipy.special import softmax

    S, kc, vc, ek, ev, q = _qjl_case(17)
    scale = 0.37
    got = o.attention(q, ek["codes"], ek["norms"], ev["codes"], ev["norms"], kc, vc, scale,
                      k_qjl=ek["qjl"], k_gamma=ek["gamma"], S=S)
    est = o.ip_scores(q, ek["codes"], ek["norms"], ek["qjl"], ek["gamma"], S, kc)
    V = o.decode(ev["codes"], ev["norms"], vc)
    want = softmax(scale * est, axis=1) @ V
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)
    # the check has teeth: the QJL term moves the output, and an unscaled QJL
    # term would move it far more than the tolerance above
    mse_only = o.ip_scores(q, ek["codes"], ek["norms"], None, None, None, o.Codec(3, kc.d, seed=5))
    corr = est - mse_only
    assert np.abs(corr).max() > 0.1
    unscaled = softmax(scale * mse_only + corr, axis=1) @ V
    assert np.abs(unscaled - want).max() > 1e-3
    assert np.abs(softmax(scale * mse_only, axis=1) @ V - want).max() > 1e-4


def test_qjl_attention_logit_unbiased():
    """Through attention outputs alone: with two keys, the logit difference
    s_0 - s_1 recovered from the output averages over S draws to its closed-form
    expectation scale * (<q, x0_hat - x1_hat> + residual parts), where
    E[sign(s.r)(s.a)] = sqrt(2/pi) <a, r>/||r|| makes the QJL term's mean
    n16 * (gamma16/||r||) * <H(Dq), rho>/d for residual rho = z - c[idx]."""
    d = m = 32
    rng = np.random.default_rng(18)
    kc, vc = o.Codec(2, d, seed=7, qjl_m=m), o.Codec(3, d, seed=8)
    x = rng.standard_normal((2, d))
    # a query leaning on key 0's quantisation residual, so the QJL part of the
    # logit is large
    e0 = o.encode(x, o.Codec(2, d, seed=7))
    q = 2.0 * (x[:1] - o.decode(e0["codes"][:1], e0["norms"][:1], o.Codec(2, d, seed=7))) \
        + 0.3 * rng.standard_normal((1, d))
    ev = o.encode(rng.standard_normal((2, d)), vc)
    V = o.decode(ev["codes"], ev["norms"], vc)
    dv = V[0] - V[1]
    scale = 0.1
    draws = 3000
    diffs = np.empty(draws)
    for i in range(draws):
        S = rng.standard_normal((m, d))
        ek = o.encode(x, kc, S)
        out = o.attention(q, ek["codes"], ek["norms"], ev["codes"], ev["norms"], kc, vc, scale,
                          k_qjl=ek["qjl"], k_gamma=ek["gamma"], S=S)[0]
        p0 = float((out - V[1]) @ dv / (dv @ dv))
        diffs[i] = math.log(p0 / (1.0 - p0))
    ek = o.encode(x, kc, rng.standard_normal((m, d)))  # S-independent parts
    a = o.rotate(q, kc)[0]
    c = kc.centroid.astype(np.float64)
    K = o.decode(ek["codes"], ek["norms"], kc)
    mean = []
    for t in range(2):
        rho = ek["z"][t] - c[ek["idx"][t]]
        n16, g16 = float(ek["norms"][t]), float(ek["gamma"][t])
        mean.append(scale * (q[0] @ K[t] + n16 * g16 / float(ek["gamma64"][t]) * (a @ rho) / d))
    want = mean[0] - mean[1]
    se = diffs.std() / math.sqrt(draws)
    assert abs(diffs.mean() - want) < 4 * se, (diffs.mean(), want, se)
    # the residual part is many standard errors away from zero: dropping the
    # QJL term, its scale or its sign would fail the check above
    resid = want - scale * (q[0] @ (K[0] - K[1]))
    assert abs(resid) > 10 * se


def test_second_sign_vector_reads_outputs_257_on():
    """signs2: bit 63 of SplitMix64 outputs 257.. (outputs 1..256 belong to
    the first sign vector, pinned by the published test vector)."""
    for seed, d in ((0, 64), (12345, 128), (2**63 + 5, 256)):
        outs = o.splitmix64(seed, 256 + d)
        want = np.array([-1.0 if (v >> 63) & 1 else 1.0 for v in outs[256:]])
        assert np.array_equal(o.second_sign_vector(seed, d), want)
        assert not np.array_equal(o.second_sign_vector(seed, d), o.sign_vector(seed, d))
        c = o.Codec(3, d, seed, residual=o.RES_SRHT)
        assert c.qjl_m == d and np.array_equal(c.signs2, want)


def test_srht_projection_is_an_orthogonal_sign_matrix():
    c = o.Codec(3, 128, 9, residual=o.RES_SRHT)
    P = c.projection()
    assert np.all(np.abs(P) == 1.0)
    np.testing.assert_array_equal(P @ P.T, 128 * np.eye(128))
    # u = S r is the second sign flip then the transform: H (signs2 * r)
    r = np.random.default_rng(30).standard_normal((3, 128))
    np.testing.assert_allclose(r @ P.T, o.rotate(r * c.signs2[None, :] * c.signs[None, :], c), rtol=1e-12, atol=1e-12)


def test_srht_estimator_nearly_unbiased():
    """Over random seeds (so random signs2), the SRHT residual term corrects the
    MSE estimate like the Gaussian QJL: the mean error of the full estimate is
    within 4 standard errors plus a 3% allowance for the bias of +-1
    projections, while the MSE-only estimate is clearly biased."""
    d = 256
    rng = np.random.default_rng(31)
    x = rng.standard_normal((1, d))
    q = x + 0.5 * rng.standard_normal((1, d))  # correlated, so the MSE error has a sign
    truth = float(q[0] @ x[0])
    err, err_mse = [], []
    for seed in range(400):
        c = o.Codec(1, d, 1000 + seed, residual=o.RES_SRHT)
        e = o.encode(x, c)
        est = o.ip_scores(q, e["codes"], e["norm"], e["qjl"], e["gamma64"], None, c)[0, 0]
        mse = o.ip_scores(q, e["codes"], e["norm"], None, None, None, o.Codec(1, d, 1000 + seed))[0, 0]
        err.append(est - truth)
        err_mse.append(mse - truth)
    err, err_mse = np.array(err), np.array(err_mse)
    se = err.std() / math.sqrt(len(err))
    assert abs(err.mean()) < 4 * se + 0.03 * abs(err_mse.mean())
    assert abs(err_mse.mean()) > 10 * se


def test_direct_sign_variance_ratio(golden_dir):
    """Direct Sign against the paper's QJL (Gaussian, m = d) on Gaussian
    residuals: the error variance of the inner-product correction is
    (1 - 2/pi)/(pi/2) = 0.2313 of QJL's, the printed 0.23 (4.3x lower)."""
    pages = _pages(golden_dir)
    d, n = 128, 400
    rng = np.random.default_rng(32)
    cs = o.Codec(2, d, 3, residual=o.RES_SIGN)
    e_ds, e_qjl = [], []
    for trial in range(25):
        r = rng.standard_normal((n, d)) * 0.2  # residuals in unit-vector units
        q = rng.standard_normal((1, d))
        a = o.rotate(q, cs)[0]
        truth = r @ a / math.sqrt(d)  # the residual part n <a/sqrt(d), r> at n = 1
        ones = np.ones(n)
        ds = o.qjl_term(q, o.pack_signs(r >= 0), ones, np.abs(r).mean(axis=1), None, cs)[0]
        S = rng.standard_normal((d, d))
        cq = o.Codec(2, d, 3, qjl_m=d)
        qj = o.qjl_term(q, o.pack_signs(r @ S.T >= 0), ones, np.linalg.norm(r, axis=1), S, cq)[0]
        e_ds.append(ds - truth)
        e_qjl.append(qj - truth)
    ratio = np.mean(np.concatenate(e_ds) ** 2) / np.mean(np.concatenate(e_qjl) ** 2)
    assert ratio == pytest.approx((1 - 2 / math.pi) / (math.pi / 2), rel=0.06)
    assert ratio == pytest.approx(float(pages["direct_sign_variance_ratio"]), abs=0.02)
    assert 1 / ratio == pytest.approx(float(pages["direct_sign_variance_reduction"]), rel=0.07)


def test_direct_sign_bits_and_scale():
    d = 128
    c = o.Codec(3, d, 4, residual=o.RES_SIGN)
    x = np.random.default_rng(33).standard_normal((10, d))
    e = o.encode(x, c)
    rho = e["z"] - c.centroid.astype(np.float64)[e["idx"]]
    assert np.array_equal(o.unpack_signs(e["qjl"], d), (rho >= 0).astype(np.uint8))
    np.testing.assert_allclose(e["gamma64"], np.abs(rho).sum(axis=1) / d / math.sqrt(d), rtol=1e-13)
    # the corrected estimate equals <q, x_hat + rebuilt residual>
    q = np.random.default_rng(34).standard_normal((2, d))
    est = o.ip_scores(q, e["codes"], e["norm"], e["qjl"], e["gamma64"], None, c)
    # rotated unit domain: centroid plus the rebuilt residual gamma*sqrt(d)*sign
    rebuilt = c.centroid.astype(np.float64)[e["idx"]] + e["gamma64"][:, None] * math.sqrt(d) * (2.0 * (rho >= 0) - 1.0)
    xr = e["norm"][:, None] * ((rebuilt @ c.H.T) / d) * c.signs[None, :]  # back through D H / d
    np.testing.assert_allclose(est, q @ xr.T, rtol=1e-11, atol=1e-11)


def test_qjl_bits_and_gamma():
    d, m = 128, 128
    rng = np.random.default_rng(14)
    S = rng.standard_normal((m, d))
    c = o.Codec(3, d, seed=0, qjl_m=m)
    x = rng.standard_normal((20, d))
    e = o.encode(x, c, S)
    assert e["qjl"].shape == (20, m // 8) and e["gamma"].dtype == np.float16
    bits = o.unpack_signs(e["qjl"], m)
    assert np.array_equal(bits, (e["u"] >= 0).astype(np.uint8))
    # gamma is the relative residual norm in orthonormal units: ~ sqrt(MSE)
    cc, tt = o.lloyd_max_gaussian(3)
    assert abs(np.mean(e["gamma64"] ** 2) / o.lloyd_max_mse(cc, tt) - 1) < 0.15
    # u = S r: each projection equals a direct dot product with the residual
    r = (e["z"] - c.centroid.astype(np.float64)[e["idx"]]) / math.sqrt(d)
    np.testing.assert_allclose(e["u"][3, 7], float(S[7] @ r[3]), rtol=1e-12)


# ----------------------------------------------------------------- Search ----
def test_topk_order_brute_force():
    scores = np.array([[0.5, 0.9, 0.9, 0.1, 0.5, 0.9, -1.0]])
    vals, ids = o.topk(scores, 5)
    brute = sorted(range(7), key=lambda i: (-scores[0, i], i))[:5]
    assert ids[0].tolist() == brute == [1, 2, 5, 0, 4]
    assert vals[0].tolist() == [0.9, 0.9, 0.9, 0.5, 0.5]


def test_ip_search_finds_planted_neighbour():
    d, m, n = 64, 64, 300
    rng = np.random.default_rng(15)
    S = rng.standard_normal((m, d))
    c = o.Codec(3, d, seed=1, qjl_m=m)
    db = rng.standard_normal((n, d))
    db /= np.linalg.norm(db, axis=1, keepdims=True)
    q = db[[17, 123]] + 0.05 * rng.standard_normal((2, d))
    e = o.encode(db, c, S)
    vals, ids = o.ip_search(q, e["codes"], e["norms"], e["qjl"], e["gamma"], S, c, 5)
    assert ids[0, 0] == 17 and ids[1, 0] == 123
    assert np.all(np.diff(vals, axis=1) <= 0)


# ---------------------------------------------------------------- Quality ----
def test_tiny_workload_quality_context():
    """Context number, not parity: the write-up reports ~99.5% attention-score
    similarity at 3 bits (idea.jsleekr, page summary).  Cosine of compressed vs
    exact score vectors on the tiny workload must be in that region."""
    import synth

    k, v, q, s = (t.numpy().astype(np.float64) for t in synth.tiny())
    c = o.Codec(3, 128, seed=0)
    e = o.encode(k, c)
    K = o.decode(e["codes"], e["norms"], c)
    exact, comp = q @ k.T, q @ K.T
    cos = np.sum(exact * comp, 1) / np.linalg.norm(exact, axis=1) / np.linalg.norm(comp, axis=1)
    assert cos.mean() > 0.98


# ------------------------------------------------- double transform (d=64) ----
def _fwht_loops(v):
    """In-place butterfly Walsh-Hadamard transform over the last axis, written
    with plain loops (an algorithm independent of the oracle's dense matrix)."""
    v = np.array(v, dtype=np.float64)
    n = v.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            for j in range(i, i + h):
                a, b = v[..., j].copy(), v[..., j + h].copy()
                v[..., j], v[..., j + h] = a + b, a - b
        h *= 2
    return v


def test_third_sign_vector_reads_outputs_513_on():
    for seed, d in ((0, 64), (77, 64), (2**63 + 5, 128)):
        outs = o.splitmix64(seed, 512 + d)
        want = np.array([-1.0 if (v >> 63) & 1 else 1.0 for v in outs[512:]])
        assert np.array_equal(o.third_sign_vector(seed, d), want)
        assert not np.array_equal(want, o.sign_vector(seed, d))
        assert not np.array_equal(want, o.second_sign_vector(seed, d))


def test_double_transform_is_two_butterflies():
    """S1 -> WHT -> S2 -> WHT ([P1] v1.5.3 item 1): the oracle's dense R D x
    equals two loop butterflies with the two sign flips, over sqrt(d); R R = d I
    exactly and R is symmetric, so decoding inverts it like H."""
    d = 64
    c = o.Codec(3, d, 21, rotation=o.ROT_DOUBLE)
    x = np.random.default_rng(40).standard_normal((5, d))
    want = _fwht_loops(_fwht_loops(x * c.signs[None, :]) * c.signs3[None, :]) / math.sqrt(d)
    np.testing.assert_allclose(o.rotate(x, c), want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(c.R @ c.R, d * np.eye(d))
    assert np.array_equal(c.R, c.R.T)
    # a plain transform in the middle would make R = sqrt(d) I: the second sign
    # flip is what mixes again (two butterflies of ones give d times the input)
    np.testing.assert_allclose(_fwht_loops(_fwht_loops(x)), d * x, rtol=1e-12)
    assert np.max(np.abs(c.R - math.sqrt(d) * np.eye(d))) > 1.0


def test_double_transform_round_trip_and_error():
    """Decode inverts the double rotation exactly (unquantised), and the
    reconstruction error of Gaussian inputs is the Lloyd-Max MSE (within 5% at
    d = 64, where the per-vector normalisation shifts it slightly)."""
    d, bits = 64, 3
    c = o.Codec(bits, d, 3, rotation=o.ROT_DOUBLE)
    x = np.random.default_rng(41).standard_normal((6000, d))
    # exact inverse: (R D)^-1 = D R / d
    y = o.rotate(x, c)
    np.testing.assert_allclose((y @ c.R.T / d) * c.signs[None, :], x, rtol=1e-11, atol=1e-11)
    e = o.encode(x, c)
    xh = o.decode(e["codes"], e["norm"], c)
    rel = np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1)
    cc, tt = o.lloyd_max_gaussian(bits)
    assert abs(rel.mean() / o.lloyd_max_mse(cc, tt) - 1) < 0.05


def test_double_transform_scores_in_the_rotated_domain():
    """The query takes the same double rotation as the keys, so scores need no
    inverse transform ([P1] v1.5.2 item 9: Q and K in the same domain)."""
    d = 64
    kc = o.Codec(4, d, 8, rotation=o.ROT_DOUBLE)
    rng = np.random.default_rng(42)
    ek = o.encode(rng.standard_normal((40, d)) * 20, kc)
    q = rng.standard_normal((3, d))
    K = o.decode(ek["codes"], ek["norms"], kc)
    rot = (o.rotate(q, kc) @ kc.centroid.astype(np.float64)[ek["idx"]].T) * ek["norms"].astype(np.float64)[None, :] / d
    np.testing.assert_allclose(q @ K.T, rot, rtol=1e-11, atol=1e-9)


def test_double_transform_brings_coordinates_closer_to_gaussian():
    """[P1] v1.5.3 item 1: at head_dim 64 one transform leaves the rotated
    coordinates far from Gaussian (excess kurtosis 0.375 on the page's keys)
    and the double transform brings them close (0.047).  On sparse inputs (four
    nonzero entries per 64) the excess kurtosis of the pooled coordinates of a
    single transform is about -1; the double transform more than halves its
    size, averaged over three seeds."""
    d, n = 64, 20000
    rng = np.random.default_rng(43)
    x = np.zeros((n, d))
    np.put_along_axis(x, rng.integers(0, d, (n, 4)), rng.standard_normal((n, 4)), 1)

    def excess(z):
        z = z.reshape(-1)
        return np.mean(z ** 4) / np.mean(z ** 2) ** 2 - 3.0

    one = np.mean([abs(excess(o.encode(x, o.Codec(3, d, s))["z"])) for s in range(3)])
    two = np.mean([abs(excess(o.encode(x, o.Codec(3, d, s, rotation=o.ROT_DOUBLE))["z"])) for s in range(3)])
    assert one > 0.8 and two < 0.5 * one, (one, two)


# ----------------------------------------------- per-block norms (d = 512) ----
def test_block_norms_split_the_norm():
    """[P1] v1.5.2 item 5: after the 512-point transform each 256-half has its
    own norm.  The block norms are the norms of the two halves of the
    orthonormally rotated vector (their squares add up to ||x||^2) and every
    block of z has unit mean square."""
    d = 512
    c = o.Codec(3, d, 4, norm_blocks=2)
    x = np.random.default_rng(44).standard_normal((7, d)) * np.linspace(0.5, 3.0, d)[None, :]
    e = o.encode(x, c)
    assert e["norms"].shape == (7, 2)
    np.testing.assert_allclose(np.sum(e["norm"] ** 2, axis=1), np.sum(x * x, axis=1), rtol=1e-12)
    y = (x * c.signs[None, :]) @ o.hadamard(d) / math.sqrt(d)  # orthonormal rotation
    np.testing.assert_allclose(e["norm"], np.linalg.norm(y.reshape(7, 2, 256), axis=2), rtol=1e-12)
    zb = e["z"].reshape(7, 2, 256)
    np.testing.assert_allclose(np.mean(zb ** 2, axis=2), 1.0, rtol=1e-12)


def test_block_norms_reduce_to_the_global_norm():
    """When both halves of the rotated vector have the same norm, the per-block
    codec gives the global codec's codes (both norms = ||x|| / sqrt(2)), and
    the decoded vectors agree up to the half rounding of the stored norms."""
    d = 512
    cb, cg = o.Codec(3, d, 6, norm_blocks=2), o.Codec(3, d, 6)
    rng = np.random.default_rng(45)
    u = rng.standard_normal((5, 256))
    y = np.concatenate([u, u[:, ::-1] * -1.0], axis=1)  # halves of equal norm
    x = (y @ o.hadamard(d) / d) * cb.signs[None, :]  # so that H D x = y
    eb, eg = o.encode(x, cb), o.encode(x, cg)
    np.testing.assert_allclose(eb["norm"], np.linalg.norm(x, axis=1)[:, None] / math.sqrt(2) * np.ones((1, 2)),
                               rtol=1e-12)
    assert np.array_equal(eb["idx"], eg["idx"])
    xb = o.decode(eb["codes"], eb["norms"], cb)
    xg = o.decode(eg["codes"], eg["norms"], cg)
    np.testing.assert_allclose(xb, xg, rtol=2e-3, atol=2e-3 * np.abs(xg).max())


def test_block_norms_follow_each_half():
    """Halves of very different size: each block is quantised at its own scale,
    so the small half keeps its Lloyd-Max relative error (a global norm would
    leave it with a fraction of its codes in use); the reconstruction error of
    each half is the Lloyd-Max MSE of that half."""
    d, bits = 512, 3
    c = o.Codec(bits, d, 7, norm_blocks=2)
    rng = np.random.default_rng(46)
    y = rng.standard_normal((3000, d))
    y[:, 256:] *= 0.01
    x = (y @ o.hadamard(d) / d) * c.signs[None, :]
    e = o.encode(x, c)
    xh = o.decode(e["codes"], e["norm"], c)
    yh = (xh * c.signs[None, :]) @ o.hadamard(d)
    cc, tt = o.lloyd_max_gaussian(bits)
    for h in range(2):
        sl = slice(256 * h, 256 * h + 256)
        rel = np.sum((y[:, sl] - yh[:, sl]) ** 2, axis=1) / np.sum(y[:, sl] ** 2, axis=1)
        assert abs(rel.mean() / o.lloyd_max_mse(cc, tt) - 1) < 0.03, (h, rel.mean())


def test_block_norms_refuse_a_residual():
    with pytest.raises(ValueError):
        o.Codec(3, 512, 1, qjl_m=64, norm_blocks=2)
