"""Plain CPU oracle for the TurboQuant KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

Everything is computed in float64 from the given inputs, one step after another
in the order the pages describe, with numpy primitives (matmul, sort, packbits)
as the only library steps.  Sources, cited as page title + section:

  [P1] "TurboQuant KV 캐시 압축 for llama.cpp" (stig.sh, AmesianX README_KO)
  [P2] "윈도우용 터보퀀트(TurboQuant) 구현을 개선하다" (idea.jsleekr.com)
  [P3] "[GitHub 탐방] TurboQuant 3-bit KV 캐시 압축 — 단일 GPU 재현 기록" (velog.io)

Readings where the pages are silent (each one is listed with its reason in the
design notes of the repository):
  * H is the unnormalised Sylvester Hadamard matrix, H[i][j] = (-1)^popcount(i&j);
    the rotated unit coordinate is z = H (D x) / ||x||, which has unit variance,
    so the codebook is the Lloyd-Max quantiser of N(0,1).
  * Sign i of D is -1 when bit 63 of the (i+1)-th SplitMix64 output for the
    seed is set.
  * idx_i = #{j : z_i > t_j} (a value exactly on a threshold goes to the lower
    cell); indices are packed as an LSB-first bit stream, index i at bits
    [b*i, b*i+b).
  * The norm is stored as IEEE half (round to nearest even, clamped to 65504).
  * QJL: residual in the rotated unit domain r = (z - c[idx]) / sqrt(d),
    gamma = ||r|| stored as half, bit_j = [(S r)_j >= 0] with S ~ N(0,1) [m][d]
    passed in by the caller; the inner-product estimator uses sqrt(pi/2)/m.

Every function here is pinned by tests/test_oracle_pins.py against values the
pages print, closed forms, textbook routines or brute force.
"""
from __future__ import annotations

import functools
import math

import numpy as np

_MASK64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15


# --------------------------------------------------------------------------
# Codebook: Lloyd-Max scalar quantiser of N(0,1)
# --------------------------------------------------------------------------
def _phi(x: float) -> float:
    """Standard normal density."""
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _upper_tail(x: float) -> float:
    """P(X > x) for X ~ N(0,1), accurate in the tail."""
    if math.isinf(x):
        return 0.0 if x > 0 else 1.0
    return 0.5 * math.erfc(x / math.sqrt(2.0))


def lloyd_max_gaussian(bits: int, tol: float = 1e-15, max_iter: int = 1_000_000):
    """Lloyd-Max quantiser for N(0,1) with 2^bits levels, in float64.

    [P1] names the scalar stage "Lloyd-Max 양자화" (page header); [P3] "GPU 세대가
    바뀌면 결과가 달라질까" describes it as mapping each coordinate to one of 2^bits
    centroids.  The quantiser is the fixed point of the two Lloyd conditions:
    every centroid is the conditional mean of its cell, and every threshold is
    the midpoint of its two neighbouring centroids.  The positive half is solved
    and mirrored, so the codebook is exactly symmetric and the middle threshold
    is exactly 0.  Start: thresholds at the uniform quantiles of N(0,1).

    Returns (centroids[L], thresholds[L-1]) in float64, ascending.
    """
    if not 1 <= bits <= 4:
        raise ValueError("bits must be 1..4")
    L = 1 << bits
    half = L // 2
    # positive-half cell edges tau[0]=0 < tau[1] < ... < tau[half-1] < tau[half]=inf
    from statistics import NormalDist

    nd = NormalDist()
    tau = [0.0] + [nd.inv_cdf(0.5 + k / L) for k in range(1, half)] + [math.inf]
    cent = [0.0] * half
    for _ in range(max_iter):
        for k in range(half):
            a, b = tau[k], tau[k + 1]
            mass = _upper_tail(a) - _upper_tail(b)
            cent[k] = (_phi(a) - _phi(b)) / mass
        new_tau = [0.0] + [0.5 * (cent[k - 1] + cent[k]) for k in range(1, half)] + [math.inf]
        delta = max((abs(new_tau[k] - tau[k]) for k in range(1, half)), default=0.0)
        tau = new_tau
        if delta < tol:
            break
    # final centroids for the final thresholds
    for k in range(half):
        a, b = tau[k], tau[k + 1]
        cent[k] = (_phi(a) - _phi(b)) / (_upper_tail(a) - _upper_tail(b))
    pos_c = np.array(cent, dtype=np.float64)
    centroids = np.concatenate([-pos_c[::-1], pos_c])
    pos_t = np.array([0.5 * (cent[k - 1] + cent[k]) for k in range(1, half)], dtype=np.float64)
    thresholds = np.concatenate([-pos_t[::-1], [0.0], pos_t])
    return centroids, thresholds


def lloyd_max_mse(centroids: np.ndarray, thresholds: np.ndarray) -> float:
    """E[(X - Q(X))^2] for X ~ N(0,1) and the quantiser (closed form per cell)."""
    edges = np.concatenate([[-np.inf], thresholds, [np.inf]])
    mse = 0.0
    for k, c in enumerate(centroids):
        a, b = float(edges[k]), float(edges[k + 1])
        mass = _upper_tail(a) - _upper_tail(b)
        # E[X^2 1_cell] = mass + a phi(a) - b phi(b);  E[X 1_cell] = phi(a) - phi(b)
        ax = 0.0 if math.isinf(a) else a * _phi(a)
        bx = 0.0 if math.isinf(b) else b * _phi(b)
        ex2 = mass + ax - bx
        ex1 = _phi(a) - _phi(b)
        mse += ex2 - 2.0 * c * ex1 + c * c * mass
    return mse


# --------------------------------------------------------------------------
# Random signs and the Hadamard matrix
# --------------------------------------------------------------------------
def splitmix64(seed: int, count: int) -> list[int]:
    """The first ``count`` outputs of SplitMix64 (Steele, Lea & Flood 2014;
    Vigna's public-domain reference) started from state ``seed``."""
    state = seed & _MASK64
    out = []
    for _ in range(count):
        state = (state + _GOLDEN) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def sign_vector(seed: int, d: int) -> np.ndarray:
    """Diagonal of D: the seeded +-1 sign flip ("tbq_signs", [P1] v1.7.0
    "핵심 설계 결정" item 4).  Sign i is -1 when bit 63 of output i+1 is set."""
    return np.array([-1.0 if (v >> 63) & 1 else 1.0 for v in splitmix64(seed, d)])


@functools.lru_cache(maxsize=None)
def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d from its definition (-1)^popcount(i&j).
    (Cached per d and returned read-only: it is a constant.)"""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    h = np.where(pc % 2 == 0, 1.0, -1.0)
    h.setflags(write=False)
    return h


# --------------------------------------------------------------------------
# Codec
# --------------------------------------------------------------------------
RES_NONE, RES_QJL, RES_SRHT, RES_SIGN = 0, 1, 2, 3


def second_sign_vector(seed: int, d: int) -> np.ndarray:
    """Second sign basis ("signs2" of [P1] v1.4.2 "MMA Tensor Core 가속" item 2,
    the SRHT QJL's own random signs): sign i is -1 when bit 63 of SplitMix64
    output 257 + i for the seed is set (outputs 1..256 belong to the first
    sign vector, whatever d)."""
    return np.array([-1.0 if (v >> 63) & 1 else 1.0 for v in splitmix64(seed, 256 + d)[256:]])


ROT_WHT, ROT_DOUBLE = 0, 1


def third_sign_vector(seed: int, d: int) -> np.ndarray:
    """Sign flip S2 of the double transform S1 -> WHT -> S2 -> WHT ([P1] v1.5.3
    "핵심 변경" item 1, head_dim 64): sign i is -1 when bit 63 of SplitMix64
    output 513 + i for the seed is set (outputs 1..512 belong to the first sign
    vector at any d up to 512, outputs 257.. to the SRHT basis)."""
    return np.array([-1.0 if (v >> 63) & 1 else 1.0 for v in splitmix64(seed, 512 + d)[512:]])


class Codec:
    """What one encoder/decoder needs: d, bits, residual kind and width,
    signs, codebook.

    The float64 Lloyd-Max values are rounded to float32 once; those float32
    centroids and thresholds define the quantiser.

    Residual kinds (one bit per projection, m of them, plus a half scale):
      RES_QJL   Gaussian projections S [m][d] given by the caller ([P1] "QJL
                보정 효과": the paper's TurboQuant_prod);
      RES_SRHT  the structured projection S = H diag(signs2), m = d: a second
                sign flip and Walsh-Hadamard transform ([P1] v1.3.0: QJL is
                SRHT-based in the original paper; v1.4.2 item 2: its second
                sign basis signs2);
      RES_SIGN  Direct Sign, m = d: the signs of the residual itself with
                their mean magnitude as the scale ([P1] v1.1.0 "Direct Sign —
                논문 QJL 대비 4.3배 낮은 분산").

    Rotation R (the transform after the sign flip D):
      ROT_WHT     R = H, the Sylvester Hadamard matrix;
      ROT_DOUBLE  R = H diag(signs3) H / sqrt(d): S1 -> WHT -> S2 -> WHT per head
                  ([P1] v1.5.3 "핵심 변경" item 1 and v1.5.2 item 9, head_dim 64,
                  where one transform leaves the coordinates too far from
                  Gaussian).  The 1/sqrt(d) keeps R R = d I, as for H, so z keeps
                  unit variance and decoding divides by d as before.
    Both R are symmetric.

    Norm blocks B ([P1] v1.5.2 "핵심 변경" item 5, d = 512: after the 512-point
    transform each 256-half gets its own norm; codecs with a residual keep the
    single norm): with y = R D x split into B blocks y_h of d/B coordinates,
    nu_h = ||y_h|| / sqrt(d) (the norm of that block of the orthonormally
    rotated vector, so sum_h nu_h^2 = ||x||^2), z_h = y_h / (nu_h sqrt(B)) and
    half(nu_h) is stored; B = 1 is the usual norm ||x||.
    """

    def __init__(self, bits: int, d: int, seed: int, qjl_m: int = 0, residual: int | None = None,
                 rotation: int = ROT_WHT, norm_blocks: int = 1):
        self.bits = int(bits)
        self.d = int(d)
        self.seed = int(seed)
        if residual is None:
            residual = RES_QJL if qjl_m else RES_NONE
        if residual in (RES_SRHT, RES_SIGN):
            qjl_m = self.d
        if residual == RES_NONE:
            qjl_m = 0
        self.residual = int(residual)
        self.qjl_m = int(qjl_m)
        c64, t64 = lloyd_max_gaussian(self.bits)
        self.centroid = c64.astype(np.float32)
        self.threshold = t64.astype(np.float32)
        self.signs = sign_vector(self.seed, self.d)
        self.signs2 = second_sign_vector(self.seed, self.d)
        self.signs3 = third_sign_vector(self.seed, self.d)
        self.H = hadamard(self.d)
        self.rotation = int(rotation)
        if self.rotation == ROT_WHT:
            self.R = self.H
        elif self.rotation == ROT_DOUBLE:
            self.R = (self.H * self.signs3[None, :]) @ self.H / math.sqrt(self.d)
        else:
            raise ValueError("unknown rotation")
        self.norm_blocks = int(norm_blocks)
        if self.norm_blocks not in (1, 2) or (self.norm_blocks > 1 and self.qjl_m):
            raise ValueError("norm blocks: 1, or 2 without a residual")

    @property
    def norm_shape_tail(self) -> tuple:
        """Trailing shape of one vector's stored norms: () or (B,)."""
        return () if self.norm_blocks == 1 else (self.norm_blocks,)

    def projection(self, S=None) -> np.ndarray:
        """The [m][d] projection of the residual: S (QJL), H diag(signs2)
        (SRHT) or the identity (Direct Sign)."""
        if self.residual == RES_QJL:
            if S is None or np.shape(S) != (self.qjl_m, self.d):
                raise ValueError("QJL needs S of shape [m][d]")
            return np.asarray(S, dtype=np.float64)
        if self.residual == RES_SRHT:
            return self.H * self.signs2[None, :]
        if self.residual == RES_SIGN:
            return np.eye(self.d)
        raise ValueError("codec has no residual")

    @property
    def residual_coef(self) -> float:
        """Estimator constant: sqrt(pi/2)/m for the projected signs (from
        E[sign(s.r)(s.a)] = sqrt(2/pi) <a, r>/||r||), 1 for Direct Sign (the
        scale is already the mean magnitude)."""
        return 1.0 if self.residual == RES_SIGN else math.sqrt(math.pi / 2) / self.qjl_m

    @property
    def code_bytes(self) -> int:
        return self.d * self.bits // 8

    @property
    def qjl_bytes(self) -> int:
        return self.qjl_m // 8


def packed_bytes(d: int, bits: int, qjl_m: int = 0) -> int:
    """Stored bytes per vector: d*bits/8 of codes + 2 B norm (+ m/8 + 2 B for QJL).

    [P1] "약간의 비하인드": a 3-bit head_dim-128 block is 50 B (48 B codes + norm);
    [P2] "핵심 발견 3": bit shifting packs several indices per byte.
    """
    total = d * bits // 8 + 2
    if qjl_m:
        total += qjl_m // 8 + 2
    return total


def to_half(x: np.ndarray) -> np.ndarray:
    """float64 -> IEEE half, round to nearest even, finite values clamped to 65504."""
    x = np.asarray(x, dtype=np.float64)
    return np.clip(x, -65504.0, 65504.0).astype(np.float16)


def pack_indices(idx: np.ndarray, bits: int) -> np.ndarray:
    """LSB-first bit stream: index i of a row occupies bits [bits*i, bits*i+bits)."""
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    shifts = np.arange(bits)
    bitplanes = (idx[:, :, None] >> shifts[None, None, :]) & 1  # [n][d][bits], bit b' of index i
    stream = bitplanes.reshape(n, d * bits).astype(np.uint8)
    return np.packbits(stream, axis=1, bitorder="little")


def unpack_indices(codes: np.ndarray, d: int, bits: int) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    stream = np.unpackbits(codes, axis=1, bitorder="little")[:, : d * bits]
    planes = stream.reshape(codes.shape[0], d, bits).astype(np.int64)
    return np.sum(planes << np.arange(bits)[None, None, :], axis=2)


def pack_signs(bits01: np.ndarray) -> np.ndarray:
    """m sign bits per row, bit j of the row stream = bits01[:, j]."""
    return np.packbits(np.asarray(bits01, dtype=np.uint8), axis=1, bitorder="little")


def unpack_signs(packed: np.ndarray, m: int) -> np.ndarray:
    return np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=1, bitorder="little")[:, :m]


def rotate(x: np.ndarray, codec: Codec) -> np.ndarray:
    """R (D x) per row: sign flip then the codec's transform R ([P1] v1.7.0
    "핵심 설계 결정" item 4: internal sign flip + butterfly WHT; R = H, or the
    double transform of v1.5.3), as a dense product."""
    x = np.asarray(x, dtype=np.float64)
    return (x * codec.signs[None, :]) @ codec.R.T


def quantize(z: np.ndarray, codec: Codec) -> np.ndarray:
    """idx = #{j : z > t_j} with the float32 thresholds (nearest centroid)."""
    t = codec.threshold.astype(np.float64)
    return np.sum(z[..., None] > t, axis=-1)


def encode(x: np.ndarray, codec: Codec, S: np.ndarray | None = None):
    """Encode rows of x (any float dtype, promoted to float64).

    Steps: norm; z = H(Dx)/norm (z = 0 for a zero vector); nearest Lloyd-Max
    index; LSB-first pack; half norm.  With QJL (codec.qjl_m > 0, S [m][d]):
    r = (z - c[idx]) / sqrt(d); gamma = ||r|| as half; bit_j = [(S r)_j >= 0].
    QJL is "the paper's TurboQuant_prod: a 1-bit residual correction on K"
    ([P1] "QJL 보정 효과"; [P1] v1.4.2 item 2 for sign bits + scalar per block).

    Returns dict(codes [n][d*b/8] u8, norms [n] f16, qjl [n][m/8] u8, gamma [n] f16,
    z [n][d] f64, idx [n][d] i64, u [n][m] f64).
    """
    x = np.asarray(x, dtype=np.float64)
    n_rows = x.shape[0]
    y = rotate(x, codec)
    if codec.norm_blocks == 1:
        norm = np.sqrt(np.sum(x * x, axis=1))
        safe = np.where(norm > 0, norm, 1.0)
        z = np.where(norm[:, None] > 0, y / safe[:, None], 0.0)
    else:
        # one norm per block of the rotated vector ([P1] v1.5.2 item 5)
        B = codec.norm_blocks
        yb = y.reshape(n_rows, B, codec.d // B)
        norm = np.sqrt(np.sum(yb * yb, axis=2)) / math.sqrt(codec.d)  # [n][B]
        safe = np.where(norm > 0, norm, 1.0) * math.sqrt(B)
        z = np.where(norm[:, :, None] > 0, yb / safe[:, :, None], 0.0).reshape(n_rows, codec.d)
    idx = quantize(z, codec)
    out = {
        "codes": pack_indices(idx, codec.bits),
        "norms": to_half(norm),
        "z": z,
        "idx": idx,
        "norm": norm,
    }
    if codec.qjl_m:
        P = codec.projection(S)
        c = codec.centroid.astype(np.float64)
        r = (z - c[idx]) / math.sqrt(codec.d)
        if codec.residual == RES_SIGN:
            gamma = np.sum(np.abs(r), axis=1) / codec.d  # mean magnitude: the best scale for fixed signs
        else:
            gamma = np.sqrt(np.sum(r * r, axis=1))
        u = r @ P.T
        out["qjl"] = pack_signs(u >= 0.0)
        out["gamma"] = to_half(gamma)
        out["gamma64"] = gamma
        out["u"] = u
        out["r"] = r
    else:
        out["qjl"] = np.zeros((n_rows, 0), dtype=np.uint8)
        out["gamma"] = np.zeros((n_rows,), dtype=np.float16)
    return out


def decode(codes: np.ndarray, norms16: np.ndarray, codec: Codec) -> np.ndarray:
    """x_hat = n16 * D * R(c[idx]) / d (R R = d I with R symmetric, D D = I);
    with norm blocks each block of c[idx] is scaled by half(nu_h) sqrt(B) first."""
    idx = unpack_indices(codes, codec.d, codec.bits)
    c = codec.centroid.astype(np.float64)[idx]
    n16 = np.asarray(norms16, dtype=np.float64)
    if codec.norm_blocks == 1:
        return n16[:, None] * (c @ codec.R.T / codec.d) * codec.signs[None, :]
    B = codec.norm_blocks
    yb = c.reshape(c.shape[0], B, codec.d // B) * (n16.reshape(-1, B)[:, :, None] * math.sqrt(B))
    return (yb.reshape(c.shape[0], codec.d) @ codec.R.T / codec.d) * codec.signs[None, :]


def append(codes, norms16, x_new, pos, codec: Codec, S=None, qjl=None, gamma16=None):
    """Decode-step append into a packed cache ([P3] "결과 — 피크 VRAM": every
    step the new K/V enters the cache before attention).

    codes [B][H][cap][row], norms16 [B][H][cap] (and with QJL qjl [B][H][cap][m/8],
    gamma16 [B][H][cap]) are updated in place: the new vector x_new[b][h] of every
    (sequence, head) is encoded and written at token pos[b]; a position outside
    [0, cap) writes nothing.  Returns the encode() result of all new vectors.
    """
    B, H, cap = norms16.shape
    flat = np.asarray(x_new, dtype=np.float64).reshape(B * H, -1)
    enc = encode(flat, codec, S)
    for b in range(B):
        p = int(pos[b])
        if not 0 <= p < cap:
            continue
        for h in range(H):
            r = b * H + h
            codes[b, h, p] = enc["codes"][r]
            norms16[b, h, p] = enc["norms"][r]
            if codec.qjl_m:
                qjl[b, h, p] = enc["qjl"][r]
                gamma16[b, h, p] = enc["gamma"][r]
    return enc


def prefill(codes, norms16, x_chunk, t0: int, codec: Codec, S=None, qjl=None, gamma16=None):
    """Chunked prefill into one sequence's packed cache ([P3] "실험 설계": the
    prompt's K/V enter the compressed cache chunk by chunk before decoding).

    codes [H][cap][row], norms16 [H][cap] (with QJL qjl [H][cap][m/8], gamma16
    [H][cap]) are updated in place: token t of head h in x_chunk [H][T][d] is
    encoded and written at slot t0 + t.  Requires 0 <= t0 and t0 + T <= cap.
    Returns the encode() result of the chunk's rows (head-major).
    """
    H, T, d = np.asarray(x_chunk).shape
    cap = norms16.shape[1]
    if t0 < 0 or t0 + T > cap:
        raise ValueError("chunk outside the cache")
    enc = encode(np.asarray(x_chunk, dtype=np.float64).reshape(H * T, d), codec, S)
    for h in range(H):
        rows = slice(h * T, (h + 1) * T)
        codes[h, t0:t0 + T] = enc["codes"][rows]
        norms16[h, t0:t0 + T] = enc["norms"][rows]
        if codec.qjl_m:
            qjl[h, t0:t0 + T] = enc["qjl"][rows]
            gamma16[h, t0:t0 + T] = enc["gamma"][rows]
    return enc


def qjl_term(q: np.ndarray, qjl_packed: np.ndarray, norms16: np.ndarray,
             gamma16: np.ndarray, S: np.ndarray, codec: Codec) -> np.ndarray:
    """QJL estimate of <q, x - x_hat> for every (query, row) pair.

    With a = H(Dq): <q, x> = n/d <a, z> and the residual part n/d <a, rho> is
    estimated by n * gamma * sqrt(pi/2)/m * <S a / sqrt(d), sign(S r)>, which is
    unbiased over S because E[sign(s.r) (s.a)] = sqrt(2/pi) <a, r>/||r|| for
    s ~ N(0, I).  ([P1] "Attention Sharpening" describes the same scalar
    correction d_qjl * sum(Q_wht2[i] * sign[i]).)  The SRHT kind uses
    S = H diag(signs2) (rows of +-1, nearly Gaussian projections); Direct Sign
    uses S = I and the constant 1: n * gamma * <a / sqrt(d), sign(r)> with gamma
    the mean |r_i|, the residual rebuilt as gamma * sign(r).  Returns
    [n_q][n_rows].
    """
    m = codec.qjl_m
    a = rotate(np.atleast_2d(q), codec)
    qhat = (a / math.sqrt(codec.d)) @ codec.projection(S).T  # [n_q][m]
    sgn = 2.0 * unpack_signs(qjl_packed, m).astype(np.float64) - 1.0  # [n][m]
    coef = np.asarray(norms16, np.float64) * np.asarray(gamma16, np.float64) * codec.residual_coef
    return (qhat @ sgn.T) * coef[None, :]


SCORE_PLAIN, SCORE_SHARPEN, SCORE_SOFTEN = 0, 1, 2


def score_factor(mode: int, n_tokens: int, sqnr: float, n0: int = 2048) -> float:
    """The factor alpha(N) multiplying every attention score of a query that
    attends over N tokens ([P1] v1.5.2 "핵심 변경" item 3 and "Attention
    Sharpening — 이론 & 동적 α 공식": quantisation noise in K flattens the
    softmax; the dynamic factor compensates, with N the current KV token count
    and N0 = 2048 the reference context):

      sharpen: alpha = 1 + c sqrt(ln N),  c = 1 / (2 SQNR_eff sqrt(ln N0));
      soften (item 11, the MMSE softening used at head_dim 64):
               alpha = SQNR / (SQNR + sqrt(ln N / ln N0));
      plain:   alpha = 1.
    N <= 1 gives ln N <= 0, read as 0 (alpha = 1): a single token's weight is 1
    whatever the factor.  The pages do not print SQNR_eff per cache type, so it
    is the caller's parameter.
    """
    if mode == SCORE_PLAIN or n_tokens <= 1:
        return 1.0
    ln_n, ln_n0 = math.log(n_tokens), math.log(n0)
    if mode == SCORE_SHARPEN:
        return 1.0 + math.sqrt(ln_n) / (2.0 * sqnr * math.sqrt(ln_n0))
    if mode == SCORE_SOFTEN:
        return sqnr / (sqnr + math.sqrt(ln_n / ln_n0))
    raise ValueError("unknown score mode")


def attention(q: np.ndarray, k_codes, k_norms, v_codes, v_norms, kc: Codec, vc: Codec,
              scale: float, k_qjl=None, k_gamma=None, S=None, k_win=None, v_win=None,
              alpha: float = 1.0, sparse_v: float = 0.0) -> np.ndarray:
    """Exact softmax attention of one query group over one decoded cache.

    Decompress-then-attend ([P3] "결과 — 피크 VRAM" describes the reference
    implementation materialising the full fp16 K/V each step): K_hat, V_hat are
    decoded, s_t = scale <q, K_hat_t> (+ the QJL estimate of the residual part),
    p = softmax(s) (max-subtracted), o = sum_t p_t V_hat_t.

    Residual window ([P3] "실험 설계" and "결과 — 피크 VRAM": the most recent
    tokens are kept uncompressed and appended to the decompressed ones before
    attention): k_win, v_win [w][d] are exact keys and values that join the
    softmax after the decoded tokens, with s = scale <q, k_win_t> (no QJL term).

    Score factor: every score (QJL part included) is multiplied by alpha
    (see score_factor).  Sparse V (the sparse V dequantisation of [P3] "왜 이걸
    보게 됐나": value rows whose softmax weight is below 1e-6 are not
    dequantised): with sparse_v = tau > 0 a token whose weight relative to the
    largest one, exp(s_t - max_u s_u), is below tau adds nothing to the output,
    while the softmax denominator keeps every token.

    q [n_q][d]; caches [ctx][...]; returns [n_q][d] float64.  With no token at
    all the output is zero.
    """
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    ctx = k_codes.shape[0]
    w = 0 if k_win is None else np.asarray(k_win).shape[0]
    if ctx + w == 0:
        return np.zeros((q.shape[0], vc.d))
    parts_s, parts_v = [], []
    if ctx:
        K = decode(k_codes, k_norms, kc)
        s = scale * (q @ K.T)
        if kc.qjl_m:
            s = s + scale * qjl_term(q, k_qjl, k_norms, k_gamma, S, kc)
        parts_s.append(s)
        parts_v.append(decode(v_codes, v_norms, vc))
    if w:
        parts_s.append(scale * (q @ np.asarray(k_win, dtype=np.float64).T))
        parts_v.append(np.asarray(v_win, dtype=np.float64))
    s = alpha * np.concatenate(parts_s, axis=1)
    V = np.concatenate(parts_v, axis=0)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    w = np.where(e < sparse_v, 0.0, e) if sparse_v > 0 else e
    return (w / e.sum(axis=1, keepdims=True)) @ V


def gqa_attention(q, ctx_len, k_codes, k_norms, v_codes, v_norms, kc, vc, scale,
                  k_qjl=None, k_gamma=None, S=None, heads=None, k_win=None, v_win=None, win_len=None):
    """Batched grouped-query attention: q [B][Hq][d], caches [B][Hkv][cap][...].

    Query head h reads kv head h // (Hq/Hkv).  ``heads`` optionally restricts the
    computation to a list of (b, h) pairs; the result then has one row per pair.
    Optional residual windows k_win, v_win [B][Hkv][win_cap][d] hold win_len[b]
    exact tokens of sequence b.
    """
    B, Hq, d = q.shape
    Hkv = k_codes.shape[1]
    g = Hq // Hkv
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    out = np.zeros((len(pairs), vc.d))
    for row, (b, h) in enumerate(pairs):
        kh = h // g
        n = int(ctx_len[b])
        args = {}
        if kc.qjl_m:
            args = dict(k_qjl=k_qjl[b, kh, :n], k_gamma=k_gamma[b, kh, :n], S=S)
        if k_win is not None:
            wl = int(win_len[b])
            args.update(k_win=k_win[b, kh, :wl], v_win=v_win[b, kh, :wl])
        out[row] = attention(q[b, h][None, :], k_codes[b, kh, :n], k_norms[b, kh, :n],
                             v_codes[b, kh, :n], v_norms[b, kh, :n], kc, vc, scale, **args)[0]
    return out


def mq_attention(q, ctx_len, k_codes, k_norms, v_codes, v_norms, kc, vc, scale,
                 k_qjl=None, k_gamma=None, S=None, cols=None, score_mode=SCORE_PLAIN, sqnr=1.0,
                 n0=2048, sparse_v=0.0):
    """Multi-query decode over the packed cache: q [B][C][Hq][d] holds the last C
    query tokens (columns) of each sequence, whose keys and values are already
    in the cache ([P1] v1.1.0 "버그 수정": prompt evaluation runs ncols = 2 query
    columns through the same attention kernel; [P1] v1.4.2 "MMA Tensor Core 가속"
    serves several columns at once).  Column c of sequence b sits at position
    ctx_len[b] - C + c and attends causally: over the first
    max(0, ctx_len[b] - (C - 1 - c)) tokens of its cache, with everything else
    as in gqa_attention.

    ``cols`` optionally restricts the computation to a list of (b, c, h)
    triples; the result then has one row per triple.  Returns [B*C*Hq][d] in
    (b, c, h) order otherwise.  score_mode / sqnr / n0 select the score factor
    alpha(N) of each column, N being the tokens it attends over; sparse_v is
    attention()'s threshold.
    """
    B, C, Hq, d = q.shape
    Hkv = k_codes.shape[1]
    g = Hq // Hkv
    trip = cols if cols is not None else [(b, c, h) for b in range(B) for c in range(C) for h in range(Hq)]
    out = np.zeros((len(trip), vc.d))
    for row, (b, c, h) in enumerate(trip):
        kh = h // g
        n = max(0, int(ctx_len[b]) - (C - 1 - c))
        args = {}
        if kc.qjl_m:
            args = dict(k_qjl=k_qjl[b, kh, :n], k_gamma=k_gamma[b, kh, :n], S=S)
        out[row] = attention(np.asarray(q[b, c, h], dtype=np.float64)[None, :], k_codes[b, kh, :n],
                             k_norms[b, kh, :n], v_codes[b, kh, :n], v_norms[b, kh, :n], kc, vc, scale,
                             alpha=score_factor(score_mode, n, sqnr, n0), sparse_v=sparse_v, **args)[0]
    return out


def ip_scores(q: np.ndarray, codes, norms16, qjl_packed, gamma16, S, codec: Codec) -> np.ndarray:
    """Unbiased inner-product estimates <q, x_t> for all (query, database row) pairs.

    est = n16 (<H(Dq), c[idx]>/d + gamma16 sqrt(pi/2)/m <S H(Dq)/sqrt(d), 2 bit - 1>);
    the vector-search use case for which the QJL term is unbiased and helps
    ([P2] "핵심 발견 1 — QJL 레이어를 제거하라": no softmax in vector search).
    """
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    X = decode(codes, norms16, codec)
    est = q @ X.T
    if codec.qjl_m:
        est = est + qjl_term(q, qjl_packed, norms16, gamma16, S, codec)
    return est


def topk(scores: np.ndarray, k: int):
    """Per row, the k largest scores ordered by (score desc, id asc)."""
    scores = np.atleast_2d(scores)
    n_q, n = scores.shape
    ids = np.zeros((n_q, k), dtype=np.int64)
    vals = np.zeros((n_q, k))
    ar = np.arange(n)
    for i in range(n_q):
        order = np.lexsort((ar, -scores[i]))[:k]
        ids[i] = order
        vals[i] = scores[i, order]
    return vals, ids


def ip_search(q, codes, norms16, qjl_packed, gamma16, S, codec: Codec, k: int):
    """Estimator over every database row, then exact top-k per query."""
    return topk(ip_scores(q, codes, norms16, qjl_packed, gamma16, S, codec), k)
