"""GPU parity of the softmax-side switches of tq_attn_decode_ex (dynamic
sharpening / MMSE softening of the scores, sparse V) against the oracle."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import tq_oracle as o
from tests import parity
from tests.test_gpu_attn import oracle_cache, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_02_amd as lib
    return lib


def gpu_ex(tq, kc, vc, q, ctx_len, dev, scale, opts, S=None):
    B, C, Hq, d = q.shape
    Hkv, cap = dev["k_codes"].shape[1], dev["k_codes"].shape[2]
    ws = tq.workspace(tq.tq_workspace_bytes(tq.TQ_OP_ATTN_DECODE_MQ, kc, vc, B, Hq, Hkv, cap, n_q=C))
    ws.fill_(0xFF)
    out = torch.full((B, C, Hq, d), float("nan"), device="cuda")
    cl = torch.tensor(ctx_len, dtype=torch.int32, device="cuda")
    tq.tq_attn_decode_ex(kc, vc, q, cl, dev["k_codes"], dev["k_norms"], dev["v_codes"], dev["v_norms"], scale, out,
                         ws, opts, dev.get("k_qjl"), dev.get("k_gamma"), S)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("mode,sqnr,C,m", [(1, 11.6, 1, 0), (1, 3.0, 3, 0), (2, 2.0, 2, 0), (1, 5.0, 2, 128)])
def test_score_factor_parity(tq, mode, sqnr, C, m):
    """Sharpened / softened scores (each row's alpha from its own token count)
    match the oracle; the factor moves the output well beyond the tolerance."""
    B, Hkv, g, cap, d = 2, 2, 4, 900, 128
    kk = torch.stack([synth.kv_block(Hkv, cap, d, 60 + b, dtype=torch.float32)[0] for b in range(B)])
    vv = torch.stack([synth.kv_block(Hkv, cap, d, 60 + b, dtype=torch.float32)[1] for b in range(B)])
    S = synth.qjl_projection(m, d, seed=61) if m else None
    S64 = None if S is None else S.numpy().astype(np.float64)
    kc_r, vc_r = o.Codec(4, d, 3, m), o.Codec(2, d, 3)
    kc, vc = tq.tq_codebook(4, d, 3, m), tq.tq_codebook(2, d, 3)
    cache = oracle_cache(kk.numpy().astype(np.float64), vv.numpy().astype(np.float64), kc_r, vc_r, S64)
    q = synth.normal((B, C, Hkv * g, d), seed=62, dtype=torch.float16)
    ctx = [900, 5]
    scale = 1 / math.sqrt(d)
    opts = tq.tq_attn_opts(mode, sqnr, 0, 0.0)
    got = gpu_ex(tq, kc, vc, q.cuda(), ctx, to_dev(cache), scale, opts, None if S is None else S.cuda())
    args = (q.float().numpy().astype(np.float64), ctx, cache["k_codes"], cache["k_norms"], cache["v_codes"],
            cache["v_norms"], kc_r, vc_r, scale, cache.get("k_qjl"), cache.get("k_gamma"), S64)
    ref = o.mq_attention(*args, score_mode=mode, sqnr=sqnr)
    plain = o.mq_attention(*args)
    got = got.reshape(-1, d)
    assert np.all(np.isfinite(got))
    assert parity.rel_rows(got, ref).max() <= parity.ATTN_TOL
    assert parity.rel_rows(plain, ref).max() > 10 * parity.ATTN_TOL


def _sparse_case(tq, tau, seed=70, g=2):
    """Keys whose 64-token tiles all open with the same dominant key, so every
    wave's running maximum is the true maximum from its first tile on and the
    kernels drop exactly the tokens the oracle drops."""
    B, Hkv, cap, d = 1, 2, 1500, 128
    rng = np.random.default_rng(seed)
    qv = rng.standard_normal(d)
    qv /= np.linalg.norm(qv)
    # scores <q, k>: N(0, 4) for the random keys (their maximum over the
    # context stays near 6.4) and 8 for the dominant keys, so many tokens carry
    # weights between 1e-4 and 0.02 of the largest
    K = rng.standard_normal((B, Hkv, cap, d)) * 2.0
    K[:, :, ::64] = 8.0 * qv  # dominant, identical keys
    V = rng.standard_normal((B, Hkv, cap, d))
    kc_r, vc_r = o.Codec(4, d, 5), o.Codec(3, d, 5)
    kc, vc = tq.tq_codebook(4, d, 5), tq.tq_codebook(3, d, 5)
    cache = oracle_cache(K, V, kc_r, vc_r)
    q = torch.from_numpy(np.broadcast_to(qv, (B, 1, Hkv * g, d)).copy()).float()  # the same query in every head
    scale = 1.0
    opts = tq.tq_attn_opts(0, 0.0, 0, tau)
    got = gpu_ex(tq, kc, vc, q.cuda(), [cap], to_dev(cache), scale, opts).reshape(-1, d)
    args = (q.numpy().astype(np.float64), [cap], cache["k_codes"], cache["k_norms"], cache["v_codes"],
            cache["v_norms"], kc_r, vc_r, scale)
    return got, o.mq_attention(*args, sparse_v=tau), o.mq_attention(*args)


@pytest.mark.parametrize("g", [2, 16])
def test_sparse_v_drops_what_the_oracle_drops(tq, g):
    """g = 16 runs blocks of 16 query rows."""
    got, ref, plain = _sparse_case(tq, 0.02, g=g)
    assert np.all(np.isfinite(got))
    assert parity.rel_rows(got, ref).max() <= parity.ATTN_TOL
    assert parity.rel_rows(plain, ref).max() > 10 * parity.ATTN_TOL  # the switch matters here


def test_sparse_v_at_the_pages_threshold(tq, golden_dir):
    """At the pages' 1e-6 the dropped weight is negligible: the output stays
    within the tolerance of both the sparse and the plain oracle."""
    import os
    tau = float([ln.split("|")[1] for ln in open(os.path.join(golden_dir, "pages_numbers.txt"), encoding="utf-8")
                 if ln.startswith("sparse_v_threshold")][0])
    got, ref, plain = _sparse_case(tq, tau, seed=71)
    assert parity.rel_rows(got, ref).max() <= parity.ATTN_TOL
    assert parity.rel_rows(got, plain).max() <= parity.ATTN_TOL


def test_sparse_v_general_bound(tq):
    """On the decode recipe (no planted maximum) the kernels' running maxima
    may keep more tokens than the oracle drops; the difference stays within the
    weight of the tokens the oracle drops (times their values' norms)."""
    B, Hkv, g, cap, d, tau = 2, 2, 7, 3000, 128, 1e-3
    kk = torch.stack([synth.kv_block(Hkv, cap, d, 80 + b, dtype=torch.float32)[0] for b in range(B)])
    vv = torch.stack([synth.kv_block(Hkv, cap, d, 80 + b, dtype=torch.float32)[1] for b in range(B)])
    kc_r, vc_r = o.Codec(4, d, 7), o.Codec(2, d, 7)
    kc, vc = tq.tq_codebook(4, d, 7), tq.tq_codebook(2, d, 7)
    cache = oracle_cache(kk.numpy().astype(np.float64), vv.numpy().astype(np.float64), kc_r, vc_r)
    q = synth.normal((B, 1, Hkv * g, d), seed=81, dtype=torch.float16)
    scale = 1 / math.sqrt(d)
    got = gpu_ex(tq, kc, vc, q.cuda(), [cap, 1234], to_dev(cache), scale, tq.tq_attn_opts(0, 0.0, 0, tau))
    got = got.reshape(B, Hkv * g, d)
    qn = q.float().numpy().astype(np.float64)
    for b, n in ((0, cap), (1, 1234)):
        for h in range(Hkv * g):
            kh = h // g
            kcd, knn = cache["k_codes"][b, kh, :n], cache["k_norms"][b, kh, :n]
            vcd, vnn = cache["v_codes"][b, kh, :n], cache["v_norms"][b, kh, :n]
            ref = o.attention(qn[b, 0, h][None], kcd, knn, vcd, vnn, kc_r, vc_r, scale, sparse_v=tau)[0]
            K = o.decode(kcd, knn, kc_r)
            Vd = o.decode(vcd, vnn, vc_r)
            s = scale * K @ qn[b, 0, h]
            e = np.exp(s - s.max())
            bound = float(np.where(e < tau, e / e.sum(), 0.0) @ np.linalg.norm(Vd, axis=1))
            err = np.linalg.norm(got[b, h] - ref)
            assert err <= bound + parity.ATTN_TOL * np.linalg.norm(ref), (b, h, err, bound)
