"""Python binding of libtq.so (include/tq.h): argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors for device buffers (torch supplies device memory and the current HIP
stream) and raises TQError on a non-zero return code.  All arithmetic runs in
the HIP kernels; there is no CPU fallback: importing this package fails if the
library has not been built (``python -m kv_cache_vector_02_amd._build`` or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EWORKSPACE, TQ_EDEVICE = 0, -1, -2, -3, -4
TQ_F32, TQ_F16, TQ_BF16 = 0, 1, 2

_DTYPES = {torch.float32: TQ_F32, torch.float16: TQ_F16, torch.bfloat16: TQ_BF16}

EXPORTS = (
    "tq_codebook", "tq_encode", "tq_encode_kv", "tq_prefill", "tq_append", "tq_decode", "tq_attn_decode", "tq_attn_prepare", "tq_attn_scan",
    "tq_attn_combine", "tq_attn_decode_rw", "tq_attn_workspace_bytes",
    "tq_ip_search", "tq_search_workspace_bytes", "tq_packed_bytes", "tq_strerror",
)


class tq_codec(ctypes.Structure):
    """Mirror of the C struct tq_codec."""

    _fields_ = [
        ("d", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("qjl_m", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
        ("sign_mask", ctypes.c_uint32 * 8),
        ("centroid", ctypes.c_float * 16),
        ("threshold", ctypes.c_float * 15),
    ]

    @property
    def code_bytes(self) -> int:
        return self.d * self.bits // 8

    @property
    def centroids(self) -> list[float]:
        return [self.centroid[i] for i in range(1 << self.bits)]

    @property
    def thresholds(self) -> list[float]:
        return [self.threshold[i] for i in range((1 << self.bits) - 1)]

    @property
    def signs(self) -> list[float]:
        return [-1.0 if (self.sign_mask[i >> 5] >> (i & 31)) & 1 else 1.0 for i in range(self.d)]


class TQError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} ({code})")
        self.code = code


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libtq.so not built at {_LIB_PATH}; run __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    CP = ctypes.POINTER(tq_codec)
    sig = {
        "tq_codebook": (I, [I, I, ctypes.c_uint64, I, CP]),
        "tq_encode": (I, [CP, P, I, I64, I64, P, I64, P, P, P, P, P]),
        "tq_encode_kv": (I, [CP, CP, P, P, I, I64, I64, P, I64, P, P, I64, P, P, P, P, P]),
        "tq_prefill": (I, [CP, CP, P, P, I, I, I64, I64, I64, P, P, P, P, P, P, P, P]),
        "tq_append": (I, [CP, CP, P, P, I, I, I, P, I64, P, P, P, P, P, P, P, P]),
        "tq_decode": (I, [CP, P, I64, P, I64, P, P]),
        "tq_attn_decode": (I, [CP, CP, P, I, I, I, I, P, I64, P, P, P, P, P, P, P, F, P, P, SZ, P]),
        "tq_attn_prepare": (I, [CP, CP, P, I, I, I, I, P, I64, P, P, P, P, P, P, P, F, P, P, SZ, P]),
        "tq_attn_scan": (I, [CP, CP, P, I, I, I, I, P, I64, P, P, P, P, P, P, P, F, P, P, SZ, P]),
        "tq_attn_combine": (I, [CP, CP, P, I, I, I, I, P, I64, P, P, P, P, P, P, P, F, P, P, SZ, P]),
        "tq_attn_decode_rw": (I, [CP, CP, P, I, I, I, I, P, I64, P, P, P, P, P, P, P, P, P, I, P, I, F, P, P, SZ, P]),
        "tq_attn_workspace_bytes": (SZ, [CP, CP, I, I, I, I64]),
        "tq_ip_search": (I, [CP, P, I, P, P, P, P, P, I64, I, P, P, P, SZ, P]),
        "tq_search_workspace_bytes": (SZ, [CP, I, I64, I]),
        "tq_packed_bytes": (SZ, [I, I, I]),
        "tq_strerror": (ctypes.c_char_p, [I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
LIB_PATH = _LIB_PATH


def strerror(code: int) -> str:
    return _lib.tq_strerror(code).decode()


def _check(code: int, where: str):
    if code != TQ_OK:
        raise TQError(code, where)


def _ptr(t):
    """Device address of a torch tensor (None passes through as NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    return t.data_ptr()


_raw_stream = torch._C._cuda_getCurrentRawStream


def _stream(stream=None, like=None):
    """hipStream_t of `stream`, else of the current stream of `like`'s device."""
    if stream is not None:
        return stream.cuda_stream
    return _raw_stream(like.get_device() if like is not None else torch.cuda.current_device())


def tq_codebook(bits: int, d: int, seed: int, qjl_m: int = 0) -> tq_codec:
    """Host-only: codec with the Lloyd-Max codebook and the seeded sign mask."""
    c = tq_codec()
    _check(_lib.tq_codebook(bits, d, ctypes.c_uint64(seed & (2**64 - 1)), qjl_m, ctypes.byref(c)), "tq_codebook")
    return c


def tq_packed_bytes(d: int, bits: int, qjl_m: int = 0) -> int:
    return _lib.tq_packed_bytes(d, bits, qjl_m)


def tq_encode(codec: tq_codec, x: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor,
              qjl_S: torch.Tensor | None = None, qjl_bits: torch.Tensor | None = None,
              qjl_gamma: torch.Tensor | None = None, stream=None) -> None:
    """x [n][>=d] (fp32/fp16/bf16, last dim contiguous); codes [n][>= d*bits/8] uint8;
    norms [n] (2-byte dtype, half bits).  Row strides are taken from the tensors."""
    if x.dim() != 2 or x.stride(1) != 1 or codes.dim() != 2 or codes.stride(1) != 1:
        raise ValueError("x and codes must be 2-D with contiguous rows")
    n = x.shape[0]
    _check(_lib.tq_encode(ctypes.byref(codec), _ptr(x), _DTYPES[x.dtype], n, x.stride(0), _ptr(codes),
                          codes.stride(0), _ptr(norms), _ptr(qjl_S), _ptr(qjl_bits), _ptr(qjl_gamma),
                          _stream(stream, x)), "tq_encode")


def tq_encode_kv(kc: tq_codec, vc: tq_codec, k: torch.Tensor, v: torch.Tensor, k_codes: torch.Tensor,
                 k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
                 qjl_S: torch.Tensor | None = None, k_qjl_bits: torch.Tensor | None = None,
                 k_qjl_gamma: torch.Tensor | None = None, stream=None) -> None:
    """tq_encode of keys and values in one call: k, v [n][>=d] of one dtype and
    row stride (last dim contiguous); codes [n][>= d*bits/8] uint8; norms [n]."""
    for t in (k, v, k_codes, v_codes):
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("k, v and the code planes must be 2-D with contiguous rows")
    if k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v must share shape, strides and dtype")
    _check(_lib.tq_encode_kv(ctypes.byref(kc), ctypes.byref(vc), _ptr(k), _ptr(v), _DTYPES[k.dtype], k.shape[0],
                             k.stride(0), _ptr(k_codes), k_codes.stride(0), _ptr(k_norms), _ptr(v_codes),
                             v_codes.stride(0), _ptr(v_norms), _ptr(qjl_S), _ptr(k_qjl_bits), _ptr(k_qjl_gamma),
                             _stream(stream, k)), "tq_encode_kv")


def tq_prefill(kc: tq_codec, vc: tq_codec, k: torch.Tensor, v: torch.Tensor, t0: int, k_codes: torch.Tensor,
               k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
               qjl_S: torch.Tensor | None = None, k_qjl_bits: torch.Tensor | None = None,
               k_qjl_gamma: torch.Tensor | None = None, stream=None) -> None:
    """k, v [H][T][d] (one dtype) contiguous; one sequence's cache planes
    [H][cap][d*bits/8] uint8 and norms [H][cap] (2-byte dtype), contiguous (a
    slice [b] of a batched cache is); writes slots [t0, t0 + T) of every head."""
    for t in (k, v, k_codes, k_norms, v_codes, v_norms):
        if not t.is_contiguous():
            raise ValueError("prefill tensors must be contiguous")
    if k.dim() != 3 or k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must be [H][T][d] of one dtype")
    if k_codes.dim() != 3 or k_codes.shape[0] != k.shape[0] or v_codes.shape[:2] != k_codes.shape[:2]:
        raise ValueError("cache planes must be [H][cap][row] matching k")
    H, T = k.shape[0], k.shape[1]
    _check(_lib.tq_prefill(ctypes.byref(kc), ctypes.byref(vc), _ptr(k), _ptr(v), _DTYPES[k.dtype], H, T, t0,
                           k_codes.shape[1], _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), _ptr(qjl_S),
                           _ptr(k_qjl_bits), _ptr(k_qjl_gamma), _stream(stream, k)), "tq_prefill")


def tq_append(kc: tq_codec, vc: tq_codec, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor,
              k_codes: torch.Tensor, k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
              qjl_S: torch.Tensor | None = None, k_qjl_bits: torch.Tensor | None = None,
              k_qjl_gamma: torch.Tensor | None = None, stream=None) -> None:
    """k, v [B][H][d] (fp32/fp16/bf16, one dtype) contiguous; pos [B] int32
    (device); cache planes [B][H][cap][d*bits/8] uint8 and norms [B][H][cap]
    (2-byte dtype), contiguous."""
    for t in (k, v, pos, k_codes, k_norms, v_codes, v_norms):
        if not t.is_contiguous():
            raise ValueError("append tensors must be contiguous")
    if k.dim() != 3 or k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must be [B][H][d] of one dtype")
    if k_codes.dim() != 4 or k_codes.shape[:2] != k.shape[:2] or v_codes.shape[:3] != k_codes.shape[:3]:
        raise ValueError("cache planes must be [B][H][cap][row] matching k")
    B, H = k.shape[0], k.shape[1]
    _check(_lib.tq_append(ctypes.byref(kc), ctypes.byref(vc), _ptr(k), _ptr(v), _DTYPES[k.dtype], B, H, _ptr(pos),
                          k_codes.shape[2], _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), _ptr(qjl_S),
                          _ptr(k_qjl_bits), _ptr(k_qjl_gamma), _stream(stream, k)), "tq_append")


def tq_decode(codec: tq_codec, codes: torch.Tensor, norms: torch.Tensor, x_hat: torch.Tensor, stream=None) -> None:
    if codes.dim() != 2 or codes.stride(1) != 1:
        raise ValueError("codes must be 2-D with contiguous rows")
    _check(_lib.tq_decode(ctypes.byref(codec), _ptr(codes), codes.stride(0), _ptr(norms), codes.shape[0],
                          _ptr(x_hat), _stream(stream, codes)), "tq_decode")


def tq_attn_workspace_bytes(kc: tq_codec, vc: tq_codec, batch: int, n_q_heads: int, n_kv_heads: int,
                            ctx_cap: int) -> int:
    return _lib.tq_attn_workspace_bytes(ctypes.byref(kc), ctypes.byref(vc), batch, n_q_heads, n_kv_heads, ctx_cap)


def _attn(name, kc, vc, q, ctx_len, k_codes, k_norms, v_codes, v_norms, scale, out, workspace,
          k_qjl, k_gamma, qjl_S, stream):
    B, Hq, _ = q.shape
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    for t in (q, k_codes, k_norms, v_codes, v_norms, out, ctx_len):
        if not t.is_contiguous():
            raise ValueError("attention tensors must be contiguous")
    fn = getattr(_lib, name)
    _check(fn(ctypes.byref(kc), ctypes.byref(vc), _ptr(q), _DTYPES[q.dtype], B, Hq, Hkv,
              _ptr(ctx_len), cap, _ptr(k_codes), _ptr(k_norms), _ptr(k_qjl), _ptr(k_gamma),
              _ptr(qjl_S), _ptr(v_codes), _ptr(v_norms), ctypes.c_float(scale), _ptr(out),
              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q)), name)


def tq_attn_decode(kc: tq_codec, vc: tq_codec, q: torch.Tensor, ctx_len: torch.Tensor,
                   k_codes: torch.Tensor, k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
                   scale: float, out: torch.Tensor, workspace: torch.Tensor,
                   k_qjl: torch.Tensor | None = None, k_gamma: torch.Tensor | None = None,
                   qjl_S: torch.Tensor | None = None, stream=None) -> None:
    """q [B][Hq][d]; caches [B][Hkv][ctx_cap][...] contiguous; out [B][Hq][d] fp32."""
    _attn("tq_attn_decode", kc, vc, q, ctx_len, k_codes, k_norms, v_codes, v_norms, scale, out, workspace,
          k_qjl, k_gamma, qjl_S, stream)


def tq_attn_decode_rw(kc: tq_codec, vc: tq_codec, q: torch.Tensor, ctx_len: torch.Tensor,
                      k_codes: torch.Tensor, k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
                      k_win: torch.Tensor, v_win: torch.Tensor, win_len: torch.Tensor,
                      scale: float, out: torch.Tensor, workspace: torch.Tensor,
                      k_qjl: torch.Tensor | None = None, k_gamma: torch.Tensor | None = None,
                      qjl_S: torch.Tensor | None = None, stream=None) -> None:
    """tq_attn_decode plus a residual window: k_win, v_win [B][Hkv][win_cap][d]
    (fp32/fp16/bf16, contiguous) holding win_len[b] exact recent tokens."""
    B, Hq, _ = q.shape
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    for t in (q, k_codes, k_norms, v_codes, v_norms, out, ctx_len, k_win, v_win, win_len):
        if not t.is_contiguous():
            raise ValueError("attention tensors must be contiguous")
    if k_win.dim() != 4 or k_win.shape != v_win.shape or k_win.dtype != v_win.dtype:
        raise ValueError("k_win and v_win must be [B][Hkv][win_cap][d] of one dtype")
    _check(_lib.tq_attn_decode_rw(ctypes.byref(kc), ctypes.byref(vc), _ptr(q), _DTYPES[q.dtype], B, Hq, Hkv,
                                  _ptr(ctx_len), cap, _ptr(k_codes), _ptr(k_norms), _ptr(k_qjl), _ptr(k_gamma),
                                  _ptr(qjl_S), _ptr(v_codes), _ptr(v_norms), _ptr(k_win), _ptr(v_win),
                                  _DTYPES[k_win.dtype], _ptr(win_len), k_win.shape[2], ctypes.c_float(scale),
                                  _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream, q)), "tq_attn_decode_rw")


def tq_attn_prepare(*args, **kw) -> None:
    """Stage 1 of tq_attn_decode (same arguments)."""
    _attn_stage("tq_attn_prepare", *args, **kw)


def tq_attn_scan(*args, **kw) -> None:
    """Stage 2 of tq_attn_decode (same arguments)."""
    _attn_stage("tq_attn_scan", *args, **kw)


def tq_attn_combine(*args, **kw) -> None:
    """Stage 3 of tq_attn_decode (same arguments)."""
    _attn_stage("tq_attn_combine", *args, **kw)


def _attn_stage(name, kc, vc, q, ctx_len, k_codes, k_norms, v_codes, v_norms, scale, out, workspace,
                k_qjl=None, k_gamma=None, qjl_S=None, stream=None):
    _attn(name, kc, vc, q, ctx_len, k_codes, k_norms, v_codes, v_norms, scale, out, workspace,
          k_qjl, k_gamma, qjl_S, stream)


def tq_search_workspace_bytes(codec: tq_codec, n_q: int, n_db: int, k: int) -> int:
    return _lib.tq_search_workspace_bytes(ctypes.byref(codec), n_q, n_db, k)


def tq_ip_search(codec: tq_codec, q: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor,
                 qjl_bits: torch.Tensor | None, qjl_gamma: torch.Tensor | None, qjl_S: torch.Tensor | None,
                 k: int, out_scores: torch.Tensor, out_ids: torch.Tensor, workspace: torch.Tensor,
                 stream=None) -> None:
    n_q = q.shape[0]
    n_db = codes.shape[0]
    _check(_lib.tq_ip_search(ctypes.byref(codec), _ptr(q), n_q, _ptr(codes), _ptr(norms), _ptr(qjl_bits),
                             _ptr(qjl_gamma), _ptr(qjl_S), n_db, k, _ptr(out_scores), _ptr(out_ids),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q)),
           "tq_ip_search")


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device byte buffer of at least nbytes (torch's allocator, 256-B aligned)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def raw_call(name: str, *args):
    """Call a C entry point with ctypes arguments as given (used by ABI tests)."""
    return getattr(_lib, name)(*args)
