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

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EWORKSPACE, TQ_EDEVICE, TQ_ESCRATCH = 0, -1, -2, -3, -4, -5
TQ_RES_NONE, TQ_RES_QJL, TQ_RES_SRHT, TQ_RES_SIGN = 0, 1, 2, 3
TQ_ROT_WHT, TQ_ROT_DOUBLE = 0, 1
TQ_NOALLOC_SCRATCH_BYTES = 16 << 20
TQ_F32, TQ_F16, TQ_BF16 = 0, 1, 2

_DTYPES = {torch.float32: TQ_F32, torch.float16: TQ_F16, torch.bfloat16: TQ_BF16}

EXPORTS = (
    "tq_codebook", "tq_codebook_ex", "tq_codebook_opts", "tq_encode", "tq_encode_kv", "tq_prefill", "tq_append", "tq_decode", "tq_attn_decode", "tq_attn_prepare", "tq_attn_scan",
    "tq_attn_combine", "tq_attn_decode_rw", "tq_attn_workspace_bytes", "tq_workspace_bytes",
    "tq_ip_search", "tq_search_workspace_bytes", "tq_packed_bytes", "tq_strerror", "tq_stream_read",
    "tq_attn_decode_noalloc", "tq_attn_decode_mq", "tq_attn_decode_ex",
)
TQ_OP_ATTN_DECODE, TQ_OP_ATTN_DECODE_RW, TQ_OP_IP_SEARCH, TQ_OP_ATTN_DECODE_MQ = 1, 2, 3, 4
TQ_MAX_QUERY_COLS = 64


class tq_codec(ctypes.Structure):
    """Mirror of the C struct tq_codec."""

    _fields_ = [
        ("d", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("qjl_m", ctypes.c_int32),
        ("residual", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
        ("sign_mask", ctypes.c_uint32 * 8),
        ("centroid", ctypes.c_float * 16),
        ("threshold", ctypes.c_float * 15),
        ("sign_mask2", ctypes.c_uint32 * 8),
        ("rotation", ctypes.c_int32),
        ("norm_blocks", ctypes.c_int32),
        ("sign_mask3", ctypes.c_uint32 * 8),
        ("sign_mask_hi", ctypes.c_uint32 * 8),
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
        def bit(i):
            return (self.sign_mask[i >> 5] >> (i & 31)) & 1 if i < 256 else \
                (self.sign_mask_hi[(i - 256) >> 5] >> (i & 31)) & 1
        return [-1.0 if bit(i) else 1.0 for i in range(self.d)]

    @property
    def signs3(self) -> list[float]:
        return [-1.0 if (self.sign_mask3[i >> 5] >> (i & 31)) & 1 else 1.0 for i in range(min(self.d, 256))]

    @property
    def signs2(self) -> list[float]:
        return [-1.0 if (self.sign_mask2[i >> 5] >> (i & 31)) & 1 else 1.0 for i in range(self.d)]


TQ_SCORE_PLAIN, TQ_SCORE_SHARPEN, TQ_SCORE_SOFTEN = 0, 1, 2


class tq_attn_opts(ctypes.Structure):
    """Mirror of the C struct tq_attn_opts (softmax-side switches, all off when zero)."""

    _fields_ = [
        ("score_mode", ctypes.c_int32),
        ("sqnr", ctypes.c_float),
        ("ref_tokens", ctypes.c_int32),
        ("sparse_v", ctypes.c_float),
    ]


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
        "tq_codebook_ex": (I, [I, I, ctypes.c_uint64, I, I, CP]),
        "tq_codebook_opts": (I, [I, I, ctypes.c_uint64, I, I, I, I, CP]),
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
        "tq_workspace_bytes": (SZ, [I, CP, CP, I, I, I, I64, I, I64, I]),
        "tq_ip_search": (I, [CP, P, I, P, P, P, P, P, I64, I, P, P, P, SZ, P]),
        "tq_search_workspace_bytes": (SZ, [CP, I, I64, I]),
        "tq_packed_bytes": (SZ, [I, I, I]),
        "tq_strerror": (ctypes.c_char_p, [I]),
        "tq_stream_read": (I, [P, SZ, P, P]),
        "tq_attn_decode_noalloc": (I, [CP, CP, P, I, I, I, I, P, I64, P, P, P, P, P, P, P, F, P, P]),
        "tq_attn_decode_mq": (I, [CP, CP, P, I, I, I, I, I, P, I64, P, P, P, P, P, P, P, F, P, P, SZ, P]),
        "tq_attn_decode_ex": (I, [CP, CP, P, I, I, I, I, I, P, I64, P, P, P, P, P, P, P, F,
                                  ctypes.POINTER(tq_attn_opts), P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
LIB_PATH = _LIB_PATH

# The per-step calls (tq_encode, tq_encode_kv, tq_prefill, tq_append,
# tq_attn_decode) go through the
# _tqcall extension when it is built and bound to _lib: the same entry points,
# with their arguments converted in C instead of by ctypes (about 0.5 us of
# host time per call saved, 7-9 % of a small encode).  Without it ctypes
# marshals them as it does the rest of the calls.
try:
    from . import _tqcall
except ImportError:
    _tqcall = None
_fast_lib = None


def _bind_fast(lib) -> bool:
    """Hands the per-step entry points of `lib` to _tqcall; True when bound."""
    global _fast_lib
    if _tqcall is None:
        return False

    def addr(name):
        return ctypes.cast(getattr(lib, name), ctypes.c_void_p).value

    try:
        _tqcall.bind(addr("tq_encode"), addr("tq_encode_kv"), addr("tq_attn_decode"), addr("tq_append"),
                     addr("tq_prefill"))
    except TypeError:  # a _tqcall built from older sources: keep ctypes
        return False
    _fast_lib = lib
    return True


_bind_fast(_lib)


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


def _shape(t, shape, name, dtype=None, elem=None):
    """Raises ValueError unless t has exactly `shape` (and dtype / element size):
    the C side trusts these sizes, so a mismatched plane would be read or
    written out of bounds on the device."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if elem is not None and t.element_size() != elem:
        raise ValueError(f"{name} must have {elem}-byte elements")


def _rows(t, n, min_width, name, dtype=None):
    """2-D tensor with n rows of at least min_width elements, contiguous rows."""
    if t is None or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    if t.shape[0] != n or t.shape[1] < min_width:
        raise ValueError(f"{name} must be [{n}][>= {min_width}], got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _vec(t, n, name):
    """n half values (any 2-byte dtype), contiguous."""
    if t is None or t.numel() != n or t.element_size() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must hold {n} contiguous 2-byte values")


def _qjl_rows(codec, n, qjl_S, qjl_bits, qjl_gamma, names=("qjl_S", "qjl_bits", "qjl_gamma")):
    """QJL planes of n rows for a QJL codec: S [m][d] float32, bits [n][m/8]
    uint8 contiguous, gamma [n] halves."""
    m = codec.qjl_m
    if not m:
        return
    if codec.residual == TQ_RES_QJL:
        _shape(qjl_S, (m, codec.d), names[0], torch.float32)
    if qjl_bits is None or qjl_bits.numel() != n * (m // 8) or qjl_bits.dtype != torch.uint8 \
            or not qjl_bits.is_contiguous() or qjl_bits.shape[-1] != m // 8:
        raise ValueError(f"{names[1]} must be contiguous uint8 [{n}][{m // 8}]")
    _vec(qjl_gamma, n, names[2])


_raw_stream = torch._C._cuda_getCurrentRawStream
_TWO_BYTE = frozenset((torch.float16, torch.bfloat16, torch.int16, torch.uint16))


def _mat(t, n, min_width, name, dtype=None):
    """_rows of a per-step tensor in one pass over its shape and strides:
    returns (address, row stride in elements); the caller checks the device
    (_on_device) once every shape has been checked."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    shp, st = t.shape, t.stride()
    if len(shp) != 2 or st[1] != 1:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    if shp[0] != n or shp[1] < min_width:
        raise ValueError(f"{name} must be [{n}][>= {min_width}], got {tuple(shp)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr(), st[0]


def _halves(t, n, name):
    """_vec of a norms plane (n contiguous 2-byte values): returns its address."""
    if not isinstance(t, torch.Tensor) or t.dtype not in _TWO_BYTE:
        raise ValueError(f"{name} must hold {n} contiguous 2-byte values")
    shp = t.shape
    if len(shp) == 1:
        ok = shp[0] == n and t.is_contiguous()
    else:
        ok = t.numel() == n and t.is_contiguous()
    if not ok:
        raise ValueError(f"{name} must hold {n} contiguous 2-byte values")
    return t.data_ptr()


def _on_device(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("device tensor expected")


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


def tq_codebook_ex(bits: int, d: int, seed: int, residual: int, qjl_m: int = 0) -> tq_codec:
    """Host-only: codec with an explicit residual kind (TQ_RES_*)."""
    c = tq_codec()
    _check(_lib.tq_codebook_ex(bits, d, ctypes.c_uint64(seed & (2**64 - 1)), residual, qjl_m, ctypes.byref(c)),
           "tq_codebook_ex")
    return c


def tq_codebook_opts(bits: int, d: int, seed: int, residual: int = TQ_RES_NONE, qjl_m: int = 0,
                     rotation: int = TQ_ROT_WHT, norm_blocks: int = 1) -> tq_codec:
    """Host-only: codec with the rotation (TQ_ROT_*) and norm blocks (1 or 2)."""
    c = tq_codec()
    _check(_lib.tq_codebook_opts(bits, d, ctypes.c_uint64(seed & (2**64 - 1)), residual, qjl_m, rotation,
                                 norm_blocks, ctypes.byref(c)), "tq_codebook_opts")
    return c


def _nshape(codec, shape):
    """Shape of a norms plane: `shape`, with a trailing block axis for a codec
    with two norm blocks."""
    return tuple(shape) + ((codec.norm_blocks,) if codec.norm_blocks > 1 else ())


def tq_packed_bytes(d: int, bits: int, qjl_m: int = 0) -> int:
    return _lib.tq_packed_bytes(d, bits, qjl_m)


def tq_encode(codec: tq_codec, x: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor,
              qjl_S: torch.Tensor | None = None, qjl_bits: torch.Tensor | None = None,
              qjl_gamma: torch.Tensor | None = None, stream=None) -> None:
    """x [n][>=d] (fp32/fp16/bf16, last dim contiguous); codes [n][>= d*bits/8] uint8;
    norms [n] (2-byte dtype, half bits).  Row strides are taken from the tensors."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be 2-D with contiguous rows")
    n = x.shape[0]
    xp, xs = _mat(x, n, codec.d, "x")
    cp, cs = _mat(codes, n, codec.code_bytes, "codes", torch.uint8)
    npp = _halves(norms, n * codec.norm_blocks, "norms")
    if codec.qjl_m:
        _qjl_rows(codec, n, qjl_S, qjl_bits, qjl_gamma)
    dt = _DTYPES.get(x.dtype)
    if dt is None:
        raise ValueError(f"x must be float32, float16 or bfloat16, got {x.dtype}")
    _on_device(x, codes, norms)
    if codec.qjl_m:
        qs, qb, qg = _ptr(qjl_S), _ptr(qjl_bits), _ptr(qjl_gamma)
    else:
        qs = qb = qg = None
    st = _stream(stream, x)
    if _lib is _fast_lib:
        rc = _tqcall.encode(ctypes.addressof(codec), xp, dt, n, xs, cp, cs, npp, qs, qb, qg, st)
    else:
        rc = _lib.tq_encode(ctypes.byref(codec), xp, dt, n, xs, cp, cs, npp, qs, qb, qg, st)
    if rc:
        _check(rc, "tq_encode")


def tq_encode_kv(kc: tq_codec, vc: tq_codec, k: torch.Tensor, v: torch.Tensor, k_codes: torch.Tensor,
                 k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
                 qjl_S: torch.Tensor | None = None, k_qjl_bits: torch.Tensor | None = None,
                 k_qjl_gamma: torch.Tensor | None = None, stream=None) -> None:
    """tq_encode of keys and values in one call: k, v [n][>=d] of one dtype and
    row stride (last dim contiguous); codes [n][>= d*bits/8] uint8; norms [n]."""
    if not isinstance(k, torch.Tensor) or not isinstance(v, torch.Tensor) or k.dim() != 2:
        raise ValueError("k, v and the code planes must be 2-D with contiguous rows")
    if k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v must share shape, strides and dtype")
    n = k.shape[0]
    kp, xs = _mat(k, n, kc.d, "k")
    vp, _ = _mat(v, n, kc.d, "v")
    kcp, kcs = _mat(k_codes, n, kc.code_bytes, "k_codes", torch.uint8)
    vcp, vcs = _mat(v_codes, n, vc.code_bytes, "v_codes", torch.uint8)
    knp = _halves(k_norms, n * kc.norm_blocks, "k_norms")
    vnp = _halves(v_norms, n * vc.norm_blocks, "v_norms")
    if kc.qjl_m:
        _qjl_rows(kc, n, qjl_S, k_qjl_bits, k_qjl_gamma, ("qjl_S", "k_qjl_bits", "k_qjl_gamma"))
    dt = _DTYPES.get(k.dtype)
    if dt is None:
        raise ValueError(f"k and v must be float32, float16 or bfloat16, got {k.dtype}")
    _on_device(k, v, k_codes, k_norms, v_codes, v_norms)
    if kc.qjl_m:
        qs, qb, qg = _ptr(qjl_S), _ptr(k_qjl_bits), _ptr(k_qjl_gamma)
    else:
        qs = qb = qg = None
    st = _stream(stream, k)
    if _lib is _fast_lib:
        rc = _tqcall.encode_kv(ctypes.addressof(kc), ctypes.addressof(vc), kp, vp, dt, n, xs, kcp, kcs, knp, vcp, vcs,
                               vnp, qs, qb, qg, st)
    else:
        rc = _lib.tq_encode_kv(ctypes.byref(kc), ctypes.byref(vc), kp, vp, dt, n, xs, kcp, kcs, knp, vcp, vcs, vnp,
                               qs, qb, qg, st)
    if rc:
        _check(rc, "tq_encode_kv")


def tq_prefill(kc: tq_codec, vc: tq_codec, k: torch.Tensor, v: torch.Tensor, t0: int, k_codes: torch.Tensor,
               k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
               qjl_S: torch.Tensor | None = None, k_qjl_bits: torch.Tensor | None = None,
               k_qjl_gamma: torch.Tensor | None = None, stream=None) -> None:
    """k, v [H][T][d] (one dtype) contiguous; one sequence's cache planes
    [H][cap][d*bits/8] uint8 and norms [H][cap] (2-byte dtype), contiguous (a
    slice [b] of a batched cache is); writes slots [t0, t0 + T) of every head."""
    for t in (k, v, k_codes, k_norms, v_codes, v_norms):
        if not isinstance(t, torch.Tensor) or not t.is_contiguous():
            raise ValueError("prefill tensors must be contiguous")
    ks, kcs = k.shape, k_codes.shape
    if len(ks) != 3 or ks != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must be [H][T][d] of one dtype")
    if len(kcs) != 3 or kcs[0] != ks[0] or v_codes.shape[:2] != kcs[:2]:
        raise ValueError("cache planes must be [H][cap][row] matching k")
    H, T, cap = ks[0], ks[1], kcs[1]
    if ks[2] != kc.d:
        raise ValueError(f"k must have shape {(H, T, kc.d)}, got {tuple(ks)}")
    if kcs[2] != kc.code_bytes or k_codes.dtype != torch.uint8:
        _shape(k_codes, (H, cap, kc.code_bytes), "k_codes", torch.uint8)
    if v_codes.shape[2] != vc.code_bytes or v_codes.dtype != torch.uint8:
        _shape(v_codes, (H, cap, vc.code_bytes), "v_codes", torch.uint8)
    for t, c, name in ((k_norms, kc, "k_norms"), (v_norms, vc, "v_norms")):
        if t.shape != _nshape(c, (H, cap)) or t.dtype not in _TWO_BYTE:
            _shape(t, _nshape(c, (H, cap)), name, elem=2)
    if kc.qjl_m:
        _qjl_rows(kc, H * cap, qjl_S, k_qjl_bits, k_qjl_gamma, ("qjl_S", "k_qjl_bits", "k_qjl_gamma"))
        _shape(k_qjl_bits, (H, cap, kc.qjl_m // 8), "k_qjl_bits", torch.uint8)
    dt = _DTYPES.get(k.dtype)
    if dt is None:
        raise ValueError(f"k and v must be float32, float16 or bfloat16, got {k.dtype}")
    _on_device(k, v, k_codes, k_norms, v_codes, v_norms)
    if kc.qjl_m:
        qs, qb, qg = _ptr(qjl_S), _ptr(k_qjl_bits), _ptr(k_qjl_gamma)
    else:
        qs = qb = qg = None
    args = (k.data_ptr(), v.data_ptr(), dt, H, T, t0, cap, k_codes.data_ptr(), k_norms.data_ptr(), v_codes.data_ptr(),
            v_norms.data_ptr(), qs, qb, qg, _stream(stream, k))
    if _lib is _fast_lib:
        rc = _tqcall.prefill(ctypes.addressof(kc), ctypes.addressof(vc), *args)
    else:
        rc = _lib.tq_prefill(ctypes.byref(kc), ctypes.byref(vc), *args)
    if rc:
        _check(rc, "tq_prefill")


def tq_append(kc: tq_codec, vc: tq_codec, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor,
              k_codes: torch.Tensor, k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
              qjl_S: torch.Tensor | None = None, k_qjl_bits: torch.Tensor | None = None,
              k_qjl_gamma: torch.Tensor | None = None, stream=None) -> None:
    """k, v [B][H][d] (fp32/fp16/bf16, one dtype) contiguous; pos [B] int32
    (device); cache planes [B][H][cap][d*bits/8] uint8 and norms [B][H][cap]
    (2-byte dtype), contiguous."""
    for t in (k, v, pos, k_codes, k_norms, v_codes, v_norms):
        if not isinstance(t, torch.Tensor) or not t.is_contiguous():
            raise ValueError("append tensors must be contiguous")
    ks, kcs = k.shape, k_codes.shape
    if len(ks) != 3 or ks != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must be [B][H][d] of one dtype")
    if len(kcs) != 4 or kcs[:2] != ks[:2] or v_codes.shape[:3] != kcs[:3]:
        raise ValueError("cache planes must be [B][H][cap][row] matching k")
    B, H, cap = kcs[0], kcs[1], kcs[2]
    if ks[2] != kc.d:
        raise ValueError(f"k must have shape {(B, H, kc.d)}, got {tuple(ks)}")
    _shape(pos, (B,), "pos", torch.int32)
    if kcs[3] != kc.code_bytes or k_codes.dtype != torch.uint8:
        _shape(k_codes, (B, H, cap, kc.code_bytes), "k_codes", torch.uint8)
    if v_codes.shape[3] != vc.code_bytes or v_codes.dtype != torch.uint8:
        _shape(v_codes, (B, H, cap, vc.code_bytes), "v_codes", torch.uint8)
    for t, c, name in ((k_norms, kc, "k_norms"), (v_norms, vc, "v_norms")):
        if t.shape != _nshape(c, (B, H, cap)) or t.dtype not in _TWO_BYTE:
            _shape(t, _nshape(c, (B, H, cap)), name, elem=2)
    if kc.qjl_m:
        _qjl_rows(kc, B * H * cap, qjl_S, k_qjl_bits, k_qjl_gamma, ("qjl_S", "k_qjl_bits", "k_qjl_gamma"))
        _shape(k_qjl_bits, (B, H, cap, kc.qjl_m // 8), "k_qjl_bits", torch.uint8)
    dt = _DTYPES.get(k.dtype)
    if dt is None:
        raise ValueError(f"k and v must be float32, float16 or bfloat16, got {k.dtype}")
    _on_device(k, v, pos, k_codes, k_norms, v_codes, v_norms)
    if kc.qjl_m:
        qs, qb, qg = _ptr(qjl_S), _ptr(k_qjl_bits), _ptr(k_qjl_gamma)
    else:
        qs = qb = qg = None
    args = (k.data_ptr(), v.data_ptr(), dt, B, H, pos.data_ptr(), cap, k_codes.data_ptr(), k_norms.data_ptr(),
            v_codes.data_ptr(), v_norms.data_ptr(), qs, qb, qg, _stream(stream, k))
    if _lib is _fast_lib:
        rc = _tqcall.append(ctypes.addressof(kc), ctypes.addressof(vc), *args)
    else:
        rc = _lib.tq_append(ctypes.byref(kc), ctypes.byref(vc), *args)
    if rc:
        _check(rc, "tq_append")


def tq_decode(codec: tq_codec, codes: torch.Tensor, norms: torch.Tensor, x_hat: torch.Tensor, stream=None) -> None:
    if codes.dim() != 2 or codes.stride(1) != 1:
        raise ValueError("codes must be 2-D with contiguous rows")
    n = codes.shape[0]
    _rows(codes, n, codec.code_bytes, "codes", torch.uint8)
    _vec(norms, n * codec.norm_blocks, "norms")
    _shape(x_hat, (n, codec.d), "x_hat", torch.float32)
    if not x_hat.is_contiguous():
        raise ValueError("x_hat must be contiguous")
    _check(_lib.tq_decode(ctypes.byref(codec), _ptr(codes), codes.stride(0), _ptr(norms), codes.shape[0],
                          _ptr(x_hat), _stream(stream, codes)), "tq_decode")


def tq_attn_workspace_bytes(kc: tq_codec, vc: tq_codec, batch: int, n_q_heads: int, n_kv_heads: int,
                            ctx_cap: int) -> int:
    return _lib.tq_attn_workspace_bytes(ctypes.byref(kc), ctypes.byref(vc), batch, n_q_heads, n_kv_heads, ctx_cap)


def _check_cache(kc, vc, q, ctx_len, k_codes, k_norms, v_codes, v_norms, out, k_qjl, k_gamma, qjl_S):
    """Shapes of a decode-attention call: q [B][Hq][d], ctx_len [B] int32,
    planes [B][Hkv][cap][row] with rows of exactly d*bits/8 bytes, norms
    [B][Hkv][cap], out [B][Hq][d] float32, QJL planes for a QJL key codec."""
    if q.dim() != 3 or k_codes.dim() != 4:
        raise ValueError("q must be [B][Hq][d] and k_codes [B][Hkv][cap][row]")
    B, Hq, _ = q.shape
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    for t in (q, k_codes, k_norms, v_codes, v_norms, out, ctx_len):
        if not t.is_contiguous():
            raise ValueError("attention tensors must be contiguous")
    _shape(q, (B, Hq, kc.d), "q")
    _shape(ctx_len, (B,), "ctx_len", torch.int32)
    _shape(k_codes, (B, Hkv, cap, kc.code_bytes), "k_codes", torch.uint8)
    _shape(v_codes, (B, Hkv, cap, vc.code_bytes), "v_codes", torch.uint8)
    _shape(k_norms, _nshape(kc, (B, Hkv, cap)), "k_norms", elem=2)
    _shape(v_norms, _nshape(vc, (B, Hkv, cap)), "v_norms", elem=2)
    _shape(out, (B, Hq, vc.d), "out", torch.float32)
    if kc.qjl_m:
        _qjl_rows(kc, B * Hkv * cap, qjl_S, k_qjl, k_gamma, ("qjl_S", "k_qjl", "k_gamma"))
        _shape(k_qjl, (B, Hkv, cap, kc.qjl_m // 8), "k_qjl", torch.uint8)
    return B, Hq, Hkv, cap


def _attn(name, kc, vc, q, ctx_len, k_codes, k_norms, v_codes, v_norms, scale, out, workspace,
          k_qjl, k_gamma, qjl_S, stream):
    B, Hq, Hkv, cap = _check_cache(kc, vc, q, ctx_len, k_codes, k_norms, v_codes, v_norms, out, k_qjl, k_gamma,
                                   qjl_S)
    if name == "tq_attn_decode" and _lib is _fast_lib:
        rc = _tqcall.attn_decode(ctypes.addressof(kc), ctypes.addressof(vc), _ptr(q), _DTYPES[q.dtype], B, Hq, Hkv,
                                 _ptr(ctx_len), cap, _ptr(k_codes), _ptr(k_norms), _ptr(k_qjl), _ptr(k_gamma),
                                 _ptr(qjl_S), _ptr(v_codes), _ptr(v_norms), float(scale), _ptr(out),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q))
    else:
        fn = getattr(_lib, name)
        rc = fn(ctypes.byref(kc), ctypes.byref(vc), _ptr(q), _DTYPES[q.dtype], B, Hq, Hkv,
                _ptr(ctx_len), cap, _ptr(k_codes), _ptr(k_norms), _ptr(k_qjl), _ptr(k_gamma),
                _ptr(qjl_S), _ptr(v_codes), _ptr(v_norms), ctypes.c_float(scale), _ptr(out),
                _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q))
    _check(rc, name)


def tq_attn_decode(kc: tq_codec, vc: tq_codec, q: torch.Tensor, ctx_len: torch.Tensor,
                   k_codes: torch.Tensor, k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
                   scale: float, out: torch.Tensor, workspace: torch.Tensor,
                   k_qjl: torch.Tensor | None = None, k_gamma: torch.Tensor | None = None,
                   qjl_S: torch.Tensor | None = None, stream=None) -> None:
    """q [B][Hq][d]; caches [B][Hkv][ctx_cap][...] contiguous; out [B][Hq][d] fp32."""
    _attn("tq_attn_decode", kc, vc, q, ctx_len, k_codes, k_norms, v_codes, v_norms, scale, out, workspace,
          k_qjl, k_gamma, qjl_S, stream)


def tq_attn_decode_mq(kc: tq_codec, vc: tq_codec, q: torch.Tensor, ctx_len: torch.Tensor,
                      k_codes: torch.Tensor, k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
                      scale: float, out: torch.Tensor, workspace: torch.Tensor,
                      k_qjl: torch.Tensor | None = None, k_gamma: torch.Tensor | None = None,
                      qjl_S: torch.Tensor | None = None, stream=None) -> None:
    """Multi-query causal decode: q and out [B][C][Hq][d] (the last C tokens of
    each sequence, already in the cache); caches [B][Hkv][ctx_cap][...]."""
    if q.dim() != 4 or out.dim() != 4:
        raise ValueError("q and out must be [B][C][Hq][d]")
    B, C, Hq, d = q.shape
    _check_cache(kc, vc, q.view(B, C * Hq, d), ctx_len, k_codes, k_norms, v_codes, v_norms, out.view(B, C * Hq, -1),
                 k_qjl, k_gamma, qjl_S)
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    _check(_lib.tq_attn_decode_mq(ctypes.byref(kc), ctypes.byref(vc), _ptr(q), _DTYPES[q.dtype], B, C, Hq, Hkv,
                                  _ptr(ctx_len), cap, _ptr(k_codes), _ptr(k_norms), _ptr(k_qjl), _ptr(k_gamma),
                                  _ptr(qjl_S), _ptr(v_codes), _ptr(v_norms), ctypes.c_float(scale), _ptr(out),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q)),
           "tq_attn_decode_mq")


def tq_attn_decode_ex(kc: tq_codec, vc: tq_codec, q: torch.Tensor, ctx_len: torch.Tensor,
                      k_codes: torch.Tensor, k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
                      scale: float, out: torch.Tensor, workspace: torch.Tensor, opts: tq_attn_opts | None = None,
                      k_qjl: torch.Tensor | None = None, k_gamma: torch.Tensor | None = None,
                      qjl_S: torch.Tensor | None = None, stream=None) -> None:
    """tq_attn_decode_mq with softmax-side switches (tq_attn_opts; None = off):
    q and out [B][C][Hq][d]."""
    if q.dim() != 4 or out.dim() != 4:
        raise ValueError("q and out must be [B][C][Hq][d]")
    B, C, Hq, d = q.shape
    _check_cache(kc, vc, q.view(B, C * Hq, d), ctx_len, k_codes, k_norms, v_codes, v_norms, out.view(B, C * Hq, -1),
                 k_qjl, k_gamma, qjl_S)
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    _check(_lib.tq_attn_decode_ex(ctypes.byref(kc), ctypes.byref(vc), _ptr(q), _DTYPES[q.dtype], B, C, Hq, Hkv,
                                  _ptr(ctx_len), cap, _ptr(k_codes), _ptr(k_norms), _ptr(k_qjl), _ptr(k_gamma),
                                  _ptr(qjl_S), _ptr(v_codes), _ptr(v_norms), ctypes.c_float(scale),
                                  ctypes.byref(opts) if opts is not None else None, _ptr(out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream, q)),
           "tq_attn_decode_ex")


def tq_attn_decode_noalloc(kc: tq_codec, vc: tq_codec, q: torch.Tensor, ctx_len: torch.Tensor,
                           k_codes: torch.Tensor, k_norms: torch.Tensor, v_codes: torch.Tensor,
                           v_norms: torch.Tensor, scale: float, out: torch.Tensor,
                           k_qjl: torch.Tensor | None = None, k_gamma: torch.Tensor | None = None,
                           qjl_S: torch.Tensor | None = None, stream=None) -> None:
    """tq_attn_decode without a workspace: the library's static per-device
    scratch (TQ_NOALLOC_SCRATCH_BYTES) is used; nothing is allocated.  Calls
    that overlap on one device race on that scratch."""
    B, Hq, Hkv, cap = _check_cache(kc, vc, q, ctx_len, k_codes, k_norms, v_codes, v_norms, out, k_qjl, k_gamma,
                                   qjl_S)
    _check(_lib.tq_attn_decode_noalloc(ctypes.byref(kc), ctypes.byref(vc), _ptr(q), _DTYPES[q.dtype], B, Hq, Hkv,
                                       _ptr(ctx_len), cap, _ptr(k_codes), _ptr(k_norms), _ptr(k_qjl), _ptr(k_gamma),
                                       _ptr(qjl_S), _ptr(v_codes), _ptr(v_norms), ctypes.c_float(scale), _ptr(out),
                                       _stream(stream, q)), "tq_attn_decode_noalloc")


def tq_attn_decode_rw(kc: tq_codec, vc: tq_codec, q: torch.Tensor, ctx_len: torch.Tensor,
                      k_codes: torch.Tensor, k_norms: torch.Tensor, v_codes: torch.Tensor, v_norms: torch.Tensor,
                      k_win: torch.Tensor, v_win: torch.Tensor, win_len: torch.Tensor,
                      scale: float, out: torch.Tensor, workspace: torch.Tensor,
                      k_qjl: torch.Tensor | None = None, k_gamma: torch.Tensor | None = None,
                      qjl_S: torch.Tensor | None = None, stream=None) -> None:
    """tq_attn_decode plus a residual window: k_win, v_win [B][Hkv][win_cap][d]
    (fp32/fp16/bf16, contiguous) holding win_len[b] exact recent tokens."""
    B, Hq, Hkv, cap = _check_cache(kc, vc, q, ctx_len, k_codes, k_norms, v_codes, v_norms, out, k_qjl, k_gamma,
                                   qjl_S)
    for t in (k_win, v_win, win_len):
        if not t.is_contiguous():
            raise ValueError("attention tensors must be contiguous")
    if k_win.dim() != 4 or k_win.shape != v_win.shape or k_win.dtype != v_win.dtype:
        raise ValueError("k_win and v_win must be [B][Hkv][win_cap][d] of one dtype")
    _shape(k_win, (B, Hkv, k_win.shape[2], kc.d), "k_win")
    _shape(win_len, (B,), "win_len", torch.int32)
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


def tq_workspace_bytes(op: int, kc: tq_codec, vc: tq_codec | None = None, batch: int = 0, n_q_heads: int = 0,
                       n_kv_heads: int = 0, ctx_cap: int = 0, n_q: int = 0, n_db: int = 0, k: int = 0) -> int:
    """Workspace bytes of operation `op` (TQ_OP_*); 0 on bad arguments."""
    return _lib.tq_workspace_bytes(op, ctypes.byref(kc), ctypes.byref(vc) if vc is not None else None, batch,
                                   n_q_heads, n_kv_heads, ctx_cap, n_q, n_db, k)


def tq_ip_search(codec: tq_codec, q: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor,
                 qjl_bits: torch.Tensor | None, qjl_gamma: torch.Tensor | None, qjl_S: torch.Tensor | None,
                 k: int, out_scores: torch.Tensor, out_ids: torch.Tensor, workspace: torch.Tensor,
                 stream=None) -> None:
    n_q = q.shape[0]
    n_db = codes.shape[0]
    _shape(q, (n_q, codec.d), "q", torch.float32)
    if not q.is_contiguous() or not codes.is_contiguous():
        raise ValueError("q and codes must be contiguous")
    _shape(codes, (n_db, codec.code_bytes), "codes", torch.uint8)
    _vec(norms, n_db, "norms")
    _qjl_rows(codec, n_db, qjl_S, qjl_bits, qjl_gamma)
    _shape(out_scores, (n_q, k), "out_scores", torch.float32)
    _shape(out_ids, (n_q, k), "out_ids", torch.int64)
    _check(_lib.tq_ip_search(ctypes.byref(codec), _ptr(q), n_q, _ptr(codes), _ptr(norms), _ptr(qjl_bits),
                             _ptr(qjl_gamma), _ptr(qjl_S), n_db, k, _ptr(out_scores), _ptr(out_ids),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q)),
           "tq_ip_search")


def tq_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read all of `src` (contiguous device tensor) with 16-byte loads; `sink`
    is a device tensor of at least 4 bytes (almost never written)."""
    if not src.is_contiguous() or sink.numel() * sink.element_size() < 4:
        raise ValueError("src must be contiguous and sink hold at least 4 bytes")
    _check(_lib.tq_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream, src)),
           "tq_stream_read")


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device byte buffer of at least nbytes (torch's allocator, 256-B aligned)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def raw_call(name: str, *args):
    """Call a C entry point with ctypes arguments as given (used by ABI tests)."""
    return getattr(_lib, name)(*args)
