"""Python binding of libtq, the MI355X rotated-basis ternary projection library.

Argument marshalling only: every function checks tensor devices, dtypes and
contiguity, allocates outputs with torch where the C function writes into
caller memory, and passes raw pointers plus torch's current HIP stream to the
C ABI declared in ``include/tq.h``.  All computation happens in the HIP
kernels of ``libtq.so``; if the library is missing, every call raises.

Entry points (same names as the C ABI without the ``tq_`` prefix):
``geometry``, ``pack_rowsplit``, ``unpack_rowsplit``, ``hadamard_signed``,
``gemv_rowsplit``, ``gemm_rowsplit``, ``embed_rows_inverse``,
``decode_rowsplit``, ``rotated_gemv_rowsplit``, ``blocks_to_planes``,
``planes_to_blocks``, ``container_parse``.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIBRARY names another build of the same C ABI (the host-only sanitizer
# build); by default the in-tree libtq.so.
LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(HERE, "libtq.so")

PQ2_0_G128 = 142
PTQ1_0_G128 = 143
FORMATS = {"PQ2_0_G128": PQ2_0_G128, "PTQ1_0_G128": PTQ1_0_G128}
F32, BF16, F16 = 0, 1, 2

GEOMETRY_FIELDS = (
    "n", "k", "k_pad", "groups_per_row", "base_bytes_per_group",
    "high_bytes_per_group", "base_row_bytes", "high_row_bytes",
    "scale_row_bytes", "base_offset", "base_bytes", "high_offset",
    "high_bytes", "scale_offset", "scale_bytes", "payload_bytes",
)

# Exported symbols of include/tq.h.
EXPORTS = (
    "tq_last_error", "tq_version", "tq_geometry_get", "tq_pack_rowsplit",
    "tq_unpack_rowsplit", "tq_hadamard_signed", "tq_gemv_rowsplit",
    "tq_gemm_rowsplit", "tq_embed_rows_inverse", "tq_decode_rowsplit",
    "tq_rotated_gemv_rowsplit", "tq_blocks_to_planes", "tq_planes_to_blocks",
    "tq_container_parse", "tq_container_object_at", "tq_g64_bytes", "tq_expand_g64",
    "tq_gemv_g64", "tq_head_argmax", "tq_hadamard_signed_grouped",
    "tq_rotated_gemv_rowsplit_grouped", "tq_stream_read", "tq_head_argmax_noalloc",
)


class TQError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("tq status %d: %s" % (status, message))
        self.status = status


class ContainerObject(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 16), ("offset", ctypes.c_uint64),
                ("bytes", ctypes.c_uint64), ("name", ctypes.c_char * 256),
                ("format", ctypes.c_char * 64), ("layout", ctypes.c_char * 64)]


class Geometry(ctypes.Structure):
    _fields_ = [(f, ctypes.c_uint64) for f in GEOMETRY_FIELDS]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f in GEOMETRY_FIELDS}


_lib = None
_i64, _u64, _i32, _vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p


def lib():
    """Load libtq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtq.so is not built (run python -m ternary_quantized_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.tq_last_error.restype = ctypes.c_char_p
        L.tq_version.restype = ctypes.c_char_p
        sigs = {
            "tq_geometry_get": [_i32, _i64, _i64, ctypes.POINTER(Geometry)],
            "tq_pack_rowsplit": [_i32, _i64, _i64, _vp, _vp, _vp, _u64],
            "tq_unpack_rowsplit": [_i32, _i64, _i64, _vp, _u64, _vp, _vp, _vp],
            "tq_hadamard_signed": [_vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp, _i32, _i64, _vp],
            "tq_gemv_rowsplit": [_vp, _u64, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _i64, _vp],
            "tq_gemm_rowsplit": [_vp, _u64, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _i32, _i64, _vp],
            "tq_rotated_gemv_rowsplit": [_vp, _u64, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _vp,
                                         _i64, _vp],
            "tq_embed_rows_inverse": [_vp, _u64, _i32, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp],
            "tq_decode_rowsplit": [_vp, _u64, _i32, _i64, _i64, _vp, _i64, _vp, _vp, _vp],
            "tq_blocks_to_planes": [_vp, _u64, _i32, _i64, _i64, _vp, _u64, _vp],
            "tq_planes_to_blocks": [_vp, _u64, _i32, _i64, _i64, _vp, _u64, _vp],
            "tq_container_parse": [_vp, _u64, ctypes.POINTER(_u64), ctypes.POINTER(_i64)],
            "tq_container_object_at": [_vp, _u64, _i64, ctypes.POINTER(ContainerObject)],
            "tq_g64_bytes": [_i64, _i64, ctypes.POINTER(_u64)],
            "tq_expand_g64": [_vp, _u64, _i32, _i64, _i64, _vp, _u64, _vp],
            "tq_head_argmax": [_vp, _u64, _i32, _i64, _i64, _vp, _i32, _vp, ctypes.c_float, _vp, _vp,
                               _vp, _vp, _vp],
            "tq_hadamard_signed_grouped": [_vp, _i32, _i64, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _i32,
                                           _i64, _vp],
            "tq_rotated_gemv_rowsplit_grouped": [_vp, _u64, _i32, _i64, _i64, _vp, _i32, _i64, _i64,
                                                 _i32, _i32, _i32, _vp, _vp, _i64, _vp],
            "tq_gemv_g64": [_vp, _u64, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _i64, _vp],
            "tq_stream_read": [_vp, _u64, _vp, _vp],
            "tq_head_argmax_noalloc": [_vp, _u64, _i32, _i64, _i64, _vp, _i32, _vp, ctypes.c_float,
                                       _vp, _vp, _vp, _vp],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise TQError(status, lib().tq_last_error().decode())


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def version():
    return lib().tq_version().decode()


def geometry(fmt, n, k):
    g = Geometry()
    _check(lib().tq_geometry_get(_fmt(fmt), n, k, ctypes.byref(g)))
    return g.as_dict()


# ------------------------------------------------------------ host codec ---
def pack_rowsplit(fmt, trits, scale_bits):
    """numpy int8 [n, k] trits + uint16 [n, G] fp16 bits -> uint8 payload."""
    trits = np.ascontiguousarray(trits, dtype=np.int8)
    scale_bits = np.ascontiguousarray(scale_bits, dtype=np.uint16)
    n, k = trits.shape
    g = geometry(fmt, n, k)
    payload = np.empty(g["payload_bytes"], dtype=np.uint8)
    _check(lib().tq_pack_rowsplit(_fmt(fmt), n, k, trits.ctypes.data, scale_bits.ctypes.data,
                                  payload.ctypes.data, payload.size))
    return payload


def unpack_rowsplit(fmt, n, k, payload):
    """uint8 payload -> (int8 values [n, k_pad], uint16 scale bits, bad codes)."""
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    g = geometry(fmt, n, k)
    values = np.empty((n, g["k_pad"]), dtype=np.int8)
    scales = np.empty((n, g["groups_per_row"]), dtype=np.uint16)
    bad = ctypes.c_uint64(0)
    _check(lib().tq_unpack_rowsplit(_fmt(fmt), n, k, payload.ctypes.data, payload.size,
                                    values.ctypes.data, scales.ctypes.data, ctypes.byref(bad)))
    return values, scales, int(bad.value)


def container_parse(data):
    """Validate a whole .ninfer container (bytes-like, host memory); return
    (payload_offset, objects) with one dict per directory entry."""
    buf = np.frombuffer(bytes(data), dtype=np.uint8)
    ptr = buf.ctypes.data if buf.size else None
    off, cnt = _u64(0), _i64(0)
    _check(lib().tq_container_parse(ptr, buf.size, ctypes.byref(off), ctypes.byref(cnt)))
    objs = []
    for i in range(cnt.value):
        o = ContainerObject()
        _check(lib().tq_container_object_at(ptr, buf.size, i, ctypes.byref(o)))
        d = {"name": o.name.decode(), "offset": int(o.offset), "bytes": int(o.bytes)}
        if o.kind == 0:
            d.update(kind="tensor", shape=[int(o.shape[j]) for j in range(o.rank)],
                     format=o.format.decode(), layout=o.layout.decode())
        else:
            d.update(kind="resource", encoding=o.format.decode())
        objs.append(d)
    return int(off.value), objs


# ---------------------------------------------------------------- device ---
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    return {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}[t.dtype]


def _dtype_of(code):
    torch = _torch()
    return {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[code]


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    return t


def _signs_ptr(signs):
    torch = _torch()
    _dev(signs, "signs")
    if signs.dtype == torch.bfloat16:
        return signs.data_ptr()
    if signs.dtype in (torch.int16, torch.uint16):
        return signs.data_ptr()
    raise ValueError("signs must be bf16 (or its int16 bit pattern)")


def hadamard_signed(x, signs, inverse=False, out_dtype=None, out=None):
    """Signed blockwise WHT of the rows of x ([rows, k] device tensor)."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit column stride")
    rows, k = x.shape
    ycode = _dtype_code(x) if out_dtype is None else {torch.float32: F32, torch.bfloat16: BF16,
                                                      torch.float16: F16}[out_dtype]
    if out is None:
        out = torch.empty((rows, k), dtype=_dtype_of(ycode), device=x.device)
    _check(lib().tq_hadamard_signed(x.data_ptr(), _dtype_code(x), rows, k, x.stride(0),
                                    _signs_ptr(signs), int(bool(inverse)), out.data_ptr(), ycode,
                                    out.stride(0), _stream(x.device)))
    return out


def gemv_rowsplit(payload, fmt, n, k, xrot, out=None):
    """y [batch, n] fp32 = decode-GEMV of rotated activations xrot [batch, k]."""
    torch = _torch()
    _dev(payload, "payload")
    _dev(xrot, "xrot")
    if xrot.dim() == 1:
        xrot = xrot.unsqueeze(0)
    batch = xrot.shape[0]
    if out is None:
        out = torch.empty((batch, n), dtype=torch.float32, device=xrot.device)
    _check(lib().tq_gemv_rowsplit(payload.data_ptr(), payload.numel() * payload.element_size(),
                                  _fmt(fmt), n, k, xrot.data_ptr(), _dtype_code(xrot), batch,
                                  xrot.stride(0), out.data_ptr(), out.stride(0),
                                  _stream(xrot.device)))
    return out


def rotated_gemv_rowsplit(payload, fmt, n, k, x, signs, out=None):
    """y [batch, n] fp32 = decode-GEMV of the signed transform of x [batch, k]
    (unrotated), in one launch."""
    torch = _torch()
    _dev(payload, "payload")
    _dev(x, "x")
    _dev(signs, "signs")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    batch = x.shape[0]
    if out is None:
        out = torch.empty((batch, n), dtype=torch.float32, device=x.device)
    _check(lib().tq_rotated_gemv_rowsplit(payload.data_ptr(), payload.numel() * payload.element_size(),
                                          _fmt(fmt), n, k, x.data_ptr(), _dtype_code(x), batch,
                                          x.stride(0), signs.data_ptr(), out.data_ptr(),
                                          out.stride(0), _stream(x.device)))
    return out


def gemm_rowsplit(payload, fmt, n, k, x, out_dtype=None, out=None):
    """Y [m, n] = prefill GEMM of rotated activations x [m, k] (f16 or bf16)."""
    torch = _torch()
    _dev(payload, "payload")
    _dev(x, "x")
    m = x.shape[0]
    ycode = F32 if out_dtype in (None, torch.float32) else BF16
    if out is None:
        out = torch.empty((m, n), dtype=_dtype_of(ycode), device=x.device)
    _check(lib().tq_gemm_rowsplit(payload.data_ptr(), payload.numel() * payload.element_size(),
                                  _fmt(fmt), n, k, x.data_ptr(), _dtype_code(x), m, x.stride(0),
                                  out.data_ptr(), ycode, out.stride(0), _stream(x.device)))
    return out


def embed_rows_inverse(payload, fmt, n, k, ids, signs, out=None, err_word=None):
    """out [count, k] fp32: inverse-transformed dequantised rows ids."""
    torch = _torch()
    _dev(payload, "payload")
    _dev(ids, "ids")
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    count = ids.numel()
    if out is None:
        out = torch.empty((count, k), dtype=torch.float32, device=ids.device)
    err_ptr = None if err_word is None else err_word.data_ptr()
    _check(lib().tq_embed_rows_inverse(payload.data_ptr(), payload.numel() * payload.element_size(),
                                       _fmt(fmt), n, k, ids.data_ptr(), count, _signs_ptr(signs),
                                       out.data_ptr(), out.stride(0) if count else k, err_ptr,
                                       _stream(ids.device)))
    return out


def decode_rowsplit(payload, fmt, n, k, rows):
    """(values int8 [count, k_pad], scale bits int16 [count, G]) for rows."""
    torch = _torch()
    _dev(payload, "payload")
    g = geometry(fmt, n, k)
    count = rows.numel()
    values = torch.empty((count, g["k_pad"]), dtype=torch.int8, device=rows.device)
    scales = torch.empty((count, g["groups_per_row"]), dtype=torch.int16, device=rows.device)
    _check(lib().tq_decode_rowsplit(payload.data_ptr(), payload.numel() * payload.element_size(),
                                    _fmt(fmt), n, k, rows.data_ptr(), count, values.data_ptr(),
                                    scales.data_ptr(), _stream(rows.device)))
    return values, scales


def blocks_to_planes(blocks, fmt, n, k, out=None):
    """Row-split payload (uint8 device tensor) of a GGUF block stream."""
    torch = _torch()
    _dev(blocks, "blocks")
    g = geometry(fmt, n, k)
    if out is None:
        out = torch.empty(g["payload_bytes"], dtype=torch.uint8, device=blocks.device)
    _check(lib().tq_blocks_to_planes(blocks.data_ptr(), blocks.numel() * blocks.element_size(),
                                     _fmt(fmt), n, k, out.data_ptr(),
                                     out.numel() * out.element_size(), _stream(blocks.device)))
    return out


def planes_to_blocks(payload, fmt, n, k, out=None):
    """GGUF block stream (uint8 device tensor) of a row-split payload."""
    torch = _torch()
    _dev(payload, "payload")
    g = geometry(fmt, n, k)
    nbytes = n * g["groups_per_row"] * (34 if _fmt(fmt) == PQ2_0_G128 else 28)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=payload.device)
    _check(lib().tq_planes_to_blocks(payload.data_ptr(), payload.numel() * payload.element_size(),
                                     _fmt(fmt), n, k, out.data_ptr(),
                                     out.numel() * out.element_size(), _stream(payload.device)))
    return out


def g64_bytes(n, k):
    """Size of the 2-bit G64 block stream of an [n, k] matrix."""
    out = _u64()
    _check(lib().tq_g64_bytes(n, k, ctypes.byref(out)))
    return int(out.value)


def expand_g64(payload, fmt, n, k, out=None):
    """2-bit G64 block stream (uint8 device tensor) of a row-split payload."""
    torch = _torch()
    _dev(payload, "payload")
    if out is None:
        out = torch.empty(g64_bytes(n, k), dtype=torch.uint8, device=payload.device)
    _check(lib().tq_expand_g64(payload.data_ptr(), payload.numel() * payload.element_size(),
                               _fmt(fmt), n, k, out.data_ptr(), out.numel() * out.element_size(),
                               _stream(payload.device)))
    return out


def gemv_g64(blocks, n, k, xrot, out=None):
    """y [batch, n] fp32 = decode-GEMV over a G64 block stream (batch 1)."""
    torch = _torch()
    _dev(blocks, "blocks")
    _dev(xrot, "xrot")
    if xrot.dim() == 1:
        xrot = xrot.unsqueeze(0)
    batch = xrot.shape[0]
    if out is None:
        out = torch.empty((batch, n), dtype=torch.float32, device=xrot.device)
    _check(lib().tq_gemv_g64(blocks.data_ptr(), blocks.numel() * blocks.element_size(), n, k,
                             xrot.data_ptr(), _dtype_code(xrot), batch, xrot.stride(0),
                             out.data_ptr(), out.stride(0), _stream(xrot.device)))
    return out


def head_argmax(payload, fmt, n, k, x, norm, eps, signs, work, logits=None, token=None):
    """Greedy token (int32 device tensor [1]) of the output head step on one
    hidden row x [k]: RMSNorm(norm, eps), signed transform, head GEMV; the
    logits go to `logits` [n] fp32 when given.  work: int64 device tensor of
    two zeroed words (left zero by every call)."""
    torch = _torch()
    for t, name in ((payload, "payload"), (x, "x"), (norm, "norm"), (signs, "signs"), (work, "work")):
        _dev(t, name)
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=x.device)
    lp = None if logits is None else logits.data_ptr()
    _check(lib().tq_head_argmax(payload.data_ptr(), payload.numel() * payload.element_size(),
                                _fmt(fmt), n, k, x.data_ptr(), _dtype_code(x), norm.data_ptr(),
                                float(eps), _signs_ptr(signs), lp, work.data_ptr(), token.data_ptr(),
                                _stream(x.device)))
    return token


def head_argmax_noalloc(payload, fmt, n, k, x, norm, eps, signs, logits=None, token=None):
    """head_argmax without a work buffer: the work words are the library's
    own per-GPU device global (calls on one GPU must not overlap).  The token
    tensor is allocated here when not given; pass `token` (and `logits`) to
    call without any allocation, e.g. under graph capture."""
    torch = _torch()
    for t, name in ((payload, "payload"), (x, "x"), (norm, "norm"), (signs, "signs")):
        _dev(t, name)
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=x.device)
    lp = None if logits is None else logits.data_ptr()
    _check(lib().tq_head_argmax_noalloc(payload.data_ptr(), payload.numel() * payload.element_size(),
                                        _fmt(fmt), n, k, x.data_ptr(), _dtype_code(x), norm.data_ptr(),
                                        float(eps), _signs_ptr(signs), lp, token.data_ptr(),
                                        _stream(x.device)))
    return token


# grouped value-head order of the model: 3 x 16 heads of 128
GDN_TILES, GDN_GROUPS, GDN_HEAD_DIM = 3, 16, 128


def hadamard_signed_grouped(x, signs, tiles=GDN_TILES, groups=GDN_GROUPS, head_dim=GDN_HEAD_DIM,
                            out_dtype=None, out=None):
    """Forward signed transform of rows x [rows, k] taken in the grouped head order."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit column stride")
    rows, k = x.shape
    if out is None:
        out = torch.empty((rows, k), dtype=out_dtype or x.dtype, device=x.device)
    _check(lib().tq_hadamard_signed_grouped(x.data_ptr(), _dtype_code(x), rows, k,
                                            x.stride(0) if rows else k, tiles, groups, head_dim,
                                            _signs_ptr(signs), out.data_ptr(), _dtype_code(out),
                                            out.stride(0) if rows else k, _stream(x.device)))
    return out


def rotated_gemv_rowsplit_grouped(payload, fmt, n, k, x, signs, tiles=GDN_TILES, groups=GDN_GROUPS,
                                  head_dim=GDN_HEAD_DIM, out=None):
    """y [batch, n] fp32 = decode-GEMV of the signed transform of x [batch, k]
    taken in the grouped head order, in one launch."""
    torch = _torch()
    _dev(payload, "payload")
    _dev(x, "x")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    batch = x.shape[0]
    if out is None:
        out = torch.empty((batch, n), dtype=torch.float32, device=x.device)
    _check(lib().tq_rotated_gemv_rowsplit_grouped(
        payload.data_ptr(), payload.numel() * payload.element_size(), _fmt(fmt), n, k, x.data_ptr(),
        _dtype_code(x), batch, x.stride(0), tiles, groups, head_dim, _signs_ptr(signs),
        out.data_ptr(), out.stride(0), _stream(x.device)))
    return out


def stream_read(src, sink=None):
    """Plain streaming read of a device tensor (the bandwidth reference the
    GEMVs are measured beside); returns the sink word tensor."""
    torch = _torch()
    _dev(src, "src")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=src.device)
    _check(lib().tq_stream_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                                _stream(src.device)))
    return sink
