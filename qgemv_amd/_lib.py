"""ctypes binding of libpingala's C ABI (include/pingala.h).

Argument marshalling only: every function has the C entry point's name and
arguments, takes torch tensors (device buffers) or numpy arrays (host
buffers) and calls the library; all arithmetic runs in the library's HIP
kernels or its host encoder.  A missing library raises -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpingala.so")

PG_OK, PG_ERR_INVALID_ARG, PG_ERR_UNSUPPORTED, PG_ERR_HIP = 0, -1, -2, -3
PG_F32, PG_F16, PG_BF16, PG_Q16 = 0, 1, 2, 3
PG_FLAG_RMSNORM = 1
PG_FLAG_CARRY_STATE = 2
PG_FLAG_KERNEL_VDOT = 4
PG_FLAG_KERNEL_MMA = 8
PG_FLAG_RATE23 = 16

EXPORTS = ("pg_version", "pg_footprint_bytes", "pg_q16_row_bytes", "pg_last_error", "pg_codebook_table", "pg_encode_ref",
           "pg_encode", "pg_encode_ex", "pg_decode_ex",
           "pg_decode", "pg_fwht_rotate", "pg_fwht_rotate_ex", "pg_qgemv", "pg_rot_qgemv", "pg_qgemm",
           "pg_qgemm_ex", "pg_qgemm_workspace_bytes", "pg_hbm_read",
           "pg_qgemm_noalloc", "pg_qgemv_ex", "pg_qgemm_tune", "pg_decode_table", "pg_rot_qgemv_table",
           "pg_encode_ref_ldlq", "pg_encode_ldlq", "pg_codebook_table_ex",
           "pg_encode_ref_table", "pg_encode_table")


class PgError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libpingala error {code}: {msg}")
        self.code = code


_LIB = None


def lib():
    """Load libpingala.so (built in-tree by qgemv_amd/build.py)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        # torch ships its own HIP runtime under the same soname
        # (libamdhip64.so.7); loading torch first makes libpingala bind to that
        # one, so the process holds a single HIP runtime and torch's device
        # buffers and streams are valid in the library
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
        L.pg_version.restype = i32
        L.pg_version.argtypes = []
        L.pg_footprint_bytes.restype = ctypes.c_size_t
        L.pg_footprint_bytes.argtypes = [i64, i64]
        L.pg_q16_row_bytes.restype = ctypes.c_size_t
        L.pg_q16_row_bytes.argtypes = [i64]
        L.pg_last_error.restype = ctypes.c_char_p
        L.pg_last_error.argtypes = []
        L.pg_codebook_table.restype = i32
        L.pg_codebook_table.argtypes = [vp]
        L.pg_codebook_table_ex.restype = i32
        L.pg_codebook_table_ex.argtypes = [u32, vp]
        L.pg_encode_ref.restype = i32
        L.pg_encode_ref.argtypes = [vp, i64, i64, vp, vp, vp, i32]
        L.pg_encode.restype = i32
        L.pg_encode.argtypes = [vp, i64, i64, vp, vp, vp, vp]
        L.pg_encode_ref_ldlq.restype = i32
        L.pg_encode_ref_ldlq.argtypes = [vp, i64, i64, vp, vp, vp, vp, i32]
        L.pg_encode_ref_table.restype = i32
        L.pg_encode_ref_table.argtypes = [vp, i64, i64, vp, vp, u32, vp, vp, i32]
        L.pg_encode_table.restype = i32
        L.pg_encode_table.argtypes = [vp, i64, i64, vp, vp, u32, vp, vp, vp]
        L.pg_encode_ldlq.restype = i32
        L.pg_encode_ldlq.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
        L.pg_encode_ex.restype = i32
        L.pg_encode_ex.argtypes = [vp, i64, i64, vp, u32, vp, vp, vp]
        L.pg_decode_ex.restype = i32
        L.pg_decode_ex.argtypes = [vp, vp, i64, i64, u32, vp, vp]
        L.pg_decode_table.restype = i32
        L.pg_decode_table.argtypes = [vp, vp, i64, i64, vp, u32, vp, vp]
        L.pg_rot_qgemv_table.restype = i32
        L.pg_rot_qgemv_table.argtypes = [vp, vp, i64, i64, vp, i32, vp, vp, u32, vp, vp]
        L.pg_decode.restype = i32
        L.pg_decode.argtypes = [vp, vp, i64, i64, vp, vp]
        L.pg_fwht_rotate.restype = i32
        L.pg_fwht_rotate.argtypes = [vp, i32, vp, i32, vp, i64, i64, u32, vp]
        L.pg_fwht_rotate_ex.restype = i32
        L.pg_fwht_rotate_ex.argtypes = [vp, i32, i64, vp, i32, vp, i64, i64, u32, vp]
        L.pg_qgemv.restype = i32
        L.pg_qgemv.argtypes = [vp, vp, i64, i64, vp, i32, i32, vp, vp]
        L.pg_rot_qgemv.restype = i32
        L.pg_rot_qgemv.argtypes = [vp, vp, i64, i64, vp, i32, i64, vp, u32, i32, vp, vp]
        L.pg_qgemm.restype = i32
        L.pg_qgemm.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp]
        L.pg_qgemm_ex.restype = i32
        L.pg_qgemm_ex.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, ctypes.c_size_t, vp]
        L.pg_qgemm_workspace_bytes.restype = ctypes.c_size_t
        L.pg_qgemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.pg_qgemv_ex.restype = i32
        L.pg_qgemv_ex.argtypes = [vp, vp, i64, i64, vp, i32, i32, u32, vp, vp]
        L.pg_qgemm_tune.restype = i32
        L.pg_qgemm_tune.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, ctypes.c_size_t, i32, i32, i64, vp]
        L.pg_qgemm_noalloc.restype = i32
        L.pg_qgemm_noalloc.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp]
        L.pg_hbm_read.restype = i32
        L.pg_hbm_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        _LIB = L
    return _LIB


def _check(rc: int) -> None:
    if rc != PG_OK:
        raise PgError(rc, lib().pg_last_error().decode())


def _ptr(t):
    """Raw address of a torch tensor or numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _esz(dtype: int) -> int:
    return 4 if dtype == PG_F32 else 2


def _need(t, nbytes: int, name: str) -> None:
    """Check a buffer handed to the library as a device pointer: a torch
    tensor must be a contiguous GPU tensor of at least nbytes bytes (a raw
    integer address is passed through unchecked; the library validates
    alignment and null pointers).  Raises ValueError before any call."""
    if t is None or isinstance(t, int):
        return
    if isinstance(t, np.ndarray):
        raise ValueError(f"{name}: a device buffer is required, got a numpy array")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name}: tensor is not on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor is not contiguous")
    have = t.numel() * t.element_size()
    if nbytes > 0 and have < nbytes:
        raise ValueError(f"{name}: {have} bytes, the call needs {nbytes}")


def _weights(codes, scales, n: int, k: int) -> None:
    if n > 0 and k > 0:
        _need(codes, n * (k // 4), "codes")
        _need(scales, n * (k // 128) * 2, "scales")


def _xbytes(dtype: int, rows: int, ldx: int, k: int) -> int:
    if rows < 1 or k < 1:
        return 0
    if dtype == PG_Q16:
        return rows * (q16_row_bytes_host(k))
    return ((rows - 1) * ldx + k) * _esz(dtype)


def q16_row_bytes_host(k: int) -> int:
    """Bytes of one PG_Q16 row (the layout in include/pingala.h)."""
    raw = 2 * k + k // 32 + k // 16
    return (raw + 63) & ~63


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _qgemm_need(codes, scales, n, k, x, m, y) -> None:
    _weights(codes, scales, n, k)
    _need(x, max(m, 0) * max(k, 0) * 2, "x_rot_bf16")
    _need(y, max(m, 0) * max(n, 0) * 4, "y")


def pg_version() -> int:
    return lib().pg_version()


def pg_footprint_bytes(n: int, k: int) -> int:
    return lib().pg_footprint_bytes(n, k)


def pg_q16_row_bytes(k: int) -> int:
    return lib().pg_q16_row_bytes(k)


def pg_last_error() -> str:
    return lib().pg_last_error().decode()


def pg_codebook_table() -> np.ndarray:
    out = np.zeros((8, 256, 4), dtype=np.int8)
    _check(lib().pg_codebook_table(out.ctypes.data))
    return out


def pg_codebook_table_ex(flags: int) -> np.ndarray:
    """A format's codebook as a table (flags 0: P8F v1; PG_FLAG_RATE23: the
    rate-2/3 variant)."""
    out = np.zeros((8, 256, 4), dtype=np.int8)
    _check(lib().pg_codebook_table_ex(flags, out.ctypes.data))
    return out


def pg_encode_ref(w: np.ndarray, n: int, k: int, sign_bits: np.ndarray, codes: np.ndarray,
                  scales: np.ndarray, n_threads: int = 0) -> None:
    """Host buffers (numpy, C-contiguous): w f32 [n][k], sign_bits u8 [k/8],
    codes u8 [n][k/4] out, scales u16 [n][k/128] out."""
    for a in (w, sign_bits, codes, scales):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("host buffers must be C-contiguous")
    _check(lib().pg_encode_ref(_ptr(w), n, k, _ptr(sign_bits), _ptr(codes), _ptr(scales), n_threads))


def _host_hessian(hessian, k: int):
    if not isinstance(hessian, np.ndarray) or hessian.dtype != np.float64 or not hessian.flags["C_CONTIGUOUS"]:
        raise ValueError("hessian: a C-contiguous float64 numpy array is required")
    if k > 0 and hessian.size < k * k:
        raise ValueError(f"hessian: {hessian.size} values, {k * k} needed")


def pg_encode_ref_ldlq(w: np.ndarray, n: int, k: int, sign_bits: np.ndarray, hessian: np.ndarray,
                       codes: np.ndarray, scales: np.ndarray, n_threads: int = 0) -> None:
    """LDLQ reference encoder.  Host buffers (numpy, C-contiguous): w f32
    [n][k], sign_bits u8 [k/8], hessian f64 [k][k], codes u8 [n][k/4] out,
    scales u16 [n][k/128] out."""
    for a, nbytes, name in ((w, n * k * 4, "w"), (sign_bits, k // 8, "sign_bits"), (codes, n * (k // 4), "codes"),
                            (scales, n * (k // 128) * 2, "scales")):
        if not isinstance(a, np.ndarray) or not a.flags["C_CONTIGUOUS"]:
            raise ValueError(f"{name}: a C-contiguous numpy array is required")
        if n > 0 and k > 0 and a.nbytes < nbytes:
            raise ValueError(f"{name}: {a.nbytes} bytes, {nbytes} needed")
    _host_hessian(hessian, k)
    _check(lib().pg_encode_ref_ldlq(_ptr(w), n, k, _ptr(sign_bits), _ptr(hessian), _ptr(codes), _ptr(scales),
                                    n_threads))


def pg_encode_ldlq(w, n: int, k: int, sign_bits, hessian: np.ndarray, codes, scales, stream=None) -> None:
    """LDLQ encoder on the GPU: w, sign_bits, codes, scales device buffers
    as pg_encode; hessian host f64 [k][k] (numpy).  Synchronous."""
    _need(w, max(n, 0) * max(k, 0) * 4, "w")
    _need(sign_bits, max(k, 0) // 8, "sign_bits")
    _weights(codes, scales, n, k)
    _host_hessian(hessian, k)
    _check(lib().pg_encode_ldlq(_ptr(w), n, k, _ptr(sign_bits), _ptr(hessian), _ptr(codes), _ptr(scales),
                                _stream(stream)))


def pg_encode_ref_table(w: np.ndarray, n: int, k: int, sign_bits: np.ndarray, table: np.ndarray, flags: int,
                        codes: np.ndarray, scales: np.ndarray, n_threads: int = 0) -> None:
    """Host encoder through a codebook table (numpy buffers, C-contiguous):
    table int8 [8][256][4]; flags 0 or PG_FLAG_RATE23."""
    for a, nbytes, name in ((w, n * k * 4, "w"), (sign_bits, k // 8, "sign_bits"), (table, 8192, "table"),
                            (codes, n * (k // 4), "codes"), (scales, n * (k // 128) * 2, "scales")):
        if not isinstance(a, np.ndarray) or not a.flags["C_CONTIGUOUS"]:
            raise ValueError(f"{name}: a C-contiguous numpy array is required")
        if n > 0 and k > 0 and a.nbytes < nbytes:
            raise ValueError(f"{name}: {a.nbytes} bytes, {nbytes} needed")
    _check(lib().pg_encode_ref_table(_ptr(w), n, k, _ptr(sign_bits), _ptr(table), flags, _ptr(codes), _ptr(scales),
                                     n_threads))


def pg_encode_table(w, n: int, k: int, sign_bits, table, flags: int, codes, scales, stream=None) -> None:
    """GPU encoder through a codebook table (device buffers as pg_encode;
    table device int8 [8][256][4])."""
    _need(w, max(n, 0) * max(k, 0) * 4, "w")
    _need(sign_bits, max(k, 0) // 8, "sign_bits")
    _need(table, TABLE_BYTES, "table")
    _weights(codes, scales, n, k)
    _check(lib().pg_encode_table(_ptr(w), n, k, _ptr(sign_bits), _ptr(table), flags, _ptr(codes), _ptr(scales),
                                 _stream(stream)))


def pg_encode(w, n: int, k: int, sign_bits, codes, scales, stream=None) -> None:
    """Device buffers: w f32 [n][k], sign_bits u8 [k/8], codes u8 [n][k/4]
    out, scales 16-bit [n][k/128] out (fp16 bits)."""
    _need(w, max(n, 0) * max(k, 0) * 4, "w")
    _need(sign_bits, max(k, 0) // 8, "sign_bits")
    _weights(codes, scales, n, k)
    _check(lib().pg_encode(_ptr(w), n, k, _ptr(sign_bits), _ptr(codes), _ptr(scales), _stream(stream)))


def pg_encode_ex(w, n: int, k: int, sign_bits, flags: int, codes, scales, stream=None) -> None:
    """pg_encode with format flags (PG_FLAG_CARRY_STATE: the carried-state variant)."""
    _need(w, max(n, 0) * max(k, 0) * 4, "w")
    _need(sign_bits, max(k, 0) // 8, "sign_bits")
    _weights(codes, scales, n, k)
    _check(lib().pg_encode_ex(_ptr(w), n, k, _ptr(sign_bits), flags, _ptr(codes), _ptr(scales), _stream(stream)))


def pg_decode_ex(codes, scales, n: int, k: int, flags: int, w_rot, stream=None) -> None:
    """pg_decode with format flags (PG_FLAG_CARRY_STATE: the carried-state variant)."""
    _weights(codes, scales, n, k)
    _need(w_rot, max(n, 0) * max(k, 0) * 4, "w_rot")
    _check(lib().pg_decode_ex(_ptr(codes), _ptr(scales), n, k, flags, _ptr(w_rot), _stream(stream)))


TABLE_BYTES = 8 * 256 * 4     # int8 [8][256][4] codebook table


def pg_decode_table(codes, scales, n: int, k: int, table, flags: int, w_rot, stream=None) -> None:
    """Decode through a codebook table (device int8 [8][256][4])."""
    _weights(codes, scales, n, k)
    _need(table, TABLE_BYTES, "table")
    _need(w_rot, max(n, 0) * max(k, 0) * 4, "w_rot")
    _check(lib().pg_decode_table(_ptr(codes), _ptr(scales), n, k, _ptr(table), flags, _ptr(w_rot), _stream(stream)))


def pg_decode(codes, scales, n: int, k: int, w_rot, stream=None) -> None:
    _weights(codes, scales, n, k)
    _need(w_rot, max(n, 0) * max(k, 0) * 4, "w_rot")
    _check(lib().pg_decode(_ptr(codes), _ptr(scales), n, k, _ptr(w_rot), _stream(stream)))


def pg_fwht_rotate(x, in_dtype: int, y, out_dtype: int, sign_bits, rows: int, k: int, flags: int = 0,
                   stream=None) -> None:
    _need(x, _xbytes(in_dtype, rows, k, k), "x")
    _need(y, _xbytes(out_dtype, rows, k, k), "y")
    _need(sign_bits, max(k, 0) // 8, "sign_bits")
    _check(lib().pg_fwht_rotate(_ptr(x), in_dtype, _ptr(y), out_dtype, _ptr(sign_bits), rows, k, flags,
                                _stream(stream)))


def pg_fwht_rotate_ex(x, in_dtype: int, ldx: int, y, out_dtype: int, sign_bits, rows: int, k: int, flags: int = 0,
                      stream=None) -> None:
    _need(x, _xbytes(in_dtype, rows, ldx, k), "x")
    _need(y, _xbytes(out_dtype, rows, k, k), "y")
    _need(sign_bits, max(k, 0) // 8, "sign_bits")
    _check(lib().pg_fwht_rotate_ex(_ptr(x), in_dtype, ldx, _ptr(y), out_dtype, _ptr(sign_bits), rows, k, flags,
                                   _stream(stream)))


def pg_qgemv(codes, scales, n: int, k: int, x_rot, x_dtype: int, batch: int, y, stream=None) -> None:
    _weights(codes, scales, n, k)
    _need(x_rot, _xbytes(x_dtype, batch, k, k), "x_rot")
    _need(y, max(batch, 0) * max(n, 0) * 4, "y")
    _check(lib().pg_qgemv(_ptr(codes), _ptr(scales), n, k, _ptr(x_rot), x_dtype, batch, _ptr(y),
                          _stream(stream)))


def pg_rot_qgemv(codes, scales, n: int, k: int, x, x_dtype: int, ldx: int, sign_bits, flags: int, batch: int, y,
                 stream=None) -> None:
    _weights(codes, scales, n, k)
    _need(x, _xbytes(x_dtype, batch, ldx, k), "x")
    _need(sign_bits, max(k, 0) // 8, "sign_bits")
    _need(y, max(batch, 0) * max(n, 0) * 4, "y")
    _check(lib().pg_rot_qgemv(_ptr(codes), _ptr(scales), n, k, _ptr(x), x_dtype, ldx, _ptr(sign_bits), flags,
                              batch, _ptr(y), _stream(stream)))


def pg_rot_qgemv_table(codes, scales, n: int, k: int, x, x_dtype: int, sign_bits, table, flags: int, y,
                       stream=None) -> None:
    """The batch-1 fused stage through a codebook table."""
    _weights(codes, scales, n, k)
    _need(x, _xbytes(x_dtype, 1, k, k), "x")
    _need(sign_bits, max(k, 0) // 8, "sign_bits")
    _need(table, TABLE_BYTES, "table")
    _need(y, max(n, 0) * 4, "y")
    _check(lib().pg_rot_qgemv_table(_ptr(codes), _ptr(scales), n, k, _ptr(x), x_dtype, _ptr(sign_bits), _ptr(table),
                                    flags, _ptr(y), _stream(stream)))


def pg_qgemm(codes, scales, n: int, k: int, x_rot_bf16, m: int, y, stream=None) -> None:
    _qgemm_need(codes, scales, n, k, x_rot_bf16, m, y)
    _check(lib().pg_qgemm(_ptr(codes), _ptr(scales), n, k, _ptr(x_rot_bf16), m, _ptr(y), _stream(stream)))


def pg_qgemm_ex(codes, scales, n: int, k: int, x_rot_bf16, m: int, y, workspace, workspace_bytes: int,
                stream=None) -> None:
    _qgemm_need(codes, scales, n, k, x_rot_bf16, m, y)
    _need(workspace, workspace_bytes, "workspace")
    _check(lib().pg_qgemm_ex(_ptr(codes), _ptr(scales), n, k, _ptr(x_rot_bf16), m, _ptr(y), _ptr(workspace),
                             workspace_bytes, _stream(stream)))


def pg_qgemm_workspace_bytes(n: int, k: int, m: int) -> int:
    return lib().pg_qgemm_workspace_bytes(n, k, m)


def pg_hbm_read(p, nbytes: int, xor_out, stream=None) -> None:
    """Streaming read of nbytes (multiple of 16) at device buffer p; the XOR of
    its 32-bit words is XOR-ed into the device u32 xor_out."""
    _need(p, nbytes, "p")
    _need(xor_out, 4, "xor_out")
    _check(lib().pg_hbm_read(_ptr(p), nbytes, _ptr(xor_out), _stream(stream)))


def pg_qgemm_noalloc(codes, scales, n: int, k: int, x_rot_bf16, m: int, y, stream=None) -> None:
    """pg_qgemm_ex on the library's own split workspace (no allocation)."""
    _qgemm_need(codes, scales, n, k, x_rot_bf16, m, y)
    _check(lib().pg_qgemm_noalloc(_ptr(codes), _ptr(scales), n, k, _ptr(x_rot_bf16), m, _ptr(y), _stream(stream)))


def pg_qgemv_ex(codes, scales, n: int, k: int, x_rot, x_dtype: int, batch: int, flags: int, y, stream=None) -> None:
    """pg_qgemv with kernel-choice flags (PG_FLAG_KERNEL_VDOT / PG_FLAG_KERNEL_MMA)."""
    _weights(codes, scales, n, k)
    _need(x_rot, _xbytes(x_dtype, batch, k, k), "x_rot")
    _need(y, max(batch, 0) * max(n, 0) * 4, "y")
    _check(lib().pg_qgemv_ex(_ptr(codes), _ptr(scales), n, k, _ptr(x_rot), x_dtype, batch, flags, _ptr(y),
                             _stream(stream)))


def pg_qgemm_tune(codes, scales, n: int, k: int, x_rot_bf16, m: int, y, workspace, workspace_bytes: int, kernel: int,
                  splits: int, first_split: int, stream=None) -> None:
    """pg_qgemm_ex with its kernel (0 the library's choice, 1..8 as in
    pingala.h) and split plan given."""
    _qgemm_need(codes, scales, n, k, x_rot_bf16, m, y)
    _need(workspace, workspace_bytes, "workspace")
    _check(lib().pg_qgemm_tune(_ptr(codes), _ptr(scales), n, k, _ptr(x_rot_bf16), m, _ptr(y), _ptr(workspace),
                               workspace_bytes, kernel, splits, first_split, _stream(stream)))
