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

EXPORTS = ("pg_version", "pg_footprint_bytes", "pg_q16_row_bytes", "pg_last_error", "pg_codebook_table", "pg_encode_ref",
           "pg_encode", "pg_encode_ex", "pg_decode_ex",
           "pg_decode", "pg_fwht_rotate", "pg_fwht_rotate_ex", "pg_qgemv", "pg_rot_qgemv", "pg_qgemm",
           "pg_qgemm_ex", "pg_qgemm_workspace_bytes")


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
        L.pg_encode_ref.restype = i32
        L.pg_encode_ref.argtypes = [vp, i64, i64, vp, vp, vp, i32]
        L.pg_encode.restype = i32
        L.pg_encode.argtypes = [vp, i64, i64, vp, vp, vp, vp]
        L.pg_encode_ex.restype = i32
        L.pg_encode_ex.argtypes = [vp, i64, i64, vp, u32, vp, vp, vp]
        L.pg_decode_ex.restype = i32
        L.pg_decode_ex.argtypes = [vp, vp, i64, i64, u32, vp, vp]
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


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


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


def pg_encode_ref(w: np.ndarray, n: int, k: int, sign_bits: np.ndarray, codes: np.ndarray,
                  scales: np.ndarray, n_threads: int = 0) -> None:
    """Host buffers (numpy, C-contiguous): w f32 [n][k], sign_bits u8 [k/8],
    codes u8 [n][k/4] out, scales u16 [n][k/128] out."""
    for a in (w, sign_bits, codes, scales):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("host buffers must be C-contiguous")
    _check(lib().pg_encode_ref(_ptr(w), n, k, _ptr(sign_bits), _ptr(codes), _ptr(scales), n_threads))


def pg_encode(w, n: int, k: int, sign_bits, codes, scales, stream=None) -> None:
    """Device buffers: w f32 [n][k], sign_bits u8 [k/8], codes u8 [n][k/4]
    out, scales 16-bit [n][k/128] out (fp16 bits)."""
    _check(lib().pg_encode(_ptr(w), n, k, _ptr(sign_bits), _ptr(codes), _ptr(scales), _stream(stream)))


def pg_encode_ex(w, n: int, k: int, sign_bits, flags: int, codes, scales, stream=None) -> None:
    """pg_encode with format flags (PG_FLAG_CARRY_STATE: the carried-state variant)."""
    _check(lib().pg_encode_ex(_ptr(w), n, k, _ptr(sign_bits), flags, _ptr(codes), _ptr(scales), _stream(stream)))


def pg_decode_ex(codes, scales, n: int, k: int, flags: int, w_rot, stream=None) -> None:
    """pg_decode with format flags (PG_FLAG_CARRY_STATE: the carried-state variant)."""
    _check(lib().pg_decode_ex(_ptr(codes), _ptr(scales), n, k, flags, _ptr(w_rot), _stream(stream)))


def pg_decode(codes, scales, n: int, k: int, w_rot, stream=None) -> None:
    _check(lib().pg_decode(_ptr(codes), _ptr(scales), n, k, _ptr(w_rot), _stream(stream)))


def pg_fwht_rotate(x, in_dtype: int, y, out_dtype: int, sign_bits, rows: int, k: int, flags: int = 0,
                   stream=None) -> None:
    _check(lib().pg_fwht_rotate(_ptr(x), in_dtype, _ptr(y), out_dtype, _ptr(sign_bits), rows, k, flags,
                                _stream(stream)))


def pg_fwht_rotate_ex(x, in_dtype: int, ldx: int, y, out_dtype: int, sign_bits, rows: int, k: int, flags: int = 0,
                      stream=None) -> None:
    _check(lib().pg_fwht_rotate_ex(_ptr(x), in_dtype, ldx, _ptr(y), out_dtype, _ptr(sign_bits), rows, k, flags,
                                   _stream(stream)))


def pg_qgemv(codes, scales, n: int, k: int, x_rot, x_dtype: int, batch: int, y, stream=None) -> None:
    _check(lib().pg_qgemv(_ptr(codes), _ptr(scales), n, k, _ptr(x_rot), x_dtype, batch, _ptr(y),
                          _stream(stream)))


def pg_rot_qgemv(codes, scales, n: int, k: int, x, x_dtype: int, ldx: int, sign_bits, flags: int, batch: int, y,
                 stream=None) -> None:
    _check(lib().pg_rot_qgemv(_ptr(codes), _ptr(scales), n, k, _ptr(x), x_dtype, ldx, _ptr(sign_bits), flags,
                              batch, _ptr(y), _stream(stream)))


def pg_qgemm(codes, scales, n: int, k: int, x_rot_bf16, m: int, y, stream=None) -> None:
    _check(lib().pg_qgemm(_ptr(codes), _ptr(scales), n, k, _ptr(x_rot_bf16), m, _ptr(y), _stream(stream)))


def pg_qgemm_ex(codes, scales, n: int, k: int, x_rot_bf16, m: int, y, workspace, workspace_bytes: int,
                stream=None) -> None:
    _check(lib().pg_qgemm_ex(_ptr(codes), _ptr(scales), n, k, _ptr(x_rot_bf16), m, _ptr(y), _ptr(workspace),
                             workspace_bytes, _stream(stream)))


def pg_qgemm_workspace_bytes(n: int, k: int, m: int) -> int:
    return lib().pg_qgemm_workspace_bytes(n, k, m)
