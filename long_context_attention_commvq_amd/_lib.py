"""ctypes binding of libcommvq (the C ABI declared in include/commvq.h).

Argument marshalling only: every computation runs in the HIP library. Tensors
are passed as device pointers (``tensor.data_ptr()``) and the stream defaults to
torch's current stream on the tensor's device. Loading fails loudly when the
library has not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import c_double, c_int32, c_int64, c_size_t, c_void_p, c_float, POINTER

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcommvq.so")

COMMVQ_OK = 0
COMMVQ_ERR_INVALID_ARG = -1
COMMVQ_ERR_UNSUPPORTED = -2
COMMVQ_ERR_WORKSPACE = -3
COMMVQ_ERR_HIP = -4
COMMVQ_NOALLOC_SCRATCH_BYTES = 16 << 20
COMMVQ_F16 = 1
COMMVQ_DECODE_EXACT = 1

STATUS_NAMES = {
    COMMVQ_OK: "COMMVQ_OK",
    COMMVQ_ERR_INVALID_ARG: "COMMVQ_ERR_INVALID_ARG",
    COMMVQ_ERR_UNSUPPORTED: "COMMVQ_ERR_UNSUPPORTED",
    COMMVQ_ERR_WORKSPACE: "COMMVQ_ERR_WORKSPACE",
    COMMVQ_ERR_HIP: "COMMVQ_ERR_HIP",
}

EXPORTED = [
    "commvq_abi_version", "commvq_last_error", "commvq_validate_codebook", "commvq_bits_per_scalar",
    "commvq_code_bytes_per_token", "commvq_decode_workspace_bytes", "commvq_encode", "commvq_append",
    "commvq_decode_attention", "commvq_decode_step", "commvq_dequantize_kv", "commvq_dense_workspace_bytes",
    "commvq_dense_decode_attention", "commvq_em_work_bytes", "commvq_em_step", "commvq_decode_attention_bitv", "commvq_decode_bitv_workspace_bytes",
    "commvq_decode_step_noalloc",
]


class CommvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class commvq_codebook(ctypes.Structure):
    _fields_ = [("head_dim", c_int32), ("group_size", c_int32), ("n_entries", c_int32),
                ("n_rounds", c_int32), ("n_kv_heads", c_int32), ("dtype", c_int32),
                ("entries", c_void_p)]


class commvq_bit_codebook(ctypes.Structure):
    _fields_ = [("n_bits", c_int32), ("dim", c_int32), ("dtype", c_int32), ("reserved", c_int32),
                ("rows", c_void_p)]


class commvq_rope(ctypes.Structure):
    _fields_ = [("theta_base", c_double), ("pairing", c_int32), ("reserved", c_int32)]


_lib = None


def lib():
    """Load libcommvq.so once (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m long_context_attention_commvq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        CB = POINTER(commvq_codebook)
        L.commvq_abi_version.restype = c_int32
        L.commvq_abi_version.argtypes = []
        L.commvq_last_error.restype = ctypes.c_char_p
        L.commvq_last_error.argtypes = []
        L.commvq_validate_codebook.restype = c_int32
        L.commvq_validate_codebook.argtypes = [CB]
        L.commvq_bits_per_scalar.restype = c_double
        L.commvq_bits_per_scalar.argtypes = [CB]
        L.commvq_code_bytes_per_token.restype = c_int64
        L.commvq_code_bytes_per_token.argtypes = [CB]
        L.commvq_decode_workspace_bytes.restype = c_int64
        L.commvq_decode_workspace_bytes.argtypes = [c_int32, c_int32, c_int32, CB, CB]
        L.commvq_encode.restype = c_int32
        L.commvq_encode.argtypes = [CB, c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64, c_void_p, c_void_p]
        L.commvq_append.restype = c_int32
        L.commvq_append.argtypes = [CB, c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_void_p]
        L.commvq_decode_attention.restype = c_int32
        L.commvq_decode_attention.argtypes = [CB, CB, POINTER(commvq_rope), c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                              c_float, c_void_p, c_void_p, c_size_t, ctypes.c_uint32, c_void_p]
        L.commvq_decode_step.restype = c_int32
        L.commvq_decode_step.argtypes = [CB, CB, POINTER(commvq_rope), c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                         c_float, c_void_p, c_void_p, c_size_t, ctypes.c_uint32, c_void_p]
        L.commvq_decode_step_noalloc.restype = c_int32
        L.commvq_decode_step_noalloc.argtypes = [CB, CB, POINTER(commvq_rope), c_void_p, c_void_p, c_void_p, c_void_p,
                                                 c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                                 c_int32, c_float, c_void_p, ctypes.c_uint32, c_void_p]
        L.commvq_dequantize_kv.restype = c_int32
        L.commvq_dequantize_kv.argtypes = [CB, CB, POINTER(commvq_rope), c_void_p, c_void_p, c_void_p, c_int32,
                                           c_int32, c_int32, c_void_p, c_void_p, c_void_p]
        L.commvq_dense_workspace_bytes.restype = c_int64
        L.commvq_dense_workspace_bytes.argtypes = [c_int32, c_int32, c_int32, c_int32, c_int32]
        L.commvq_dense_decode_attention.restype = c_int32
        L.commvq_dense_decode_attention.argtypes = [POINTER(commvq_rope), c_void_p, c_void_p, c_void_p, c_void_p,
                                                    c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                                    c_float, c_void_p, c_void_p, c_size_t, c_void_p]
        L.commvq_decode_attention_bitv.restype = c_int32
        L.commvq_decode_attention_bitv.argtypes = [CB, POINTER(commvq_bit_codebook), POINTER(commvq_rope), c_void_p,
                                                   c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                                   c_int32, c_float, c_void_p, c_void_p, c_size_t, ctypes.c_uint32,
                                                   c_void_p]
        L.commvq_decode_bitv_workspace_bytes.restype = c_int64
        L.commvq_decode_bitv_workspace_bytes.argtypes = [c_int32, c_int32, c_int32, CB, POINTER(commvq_bit_codebook)]
        L.commvq_em_work_bytes.restype = c_int64
        L.commvq_em_work_bytes.argtypes = [CB]
        L.commvq_em_step.restype = c_int32
        L.commvq_em_step.argtypes = [CB, c_void_p, c_int64, c_int64, c_int32, c_float, c_float, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if hasattr(t, "device") and t.device.type == "cuda":
            return torch.cuda.current_stream(t.device).cuda_stream
    return torch.cuda.current_stream().cuda_stream


def _check(status: int) -> int:
    if status != COMMVQ_OK:
        raise CommvqError(status, commvq_last_error())
    return status


def make_codebook(entries, head_dim: int, group_size: int, n_entries: int, n_rounds: int,
                  n_kv_heads: int) -> commvq_codebook:
    """Descriptor for fp16 entries [Hkv][D/g][R][Nc'][g] (keep `entries` alive)."""
    return commvq_codebook(head_dim, group_size, n_entries, n_rounds, n_kv_heads, COMMVQ_F16,
                           _ptr(entries) if entries is not None else None)


def make_bit_codebook(rows, n_bits: int, dim: int) -> commvq_bit_codebook:
    """Descriptor for fp16 rows [n_bits][dim] (keep `rows` alive)."""
    return commvq_bit_codebook(n_bits, dim, COMMVQ_F16, 0, _ptr(rows) if rows is not None else None)


def make_rope(theta_base: float, pairing: int = 0) -> commvq_rope:
    return commvq_rope(float(theta_base), int(pairing), 0)


# ---- same names as the C ABI ------------------------------------------------

def commvq_abi_version() -> int:
    return lib().commvq_abi_version()


def commvq_last_error() -> str:
    return lib().commvq_last_error().decode()


def commvq_validate_codebook(cb: commvq_codebook) -> int:
    return lib().commvq_validate_codebook(ctypes.byref(cb))


def commvq_bits_per_scalar(cb: commvq_codebook) -> float:
    return lib().commvq_bits_per_scalar(ctypes.byref(cb))


def commvq_code_bytes_per_token(cb: commvq_codebook) -> int:
    return lib().commvq_code_bytes_per_token(ctypes.byref(cb))


def commvq_decode_workspace_bytes(batch: int, n_q_heads: int, max_seq_len: int, kcb: commvq_codebook,
                                  vcb: commvq_codebook) -> int:
    return lib().commvq_decode_workspace_bytes(batch, n_q_heads, max_seq_len, ctypes.byref(kcb),
                                               ctypes.byref(vcb))


def commvq_encode(cb: commvq_codebook, x, n_tokens: int, x_token_stride: int, codes, code_token_stride: int,
                  code_head_stride: int, gap_out=None, stream=None) -> int:
    return _check(lib().commvq_encode(ctypes.byref(cb), _ptr(x), n_tokens, x_token_stride, _ptr(codes),
                                      code_token_stride, code_head_stride, _ptr(gap_out), _stream(stream, x, codes)))


def commvq_append(cb: commvq_codebook, x, batch: int, positions, cache, cache_len: int, stream=None) -> int:
    return _check(lib().commvq_append(ctypes.byref(cb), _ptr(x), batch, _ptr(positions), _ptr(cache), cache_len,
                                      _stream(stream, x, cache)))


def commvq_decode_attention(kcb: commvq_codebook, vcb: commvq_codebook, rope: commvq_rope, q, q_pos, kcodes,
                            vcodes, seq_lens, batch: int, n_q_heads: int, cache_len: int, max_seq_len: int,
                            sm_scale: float, out, workspace, workspace_bytes: int, flags: int = 0,
                            stream=None) -> int:
    return _check(lib().commvq_decode_attention(
        ctypes.byref(kcb), ctypes.byref(vcb), ctypes.byref(rope), _ptr(q), _ptr(q_pos), _ptr(kcodes),
        _ptr(vcodes), _ptr(seq_lens), batch, n_q_heads, cache_len, max_seq_len, float(sm_scale), _ptr(out),
        _ptr(workspace), int(workspace_bytes), int(flags), _stream(stream, q, out)))


def commvq_decode_step(kcb: commvq_codebook, vcb: commvq_codebook, rope: commvq_rope, k_new, v_new, positions, q,
                       q_pos, kcodes, vcodes, seq_lens, batch: int, n_q_heads: int, cache_len: int, max_seq_len: int,
                       sm_scale: float, out, workspace, workspace_bytes: int, flags: int = 0, stream=None) -> int:
    return _check(lib().commvq_decode_step(
        ctypes.byref(kcb), ctypes.byref(vcb), ctypes.byref(rope), _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(q),
        _ptr(q_pos), _ptr(kcodes), _ptr(vcodes), _ptr(seq_lens), batch, n_q_heads, cache_len, max_seq_len,
        float(sm_scale), _ptr(out), _ptr(workspace), int(workspace_bytes), int(flags), _stream(stream, q, out)))


def commvq_decode_step_noalloc(kcb: commvq_codebook, vcb: commvq_codebook, rope: commvq_rope, k_new, v_new,
                               positions, q, q_pos, kcodes, vcodes, seq_lens, batch: int, n_q_heads: int,
                               cache_len: int, max_seq_len: int, sm_scale: float, out, flags: int = 0,
                               stream=None) -> int:
    return _check(lib().commvq_decode_step_noalloc(
        ctypes.byref(kcb), ctypes.byref(vcb), ctypes.byref(rope), _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(q),
        _ptr(q_pos), _ptr(kcodes), _ptr(vcodes), _ptr(seq_lens), batch, n_q_heads, cache_len, max_seq_len,
        float(sm_scale), _ptr(out), int(flags), _stream(stream, q, out)))


def commvq_dequantize_kv(kcb: commvq_codebook, vcb: commvq_codebook, rope: commvq_rope, kcodes, vcodes, seq_lens,
                         batch: int, cache_len: int, max_seq_len: int, k_out, v_out, stream=None) -> int:
    return _check(lib().commvq_dequantize_kv(
        ctypes.byref(kcb), ctypes.byref(vcb), ctypes.byref(rope), _ptr(kcodes), _ptr(vcodes), _ptr(seq_lens), batch,
        cache_len, max_seq_len, _ptr(k_out), _ptr(v_out), _stream(stream, k_out, kcodes)))


def commvq_dense_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                                 max_seq_len: int) -> int:
    return lib().commvq_dense_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_seq_len)


def commvq_dense_decode_attention(rope: commvq_rope, q, q_pos, k, v, seq_lens, batch: int, n_q_heads: int,
                                  n_kv_heads: int, head_dim: int, cache_len: int, max_seq_len: int, sm_scale: float,
                                  out, workspace, workspace_bytes: int, stream=None) -> int:
    return _check(lib().commvq_dense_decode_attention(
        ctypes.byref(rope), _ptr(q), _ptr(q_pos), _ptr(k), _ptr(v), _ptr(seq_lens), batch, n_q_heads, n_kv_heads,
        head_dim, cache_len, max_seq_len, float(sm_scale), _ptr(out), _ptr(workspace), int(workspace_bytes),
        _stream(stream, q, out)))


def commvq_em_work_bytes(cb: commvq_codebook) -> int:
    return lib().commvq_em_work_bytes(ctypes.byref(cb))


def commvq_em_step(cb: commvq_codebook, x, n_tokens: int, x_token_stride: int, round_index: int, temperature: float,
                   min_mass: float, new_entries, mass_out, work, work_bytes: int, stream=None) -> int:
    return _check(lib().commvq_em_step(
        ctypes.byref(cb), _ptr(x), n_tokens, x_token_stride, round_index, float(temperature), float(min_mass),
        _ptr(new_entries), _ptr(mass_out), _ptr(work), int(work_bytes), _stream(stream, x, new_entries)))


def commvq_decode_bitv_workspace_bytes(batch: int, n_q_heads: int, max_seq_len: int, kcb: commvq_codebook,
                                      vcb: commvq_bit_codebook) -> int:
    return lib().commvq_decode_bitv_workspace_bytes(batch, n_q_heads, max_seq_len, ctypes.byref(kcb),
                                                    ctypes.byref(vcb))


def commvq_decode_attention_bitv(kcb: commvq_codebook, vcb: commvq_bit_codebook, rope: commvq_rope, q, q_pos, kcodes,
                                 vbits, seq_lens, batch: int, n_q_heads: int, cache_len: int, max_seq_len: int,
                                 sm_scale: float, out, workspace, workspace_bytes: int, flags: int = 0,
                                 stream=None) -> int:
    return _check(lib().commvq_decode_attention_bitv(
        ctypes.byref(kcb), ctypes.byref(vcb), ctypes.byref(rope), _ptr(q), _ptr(q_pos), _ptr(kcodes), _ptr(vbits),
        _ptr(seq_lens), batch, n_q_heads, cache_len, max_seq_len, float(sm_scale), _ptr(out), _ptr(workspace),
        int(workspace_bytes), int(flags), _stream(stream, q, out)))
