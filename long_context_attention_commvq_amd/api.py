"""Tensor-level conveniences over the C ABI: allocate outputs and workspace with
torch (device memory and streams only) and call the HIP library."""

from __future__ import annotations

import math

import torch

from . import _lib


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, device, shape: tuple | None = None) -> torch.Tensor:
    """The C ABI reads raw pointers: check what it cannot (dtype, device, shape)
    and hand it a contiguous tensor."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.contiguous()


def _need_cache(t: torch.Tensor, name: str, quant: "Quantizer", batch: int, device) -> torch.Tensor:
    """A packed cache: uint8 [B, Hkv, Lmax, bytes_per_token], contiguous (written in place, so never copied)."""
    if t.dtype != torch.uint8 or t.dim() != 4:
        raise TypeError(f"{name} must be uint8 [B, Hkv, Lmax, bytes_per_token]")
    if t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.shape[0] != batch or t.shape[1] != quant.n_kv_heads or t.shape[3] != quant.bytes_per_token:
        raise ValueError(f"{name} has shape {tuple(t.shape)}; expected [{batch}, {quant.n_kv_heads}, Lmax, "
                         f"{quant.bytes_per_token}]")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (it is read and written in place)")
    return t


class Quantizer:
    """One residual codebook (keys or values) living on the GPU.

    entries: fp16 tensor [Hkv, D/g, R, Nc', g] on a CUDA/HIP device."""

    def __init__(self, entries: torch.Tensor, group_size: int):
        if entries.dtype != torch.float16 or entries.dim() != 5:
            raise ValueError("entries must be fp16 [Hkv, D/g, R, Nc', g]")
        self.entries = entries.contiguous()
        Hkv, G, R, Nc, g = self.entries.shape
        if g != group_size:
            raise ValueError("group_size does not match the entries' last axis")
        self.head_dim, self.group_size, self.n_entries, self.n_rounds, self.n_kv_heads = G * g, g, Nc, R, Hkv
        self.desc = _lib.make_codebook(self.entries, self.head_dim, g, Nc, R, Hkv)

    @property
    def bytes_per_token(self) -> int:
        n = _lib.commvq_code_bytes_per_token(self.desc)
        if n < 0:
            raise _lib.CommvqError(int(n), _lib.commvq_last_error())
        return int(n)

    @property
    def bits_per_scalar(self) -> float:
        return _lib.commvq_bits_per_scalar(self.desc)


def encode(quant: Quantizer, x: torch.Tensor, out: torch.Tensor | None = None,
           gaps: torch.Tensor | None = None) -> torch.Tensor:
    """x fp16 [N, Hkv, D] -> packed codes uint8 [N, Hkv, bytes_per_token]; with
    gaps (fp32 [N, Hkv, R, G], contiguous) also each field's near-tie margin."""
    N, H, D = x.shape
    x = x.contiguous()
    bpt = quant.bytes_per_token
    if out is None:
        out = torch.empty((N, H, bpt), dtype=torch.uint8, device=x.device)
    if gaps is not None:
        _need(gaps, "gaps", torch.float32, x.device, (N, H, quant.n_rounds, quant.head_dim // quant.group_size))
        if not gaps.is_contiguous():
            raise ValueError("gaps must be contiguous")
    _lib.commvq_encode(quant.desc, x, N, H * D, out, out.stride(0), out.stride(1), gaps)
    return out


def encode_into_cache(quant: Quantizer, x: torch.Tensor, cache: torch.Tensor, b: int, pos0: int) -> None:
    """Prefill: x fp16 [N, Hkv, D] -> cache[b, :, pos0:pos0+N] (cache uint8 [B, Hkv, Lmax, bpt])."""
    N, H, D = x.shape
    x = x.contiguous()
    view = cache[b, :, pos0:pos0 + N]
    _lib.commvq_encode(quant.desc, x, N, H * D, view, cache.stride(2), cache.stride(1))


def append(quant: Quantizer, x: torch.Tensor, positions: torch.Tensor, cache: torch.Tensor) -> None:
    """x fp16 [B, Hkv, D], positions int32 [B] (device) -> cache[b, :, positions[b]]."""
    B = x.shape[0]
    dev = x.device
    x = _need(x, "x", torch.float16, dev, (B, quant.n_kv_heads, quant.head_dim))
    positions = _need(positions, "positions", torch.int32, dev, (B,))
    cache = _need_cache(cache, "cache", quant, B, dev)
    _lib.commvq_append(quant.desc, x, B, positions, cache, cache.shape[2])


class DecodeWorkspace:
    """Workspace sized for (batch, n_q_heads, max_seq_len) and reused across calls."""

    def __init__(self, kq: Quantizer, vq: Quantizer, batch: int, n_q_heads: int, max_seq_len: int, device):
        n = _lib.commvq_decode_workspace_bytes(batch, n_q_heads, max_seq_len, kq.desc, vq.desc)
        if n < 0:
            raise _lib.CommvqError(int(n), _lib.commvq_last_error())
        self.nbytes = int(n)
        # chunk partials and new-token terms: no initialisation needed
        self.buf = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=device)


def decode_attention(kq: Quantizer, vq: Quantizer, q: torch.Tensor, q_pos: torch.Tensor, kcache: torch.Tensor,
                     vcache: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, theta_base: float,
                     sm_scale: float | None = None, out: torch.Tensor | None = None,
                     workspace: DecodeWorkspace | None = None, exact: bool = False) -> torch.Tensor:
    """q fp32 [B, Hq, D] -> out fp32 [B, Hq, D] over packed caches [B, Hkv, Lmax, bpt]."""
    B, Hq, D = q.shape
    dev = q.device
    q = _need(q, "q", torch.float32, dev, (B, Hq, kq.head_dim))
    q_pos = _need(q_pos, "q_pos", torch.int32, dev, (B,))
    seq_lens = _need(seq_lens, "seq_lens", torch.int32, dev, (B,))
    kcache = _need_cache(kcache, "kcache", kq, B, dev)
    vcache = _need_cache(vcache, "vcache", vq, B, dev)
    if out is not None:
        _need(out, "out", torch.float32, dev, (B, Hq, D))
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = DecodeWorkspace(kq, vq, B, Hq, max_seq_len, q.device)
    rope = _lib.make_rope(theta_base)
    _lib.commvq_decode_attention(kq.desc, vq.desc, rope, q, q_pos, kcache, vcache, seq_lens, B, Hq,
                                 kcache.shape[2], max_seq_len, sm_scale, out, workspace.buf, workspace.nbytes,
                                 _lib.COMMVQ_DECODE_EXACT if exact else 0)
    return out


def decode_step(kq: Quantizer, vq: Quantizer, k_new: torch.Tensor, v_new: torch.Tensor, positions: torch.Tensor,
                q: torch.Tensor, q_pos: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                seq_lens: torch.Tensor, max_seq_len: int, theta_base: float, sm_scale: float | None = None,
                out: torch.Tensor | None = None, workspace: DecodeWorkspace | None = None,
                exact: bool = False) -> torch.Tensor:
    """Append k_new/v_new fp16 [B, Hkv, D] at positions[b], then attend (one call)."""
    B, Hq, D = q.shape
    dev = q.device
    q = _need(q, "q", torch.float32, dev, (B, Hq, kq.head_dim))
    k_new = _need(k_new, "k_new", torch.float16, dev, (B, kq.n_kv_heads, kq.head_dim))
    v_new = _need(v_new, "v_new", torch.float16, dev, (B, vq.n_kv_heads, vq.head_dim))
    positions = _need(positions, "positions", torch.int32, dev, (B,))
    q_pos = _need(q_pos, "q_pos", torch.int32, dev, (B,))
    seq_lens = _need(seq_lens, "seq_lens", torch.int32, dev, (B,))
    kcache = _need_cache(kcache, "kcache", kq, B, dev)
    vcache = _need_cache(vcache, "vcache", vq, B, dev)
    if out is not None:
        _need(out, "out", torch.float32, dev, (B, Hq, D))
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = DecodeWorkspace(kq, vq, B, Hq, max_seq_len, q.device)
    rope = _lib.make_rope(theta_base)
    _lib.commvq_decode_step(kq.desc, vq.desc, rope, k_new, v_new, positions, q, q_pos,
                            kcache, vcache, seq_lens, B, Hq, kcache.shape[2], max_seq_len, sm_scale, out,
                            workspace.buf, workspace.nbytes, _lib.COMMVQ_DECODE_EXACT if exact else 0)
    return out


# ---- comparison path: dequantise to fp16, then dense attention ---------------

def dequantize_kv(kq: Quantizer, vq: Quantizer, kcache: torch.Tensor, vcache: torch.Tensor, seq_lens: torch.Tensor,
                  max_seq_len: int, theta_base: float, k_out: torch.Tensor | None = None,
                  v_out: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Packed caches [B, Hkv, Lmax, bpt] -> fp16 keys (rotated to their positions)
    and values [B, Hkv, Lmax, D]; positions at or past seq_lens[b] are left as
    they were in k_out / v_out."""
    B, H, Lmax, _ = kcache.shape
    D = kq.head_dim
    if k_out is None:
        k_out = torch.zeros((B, H, Lmax, D), dtype=torch.float16, device=kcache.device)
    if v_out is None:
        v_out = torch.zeros((B, H, Lmax, D), dtype=torch.float16, device=kcache.device)
    rope = _lib.make_rope(theta_base)
    _lib.commvq_dequantize_kv(kq.desc, vq.desc, rope, kcache, vcache, seq_lens, B, Lmax, max_seq_len, k_out, v_out)
    return k_out, v_out


class DenseWorkspace:
    """Workspace of commvq_dense_decode_attention for one shape."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, max_seq_len: int, device):
        n = _lib.commvq_dense_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_seq_len)
        if n < 0:
            raise _lib.CommvqError(int(n), _lib.commvq_last_error())
        self.nbytes = int(n)
        self.buf = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=device)


def dense_decode_attention(q: torch.Tensor, q_pos: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           seq_lens: torch.Tensor, max_seq_len: int, theta_base: float,
                           sm_scale: float | None = None, out: torch.Tensor | None = None,
                           workspace: DenseWorkspace | None = None) -> torch.Tensor:
    """q fp32 [B, Hq, D] (not rotated) over fp16 k (rotated), v [B, Hkv, Lmax, D]."""
    B, Hq, D = q.shape
    Hkv, Lmax = k.shape[1], k.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = DenseWorkspace(B, Hq, Hkv, D, max_seq_len, q.device)
    rope = _lib.make_rope(theta_base)
    _lib.commvq_dense_decode_attention(rope, q, q_pos, k, v, seq_lens, B, Hq, Hkv, D, Lmax, max_seq_len, sm_scale,
                                       out, workspace.buf, workspace.nbytes)
    return out


# ---- codebook fitting -----------------------------------------------------------

def em_step(quant: Quantizer, x: torch.Tensor, round_index: int, temperature: float = 0.0, min_mass: float = 0.0,
            new_entries: torch.Tensor | None = None, work: torch.Tensor | None = None,
            with_mass: bool = False):
    """One EM iteration for round `round_index` of `quant`'s codebook on x fp16
    [N, Hkv, D]. Returns the entries tensor holding the update (in place in
    quant.entries unless new_entries is given) and, with with_mass, the mass
    fp32 [Hkv, D/g, Nc']."""
    N, H, D = x.shape
    x = x.contiguous()
    if new_entries is None:
        new_entries = quant.entries
    if work is None:
        n = _lib.commvq_em_work_bytes(quant.desc)
        if n < 0:
            raise _lib.CommvqError(int(n), _lib.commvq_last_error())
        work = torch.empty(int(n), dtype=torch.uint8, device=x.device)
    mass = None
    if with_mass:
        mass = torch.empty((quant.n_kv_heads, quant.head_dim // quant.group_size, quant.n_entries),
                           dtype=torch.float32, device=x.device)
    _lib.commvq_em_step(quant.desc, x, N, H * D, round_index, temperature, min_mass, new_entries, mass, work,
                        work.numel())
    return (new_entries, mass) if with_mass else new_entries


# ---- binary value codes ---------------------------------------------------------

class BitvWorkspace:
    """Workspace of commvq_decode_attention_bitv for one shape (either path)."""

    def __init__(self, kq: Quantizer, n_bits: int, dim: int, batch: int, n_q_heads: int, max_seq_len: int,
                 device):
        vcb = _lib.make_bit_codebook(None, n_bits, dim)
        n = _lib.commvq_decode_bitv_workspace_bytes(batch, n_q_heads, max_seq_len, kq.desc, vcb)
        if n < 0:
            raise _lib.CommvqError(int(n), _lib.commvq_last_error())
        self.nbytes = int(n)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)


def bitv_storage(bits):
    """Token-major bit strings [B, L, Nc/8] (bit i of a token = bit i % 8 of byte
    i / 8) -> the library's range-major storage [B, Nc/128, L, 16] (one range of
    Nc/8 bytes when Nc < 128). A copy; works on torch tensors and numpy arrays."""
    B, L, nby = bits.shape
    rb = min(16, nby)
    v = bits.reshape(B, L, nby // rb, rb)
    if isinstance(v, torch.Tensor):
        return v.permute(0, 2, 1, 3).contiguous()
    import numpy as np
    return np.ascontiguousarray(v.transpose(0, 2, 1, 3))


def decode_attention_bitv(kq: Quantizer, rows: torch.Tensor, q: torch.Tensor, q_pos: torch.Tensor,
                          kcache: torch.Tensor, vbits: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                          theta_base: float, sm_scale: float | None = None, out: torch.Tensor | None = None,
                          workspace: BitvWorkspace | None = None, flags: int = 0) -> torch.Tensor:
    """Keys from packed caches [B, Hkv, Lmax, bpt]; values from binary codes in
    the range-major storage vbits uint8 [B, Nc/128, Lmax, 16] (bitv_storage of
    the token-major strings) and rows fp16 [Nc, Hkv * D]."""
    B, Hq, D = q.shape
    nby = rows.shape[0] // 8
    rb = min(16, nby)
    want = (B, nby // rb, kcache.shape[2], rb)
    if vbits.dtype != torch.uint8 or tuple(vbits.shape) != want or not vbits.is_contiguous():
        raise ValueError(f"vbits must be contiguous uint8 {want} (range-major storage), got {vbits.dtype} "
                         f"{tuple(vbits.shape)}")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = BitvWorkspace(kq, rows.shape[0], rows.shape[1], B, Hq, max_seq_len, q.device)
    rows = rows.contiguous()
    vcb = _lib.make_bit_codebook(rows, rows.shape[0], rows.shape[1])
    rope = _lib.make_rope(theta_base)
    _lib.commvq_decode_attention_bitv(kq.desc, vcb, rope, q, q_pos, kcache, vbits, seq_lens, B, Hq, kcache.shape[2],
                                      max_seq_len, sm_scale, out, workspace.buf, workspace.nbytes, flags)
    return out
