"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, answers size queries, and rejects bad arguments with the
documented status before any GPU call."""

import ctypes
import os
import re

import pytest

from long_context_attention_commvq_amd import _lib
from oracle import commvq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "commvq.h")
FAKE = 0x10000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(commvq_\w+)\s*\(", text, flags=re.M)))


def cb(D=128, g=8, Nc=256, R=2, H=8, entries=FAKE):
    return _lib.make_codebook(entries, D, g, Nc, R, H)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n
    assert _lib.commvq_abi_version() == 2


def test_size_queries_match_the_oracle():
    for (D, g, Nc, R) in [(128, 8, 256, 2), (128, 8, 256, 1), (64, 16, 64, 2), (48, 6, 2, 3), (128, 4, 8, 3)]:
        c = cb(D, g, Nc, R)
        assert _lib.commvq_validate_codebook(c) == 0
        assert _lib.commvq_bits_per_scalar(c) == O.bits_per_scalar(g, Nc, R)
        assert _lib.commvq_code_bytes_per_token(c) == O.code_bytes_per_token(D, g, Nc, R)


def test_workspace_query():
    k = cb()
    n = _lib.commvq_decode_workspace_bytes(1, 32, 131072, k, k)
    assert n > 0 and n % 4 == 0
    assert _lib.commvq_decode_workspace_bytes(1, 32, 1, k, k) > 0
    assert _lib.commvq_decode_workspace_bytes(1, 30, 1000, k, k) == _lib.COMMVQ_ERR_INVALID_ARG
    assert _lib.commvq_decode_workspace_bytes(1, 24, 1000, k, k) == _lib.COMMVQ_ERR_UNSUPPORTED  # 3 q per kv
    assert _lib.commvq_decode_workspace_bytes(0, 32, 1000, k, k) == _lib.COMMVQ_ERR_INVALID_ARG
    assert _lib.commvq_decode_workspace_bytes(1, 32, 0, k, k) == _lib.COMMVQ_ERR_INVALID_ARG
    assert _lib.commvq_decode_workspace_bytes(1, 32, 1000, k, cb(D=64)) == _lib.COMMVQ_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [
    dict(D=127), dict(D=0), dict(D=512), dict(g=7), dict(g=0), dict(g=18), dict(D=128, g=12),
    dict(Nc=100), dict(Nc=1), dict(Nc=512), dict(R=0), dict(R=33), dict(H=0), dict(D=256, g=256), dict(D=130, g=130),
])
def test_invalid_descriptors(bad):
    c = cb(**bad)
    assert _lib.commvq_validate_codebook(c) == _lib.COMMVQ_ERR_INVALID_ARG
    assert _lib.commvq_last_error() != ""
    assert _lib.commvq_bits_per_scalar(c) < 0
    assert _lib.commvq_code_bytes_per_token(c) == _lib.COMMVQ_ERR_INVALID_ARG


def test_null_descriptor():
    L = _lib.lib()
    assert L.commvq_validate_codebook(None) == _lib.COMMVQ_ERR_INVALID_ARG
    assert "null" in _lib.commvq_last_error()


def _raw_encode(c, x, n, xs, codes, ts, hs, gap=None):
    return _lib.lib().commvq_encode(ctypes.byref(c), x, n, xs, codes, ts, hs, gap, None)


def test_encode_validation_without_launch():
    c = cb(H=2)
    bpt = 32
    assert _raw_encode(c, FAKE, 0, 256, FAKE, 64, 32) == 0          # nothing to do
    assert _raw_encode(c, None, 4, 256, FAKE, 64, 32) == _lib.COMMVQ_ERR_INVALID_ARG
    assert _raw_encode(c, FAKE, 4, 256, None, 64, 32) == _lib.COMMVQ_ERR_INVALID_ARG
    assert _raw_encode(c, FAKE, -1, 256, FAKE, 64, 32) == _lib.COMMVQ_ERR_INVALID_ARG
    assert _raw_encode(c, FAKE, 4, 255, FAKE, 64, 32) == _lib.COMMVQ_ERR_INVALID_ARG   # stride < H*D
    assert _raw_encode(c, FAKE + 2, 4, 256, FAKE, 64, 32) == _lib.COMMVQ_ERR_INVALID_ARG  # misaligned x
    assert _raw_encode(c, FAKE, 4, 256, FAKE, bpt, bpt) == _lib.COMMVQ_ERR_INVALID_ARG   # records overlap
    assert _raw_encode(c, FAKE, 4, 256, FAKE, -64, 32) == _lib.COMMVQ_ERR_INVALID_ARG
    assert _raw_encode(cb(H=2, entries=None), FAKE, 4, 256, FAKE, 64, 32) == _lib.COMMVQ_ERR_INVALID_ARG
    assert _raw_encode(cb(H=2, entries=FAKE + 8), FAKE, 4, 256, FAKE, 64, 32) == _lib.COMMVQ_ERR_INVALID_ARG
    assert _raw_encode(c, FAKE, 4, 256, FAKE, 64, 32, gap=FAKE + 2) == _lib.COMMVQ_ERR_INVALID_ARG  # misaligned gap_out
    assert "gap_out" in _lib.commvq_last_error()


def test_append_validation_without_launch():
    c = cb()
    L = _lib.lib()
    assert L.commvq_append(ctypes.byref(c), FAKE, 0, FAKE, FAKE, 16, None) == 0
    assert L.commvq_append(ctypes.byref(c), FAKE, -1, FAKE, FAKE, 16, None) == _lib.COMMVQ_ERR_INVALID_ARG
    assert L.commvq_append(ctypes.byref(c), FAKE, 2, None, FAKE, 16, None) == _lib.COMMVQ_ERR_INVALID_ARG
    assert L.commvq_append(ctypes.byref(c), FAKE, 2, FAKE, FAKE, 0, None) == _lib.COMMVQ_ERR_INVALID_ARG


def _raw_decode(k, v, rope, B=1, Hq=32, cache_len=1024, max_len=1024, scale=0.088, ws=FAKE, ws_bytes=1 << 30,
                q=FAKE, out=FAKE, codes=FAKE, flags=0):
    L = _lib.lib()
    return L.commvq_decode_attention(ctypes.byref(k), ctypes.byref(v), ctypes.byref(rope) if rope else None,
                                     q, FAKE, codes, codes, FAKE, B, Hq, cache_len, max_len, scale, out, ws,
                                     ws_bytes, flags, None)


def test_decode_validation_without_launch():
    k, rope = cb(), _lib.make_rope(500000.0)
    E = _lib
    assert _raw_decode(k, k, None) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(k, k, _lib.make_rope(1.0)) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(k, k, _lib.make_rope(float("nan"))) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(k, k, _lib.make_rope(500000.0, pairing=1)) == E.COMMVQ_ERR_UNSUPPORTED
    assert _raw_decode(k, k, rope, Hq=31) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(k, k, rope, Hq=24) == E.COMMVQ_ERR_UNSUPPORTED
    assert _raw_decode(k, k, rope, max_len=2048) == E.COMMVQ_ERR_INVALID_ARG  # beyond the cache
    assert _raw_decode(k, k, rope, B=0) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(k, k, rope, scale=float("inf")) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(k, k, rope, flags=2) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(k, k, rope, ws_bytes=16) == E.COMMVQ_ERR_WORKSPACE
    assert _raw_decode(k, k, rope, ws=None) == E.COMMVQ_ERR_WORKSPACE
    assert _raw_decode(k, k, rope, ws=FAKE + 64) == E.COMMVQ_ERR_WORKSPACE  # 256-byte alignment
    assert _raw_decode(k, k, rope, q=FAKE + 4) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(k, k, rope, codes=FAKE + 1) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(k, k, rope, out=None) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(k, cb(D=64), rope) == E.COMMVQ_ERR_INVALID_ARG
    assert _raw_decode(cb(g=6, D=96), cb(g=6, D=96), rope) == E.COMMVQ_ERR_UNSUPPORTED
    # launch-grid limits: batch on the grid's y axis, chunks x KV heads on x
    assert _raw_decode(k, k, rope, B=65536) == E.COMMVQ_ERR_UNSUPPORTED
    assert "batch" in _lib.commvq_last_error()
    assert _raw_decode(cb(H=65536), cb(H=65536), rope, Hq=65536) == E.COMMVQ_ERR_UNSUPPORTED
    big = 2**31 - 1
    assert _raw_decode(cb(H=2048), cb(H=2048), rope, Hq=8192, cache_len=big, max_len=big) == E.COMMVQ_ERR_UNSUPPORTED
    assert "launch grid" in _lib.commvq_last_error()
    assert "workspace" in (_raw_decode(k, k, rope, ws_bytes=16) and _lib.commvq_last_error())


def test_decode_step_validation_without_launch():
    k, rope = cb(), _lib.make_rope(500000.0)
    L = _lib.lib()

    def step(k_new=FAKE, v_new=FAKE, positions=FAKE, ws_bytes=1 << 30):
        return L.commvq_decode_step(ctypes.byref(k), ctypes.byref(k), ctypes.byref(rope), k_new, v_new, positions,
                                    FAKE, FAKE, FAKE, FAKE, FAKE, 1, 32, 1024, 1024, 0.088, FAKE, FAKE, ws_bytes, 0,
                                    None)
    assert step(k_new=None) == _lib.COMMVQ_ERR_INVALID_ARG
    assert step(v_new=None) == _lib.COMMVQ_ERR_INVALID_ARG
    assert step(positions=None) == _lib.COMMVQ_ERR_INVALID_ARG
    assert step(k_new=FAKE + 8) == _lib.COMMVQ_ERR_INVALID_ARG
    assert step(ws_bytes=16) == _lib.COMMVQ_ERR_WORKSPACE


def test_decode_step_noalloc_validation_without_launch():
    """The allocation-free step checks every argument, and its static scratch's
    size against the shape's need, before any GPU call."""
    k, rope = cb(R=1), _lib.make_rope(500000.0)
    L = _lib.lib()

    def step(k_new=FAKE, batch=1, lmax=1024, flags=0):
        return L.commvq_decode_step_noalloc(ctypes.byref(k), ctypes.byref(k), ctypes.byref(rope), k_new, FAKE, FAKE,
                                            FAKE, FAKE, FAKE, FAKE, FAKE, batch, 32, lmax, lmax, 0.088, FAKE, flags,
                                            None)
    assert step(k_new=None) == _lib.COMMVQ_ERR_INVALID_ARG
    assert step(flags=2) == _lib.COMMVQ_ERR_INVALID_ARG
    assert step(batch=0) == _lib.COMMVQ_ERR_INVALID_ARG
    big = (64, 131072)
    assert _lib.commvq_decode_workspace_bytes(big[0], 32, big[1], k, k) > _lib.COMMVQ_NOALLOC_SCRATCH_BYTES
    assert step(batch=big[0], lmax=big[1]) == _lib.COMMVQ_ERR_WORKSPACE
    assert "scratch" in _lib.commvq_last_error()


def test_dense_workspace_query():
    E = _lib
    assert E.commvq_dense_workspace_bytes(1, 32, 8, 128, 131072) == 32 * 128 * 130 * 4  # chunks of 1024 positions
    assert E.commvq_dense_workspace_bytes(2, 4, 1, 128, 1025) == 2 * 4 * 2 * 130 * 4
    assert E.commvq_dense_workspace_bytes(1, 32, 8, 64, 1000) == E.COMMVQ_ERR_UNSUPPORTED
    assert E.commvq_dense_workspace_bytes(1, 32, 8, 127, 1000) == E.COMMVQ_ERR_INVALID_ARG
    assert E.commvq_dense_workspace_bytes(1, 30, 8, 128, 1000) == E.COMMVQ_ERR_INVALID_ARG
    assert E.commvq_dense_workspace_bytes(1, 24, 8, 128, 1000) == E.COMMVQ_ERR_UNSUPPORTED  # 3 q per kv
    assert E.commvq_dense_workspace_bytes(0, 32, 8, 128, 1000) == E.COMMVQ_ERR_INVALID_ARG
    assert E.commvq_dense_workspace_bytes(1, 32, 8, 128, 0) == E.COMMVQ_ERR_INVALID_ARG
    assert E.commvq_dense_workspace_bytes(1, 32, 0, 128, 10) == E.COMMVQ_ERR_INVALID_ARG
    assert E.commvq_dense_workspace_bytes(65536, 32, 8, 128, 10) == E.COMMVQ_ERR_UNSUPPORTED


def test_dequantize_validation_without_launch():
    k, rope = cb(R=1), _lib.make_rope(500000.0)
    L = _lib.lib()

    def deq(kc=k, vc=k, rp=rope, codes=FAKE, lens=FAKE, B=1, cache_len=1024, max_len=1024, ko=FAKE, vo=FAKE):
        return L.commvq_dequantize_kv(ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(rp) if rp else None, codes,
                                      codes, lens, B, cache_len, max_len, ko, vo, None)
    E = _lib
    assert deq(rp=None) == E.COMMVQ_ERR_INVALID_ARG
    assert deq(rp=_lib.make_rope(500000.0, pairing=1)) == E.COMMVQ_ERR_UNSUPPORTED
    assert deq(vc=cb(D=64)) == E.COMMVQ_ERR_INVALID_ARG
    assert deq(vc=cb(g=4)) == E.COMMVQ_ERR_INVALID_ARG
    assert deq(B=0) == E.COMMVQ_ERR_INVALID_ARG
    assert deq(max_len=0) == E.COMMVQ_ERR_INVALID_ARG
    assert deq(max_len=1025) == E.COMMVQ_ERR_INVALID_ARG  # beyond the cache
    assert deq(B=65536) == E.COMMVQ_ERR_UNSUPPORTED
    assert deq(codes=None) == E.COMMVQ_ERR_INVALID_ARG
    assert deq(lens=None) == E.COMMVQ_ERR_INVALID_ARG
    assert deq(ko=None) == E.COMMVQ_ERR_INVALID_ARG
    assert deq(vo=FAKE + 8) == E.COMMVQ_ERR_INVALID_ARG  # 16-byte alignment
    assert deq(kc=cb(R=1, entries=None)) == E.COMMVQ_ERR_INVALID_ARG
    assert deq(kc=cb(D=0)) == E.COMMVQ_ERR_INVALID_ARG


def test_dense_attention_validation_without_launch():
    rope = _lib.make_rope(500000.0)
    L = _lib.lib()

    def dense(rp=rope, q=FAKE, k=FAKE, out=FAKE, B=1, Hq=32, Hkv=8, D=128, cache_len=1024, max_len=1024,
              scale=0.088, ws=FAKE, ws_bytes=1 << 30):
        return L.commvq_dense_decode_attention(ctypes.byref(rp) if rp else None, q, FAKE, k, k, FAKE, B, Hq, Hkv, D,
                                               cache_len, max_len, scale, out, ws, ws_bytes, None)
    E = _lib
    assert dense(rp=None) == E.COMMVQ_ERR_INVALID_ARG
    assert dense(rp=_lib.make_rope(0.5)) == E.COMMVQ_ERR_INVALID_ARG
    assert dense(D=64) == E.COMMVQ_ERR_UNSUPPORTED
    assert dense(Hq=12) == E.COMMVQ_ERR_INVALID_ARG
    assert dense(Hq=24) == E.COMMVQ_ERR_UNSUPPORTED
    assert dense(max_len=1025) == E.COMMVQ_ERR_INVALID_ARG
    assert dense(scale=float("nan")) == E.COMMVQ_ERR_INVALID_ARG
    assert dense(q=None) == E.COMMVQ_ERR_INVALID_ARG
    assert dense(k=FAKE + 2) == E.COMMVQ_ERR_INVALID_ARG
    assert dense(out=FAKE + 4) == E.COMMVQ_ERR_INVALID_ARG
    assert dense(ws_bytes=16) == E.COMMVQ_ERR_WORKSPACE
    assert dense(ws=None) == E.COMMVQ_ERR_WORKSPACE
    assert dense(ws=FAKE + 64) == E.COMMVQ_ERR_WORKSPACE
    assert dense(B=0) == E.COMMVQ_ERR_INVALID_ARG


def test_em_validation_without_launch():
    c = cb(D=128, g=8, Nc=256, R=2, H=8)
    E = _lib
    assert E.commvq_em_work_bytes(c) == 8 * 16 * 256 * 9 * 4 + (4 << 20)  # accumulators + a batch of codes
    assert E.commvq_em_work_bytes(cb(D=64, g=4, Nc=16, R=3, H=2)) == (2 * 16 * 16 * 5 * 4 + 255) // 256 * 256
    assert E.commvq_em_work_bytes(cb(D=127)) == E.COMMVQ_ERR_INVALID_ARG
    L = _lib.lib()

    def em(cc=c, x=FAKE, n=100, stride=1024, r=0, T=0.0, mm=0.0, new=FAKE, mass=None, work=FAKE, wb=1 << 30):
        return L.commvq_em_step(ctypes.byref(cc), x, n, stride, r, T, mm, new, mass, work, wb, None)
    assert em(n=0) == E.COMMVQ_ERR_INVALID_ARG
    assert em(r=2) == E.COMMVQ_ERR_INVALID_ARG
    assert em(r=-1) == E.COMMVQ_ERR_INVALID_ARG
    assert em(T=-1.0) == E.COMMVQ_ERR_INVALID_ARG
    assert em(T=float("inf")) == E.COMMVQ_ERR_INVALID_ARG
    assert em(mm=float("nan")) == E.COMMVQ_ERR_INVALID_ARG
    assert em(stride=1023) == E.COMMVQ_ERR_INVALID_ARG
    assert em(x=None) == E.COMMVQ_ERR_INVALID_ARG
    assert em(x=FAKE + 2) == E.COMMVQ_ERR_INVALID_ARG
    assert em(stride=1025) == E.COMMVQ_ERR_INVALID_ARG
    assert em(new=FAKE + 8) == E.COMMVQ_ERR_INVALID_ARG
    assert em(mass=FAKE + 2) == E.COMMVQ_ERR_INVALID_ARG
    assert em(wb=16) == E.COMMVQ_ERR_WORKSPACE
    assert em(work=None) == E.COMMVQ_ERR_WORKSPACE
    assert em(work=FAKE + 64) == E.COMMVQ_ERR_WORKSPACE
    assert em(cc=cb(entries=None)) == E.COMMVQ_ERR_INVALID_ARG


def test_wide_groups_and_many_rounds():
    """The paper's own hyperparameters (g = 64 scalars, Nc' = 64, R = 11 or 21)
    and g = 128 are valid descriptors; the entry points that have no kernel for
    a shape say so with COMMVQ_ERR_UNSUPPORTED before any GPU call."""
    E = _lib
    L = _lib.lib()
    for R, bits in [(11, 11 * 6 / 64), (21, 21 * 6 / 64)]:
        c = cb(D=128, g=64, Nc=64, R=R)
        assert E.commvq_validate_codebook(c) == 0
        assert E.commvq_bits_per_scalar(c) == bits
        assert E.commvq_code_bytes_per_token(c) == -(-R * 2 * 6 // 8)
    assert E.commvq_validate_codebook(cb(D=128, g=128, Nc=64, R=32)) == 0
    rope = _lib.make_rope(500000.0)

    def enc(c):
        return L.commvq_encode(ctypes.byref(c), FAKE, 4, c.n_kv_heads * c.head_dim, FAKE, 4096, 512, None, None)
    assert enc(cb(D=96, g=24, Nc=16, R=1)) == E.COMMVQ_ERR_UNSUPPORTED          # no kernel for g = 24
    assert enc(cb(D=256, g=2, Nc=256, R=32)) == E.COMMVQ_ERR_UNSUPPORTED        # 4096 fields per record
    k = cb(D=128, g=64, Nc=256, R=16)
    assert _raw_decode(k, k, rope) == E.COMMVQ_ERR_UNSUPPORTED                  # 16 rounds x 256 entries of a slice
    assert "LDS" in _lib.commvq_last_error()
    assert _raw_decode(cb(D=96, g=24), cb(D=96, g=24), rope) == E.COMMVQ_ERR_UNSUPPORTED
    w = cb(D=128, g=32, Nc=64, R=2)
    assert L.commvq_dequantize_kv(ctypes.byref(w), ctypes.byref(w), ctypes.byref(rope), FAKE, FAKE, FAKE, 1, 64, 64,
                                  FAKE, FAKE, None) == E.COMMVQ_ERR_UNSUPPORTED
    assert L.commvq_em_step(ctypes.byref(w), FAKE, 10, 1024, 0, 0.0, 0.0, FAKE, None, FAKE, 1 << 30,
                            None) == E.COMMVQ_ERR_UNSUPPORTED
    big = cb(D=128, g=16, Nc=256, R=32)
    assert L.commvq_em_step(ctypes.byref(big), FAKE, 10, 1024, 31, 0.0, 0.0, FAKE, None, FAKE, 1 << 30,
                            None) == E.COMMVQ_ERR_UNSUPPORTED  # 32 rounds of fp32 codebook in LDS


def test_bit_value_decode_validation_without_launch():
    k, rope = cb(D=128, g=8, Nc=256, R=1, H=8), _lib.make_rope(500000.0)
    L = _lib.lib()
    E = _lib

    def bitv(nb=1024, dim=1024, rows=FAKE, Hq=32, bits=FAKE, ws_bytes=1 << 30, flags=0):
        v = _lib.make_bit_codebook(rows, nb, dim)
        return L.commvq_decode_attention_bitv(ctypes.byref(k), ctypes.byref(v), ctypes.byref(rope), FAKE, FAKE, FAKE,
                                              bits, FAKE, 1, Hq, 1024, 1024, 0.088, FAKE, FAKE, ws_bytes, flags, None)
    assert bitv(flags=2) == E.COMMVQ_ERR_INVALID_ARG
    assert bitv(nb=1000) == E.COMMVQ_ERR_INVALID_ARG
    assert bitv(nb=4096) == E.COMMVQ_ERR_INVALID_ARG
    assert bitv(dim=512) == E.COMMVQ_ERR_INVALID_ARG
    assert bitv(rows=None) == E.COMMVQ_ERR_INVALID_ARG
    assert bitv(rows=FAKE + 8) == E.COMMVQ_ERR_INVALID_ARG
    assert bitv(bits=None) == E.COMMVQ_ERR_INVALID_ARG
    assert bitv(bits=FAKE + 4) == E.COMMVQ_ERR_INVALID_ARG
    assert bitv(Hq=24) == E.COMMVQ_ERR_UNSUPPORTED
    assert bitv(ws_bytes=16) == E.COMMVQ_ERR_WORKSPACE


def test_bit_value_workspace_sizes():
    """Workspace of the binary-value decode, in closed form. 128K positions, 32
    query / 8 KV heads, 1-bit keys, 1024-bit codes (fast path, chunks of 4096):
    partial slots [1][32][32 chunks x 8 ranges][130] fp32 plus fp16 weights
    [1][32][131072]; the generic kernel's need (chunks of 1024, and the
    new-token area) is smaller. 64-bit codes: the generic path only."""
    k = cb(D=128, g=8, Nc=256, R=1, H=8)
    v = _lib.make_bit_codebook(None, 1024, 1024)
    fast = 32 * 32 * 8 * 130 * 4 + 32 * 131072 * 2
    assert _lib.commvq_decode_bitv_workspace_bytes(1, 32, 131072, k, v) == fast
    generic = 32 * 128 * 130 * 4 + 8 * 192 * 4
    v64 = _lib.make_bit_codebook(None, 64, 1024)
    assert _lib.commvq_decode_bitv_workspace_bytes(1, 32, 131072, k, v64) == generic
    assert _lib.commvq_decode_bitv_workspace_bytes(1, 32, 131072, k, _lib.make_bit_codebook(None, 1000, 1024)) == \
        _lib.COMMVQ_ERR_INVALID_ARG


def test_bitv_storage_layout():
    """bitv_storage puts bits 128 r .. 128 r + 127 of token t at [b, r, t, :]
    (the layout commvq.h documents for vbits); strings under 128 bits stay one
    range per token."""
    import numpy as np
    from long_context_attention_commvq_amd import api
    rng = np.random.default_rng(5)
    tm = rng.integers(0, 256, size=(2, 7, 128), dtype=np.uint8)  # 1024 bits per token
    st = api.bitv_storage(tm)
    assert st.shape == (2, 8, 7, 16) and st.flags["C_CONTIGUOUS"]
    flat = st.reshape(-1)
    for b, t, byte in [(0, 0, 0), (1, 6, 127), (0, 3, 17), (1, 2, 64)]:
        r, k = divmod(byte, 16)
        assert flat[((b * 8 + r) * 7 + t) * 16 + k] == tm[b, t, byte]
    small = rng.integers(0, 256, size=(1, 5, 8), dtype=np.uint8)  # 64 bits per token
    assert np.array_equal(api.bitv_storage(small).reshape(1, 5, 8), small)
    import torch  # the same on torch tensors
    tt = api.bitv_storage(torch.from_numpy(tm))
    assert tt.is_contiguous() and np.array_equal(tt.numpy(), st)
