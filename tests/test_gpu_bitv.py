"""GPU parity of decode attention with the paper's binary value codes
(commvq_decode_attention_bitv, through the C ABI) against the oracle's
decode_attention_bit_values on the same seeded inputs: keys from the residual
commutative codebook, values as the sum of the rows whose bits are set, within
2e-3 of each row's max |ref|."""

import math

import numpy as np
import pytest
import torch

from long_context_attention_commvq_amd import api, synth, _lib
from oracle import commvq_oracle as O
from tests.parity import ATTN_TOL, row_errors

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _pack_cache(codes, n_entries):
    """codes [B, L, Hkv, R, G] -> packed [B, Hkv, L, bpt] via the oracle's packer."""
    return np.ascontiguousarray(np.stack([O.pack_codes(codes[b], n_entries) for b in range(codes.shape[0])])
                                .transpose(0, 2, 1, 3))


def bit_rows(seed, n_bits, dim):
    """Rows C [n_bits, dim] fp16, scaled so a sum of about n_bits / 2 rows is O(1)."""
    r = np.random.default_rng(seed).standard_normal((n_bits, dim)) / math.sqrt(n_bits / 2)
    return r.astype(np.float16)


@pytest.mark.parametrize("case", [
    dict(B=1, Hq=32, Hkv=8, D=128, g=8, Nc=256, R=1, nbits=1024, lens=[3000], Lmax=3000),   # 1 bit per scalar
    dict(B=1, Hq=32, Hkv=8, D=128, g=64, Nc=64, R=11, nbits=2048, lens=[1500], Lmax=1500),  # the paper's 2-bit pair
    dict(B=2, Hq=4, Hkv=2, D=64, g=4, Nc=16, R=2, nbits=256, lens=[700, 1], Lmax=800),
    dict(B=1, Hq=8, Hkv=1, D=128, g=8, Nc=256, R=2, nbits=512, lens=[2049], Lmax=2100),     # 8 query heads; chunk edge
    dict(B=3, Hq=8, Hkv=4, D=32, g=2, Nc=4, R=3, nbits=32, lens=[1024, 0, 5], Lmax=1100),   # a zero length
    dict(B=2, Hq=4, Hkv=1, D=64, g=8, Nc=16, R=1, nbits=64, lens=[300, 17], Lmax=320),      # one 8-byte range per token
])
def test_bit_value_decode_matches_oracle(case):
    B, Hq, Hkv, D, g, Nc, R, nb, Lmax = (case[k] for k in ("B", "Hq", "Hkv", "D", "g", "Nc", "R", "nbits", "Lmax"))
    lens = np.asarray(case["lens"], dtype=np.int32)
    seed = 9000 + D + g + Nc + R + nb
    rng = np.random.default_rng(seed)
    kcb = synth.codebook(seed + 1, Hkv, D, g, Nc, R)
    kp = _pack_cache(rng.integers(0, Nc, size=(B, Lmax, Hkv, R, D // g)), Nc)
    vbits = rng.integers(0, 256, size=(B, Lmax, nb // 8), dtype=np.uint8)
    rows = bit_rows(seed + 2, nb, Hkv * D)
    q = synth.queries(seed + 3, B, Hq, D)
    qpos = np.maximum(lens, 1) - 1
    ref = O.decode_attention_bit_values(q, qpos, kp, vbits, lens, kcb, rows, 500000.0)
    kq = api.Quantizer(dev(kcb), g)
    out = api.decode_attention_bitv(kq, dev(rows), dev(q), dev(qpos), dev(kp), dev(api.bitv_storage(vbits)), dev(lens), Lmax, 500000.0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = row_errors(got.reshape(-1, D), ref.reshape(-1, D))
    print(f"[bit values {case}] max row rel err {err.max():.3e}", flush=True)
    for b in range(B):
        if lens[b] == 0:
            assert np.all(got[b] == 0.0)
    assert err.max() <= ATTN_TOL


@pytest.mark.parametrize("case", [
    # the fast kernel's key shapes (g 8, Nc' 256, R 1 or 2, 4 query heads per KV head), >= 128-bit codes
    dict(B=2, Hq=4, Hkv=1, R=2, nbits=128, lens=[1500, 0], Lmax=2048),          # one range; 12 padded heads; a zero length
    dict(B=3, Hq=16, Hkv=4, R=1, nbits=256, lens=[1, 33, 1025], Lmax=1100),     # ragged tails inside a k-step
    dict(B=1, Hq=32, Hkv=8, R=2, nbits=2048, lens=[5000], Lmax=5000),           # 16 ranges (the paper's 2-bit width)
    dict(B=1, Hq=32, Hkv=8, R=1, nbits=1024, lens=[9000], Lmax=9000, qscale=8.0),  # peaked scores
    dict(B=2, Hq=8, Hkv=2, R=1, nbits=512, lens=[2047, 2049], Lmax=4100),       # chunk and range edges
])
def test_bit_value_fast_path_matches_oracle_and_generic(case):
    """On the fast kernel's shapes commvq_decode_attention_bitv takes the fast
    path (fp16 weights on the matrix cores); COMMVQ_DECODE_EXACT takes the
    generic kernel. Both meet the bar against the oracle, and they differ (two
    paths ran)."""
    B, Hq, Hkv, R, nb, Lmax = (case[k] for k in ("B", "Hq", "Hkv", "R", "nbits", "Lmax"))
    D, g, Nc = 128, 8, 256
    lens = np.asarray(case["lens"], dtype=np.int32)
    seed = 9300 + R + nb + Hq + int(lens.sum()) % 97
    rng = np.random.default_rng(seed)
    kcb = synth.codebook(seed + 1, Hkv, D, g, Nc, R)
    kp = rng.integers(0, 256, size=(B, Hkv, Lmax, 16 * R), dtype=np.uint8)  # every byte string is a valid record
    vbits = rng.integers(0, 256, size=(B, Lmax, nb // 8), dtype=np.uint8)
    rows = bit_rows(seed + 2, nb, Hkv * D)
    q = synth.queries(seed + 3, B, Hq, D) * np.float32(case.get("qscale", 1.0))
    qpos = np.maximum(lens, 1) - 1
    ref = O.decode_attention_bit_values(q, qpos, kp, vbits, lens, kcb, rows, 500000.0)
    kq = api.Quantizer(dev(kcb), g)
    args = (kq, dev(rows), dev(q), dev(qpos), dev(kp), dev(api.bitv_storage(vbits)), dev(lens), Lmax, 500000.0)
    fast = api.decode_attention_bitv(*args)
    exact = api.decode_attention_bitv(*args, flags=_lib.COMMVQ_DECODE_EXACT)
    torch.cuda.synchronize()
    fast, exact = fast.cpu().numpy(), exact.cpu().numpy()
    for name, got in (("fast", fast), ("generic", exact)):
        err = row_errors(got.reshape(-1, D), ref.reshape(-1, D))
        print(f"[bit values {name} {case}] max row rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL
        for b in range(B):
            if lens[b] == 0:
                assert np.all(got[b] == 0.0)
    assert not np.array_equal(fast, exact)


def test_bit_value_decode_rejects_bad_arguments():
    kcb = synth.codebook(9100, 2, 64, 8, 16, 1)
    kq = api.Quantizer(dev(kcb), 8)
    q = torch.zeros((1, 4, 64), dtype=torch.float32, device=DEV)
    pos = torch.zeros(1, dtype=torch.int32, device=DEV)
    codes = torch.zeros((1, 2, 16, kq.bytes_per_token), dtype=torch.uint8, device=DEV)
    def bits(nb):  # zero codes of nb bits for the 16 cached positions, in the library's storage
        return api.bitv_storage(torch.zeros((1, 16, nb // 8), dtype=torch.uint8, device=DEV))
    with pytest.raises(_lib.CommvqError) as e:
        api.decode_attention_bitv(kq, torch.zeros((256, 100), dtype=torch.float16, device=DEV), q, pos, codes,
                                  bits(256), pos + 1, 16, 500000.0)  # dim != Hkv * D
    assert e.value.status == _lib.COMMVQ_ERR_INVALID_ARG
    with pytest.raises(_lib.CommvqError) as e:
        api.decode_attention_bitv(kq, torch.zeros((96, 128), dtype=torch.float16, device=DEV), q, pos, codes,
                                  bits(96), pos + 1, 16, 500000.0)  # 96 bits: not a power of two
    assert e.value.status == _lib.COMMVQ_ERR_INVALID_ARG
    with pytest.raises(ValueError):  # token-major strings instead of the range-major storage
        api.decode_attention_bitv(kq, torch.zeros((256, 128), dtype=torch.float16, device=DEV), q, pos, codes,
                                  torch.zeros((1, 16, 32), dtype=torch.uint8, device=DEV), pos + 1, 16, 500000.0)


def test_bit_value_decode_full_size_128k_sampled():
    """128K positions, 32 query / 8 KV heads, 1024-bit value codes over the
    1024 value scalars of a token (1 bit per scalar) and the 1-bit key
    codebook, every head and chunk in one call; the oracle recomputes two KV
    heads over all positions."""
    B, Hq, Hkv, D, g, Nc, R, nb, L = 1, 32, 8, 128, 8, 256, 1, 1024, 131072
    rep = Hq // Hkv
    rng = np.random.default_rng(9200)
    kcb = synth.codebook(9201, Hkv, D, g, Nc, R)
    kp = rng.integers(0, 256, size=(B, Hkv, L, 16), dtype=np.uint8)  # every byte string is a valid 1-round record
    vbits = rng.integers(0, 256, size=(B, L, nb // 8), dtype=np.uint8)
    rows = bit_rows(9202, nb, Hkv * D)
    q = synth.queries(9203, B, Hq, D)
    lens = np.array([L], dtype=np.int32)
    kq = api.Quantizer(dev(kcb), g)
    print("[bit values full size] launching", flush=True)
    out = api.decode_attention_bitv(kq, dev(rows), dev(q), dev(lens - 1), dev(kp), dev(api.bitv_storage(vbits)), dev(lens), L, 500000.0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    for h in (int(rng.integers(0, Hkv)), Hkv - 1):
        ref = O.decode_attention_bit_values(q[:, h * rep:(h + 1) * rep], lens - 1, kp[:, h:h + 1], vbits, lens,
                                            kcb[h:h + 1], rows[:, h * D:(h + 1) * D], 500000.0)[0]
        err = row_errors(got[0, h * rep:(h + 1) * rep], ref)
        print(f"[bit values full size] head {h} max row rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL


def test_bit_value_fast_path_graph_replay():
    """Fast-path binary-value calls recorded into one HIP graph give the eager
    result bit for bit on every replay, with eager work between replays (its
    three kernels use no atomics, no memset, and no initialised workspace)."""
    B, Hq, Hkv, D, g, Nc, R, nb, L = 1, 32, 8, 128, 8, 256, 1, 1024, 5000
    rng = np.random.default_rng(9400)
    kcb = synth.codebook(9401, Hkv, D, g, Nc, R)
    kp = dev(rng.integers(0, 256, size=(B, Hkv, L, 16), dtype=np.uint8))
    vb = dev(api.bitv_storage(rng.integers(0, 256, size=(B, L, nb // 8), dtype=np.uint8)))
    rows = dev(bit_rows(9402, nb, Hkv * D))
    kq = api.Quantizer(dev(kcb), g)
    qs = [dev(synth.queries(9403 + i, B, Hq, D)) for i in range(2)]
    lens = dev(np.array([L - 3], dtype=np.int32))
    qpos = lens - 1
    ws = api.BitvWorkspace(kq, nb, Hkv * D, B, Hq, L, DEV)
    outs = [torch.empty((B, Hq, D), dtype=torch.float32, device=DEV) for _ in range(2)]
    for i in range(2):
        api.decode_attention_bitv(kq, rows, qs[i], qpos, kp, vb, lens, L, 500000.0, out=outs[i], workspace=ws)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(2):
            api.decode_attention_bitv(kq, rows, qs[i], qpos, kp, vb, lens, L, 500000.0, out=outs[i], workspace=ws)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        other = api.decode_attention_bitv(kq, rows, qs[rep % 2], qpos, kp, vb, lens, L, 500000.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], eager[i]), (rep, i)
        assert torch.equal(other, eager[rep % 2])


def test_bit_value_fast_path_batch_two_long():
    """Two sequences of 40,000 and 33,001 positions on the fast path (chunks of
    2048, a ragged last chunk each, 1024-bit codes): every query head of one
    KV head per sequence against the oracle."""
    B, Hq, Hkv, D, g, Nc, R, nb, Lmax = 2, 32, 8, 128, 8, 256, 1, 1024, 40000
    rep = Hq // Hkv
    rng = np.random.default_rng(9500)
    kcb = synth.codebook(9501, Hkv, D, g, Nc, R)
    kp = rng.integers(0, 256, size=(B, Hkv, Lmax, 16), dtype=np.uint8)
    vbits = rng.integers(0, 256, size=(B, Lmax, nb // 8), dtype=np.uint8)
    rows = bit_rows(9502, nb, Hkv * D)
    q = synth.queries(9503, B, Hq, D)
    lens = np.array([40000, 33001], dtype=np.int32)
    kq = api.Quantizer(dev(kcb), g)
    out = api.decode_attention_bitv(kq, dev(rows), dev(q), dev(lens - 1), dev(kp), dev(api.bitv_storage(vbits)), dev(lens), Lmax, 500000.0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b, h in ((0, 3), (1, 6)):
        ref = O.decode_attention_bit_values(q[b:b + 1, h * rep:(h + 1) * rep], lens[b:b + 1] - 1, kp[b:b + 1, h:h + 1],
                                            vbits[b:b + 1], lens[b:b + 1], kcb[h:h + 1], rows[:, h * D:(h + 1) * D],
                                            500000.0)[0]
        err = row_errors(got[b, h * rep:(h + 1) * rep], ref)
        print(f"[bit values B2] sequence {b} head {h} max row rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL
