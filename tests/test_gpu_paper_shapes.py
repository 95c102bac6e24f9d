"""GPU parity at the paper's own quantizer hyperparameters ("Pith review of
CommVQ", "Assumptions & free parameters": Nc' = 64 entries, g = 64, R = 11
rounds for 1 bit and 21 for 2 bits), with g counted in scalars as everywhere in
this library (11 x 6 / 64 = 1.03 and 21 x 6 / 64 = 1.97 bits per scalar, the
review's Table 8 labels), and at g = 128 (one index per head and round): 6-bit
fields that straddle bytes, records of 17 and 32 bytes, a query x codebook
table per (group, round) of up to 64 pairs. Through the C ABI against the
oracle on the same seeded inputs: records bit-exact up to logged near ties,
attention within 2e-3 of each row's max |ref|."""


import numpy as np
import pytest
import torch

from long_context_attention_commvq_amd import api, synth
from oracle import commvq_oracle as O
from tests.parity import ATTN_TOL, check_encoding, row_errors

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _pack_cache(codes, n_entries):
    """codes [B, L, Hkv, R, G] -> packed [B, Hkv, L, bpt] via the oracle's packer."""
    return np.ascontiguousarray(np.stack([O.pack_codes(codes[b], n_entries) for b in range(codes.shape[0])])
                                .transpose(0, 2, 1, 3))


@pytest.mark.parametrize("D,g,Nc,R,H,N", [
    (128, 64, 64, 11, 2, 300),    # the paper's 1-bit keys: bulk encoder (one round of one group staged at a time)
    (128, 64, 64, 21, 1, 257),    # the paper's 2-bit keys
    (128, 64, 64, 11, 2, 5),      # few tokens: one wavefront per group
    (128, 128, 64, 21, 1, 100),   # one index per head and round
    (128, 32, 16, 6, 2, 70),
])
def test_encode_paper_hyperparameters(D, g, Nc, R, H, N):
    seed = 7000 + g + R + N
    x = synth.kv(seed, N, H, D)
    cb = synth.codebook(seed + 1, H, D, g, Nc, R)
    q = api.Quantizer(dev(cb), g)
    got = api.encode(q, dev(x))
    torch.cuda.synchronize()
    hard, ties = check_encoding(x, cb, got.cpu().numpy(), Nc)
    print(f"[encode g{g} Nc{Nc} R{R}] {len(ties)} near ties accepted of {N * H * R * (D // g)} fields", flush=True)
    assert not hard, hard[:5]


@pytest.mark.parametrize("case", [
    dict(B=1, Hq=4, Hkv=1, g=64, Nc=64, R=11, lens=[2048], Lmax=2048),
    dict(B=2, Hq=8, Hkv=2, g=64, Nc=64, R=21, lens=[1000, 1537], Lmax=1600),
    dict(B=1, Hq=8, Hkv=1, g=64, Nc=64, R=11, lens=[1200], Lmax=1200),     # eight query heads: 128 KiB table
    dict(B=2, Hq=4, Hkv=1, g=128, Nc=64, R=21, lens=[700, 1], Lmax=800),
    dict(B=1, Hq=4, Hkv=2, g=32, Nc=16, R=6, lens=[999], Lmax=1024),
    # four query heads per KV head, g = 32: four groups of one slice; a cache
    # length off the 64-position grid (the last wavefront's lanes past it)
    dict(B=2, Hq=8, Hkv=2, g=32, Nc=256, R=3, lens=[999, 517], Lmax=1000),
    # 8 entries and 3 rounds: 24 bins per group, not whole 16-bin steps, so the
    # contraction takes the per-lane path
    dict(B=1, Hq=4, Hkv=1, g=64, Nc=8, R=3, lens=[777], Lmax=800),
    # exact mode (exact phases, dot products on the vector ALUs) with the
    # matrix-core contraction
    dict(B=2, Hq=4, Hkv=1, g=64, Nc=64, R=11, lens=[1500, 90], Lmax=1536, exact=True),
])
def test_decode_paper_hyperparameters(case):
    B, Hq, Hkv, g, Nc, R, Lmax = (case[k] for k in ("B", "Hq", "Hkv", "g", "Nc", "R", "Lmax"))
    D = 128
    lens = np.asarray(case["lens"], dtype=np.int32)
    seed = 7100 + g + R + Hq
    G = D // g
    rng = np.random.default_rng(seed)
    kcb = synth.codebook(seed + 1, Hkv, D, g, Nc, R)
    vcb = synth.codebook(seed + 2, Hkv, D, g, Nc, R)
    kp = _pack_cache(rng.integers(0, Nc, size=(B, Lmax, Hkv, R, G)), Nc)
    vp = _pack_cache(rng.integers(0, Nc, size=(B, Lmax, Hkv, R, G)), Nc)
    q = synth.queries(seed + 3, B, Hq, D)
    qpos = lens - 1
    ref = O.decode_attention_from_packed(q, qpos, kp, vp, lens, kcb, vcb, 500000.0)
    kq, vq = api.Quantizer(dev(kcb), g), api.Quantizer(dev(vcb), g)
    out = api.decode_attention(kq, vq, dev(q), dev(qpos), dev(kp), dev(vp), dev(lens), Lmax, 500000.0,
                               exact=bool(case.get("exact", False)))
    torch.cuda.synchronize()
    err = row_errors(out.cpu().numpy().reshape(-1, D), ref.reshape(-1, D))
    print(f"[decode {case}] max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= ATTN_TOL


def test_decode_step_paper_hyperparameters():
    """Append (the few-token encoder) then attend (the generic kernel) in one
    call at g = 64, Nc' = 64, R = 11; the new records must equal the oracle's."""
    B, Hq, Hkv, D, g, Nc, R, Lmax = 2, 8, 2, 128, 64, 64, 11, 1500
    G = D // g
    lens = np.array([1200, 1500], dtype=np.int32)
    positions = lens - 1
    rng = np.random.default_rng(7200)
    kcb = synth.codebook(7201, Hkv, D, g, Nc, R)
    vcb = synth.codebook(7202, Hkv, D, g, Nc, R)
    kp = _pack_cache(rng.integers(0, Nc, size=(B, Lmax, Hkv, R, G)), Nc)
    vp = _pack_cache(rng.integers(0, Nc, size=(B, Lmax, Hkv, R, G)), Nc)
    k_new = synth.kv(7203, B, Hkv, D)
    v_new = synth.kv(7204, B, Hkv, D)
    q = synth.queries(7205, B, Hq, D)
    kq, vq = api.Quantizer(dev(kcb), g), api.Quantizer(dev(vcb), g)
    kd, vd = dev(kp), dev(vp)
    out = api.decode_step(kq, vq, dev(k_new), dev(v_new), dev(positions), dev(q), dev(positions), kd, vd, dev(lens),
                          Lmax, 500000.0)
    torch.cuda.synchronize()
    kgot, vgot = kd.cpu().numpy(), vd.cpu().numpy()
    # the oracle's cache: its own records of the new tokens at their positions
    kexp, vexp = kp.copy(), vp.copy()
    kn_codes, _ = O.encode(k_new, kcb)
    vn_codes, _ = O.encode(v_new, vcb)
    for b in range(B):
        p = positions[b]
        kexp[b, :, p] = O.pack_codes(kn_codes[b], Nc)
        vexp[b, :, p] = O.pack_codes(vn_codes[b], Nc)
        hard, _ = check_encoding(k_new[b][None], kcb, kgot[b, :, p][None], Nc)
        assert not hard, (b, hard)
        hard, _ = check_encoding(v_new[b][None], vcb, vgot[b, :, p][None], Nc)
        assert not hard, (b, hard)
        kgot[b, :, p] = kexp[b, :, p]  # (equal up to the near ties just checked)
        vgot[b, :, p] = vexp[b, :, p]
    assert np.array_equal(kgot, kexp) and np.array_equal(vgot, vexp)  # nothing else written
    ref = O.decode_attention_from_packed(q, positions, kexp, vexp, lens, kcb, vcb, 500000.0)
    err = row_errors(out.cpu().numpy().reshape(-1, D), ref.reshape(-1, D))
    print(f"[decode step paper shape] max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= ATTN_TOL
