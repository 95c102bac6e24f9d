"""GPU parity of the comparison path (dequantise the codes to fp16, then dense
attention) through the C ABI, against the CPU oracle on the same seeded inputs.

- commvq_dequantize_kv: values must equal the oracle's dequantised values
  rounded to fp16 (bit-exact: the fp32 sum of fp16 entries is exact); rotated
  keys must lie within half an fp16 ulp of the oracle's fp64 rotation, plus
  3e-7 of the row's largest magnitude for the fp32 rotation and the hardware
  sine/cosine. Positions at or past the length stay untouched.
- commvq_dense_decode_attention: within 2e-3 of each row's max |ref| (the
  rotated query carried as two fp16 parts, products summed in fp32).
- The whole comparison path on packed caches against the oracle's
  unpack -> dequantise -> RoPE -> dense softmax, and at the 128K 1-bit
  workload's full size on sampled KV heads."""

import math
import zlib

import numpy as np
import pytest
import torch

from long_context_attention_commvq_amd import api, synth, _lib
from oracle import commvq_oracle as O
from tests.parity import ATTN_TOL, row_errors

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = 1234.0  # exactly representable in fp16


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _pack_cache(codes, n_entries):
    """codes [B, L, Hkv, R, G] -> packed [B, Hkv, L, bpt] via the oracle's packer."""
    return np.ascontiguousarray(np.stack([O.pack_codes(codes[b], n_entries) for b in range(codes.shape[0])])
                                .transpose(0, 2, 1, 3))


def _seed(case):
    return zlib.crc32(repr(sorted(case.items())).encode()) % 10000


@pytest.mark.parametrize("case", [
    dict(B=1, H=1, D=128, g=8, Nc=256, R=2, lens=[2048], Lmax=2048),
    dict(B=1, H=8, D=128, g=8, Nc=256, R=1, lens=[1000], Lmax=1024),
    dict(B=3, H=2, D=48, g=6, Nc=8, R=3, lens=[1, 300, 0], Lmax=320),      # 3-bit fields straddle bytes
    dict(B=2, H=3, D=64, g=16, Nc=64, R=2, lens=[37, 200], Lmax=256),      # 6-bit fields
    dict(B=1, H=1, D=256, g=16, Nc=256, R=1, lens=[513], Lmax=513),
    dict(B=1, H=2, D=256, g=16, Nc=256, R=2, lens=[4100], Lmax=4100),   # 256 KiB codebooks: read from L2
    dict(B=2, H=1, D=128, g=8, Nc=256, R=1, lens=[4096, 8193], Lmax=8200),  # chunks of 4096 positions
    dict(B=2, H=2, D=128, g=2, Nc=16, R=4, lens=[100, 129], Lmax=130, max_len=120),  # clamped to max_len
])
def test_dequantize_matches_oracle(case):
    case = dict(case)
    seed = _seed(case)
    B, H, D, g, Nc, R, Lmax = (case[k] for k in ("B", "H", "D", "g", "Nc", "R", "Lmax"))
    max_len = case.get("max_len", Lmax)
    lens = np.asarray(case["lens"], dtype=np.int32)
    G = D // g
    theta = 500000.0
    rng = np.random.default_rng(seed)
    kcb = synth.codebook(seed + 1, H, D, g, Nc, R)
    vcb = synth.codebook(seed + 2, H, D, g, Nc, R)
    kc = rng.integers(0, Nc, size=(B, Lmax, H, R, G))
    vc = rng.integers(0, Nc, size=(B, Lmax, H, R, G))
    kp, vp = _pack_cache(kc, Nc), _pack_cache(vc, Nc)
    kq, vq = api.Quantizer(dev(kcb), g), api.Quantizer(dev(vcb), g)
    k_out = torch.full((B, H, Lmax, D), SENTINEL, dtype=torch.float16, device=DEV)
    v_out = torch.full((B, H, Lmax, D), SENTINEL, dtype=torch.float16, device=DEV)
    api.dequantize_kv(kq, vq, dev(kp), dev(vp), dev(lens), max_len, theta, k_out, v_out)
    torch.cuda.synchronize()
    kg = k_out.cpu().numpy().astype(np.float64)
    vg = v_out.cpu().numpy().astype(np.float64)
    thetas = O.rope_thetas(D, theta)
    worst = 0.0
    for b in range(B):
        L = int(min(max(lens[b], 0), max_len))
        assert np.all(kg[b, :, L:] == SENTINEL) and np.all(vg[b, :, L:] == SENTINEL)
        if L == 0:
            continue
        kh = O.dequantize(kc[b, :L], kcb).transpose(1, 0, 2)  # [H, L, D]
        vh = O.dequantize(vc[b, :L], vcb).transpose(1, 0, 2)
        kr = O.apply_rope(kh, np.arange(L), thetas)
        v16 = vh.astype(np.float16).astype(np.float64)
        assert np.array_equal(vg[b, :, :L], v16), np.abs(vg[b, :, :L] - v16).max()
        big = np.maximum(np.abs(kr), np.abs(kg[b, :, :L]))
        ulp = np.spacing(big.astype(np.float16)).astype(np.float64)
        bound = 0.5 * ulp + 3e-7 * np.abs(kr).max(axis=-1, keepdims=True)
        excess = np.abs(kg[b, :, :L] - kr) / bound
        worst = max(worst, float(excess.max()))
        assert excess.max() <= 1.0, (b, np.unravel_index(np.argmax(excess), excess.shape))
    print(f"[dequantize {case}] max key error / bound {worst:.3f}", flush=True)


def run_dense_case(seed, B, Hq, Hkv, lens, Lmax, max_len=None, q_pos=None, q_scale=1.0, theta=500000.0):
    D = 128
    kv = synth.kv(seed + 1, Lmax, Hkv, D, batch=B)  # [B, L, H, D]
    vv = synth.kv(seed + 2, Lmax, Hkv, D, batch=B)
    k16 = np.ascontiguousarray(kv.transpose(0, 2, 1, 3))
    v16 = np.ascontiguousarray(vv.transpose(0, 2, 1, 3))
    q = synth.queries(seed + 3, B, Hq, D) * np.float32(q_scale)
    lens = np.asarray(lens, dtype=np.int32)
    max_len = Lmax if max_len is None else max_len
    qpos = (np.maximum(lens, 1) - 1) if q_pos is None else np.asarray(q_pos, dtype=np.int32)
    scale = 1.0 / math.sqrt(D)
    thetas = O.rope_thetas(D, theta)
    rep = Hq // Hkv
    ref = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(min(max(lens[b], 0), max_len))
        if L == 0:
            continue
        qr = O.apply_rope(q[b], np.full(Hq, int(qpos[b])), thetas)
        for hq in range(Hq):
            h = hq // rep
            ref[b, hq] = O.attend_one(qr[hq], k16[b, h, :L].astype(np.float64), v16[b, h, :L].astype(np.float64),
                                      scale)
    out = api.dense_decode_attention(dev(q), dev(qpos), dev(k16), dev(v16), dev(lens), max_len, theta, scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    return got, ref, row_errors(got.reshape(-1, D), ref.reshape(-1, D))


@pytest.mark.parametrize("case", [
    dict(B=1, Hq=4, Hkv=1, lens=[2048], Lmax=2048),
    dict(B=3, Hq=8, Hkv=8, lens=[1, 1024, 1025], Lmax=1100),        # one query head per KV head; chunk edges
    dict(B=2, Hq=16, Hkv=8, lens=[1024, 777], Lmax=1100),
    dict(B=2, Hq=8, Hkv=1, lens=[1500, 0], Lmax=1536),              # eight query heads; a zero length
    dict(B=1, Hq=4, Hkv=1, lens=[5000], Lmax=6000, max_len=4096),   # clamped to max_seq_len
    dict(B=2, Hq=4, Hkv=1, lens=[300, 1000], Lmax=1024, q_pos=[2_000_000_000, 131071]),
    dict(B=1, Hq=32, Hkv=8, lens=[3000], Lmax=3000, q_scale=4.0),   # peaked scores
])
def test_dense_attention_matches_oracle(case):
    got, ref, err = run_dense_case(_seed(case), **case)
    print(f"[dense {case}] max row rel err {err.max():.3e}", flush=True)
    assert np.all(np.isfinite(got))
    for b, L in enumerate(case["lens"]):
        if L == 0:
            assert np.all(got[b] == 0.0)
    assert err.max() <= ATTN_TOL


def test_dense_attention_rejects_bad_arguments():
    q = torch.zeros((1, 4, 128), dtype=torch.float32, device=DEV)
    kv = torch.zeros((1, 1, 64, 128), dtype=torch.float16, device=DEV)
    pos = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = api.DenseWorkspace(1, 4, 1, 128, 64, DEV)
    rope = _lib.make_rope(500000.0)
    out = torch.zeros_like(q)
    with pytest.raises(_lib.CommvqError) as e:
        _lib.commvq_dense_decode_attention(rope, q, pos, kv, kv, pos, 1, 4, 1, 128, 64, 65, 0.1, out, ws.buf,
                                           ws.nbytes)  # max_seq_len > cache_len
    assert e.value.status == _lib.COMMVQ_ERR_INVALID_ARG
    with pytest.raises(_lib.CommvqError) as e:
        _lib.commvq_dense_decode_attention(rope, q, pos, kv, kv, pos, 1, 4, 1, 128, 64, 64, 0.1, out, ws.buf,
                                           ws.nbytes - 4)
    assert e.value.status == _lib.COMMVQ_ERR_WORKSPACE
    with pytest.raises(_lib.CommvqError) as e:
        _lib.commvq_dense_decode_attention(rope, q, pos, kv, kv, pos, 1, 4, 1, 64, 64, 64, 0.1, out, ws.buf,
                                           ws.nbytes)
    assert e.value.status == _lib.COMMVQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("R,B,Hq,Hkv,lens,Lmax", [
    (2, 1, 4, 1, [2048], 2048),
    (1, 2, 8, 2, [1500, 3001], 3100),
])
def test_comparison_path_matches_oracle(R, B, Hq, Hkv, lens, Lmax):
    """Packed caches -> commvq_dequantize_kv -> commvq_dense_decode_attention
    against the oracle's unpack -> dequantise -> RoPE -> dense softmax; the
    table/histogram path on the same inputs meets the same bar."""
    D, g, Nc, theta = 128, 8, 256, 500000.0
    seed = 300 + 10 * R + B
    G = D // g
    rng = np.random.default_rng(seed)
    kcb = synth.codebook(seed + 1, Hkv, D, g, Nc, R)
    vcb = synth.codebook(seed + 2, Hkv, D, g, Nc, R)
    kp = _pack_cache(rng.integers(0, Nc, size=(B, Lmax, Hkv, R, G)), Nc)
    vp = _pack_cache(rng.integers(0, Nc, size=(B, Lmax, Hkv, R, G)), Nc)
    q = synth.queries(seed + 3, B, Hq, D)
    lens = np.asarray(lens, dtype=np.int32)
    qpos = lens - 1
    ref = O.decode_attention_from_packed(q, qpos, kp, vp, lens, kcb, vcb, theta)
    kq, vq = api.Quantizer(dev(kcb), g), api.Quantizer(dev(vcb), g)
    kd, vd, ld = dev(kp), dev(vp), dev(lens)
    k16, v16 = api.dequantize_kv(kq, vq, kd, vd, ld, Lmax, theta)
    naive = api.dense_decode_attention(dev(q), dev(qpos), k16, v16, ld, Lmax, theta)
    table = api.decode_attention(kq, vq, dev(q), dev(qpos), kd, vd, ld, Lmax, theta)
    torch.cuda.synchronize()
    e1 = row_errors(naive.cpu().numpy().reshape(-1, D), ref.reshape(-1, D))
    e2 = row_errors(table.cpu().numpy().reshape(-1, D), ref.reshape(-1, D))
    print(f"[comparison R{R} B{B}] naive {e1.max():.3e}, table path {e2.max():.3e}", flush=True)
    assert e1.max() <= ATTN_TOL and e2.max() <= ATTN_TOL


def test_comparison_path_full_size_128k_1bit_sampled():
    """The 128K 1-bit workload's shape (8 KV heads, 32 query heads, 131072
    positions) in the launch configuration the benchmark times: every head
    dequantised and attended at once; the oracle recomputes sampled positions
    of every head and two whole KV heads."""
    w = synth.WORKLOADS["llama8b_ctx128k_1bit_64steps"]
    B, Hq, H, D, Lmax = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.context
    rep = Hq // H
    kcb = synth.codebook(w.seed + 1, H, D, w.group_size, w.n_entries, w.n_rounds)
    vcb = synth.codebook(w.seed + 2, H, D, w.group_size, w.n_entries, w.n_rounds)
    kq, vq = api.Quantizer(dev(kcb), w.group_size), api.Quantizer(dev(vcb), w.group_size)
    bpt = kq.bytes_per_token
    rng = np.random.default_rng(w.seed + 70)
    kp = rng.integers(0, 256, size=(B, H, Lmax, bpt), dtype=np.uint8)  # every byte string is a valid record
    vp = rng.integers(0, 256, size=(B, H, Lmax, bpt), dtype=np.uint8)
    q = synth.queries(w.seed + 71, B, Hq, D)
    lens = np.array([Lmax], dtype=np.int32)
    qpos = lens - 1
    print(f"[comparison full size] B={B} Hq={Hq} Hkv={H} L={Lmax}", flush=True)
    kq_d, vq_d, ld = dev(kp), dev(vp), dev(lens)
    k16, v16 = api.dequantize_kv(kq, vq, kq_d, vq_d, ld, Lmax, w.theta_base)
    out = api.dense_decode_attention(dev(q), dev(qpos), k16, v16, ld, Lmax, w.theta_base)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    # dequantised vectors at sampled positions (first, last, random) of every head
    pos = np.unique(np.concatenate([[0, 1, Lmax - 1], rng.integers(0, Lmax, 500)]))
    thetas = O.rope_thetas(D, w.theta_base)
    kg = k16[0][:, torch.from_numpy(pos).to(DEV)].cpu().numpy().astype(np.float64)  # [H, P, D]
    vg = v16[0][:, torch.from_numpy(pos).to(DEV)].cpu().numpy().astype(np.float64)
    kc = O.unpack_codes(kp[0][:, pos].transpose(1, 0, 2), w.n_rounds, D // w.group_size, w.n_entries)  # [P, H, R, G]
    vc = O.unpack_codes(vp[0][:, pos].transpose(1, 0, 2), w.n_rounds, D // w.group_size, w.n_entries)
    kr = O.apply_rope(O.dequantize(kc, kcb).transpose(1, 0, 2), pos, thetas)
    vh = O.dequantize(vc, vcb).transpose(1, 0, 2)
    assert np.array_equal(vg, vh.astype(np.float16).astype(np.float64))
    big = np.maximum(np.abs(kr), np.abs(kg))
    bound = 0.5 * np.spacing(big.astype(np.float16)).astype(np.float64) + 3e-7 * np.abs(kr).max(-1, keepdims=True)
    assert (np.abs(kg - kr) / bound).max() <= 1.0
    # attention rows of two whole KV heads
    for h in (int(rng.integers(0, H)), H - 1):
        ref = O.decode_attention_from_packed(q[:, h * rep:(h + 1) * rep], qpos, kp[:, h:h + 1], vp[:, h:h + 1], lens,
                                             kcb[h:h + 1], vcb[h:h + 1], w.theta_base)[0]
        err = row_errors(got[0, h * rep:(h + 1) * rep], ref)
        print(f"[comparison full size] head {h} max row rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL
