"""Pins for the CPU oracle: each test ties the oracle to something other than
itself (numbers printed on the pages, closed forms, invariants, brute force,
library routines). No GPU needed."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import commvq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- storage cost

def test_bit_rate_table9_printed_values():
    for row in _golden("pages_numbers.json")["bit_rate_table9"]["rows"]:
        got = O.bits_per_scalar(row["g"], row["n_entries"], row["n_rounds"])
        assert got == row["avg_bits"], row


def test_bit_rate_table8_labels():
    for row in _golden("pages_numbers.json")["table8_configs"]["rows"]:
        got = O.bits_per_scalar(row["g"], row["n_entries"], row["n_rounds"])
        assert round(got) == row["label_bits"] and abs(got - row["label_bits"]) < 0.05, (row, got)


def test_size_cuts_vs_fp16_and_packed_length():
    # 2-bit and 1-bit workload quantisers: g = 8 scalars, Nc' = 256, R = 2 or 1.
    for row in _golden("pages_numbers.json")["size_cuts_vs_fp16"]["rows"]:
        R = row["bits"]
        bits = O.bits_per_scalar(8, 256, R)
        assert bits == row["bits"]
        assert 100.0 * (1.0 - bits / 16.0) == row["cut_percent"]
        # a real packed record has exactly bits/16 of the fp16 record's bytes
        codes = np.random.default_rng(R).integers(0, 256, size=(5, 3, R, 16))
        packed = O.pack_codes(codes, 256)
        assert packed.shape[-1] == O.code_bytes_per_token(128, 8, 256, R)
        assert packed.shape[-1] / (128 * 2) == bits / 16


def test_fp16_cache_sizes_from_referee():
    for row in _golden("pages_numbers.json")["fp16_cache_sizes"]["rows"]:
        b = O.fp16_kv_cache_bytes(row["batch"], row["tokens"], row["layers"], row["kv_dim"])
        assert round(b / 1e9, 1) == row["approx_gb"], (row, b)


def test_field_bits_rejects_non_power_of_two():
    assert O.field_bits(1) == 0 and O.field_bits(256) == 8 and O.field_bits(64) == 6
    for bad in (0, 3, 100, 255):
        with pytest.raises(ValueError):
            O.field_bits(bad)


# ---------------------------------------------------------------- commutation, RoPE

def test_commutative_block_commutes_with_rotation():
    g = np.random.default_rng(0)
    for _ in range(200):
        x, y = g.standard_normal(2)
        ang = g.uniform(-50, 50)
        C = O.commutative_block(x, y)
        Rm = O.rotation_matrix(ang)
        lhs, rhs = Rm @ C, C @ Rm
        assert np.max(np.abs(lhs - rhs)) <= 1e-15 * max(1.0, np.max(np.abs(lhs)))


def test_non_commutative_block_fails_the_same_check():
    # negative control: [[x, y], [y, x]] is not of the commutative form
    Rm = O.rotation_matrix(0.7)
    M = np.array([[0.3, 1.1], [1.1, 0.3]])
    assert np.max(np.abs(Rm @ M - M @ Rm)) > 0.1


def test_rope_thetas_closed_forms():
    th = O.rope_thetas(128, 500000.0)
    assert th.shape == (64,)
    assert th[0] == 1.0
    assert math.isclose(th[32], 1.0 / math.sqrt(500000.0), rel_tol=1e-14)
    assert math.isclose(th[16], 500000.0 ** -0.25, rel_tol=1e-14)
    assert np.all(np.diff(th) < 0)


def test_rope_rotation_closed_form():
    th = np.array([1.0, 0.5])
    x = np.array([[1.0, 0.0, 0.0, 1.0]])
    out = O.apply_rope(x, np.array([1]), th)[0]
    # pair 0: (1, 0) rotated by 1 rad -> (cos 1, sin 1); pair 1: (0, 1) by 0.5 -> (-sin .5, cos .5)
    np.testing.assert_allclose(out, [math.cos(1), math.sin(1), -math.sin(0.5), math.cos(0.5)], rtol=0, atol=1e-15)
    # the same as the explicit 2x2 block and as complex multiplication by e^{i angle}
    v = np.array([0.3, -1.7])
    ref_m = O.rotation_matrix(2.5) @ v
    z = complex(v[0], v[1]) * complex(math.cos(2.5), math.sin(2.5))
    got = O.apply_rope(np.array([[v[0], v[1]]]), np.array([5]), np.array([0.5]))[0]
    np.testing.assert_allclose(got, ref_m, atol=1e-15)
    np.testing.assert_allclose(got, [z.real, z.imag], atol=1e-15)


def test_rope_inverse_norm_and_relativity():
    g = np.random.default_rng(1)
    th = O.rope_thetas(64, 10000.0)
    x = g.standard_normal((7, 64))
    pos = g.integers(0, 100000, size=7)
    r = O.apply_rope(x, pos, th)
    np.testing.assert_allclose(O.apply_rope(r, -pos, th), x, atol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    q, k = g.standard_normal(64), g.standard_normal(64)
    d0 = O.apply_rope(q[None], np.array([900]), th)[0] @ O.apply_rope(k[None], np.array([37]), th)[0]
    d1 = O.apply_rope(q[None], np.array([900 + 5000]), th)[0] @ O.apply_rope(k[None], np.array([37 + 5000]), th)[0]
    assert abs(d0 - d1) < 1e-9 * max(1.0, abs(d0))


# ---------------------------------------------------------------- packing

def test_pack_golden_records():
    for case in _golden("pack_fields.json")["cases"]:
        codes = np.array(case["codes"], dtype=np.int64)
        got = O.pack_codes(codes, case["n_entries"])
        assert got.tolist() == case["bytes"], case
        back = O.unpack_codes(got, codes.shape[0], codes.shape[1], case["n_entries"])
        assert np.array_equal(back, codes)


@pytest.mark.parametrize("n_entries", [1, 2, 4, 8, 16, 64, 256, 1024, 65536])
def test_pack_roundtrip(n_entries):
    g = np.random.default_rng(n_entries)
    codes = g.integers(0, n_entries, size=(3, 2, 3, 5))
    packed = O.pack_codes(codes, n_entries)
    assert packed.shape == (3, 2, (3 * 5 * O.field_bits(n_entries) + 7) // 8)
    assert np.array_equal(O.unpack_codes(packed, 3, 5, n_entries), codes)


# ---------------------------------------------------------------- encoder

def _brute_nearest(e, entries):
    """Nearest entry by an explicit Python loop; first index wins exact ties."""
    best, bd = 0, None
    for l in range(entries.shape[0]):
        d = 0.0
        for i in range(entries.shape[1]):
            diff = float(e[i]) - float(entries[l, i])
            d += diff * diff
        if bd is None or d < bd:
            best, bd = l, d
    return best


@pytest.mark.parametrize("g,Nc", [(2, 16), (4, 8), (8, 16)])
def test_encoder_r1_is_exact_nearest_neighbour(g, Nc):
    rng = np.random.default_rng(g * 100 + Nc)
    H, G, N = 2, 2, 9
    cb = rng.standard_normal((H, G, 1, Nc, g)).astype(np.float16)
    x = rng.standard_normal((N, H, G * g)).astype(np.float16)
    codes, _ = O.encode(x, cb)
    for n, h, j in itertools.product(range(N), range(H), range(G)):
        e = x[n, h, j * g:(j + 1) * g].astype(np.float64)
        assert codes[n, h, 0, j] == _brute_nearest(e, cb[h, j, 0].astype(np.float64))


def test_encoder_greedy_vs_joint_optimum():
    rng = np.random.default_rng(7)
    g, Nc = 4, 6
    for R in (1, 2, 3):
        cb = rng.standard_normal((1, 1, R, Nc, g))
        x = rng.standard_normal((12, 1, g))
        codes, _ = O.encode(x, cb)
        xh = O.dequantize(codes, cb)
        for n in range(12):
            greedy_err = np.sum((x[n, 0] - xh[n, 0]) ** 2)
            joint = min(np.sum((x[n, 0] - sum(cb[0, 0, r, c[r]] for r in range(R))) ** 2)
                        for c in itertools.product(range(Nc), repeat=R))
            assert greedy_err >= joint - 1e-12
            if R == 1:
                assert abs(greedy_err - joint) < 1e-12
            # greedy round-by-round choice is the nearest entry to the running residual
            e = x[n, 0].copy()
            for r in range(R):
                assert codes[n, 0, r, 0] == _brute_nearest(e, cb[0, 0, r])
                e = e - cb[0, 0, r, codes[n, 0, r, 0]]


def test_encoder_known_codebook_reconstructs_exactly():
    rng = np.random.default_rng(11)
    g, Nc, G, N = 8, 16, 3, 5
    x = rng.standard_normal((N, 1, G * g))
    cb = rng.standard_normal((1, G, 2, Nc, g)) * 10 + 40  # far from the inputs
    want0 = rng.integers(0, Nc, size=(N, G))
    for j in range(G):
        # distinct slots per token inside this group
        want0[:, j] = rng.permutation(Nc)[:N]
        for n in range(N):
            cb[0, j, 0, want0[n, j]] = x[n, 0, j * g:(j + 1) * g]
        cb[0, j, 1, 9] = 0.0  # zero entry: the residual after round 0 is exactly zero
    codes, _ = O.encode(x, cb)
    assert np.array_equal(codes[:, 0, 0, :], want0)
    assert np.all(codes[:, 0, 1, :] == 9)
    np.testing.assert_array_equal(O.dequantize(codes, cb), x)


def test_encoder_ties_take_lowest_index_and_permutation_equivariance():
    rng = np.random.default_rng(3)
    g, Nc = 4, 8
    cb = rng.standard_normal((1, 1, 1, Nc, g))
    cb[0, 0, 0, 6] = cb[0, 0, 0, 2]  # duplicate entry
    x = cb[0, 0, 0, 2][None, None, :] + 1e-3
    codes, gaps = O.encode(x, cb)
    assert codes[0, 0, 0, 0] == 2 and gaps[0, 0, 0, 0] == 0.0
    perm = rng.permutation(Nc)
    cbp = cb[:, :, :, perm]
    y = rng.standard_normal((20, 1, g))
    c1, _ = O.encode(y, cb)
    c2, _ = O.encode(y, cbp)
    inv = np.argsort(perm)
    # distinct entries only (drop the duplicated pair from this comparison)
    ok = (c1[..., 0] != 2) & (c1[..., 0] != 6)
    assert np.array_equal(inv[c1[..., 0][ok]], c2[..., 0][ok]) or np.array_equal(perm[c2[..., 0][ok]], c1[..., 0][ok])


def test_encoder_single_entry_codebook():
    cb = np.random.default_rng(0).standard_normal((2, 4, 2, 1, 4))
    x = np.random.default_rng(1).standard_normal((3, 2, 16))
    codes, _ = O.encode(x, cb)
    assert np.all(codes == 0)
    assert O.code_bytes_per_token(16, 4, 1, 2) == 0


# ---------------------------------------------------------------- attention

def _rand_attention_case(seed, B=2, Hq=4, Hkv=2, D=32, L=40, g=4, Nc=16, R=2):
    rng = np.random.default_rng(seed)
    G = D // g
    kcb = rng.standard_normal((Hkv, G, R, Nc, g))
    vcb = rng.standard_normal((Hkv, G, R, Nc, g))
    kc = rng.integers(0, Nc, size=(B, L, Hkv, R, G))
    vc = rng.integers(0, Nc, size=(B, L, Hkv, R, G))
    kh = np.stack([O.dequantize(kc[b], kcb) for b in range(B)]).transpose(0, 2, 1, 3)  # [B, Hkv, L, D]
    vh = np.stack([O.dequantize(vc[b], vcb) for b in range(B)]).transpose(0, 2, 1, 3)
    q = rng.standard_normal((B, Hq, D))
    lens = rng.integers(1, L + 1, size=B)
    return dict(q=q, kh=kh, vh=vh, kc=kc, vc=vc, kcb=kcb, vcb=vcb, lens=lens, Nc=Nc)


def test_attention_matches_torch_sdpa_with_gqa():
    c = _rand_attention_case(5)
    B, Hq, D = c["q"].shape
    Hkv = c["kh"].shape[1]
    th = O.rope_thetas(D, 500000.0)
    qpos = c["lens"] - 1
    got = O.decode_attention(c["q"], qpos, c["kh"], c["vh"], c["lens"], th, 1 / math.sqrt(D))
    for b in range(B):
        L = int(c["lens"][b])
        pos = np.arange(L)
        kr = np.stack([O.apply_rope(c["kh"][b, h, :L], pos, th) for h in range(Hkv)])
        qr = O.apply_rope(c["q"][b], np.full(Hq, qpos[b]), th)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qr)[None, :, None, :], torch.from_numpy(kr)[None],
            torch.from_numpy(c["vh"][b, :, :L])[None], enable_gqa=True)[0, :, 0, :].numpy()
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    c = _rand_attention_case(6, B=1)
    D = c["q"].shape[2]
    th = O.rope_thetas(D, 500000.0)
    rep = c["q"].shape[1] // c["kh"].shape[1]
    # L = 1: output is the single value row
    one = O.decode_attention(c["q"], [0], c["kh"], c["vh"], [1], th, 0.2)
    for hq in range(c["q"].shape[1]):
        np.testing.assert_allclose(one[0, hq], c["vh"][0, hq // rep, 0], rtol=0, atol=1e-15)
    # q = 0: uniform weights -> mean of values
    L = 17
    z = O.decode_attention(np.zeros_like(c["q"]), [L - 1], c["kh"], c["vh"], [L], th, 0.2)
    for hq in range(c["q"].shape[1]):
        np.testing.assert_allclose(z[0, hq], c["vh"][0, hq // rep, :L].mean(0), rtol=1e-13, atol=1e-14)
    # huge q stays finite (max subtraction)
    big = O.decode_attention(c["q"] * 1e4, [L - 1], c["kh"], c["vh"], [L], th, 0.2)
    assert np.all(np.isfinite(big))
    # positions beyond the length are ignored
    kh2, vh2 = c["kh"].copy(), c["vh"].copy()
    kh2[:, :, L:] = 1e6
    vh2[:, :, L:] = -1e6
    a = O.decode_attention(c["q"], [L - 1], c["kh"], c["vh"], [L], th, 0.2)
    b = O.decode_attention(c["q"], [L - 1], kh2, vh2, [L], th, 0.2)
    np.testing.assert_array_equal(a, b)


def test_table_form_scores_equal_dense_scores():
    """The reordering the fast path relies on: query x codebook table, gathered per
    code and multiplied by the position's phase, equals dense RoPE'd dot products."""
    rng = np.random.default_rng(8)
    D, g, Nc, R, L = 32, 8, 16, 2, 50
    G = D // g
    cb = rng.standard_normal((1, G, R, Nc, g))
    codes = rng.integers(0, Nc, size=(L, 1, R, G))
    q = rng.standard_normal(D)
    th = O.rope_thetas(D, 10000.0)
    for qpos in (L - 1, 123456):
        kh = O.dequantize(codes, cb)[:, 0]
        kr = O.apply_rope(kh, np.arange(L), th)
        qr = O.apply_rope(q[None], np.array([qpos]), th)[0]
        dense = kr @ qr * 0.3
        table = O.scores_table_form(q, qpos, codes[:, 0], cb[0], th, 0.3)
        np.testing.assert_allclose(table, dense, rtol=1e-12, atol=1e-12)


def test_histogram_value_form_equals_dense_values():
    rng = np.random.default_rng(9)
    D, g, Nc, R, L = 32, 4, 16, 3, 200
    G = D // g
    cb = rng.standard_normal((1, G, R, Nc, g))
    codes = rng.integers(0, Nc, size=(L, 1, R, G))
    w = rng.random(L)
    dense = w @ O.dequantize(codes, cb)[:, 0]
    hist = O.values_histogram_form(w, codes[:, 0], cb[0])
    np.testing.assert_allclose(hist, dense, rtol=1e-12, atol=1e-12)


def test_packed_path_equals_dequantised_path():
    c = _rand_attention_case(10, B=2, Hq=4, Hkv=2, D=32, L=30, g=4, Nc=16, R=2)
    D = c["q"].shape[2]
    th = O.rope_thetas(D, 500000.0)
    kp = np.stack([O.pack_codes(c["kc"][b], c["Nc"]) for b in range(2)]).transpose(0, 2, 1, 3)
    vp = np.stack([O.pack_codes(c["vc"][b], c["Nc"]) for b in range(2)]).transpose(0, 2, 1, 3)
    qpos = c["lens"] - 1
    a = O.decode_attention_from_packed(c["q"], qpos, kp, vp, c["lens"], c["kcb"], c["vcb"], 500000.0)
    b = O.decode_attention(c["q"], qpos, c["kh"], c["vh"], c["lens"], th, 1 / math.sqrt(D))
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_encode_then_attend_end_to_end_small():
    """Encoding then attending stays close to attention on the raw vectors when the
    codebook is rich (sanity that encoder and decoder use the same layout)."""
    rng = np.random.default_rng(12)
    D, g, Nc, R, L = 16, 2, 256, 3, 25
    G = D // g
    cb = rng.standard_normal((1, G, R, Nc, g)) * np.array([1.0, 0.1, 0.01])[None, None, :, None, None]
    x = rng.standard_normal((L, 1, D)) * 0.8
    codes, _ = O.encode(x, cb)
    err = np.abs(O.dequantize(codes, cb) - x).max()
    assert err < 0.1


# ---------------------------------------------------------------- codebook fitting (EM)

def _em_data(seed, N, H, G, g, Nc, R):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, H, G * g))
    cb = rng.standard_normal((H, G, R, Nc, g))
    return x, cb


def test_em_hard_step_equals_brute_force_lloyd_step():
    """T = 0, round 0: every entry becomes the plain mean of the vectors whose
    nearest entry it is, found here by explicit loops over every entry."""
    x, cb = _em_data(11, 60, 2, 2, 2, 5, 1)
    new, mass = O.em_step(x, cb, 0, 0.0)
    N, H, D = x.shape
    G, g, Nc = 2, 2, 5
    for h in range(H):
        for j in range(G):
            members = [[] for _ in range(Nc)]
            for n in range(N):
                e = x[n, h, j * g:(j + 1) * g]
                best, bd = 0, None
                for l in range(Nc):
                    d = sum((e[i] - cb[h, j, 0, l, i]) ** 2 for i in range(g))
                    if bd is None or d < bd:
                        best, bd = l, d
                members[best].append(e)
            for l in range(Nc):
                assert mass[h, j, l] == len(members[l])
                want = np.mean(members[l], axis=0) if members[l] else cb[h, j, 0, l]
                assert np.allclose(new[h, j, l], want, rtol=0, atol=1e-12)


def _explicit_soft_em(x, cb, r, T):
    """One soft EM iteration written as plain loops over every (vector, entry):
    residuals by an explicit nearest-entry search of each earlier round, then
    weights exp(-(d_l - min d) / T) / sum, masses and weighted means."""
    N, H, D = x.shape
    _, G, R, Nc, g = cb.shape
    new = cb[:, :, r].copy()
    mass = np.zeros((H, G, Nc))
    for h in range(H):
        for j in range(G):
            sums = np.zeros((Nc, g))
            for n in range(N):
                e = [float(v) for v in x[n, h, j * g:(j + 1) * g]]
                for rr in range(r):
                    best, bd = 0, None
                    for l in range(Nc):
                        d = sum((e[i] - cb[h, j, rr, l, i]) ** 2 for i in range(g))
                        if bd is None or d < bd:
                            best, bd = l, d
                    e = [e[i] - cb[h, j, rr, best, i] for i in range(g)]
                d = [sum((e[i] - cb[h, j, r, l, i]) ** 2 for i in range(g)) for l in range(Nc)]
                dmin = min(d)
                w = [math.exp(-(d[l] - dmin) / T) for l in range(Nc)]
                tot = sum(w)
                for l in range(Nc):
                    mass[h, j, l] += w[l] / tot
                    for i in range(g):
                        sums[l, i] += w[l] / tot * e[i]
            for l in range(Nc):
                if mass[h, j, l] > 0:
                    new[h, j, l] = sums[l] / mass[h, j, l]
    return new, mass


@pytest.mark.parametrize("T,r", [(0.3, 0), (2.0, 1), (0.3, 2)])
def test_em_soft_step_equals_explicit_loops(T, r):
    """Finite temperature: the annealed soft E-step and the weighted-mean M-step
    (review, "Assumptions & free parameters": soft assignment and annealing;
    "Referee Report", Significance: closed-form update), against plain loops.
    Unit-scale data, so a temperature off by a factor moves the weights."""
    x, cb = _em_data(17 + r, 40, 2, 2, 3, 5, 3)
    new, mass = O.em_step(x, cb, r, T)
    want, wmass = _explicit_soft_em(x, cb, r, T)
    assert np.allclose(mass, wmass, rtol=1e-12, atol=1e-12)
    assert np.allclose(mass.sum(axis=-1), 40.0, rtol=1e-12)  # each vector's weights sum to one
    assert np.allclose(new, want, rtol=1e-10, atol=1e-12)


def test_encode_gaps_equal_brute_force_top2():
    """The near-tie diagnostic: for each decision, the two smallest distances found
    by sorting every entry's distance (explicit loops), relative to max(d_best,
    1e-12 |e|^2), with the residual of the greedy rounds before it."""
    rng = np.random.default_rng(19)
    N, H, G, g, Nc, R = 25, 2, 3, 2, 6, 3
    x = rng.standard_normal((N, H, G * g))
    cb = rng.standard_normal((H, G, R, Nc, g))
    cb[1, 2, 1, 4] = cb[1, 2, 1, 1]  # an exact duplicate: gap 0 wherever either is nearest
    codes, gaps = O.encode(x, cb)
    for n in range(N):
        for h in range(H):
            for j in range(G):
                e = [float(v) for v in x[n, h, j * g:(j + 1) * g]]
                for r in range(R):
                    d = sorted((sum((e[i] - cb[h, j, r, l, i]) ** 2 for i in range(g)), l) for l in range(Nc))
                    (d1, l1), (d2, _) = d[0], d[1]
                    norm2 = sum(v * v for v in e)
                    want = (d2 - d1) / max(d1, 1e-12 * norm2, 1e-300)
                    assert codes[n, h, r, j] == l1
                    assert math.isclose(gaps[n, h, r, j], want, rel_tol=1e-9, abs_tol=1e-12)
                    e = [e[i] - cb[h, j, r, l1, i] for i in range(g)]
    assert (gaps[:, 1, 1, 2] == 0).any() or not (codes[:, 1, 1, 2] == 1).any()


def test_em_infinite_temperature_gives_the_mean_of_all_residuals():
    """T -> infinity: uniform responsibilities, so every entry becomes the mean of
    all residuals (round 1: x minus the nearest round-0 entry) with mass N / Nc."""
    x, cb = _em_data(12, 80, 1, 3, 4, 6, 2)
    new, mass = O.em_step(x, cb, 1, 1e15)
    e = O.em_round_residuals(x, cb, 1)  # [N, 1, 3, 4]
    # round-0 residual by explicit nearest-entry search
    for j in range(3):
        for n in range(80):
            v = x[n, 0, 4 * j:4 * j + 4]
            l = int(np.argmin([np.sum((v - cb[0, j, 0, k]) ** 2) for k in range(6)]))
            assert np.allclose(e[n, 0, j], v - cb[0, j, 0, l], atol=1e-15)
        assert np.allclose(mass[0, j], 80 / 6, rtol=1e-12)
        assert np.allclose(new[0, j], e[:, 0, j].mean(axis=0)[None, :], atol=1e-9)


def test_em_small_temperature_approaches_hard_assignment():
    x, cb = _em_data(13, 200, 1, 2, 8, 16, 1)
    hard, mh = O.em_step(x, cb, 0, 0.0)
    soft, ms = O.em_step(x, cb, 0, 1e-6)
    d = O.sq_distances(x.reshape(200, 1, 2, 8), cb[:, :, 0][None])
    part = np.partition(d, 1, axis=-1)
    assert (part[..., 1] - part[..., 0]).min() > 1e-3  # no near-ties: 1e-3 / 1e-6 makes the runner-up weight < e^-1000
    assert np.allclose(soft, hard, atol=1e-12) and np.allclose(ms, mh, atol=1e-12)


def test_em_hard_iterations_never_increase_the_reconstruction_error():
    """Lloyd's iteration: neither the closed-form update nor the re-assignment
    can raise the squared error of a one-round quantiser."""
    x, cb = _em_data(14, 500, 2, 4, 4, 8, 1)
    err = [O.reconstruction_error(x, cb)]
    for _ in range(6):
        new, _ = O.em_step(x, cb, 0, 0.0)
        cb = cb.copy()
        cb[:, :, 0] = new
        err.append(O.reconstruction_error(x, cb))
    assert all(b <= a + 1e-12 for a, b in zip(err, err[1:])), err
    assert err[-1] < 0.8 * err[0]


def test_em_fixed_point_and_unused_entries():
    """A codebook holding the data points themselves is a fixed point of the hard
    step; entries no vector picks keep their value, and min_mass keeps entries
    whose mass is too small."""
    rng = np.random.default_rng(15)
    pts = rng.standard_normal((5, 4))
    x = np.repeat(pts, [3, 1, 4, 2, 5], axis=0)[:, None, :]  # [15, 1, 4]: one group of g = 4
    cb = np.zeros((1, 1, 1, 8, 4))
    cb[0, 0, 0, :5] = pts
    cb[0, 0, 0, 5:] = 100.0 + rng.standard_normal((3, 4))  # far away: never chosen
    new, mass = O.em_step(x, cb, 0, 0.0)
    assert np.allclose(new, cb[:, :, 0], rtol=0, atol=1e-14) and list(mass[0, 0]) == [3, 1, 4, 2, 5, 0, 0, 0]
    assert np.array_equal(new[0, 0, 5:], cb[0, 0, 0, 5:])  # unused entries: bit-identical
    moved = cb.copy()
    moved[0, 0, 0, :5] += 0.01
    new2, _ = O.em_step(x, moved, 0, 0.0, min_mass=2.5)
    assert np.allclose(new2[0, 0, [0, 2, 4]], pts[[0, 2, 4]], atol=1e-14)   # mass 3, 4, 5 -> the mean
    assert np.array_equal(new2[0, 0, [1, 3]], moved[0, 0, 0, [1, 3]])       # mass 1, 2 <= 2.5 -> kept


def test_em_later_round_fits_what_earlier_rounds_leave():
    """Round 1 is fitted on x minus round 0's choice: with round 0 holding the
    exact data points the residuals are zero, so every used round-1 entry moves
    to 0; the fitted codebook then reconstructs x exactly."""
    rng = np.random.default_rng(16)
    pts = rng.standard_normal((4, 6))
    x = np.repeat(pts, 3, axis=0)[:, None, :]  # [12, 1, 6]
    cb = np.zeros((1, 1, 2, 4, 6))
    cb[0, 0, 0] = pts
    cb[0, 0, 1] = rng.standard_normal((4, 6))
    new, mass = O.em_step(x, cb, 1, 0.0)
    used = mass[0, 0] > 0
    assert used.any() and np.allclose(new[0, 0][used], 0.0, atol=1e-15)
    cb[0, 0, 1] = new[0, 0]
    assert O.reconstruction_error(x, cb) < 1e-30


# ---------------------------------------------------------------- binary value codes

def test_unpack_bits_hand_built_record():
    # bytes 0b00000101, 0b10000000: bits 0 and 2 of byte 0, bit 7 of byte 1 -> indices 0, 2, 15
    bits = O.unpack_bits(np.array([[0b00000101, 0b10000000]], dtype=np.uint8), 16)
    assert list(np.flatnonzero(bits[0])) == [0, 2, 15]
    rng = np.random.default_rng(20)
    raw = rng.integers(0, 256, size=(5, 32), dtype=np.uint8)
    assert np.array_equal(O.unpack_bits(raw, 256), np.unpackbits(raw, axis=-1, bitorder="little"))  # library routine


def test_binary_values_special_cases():
    rng = np.random.default_rng(21)
    C = rng.standard_normal((64, 12))
    one = np.zeros((1, 8), dtype=np.uint8)
    one[0, 37 // 8] = 1 << (37 % 8)
    assert np.array_equal(O.binary_values(one, C)[0], C[37])            # one bit: that row
    ones = np.full((1, 8), 255, dtype=np.uint8)
    assert np.allclose(O.binary_values(ones, C)[0], C.sum(axis=0), atol=1e-12)  # every bit: the column sums
    assert np.array_equal(O.binary_values(np.zeros((1, 8), dtype=np.uint8), C)[0], np.zeros(12))


def test_bit_values_reordered_equals_dense():
    """(sum_m w_m s_m)^T C = sum_m w_m (s_m^T C): the reordering the decode
    kernel relies on."""
    rng = np.random.default_rng(22)
    C = rng.standard_normal((256, 40))
    packed = rng.integers(0, 256, size=(300, 32), dtype=np.uint8)
    w = rng.random(300)
    dense = w @ O.binary_values(packed, C)
    assert np.allclose(O.bit_values_reordered(w, packed, C), dense, rtol=1e-12, atol=1e-10)


def test_bit_value_attention_matches_torch_sdpa():
    rng = np.random.default_rng(23)
    B, Hq, Hkv, D, g, Nc, R, L, Nb = 1, 4, 2, 16, 4, 8, 2, 40, 64
    kcb = rng.standard_normal((Hkv, D // g, R, Nc, g))
    kc = rng.integers(0, Nc, size=(L, Hkv, R, D // g))
    kp = O.pack_codes(kc, Nc).transpose(1, 0, 2)[None]
    vb = rng.integers(0, 256, size=(B, L, Nb // 8), dtype=np.uint8)
    C = rng.standard_normal((Nb, Hkv * D))
    q = rng.standard_normal((B, Hq, D))
    got = O.decode_attention_bit_values(q, [L - 1], kp, vb, [L], kcb, C, 10000.0)
    th = O.rope_thetas(D, 10000.0)
    kr = O.apply_rope(O.dequantize(kc, kcb).transpose(1, 0, 2), np.arange(L), th)  # [Hkv, L, D]
    vv = (np.unpackbits(vb[0], axis=-1, bitorder="little").astype(np.float64) @ C).reshape(L, Hkv, D).transpose(1, 0, 2)
    qr = O.apply_rope(q[0], np.full(Hq, L - 1), th)
    rep = Hq // Hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qr).reshape(Hq, 1, 1, D), torch.from_numpy(np.repeat(kr, rep, axis=0))[:, None],
        torch.from_numpy(np.repeat(vv, rep, axis=0))[:, None], scale=1 / math.sqrt(D)).reshape(Hq, D).numpy()
    assert np.allclose(got[0], ref, atol=1e-10)
