"""Planted mistakes in the oracle (CPU only): each mutant must make at least one
pin fail, which shows the pins can tell a wrong oracle from a right one."""

import numpy as np
import pytest

from oracle import commvq_oracle as O
from tests import test_oracle_pins as P


def _expect_fail(fn):
    with pytest.raises(AssertionError):
        fn()


def test_mutant_rope_sign(monkeypatch):
    def bad(x, positions, thetas):
        x = np.asarray(x, dtype=np.float64)
        ang = np.asarray(positions, dtype=np.float64)[:, None] * thetas[None, :]
        c, s = np.cos(ang), np.sin(ang)
        out = np.empty_like(x)
        out[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s
        out[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c
        return out
    monkeypatch.setattr(O, "apply_rope", bad)
    _expect_fail(P.test_rope_rotation_closed_form)


def test_mutant_theta_exponent(monkeypatch):
    monkeypatch.setattr(O, "rope_thetas", lambda D, base: np.power(float(base), -np.arange(D // 2) / D))
    _expect_fail(P.test_rope_thetas_closed_forms)


def test_mutant_bit_rate_formula(monkeypatch):
    monkeypatch.setattr(O, "bits_per_scalar", lambda g, n, R: R * n / g)
    _expect_fail(P.test_bit_rate_table9_printed_values)


def test_mutant_pack_group_major(monkeypatch):
    real = O.pack_codes

    def bad(codes, n_entries):
        codes = np.asarray(codes)
        return real(np.swapaxes(codes, -1, -2), n_entries)  # j outer, r inner
    monkeypatch.setattr(O, "pack_codes", bad)
    _expect_fail(P.test_pack_golden_records)


def test_mutant_pack_msb_first(monkeypatch):
    def bad(codes, n_entries):
        b = O.field_bits(n_entries)
        codes = np.asarray(codes, dtype=np.int64)
        R, G = codes.shape[-2:]
        flat = codes.reshape(-1, R * G)
        nbytes = (R * G * b + 7) // 8
        out = np.zeros((flat.shape[0], nbytes), dtype=np.uint8)
        for f in range(R * G):
            for i in range(b):
                P_ = f * b + i
                out[:, P_ // 8] |= (((flat[:, f] >> i) & 1) << (7 - P_ % 8)).astype(np.uint8)
        return out.reshape(codes.shape[:-2] + (nbytes,))
    monkeypatch.setattr(O, "pack_codes", bad)
    _expect_fail(P.test_pack_golden_records)


def test_mutant_l1_distance(monkeypatch):
    monkeypatch.setattr(O, "sq_distances", lambda e, entries: np.sum(np.abs(e[..., None, :] - entries), axis=-1))
    _expect_fail(lambda: P.test_encoder_r1_is_exact_nearest_neighbour(8, 16))


def test_mutant_dequant_drops_last_round(monkeypatch):
    real = O.dequantize

    def bad(codes, codebook):
        cb = np.asarray(codebook, dtype=np.float64).copy()
        cb[:, :, -1] = 0.0
        return real(codes, cb)
    monkeypatch.setattr(O, "dequantize", bad)
    _expect_fail(P.test_histogram_value_form_equals_dense_values)


def test_mutant_attention_scale_dropped(monkeypatch):
    real = O.attend_one
    monkeypatch.setattr(O, "attend_one", lambda q, k, v, s: real(q, k, v, 1.0))
    _expect_fail(P.test_attention_matches_torch_sdpa_with_gqa)


def test_mutant_attention_no_max_subtraction(monkeypatch):
    def bad(q_rot, k_rot, v, sm_scale):
        w = np.exp((k_rot @ q_rot) * sm_scale)
        return (w / np.sum(w)) @ v
    monkeypatch.setattr(O, "attend_one", bad)
    with np.errstate(all="ignore"):
        _expect_fail(P.test_attention_special_cases)


def test_mutant_gqa_head_mapping(monkeypatch):
    def bad(q, q_pos, k_hat, v_hat, seq_lens, thetas, sm_scale):
        q = np.asarray(q, dtype=np.float64)
        B, Hq, D = q.shape
        Hkv = k_hat.shape[1]
        out = np.zeros((B, Hq, D))
        for b in range(B):
            L = int(seq_lens[b])
            qr = O.apply_rope(q[b], np.full(Hq, int(q_pos[b])), thetas)
            for hq in range(Hq):
                h = hq % Hkv  # wrong mapping
                kr = O.apply_rope(k_hat[b, h, :L], np.arange(L), thetas)
                out[b, hq] = O.attend_one(qr[hq], kr, v_hat[b, h, :L], sm_scale)
        return out
    monkeypatch.setattr(O, "decode_attention", bad)
    _expect_fail(P.test_attention_matches_torch_sdpa_with_gqa)


def test_mutant_table_form_conjugate(monkeypatch):
    def bad(q, q_pos, codes, codebook, thetas, sm_scale):
        G, R, Nc, g = codebook.shape
        P_ = g // 2
        qr = O.apply_rope(np.asarray(q)[None], np.array([q_pos]), thetas)[0]
        qz = qr[0::2] + 1j * qr[1::2]
        cbz = codebook[..., 0::2] + 1j * codebook[..., 1::2]
        T = qz.reshape(G, 1, 1, P_) * cbz  # conjugate missing
        L = codes.shape[0]
        ph = np.exp(1j * np.arange(L)[:, None] * thetas[None, :]).reshape(L, G, P_)
        s = np.zeros(L)
        for j in range(G):
            for r in range(R):
                s += np.sum(np.real(T[j, r, codes[:, r, j], :] * ph[:, j, :]), axis=-1)
        return s * sm_scale
    monkeypatch.setattr(O, "scores_table_form", bad)
    _expect_fail(P.test_table_form_scores_equal_dense_scores)


def test_mutant_em_unnormalised_soft_weights(monkeypatch):
    def bad(x, codebook, round_index, temperature, min_mass=0.0):
        cb = np.asarray(codebook, dtype=np.float64)
        e = O.em_round_residuals(x, cb, round_index)
        entries = cb[:, :, round_index]
        d = O.sq_distances(e, entries[None])
        w = np.exp(-(d - d.min(axis=-1, keepdims=True)) / temperature) if temperature > 0 else \
            (d == d.min(axis=-1, keepdims=True)).astype(float)
        mass = w.sum(axis=0)
        new = np.einsum("nhgl,nhgi->hgli", w, e) / np.maximum(mass, 1e-300)[..., None]
        return new, mass  # weights not normalised per vector
    monkeypatch.setattr(O, "em_step", bad)
    _expect_fail(P.test_em_infinite_temperature_gives_the_mean_of_all_residuals)


def test_mutant_em_ignores_earlier_rounds(monkeypatch):
    real = O.em_round_residuals
    monkeypatch.setattr(O, "em_round_residuals", lambda x, cb, r: real(x, cb, 0))
    _expect_fail(P.test_em_later_round_fits_what_earlier_rounds_leave)


def test_mutant_em_update_is_not_the_mean(monkeypatch):
    real = O.em_step

    def bad(x, codebook, round_index, temperature, min_mass=0.0):
        new, mass = real(x, codebook, round_index, temperature, min_mass)
        return 0.5 * (new + np.asarray(codebook, dtype=np.float64)[:, :, round_index]), mass  # half step
    monkeypatch.setattr(O, "em_step", bad)
    _expect_fail(P.test_em_hard_step_equals_brute_force_lloyd_step)


def test_mutant_bits_msb_first(monkeypatch):
    def bad(packed, n_bits):
        packed = np.asarray(packed, dtype=np.uint8)
        out = np.zeros(packed.shape[:-1] + (n_bits,), dtype=np.int64)
        for i in range(n_bits):
            out[..., i] = (packed[..., i // 8] >> (7 - i % 8)) & 1
        return out
    monkeypatch.setattr(O, "unpack_bits", bad)
    _expect_fail(P.test_unpack_bits_hand_built_record)


def test_mutant_bit_values_wrong_head_slice(monkeypatch):
    real = O.binary_values
    monkeypatch.setattr(O, "binary_values", lambda packed, rows: real(packed, rows)[..., ::-1])  # columns reversed
    _expect_fail(P.test_bit_value_attention_matches_torch_sdpa)


def test_mutant_em_double_temperature(monkeypatch):
    real = O.em_step
    monkeypatch.setattr(O, "em_step", lambda x, cb, r, T, min_mass=0.0: real(x, cb, r, 2 * T, min_mass))
    _expect_fail(lambda: P.test_em_soft_step_equals_explicit_loops(0.3, 0))
    _expect_fail(lambda: P.test_em_soft_step_equals_explicit_loops(2.0, 1))


def test_mutant_em_soft_weights_without_min_shift_sign(monkeypatch):
    """exp(+(d - min d) / T): weights that grow with distance."""
    def bad(x, codebook, round_index, temperature, min_mass=0.0):
        cb = np.asarray(codebook, dtype=np.float64)
        e = O.em_round_residuals(x, cb, round_index)
        entries = cb[:, :, round_index]
        d = O.sq_distances(e, entries[None])
        w = np.exp((d - d.max(axis=-1, keepdims=True)) / temperature)
        w = w / w.sum(axis=-1, keepdims=True)
        mass = w.sum(axis=0)
        new = np.einsum("nhgl,nhgi->hgli", w, e) / mass[..., None]
        return new, mass
    monkeypatch.setattr(O, "em_step", bad)
    _expect_fail(lambda: P.test_em_soft_step_equals_explicit_loops(0.3, 0))


def test_mutant_encode_gap_absolute(monkeypatch):
    real = O.encode

    def bad(x, codebook, chunk=256):
        codes, gaps = real(x, codebook, chunk)
        return codes, gaps * 0.5  # a gap off by a factor (e.g. measured on distances, not squared)
    monkeypatch.setattr(O, "encode", bad)
    _expect_fail(P.test_encode_gaps_equal_brute_force_top2)
