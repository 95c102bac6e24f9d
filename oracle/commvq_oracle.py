"""CommVQ reference oracle: plain, slow, float64 NumPy.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it. It shares no code, constants or helpers with the HIP
library under ``long_context_attention_commvq_amd/``.

Sources (the pages this implements):
  * "CommVQ: Commutative Vector Quantization for KV Cache Compression" abstract
    (catalyzex / chatpaper / vectordb.ever.works pages): additive quantization of
    each K/V vector, decoded by summing codebook vectors; RoPE-commutative
    codebook.
  * pith.science review of arXiv 2506.18879 ("Pith review of CommVQ"):
      - "What carries the argument": RoPE as block-diagonal 2x2 rotations
        R_m^i on 2-D sub-vectors; codebook blocks C = [[x, y], [-y, x]] that
        commute with R_m^i (paper Eq. 7); index sharing over a group of size g;
        R residual rounds; average bit rate R*log2(Nc')/g (paper Eq. 21);
        query-dependent and codebook-dependent factors computed once and reused
        over all cached positions.
      - "Editorial extensions / If this is right", fourth bullet: softmax weights
        multiply the quantized value codes before the codebook multiply.
      - "Assumptions & free parameters": RoPE is block-diagonal 2x2 rotations
        (Eqns 5-6); matrices [[x, y], [-y, x]] commute with every 2-D rotation
        (Eqn 8, Property 1); R = residual rounds, g = group size, Nc' = entries;
        the codebook is fitted by alternating assignment and update (k-means
        style) with soft assignment and annealing ("Referee Report",
        Significance: the update has a closed form).

Readings taken where the pages are silent or ambiguous (each listed in the
repository's design notes):
  * g counts scalars (g = 8 -> four complex pairs per shared index).
  * A codebook entry's pair (x, y) reconstructs the 2-vector (x, y), i.e. the
    complex number x + iy; rotating it by angle phi is multiplication by e^{i phi}.
  * RoPE pairs are interleaved channels (2p, 2p+1); R(phi) = [[cos, -sin], [sin, cos]];
    theta_p = base^(-2p/D); no frequency scaling.
  * The residual search is greedy: per round, the nearest entry in squared
    Euclidean distance, lowest index on exact ties.
  * Packed record per (token, head): R*G fields of log2(Nc') bits, round-major
    (round outer, group inner), LSB-first, padded to whole bytes.
  * The query arrives un-rotated and sits at position q_pos = L - 1; attention
    covers cached positions [0, L); scale 1/sqrt(D) by default.
  * Values use the same greedy residual codebook as keys, without RoPE.
  * Codebook fitting: round r is fitted on the residuals of the earlier rounds;
    soft assignment = softmax of -distance / temperature, temperature 0 = the
    nearest entry; the update is the responsibility-weighted mean.

Array conventions:
  codebook  [Hkv, G, R, Nc, g]   float (fp16 values are used exactly as float64)
  x (K/V)   [N, Hkv, D]
  codes     [N, Hkv, R, G]       int64
  packed    [N, Hkv, nbytes]     uint8
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Storage cost (review page, "What carries the argument": bit rate, paper Eq. 21)
# ---------------------------------------------------------------------------


def field_bits(n_entries: int) -> int:
    """Bits of one code field: log2(Nc'); Nc' must be a power of two."""
    if n_entries < 1 or (n_entries & (n_entries - 1)) != 0:
        raise ValueError("n_entries must be a power of two >= 1")
    return n_entries.bit_length() - 1


def bits_per_scalar(group_size: int, n_entries: int, n_rounds: int) -> float:
    """Average stored bits per scalar, R * log2(Nc') / g (paper Eq. 21, quoted in
    the review's "What carries the argument"; the circularity check calls it a
    definition of storage cost)."""
    return n_rounds * math.log2(n_entries) / group_size


def code_bytes_per_token(head_dim: int, group_size: int, n_entries: int, n_rounds: int) -> int:
    """Bytes of one packed (token, KV head) record: R*(D/g) fields, padded to bytes."""
    if head_dim % group_size:
        raise ValueError("group_size must divide head_dim")
    nbits = n_rounds * (head_dim // group_size) * field_bits(n_entries)
    return (nbits + 7) // 8


def fp16_kv_cache_bytes(batch: int, tokens: int, layers: int, kv_dim: int) -> int:
    """Uncompressed FP16 KV cache size: K and V, 2 bytes per scalar. This is the
    arithmetic the review's referee report (major comment 2) uses for the FP16
    baseline of LLaMA-3.1-8B (32 layers, KV dimension 1024)."""
    return 2 * batch * tokens * layers * kv_dim * 2


# ---------------------------------------------------------------------------
# RoPE and the commutative block (review: "What carries the argument"; Eqns 5-8)
# ---------------------------------------------------------------------------


def rope_thetas(head_dim: int, base: float) -> np.ndarray:
    """Per-pair angular frequency theta_p = base^(-2p/D), p = 0..D/2-1."""
    p = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * p / head_dim)


def rotation_matrix(angle: float) -> np.ndarray:
    """The 2x2 RoPE block R = [[cos a, -sin a], [sin a, cos a]] (Eqns 5-6)."""
    c, s = math.cos(angle), math.sin(angle)
    return np.array([[c, -s], [s, c]], dtype=np.float64)


def commutative_block(x: float, y: float) -> np.ndarray:
    """A codebook block in the RoPE-commutative form [[x, y], [-y, x]] (Eq. 7)."""
    return np.array([[x, y], [-y, x]], dtype=np.float64)


def apply_rope(x: np.ndarray, positions: np.ndarray, thetas: np.ndarray) -> np.ndarray:
    """Rotate each interleaved pair (x[2p], x[2p+1]) of the last axis by
    positions * theta_p with the 2x2 rotation written out explicitly.

    x: [..., T, D]; positions: [T] (broadcast against x's token axis)."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.float64)
    ang = pos[:, None] * thetas[None, :]  # [T, D/2]
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


# ---------------------------------------------------------------------------
# Encoder: greedy residual nearest-codeword search (review: "What carries the
# argument": shared index per group, R residual rounds; "free parameters":
# R = number of iterative clustering passes on residuals)
# ---------------------------------------------------------------------------


def sq_distances(e: np.ndarray, entries: np.ndarray) -> np.ndarray:
    """Squared Euclidean distance from residual vectors to every entry.

    e: [..., g]; entries: [..., Nc, g] (same leading dims) -> [..., Nc].
    Written as the plain sum of squared differences."""
    diff = e[..., None, :] - entries
    return np.sum(diff * diff, axis=-1)


def encode(x: np.ndarray, codebook: np.ndarray, chunk: int = 256):
    """Greedy residual encoding of every (token, head, group).

    Returns (codes [N, H, R, G] int64, gaps [N, H, R, G] float64) where gap is the
    relative distance margin (d_second - d_best) / max(d_best, 1e-12*|e|^2) of the
    round's decision (diagnostic for near-ties)."""
    x = np.asarray(x, dtype=np.float64)
    cb = np.asarray(codebook, dtype=np.float64)
    N, H, D = x.shape
    Hc, G, R, Nc, g = cb.shape
    if Hc != H or G * g != D:
        raise ValueError("codebook shape does not match x")
    codes = np.zeros((N, H, R, G), dtype=np.int64)
    gaps = np.full((N, H, R, G), np.inf, dtype=np.float64)
    for t0 in range(0, N, chunk):
        t1 = min(N, t0 + chunk)
        e = x[t0:t1].reshape(t1 - t0, H, G, g).copy()  # residual [n, H, G, g]
        for r in range(R):
            entries = cb[:, :, r]  # [H, G, Nc, g]
            d = sq_distances(e, entries[None])  # [n, H, G, Nc]
            best = np.argmin(d, axis=-1)  # first index on exact ties
            codes[t0:t1, :, r, :] = best
            if Nc > 1:
                part = np.partition(d, 1, axis=-1)
                d1, d2 = part[..., 0], part[..., 1]
                norm2 = np.sum(e * e, axis=-1)
                gaps[t0:t1, :, r, :] = (d2 - d1) / np.maximum(np.maximum(d1, 1e-12 * norm2), 1e-300)
            chosen = np.take_along_axis(entries[None], best[..., None, None], axis=-2)[..., 0, :]
            e = e - chosen
    return codes, gaps


# ---------------------------------------------------------------------------
# Bit packing (reading: fields round-major, LSB-first, padded to bytes)
# ---------------------------------------------------------------------------


def pack_codes(codes: np.ndarray, n_entries: int) -> np.ndarray:
    """codes [..., R, G] -> bytes [..., nbytes]; field f = r*G + j occupies bits
    [f*b, f*b + b) of the record, bit i of the field at record bit f*b + i,
    record bit P stored in byte P // 8 at bit P % 8."""
    b = field_bits(n_entries)
    codes = np.asarray(codes, dtype=np.int64)
    lead = codes.shape[:-2]
    R, G = codes.shape[-2:]
    flat = codes.reshape(-1, R * G)
    nbytes = (R * G * b + 7) // 8
    out = np.zeros((flat.shape[0], nbytes), dtype=np.uint8)
    for f in range(R * G):
        for i in range(b):
            P = f * b + i
            bit = (flat[:, f] >> i) & 1
            out[:, P // 8] |= (bit << (P % 8)).astype(np.uint8)
    return out.reshape(lead + (nbytes,))


def unpack_codes(packed: np.ndarray, n_rounds: int, n_groups: int, n_entries: int) -> np.ndarray:
    """Inverse of pack_codes: bytes [..., nbytes] -> codes [..., R, G]."""
    b = field_bits(n_entries)
    packed = np.asarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    flat = packed.reshape(int(np.prod(lead, dtype=np.int64)), packed.shape[-1]).astype(np.int64)
    nf = n_rounds * n_groups
    out = np.zeros((flat.shape[0], nf), dtype=np.int64)
    for f in range(nf):
        for i in range(b):
            P = f * b + i
            out[:, f] |= ((flat[:, P // 8] >> (P % 8)) & 1) << i
    return out.reshape(lead + (n_rounds, n_groups))


# ---------------------------------------------------------------------------
# Decoder: additive reconstruction (abstract: decoded as a sum of codebook vectors)
# ---------------------------------------------------------------------------


def dequantize(codes: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """x_hat[n, h, g*j:g*j+g] = sum_r codebook[h, j, r, codes[n, h, r, j]]."""
    cb = np.asarray(codebook, dtype=np.float64)
    H, G, R, Nc, g = cb.shape
    codes = np.asarray(codes, dtype=np.int64)
    N = codes.shape[0]
    out = np.zeros((N, H, G, g), dtype=np.float64)
    hh = np.arange(H)[None, :, None]
    jj = np.arange(G)[None, None, :]
    for r in range(R):
        out += cb[hh, jj, r, codes[:, :, r, :]]
    return out.reshape(N, H, G * g)


# ---------------------------------------------------------------------------
# Attention: dense softmax over explicitly rotated, fully dequantised K/V
# ---------------------------------------------------------------------------


def attend_one(q_rot: np.ndarray, k_rot: np.ndarray, v: np.ndarray, sm_scale: float) -> np.ndarray:
    """Dense single-query softmax attention. q_rot [D], k_rot [L, D], v [L, D]."""
    s = (k_rot @ q_rot) * sm_scale
    s = s - np.max(s)
    w = np.exp(s)
    w = w / np.sum(w)
    return w @ v


def decode_attention(q, q_pos, k_hat, v_hat, seq_lens, thetas, sm_scale):
    """Decode-step attention for B sequences with grouped-query heads.

    q [B, Hq, D] (not rotated), q_pos [B], k_hat/v_hat [B, Hkv, Lmax, D]
    (dequantised, not rotated), seq_lens [B]. Query head hq reads KV head
    hq // (Hq // Hkv). Returns [B, Hq, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_hat.shape[1]
    rep = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue  # nothing to attend: the row stays zero
        pos = np.arange(L)
        qr = apply_rope(q[b], np.full(Hq, int(q_pos[b])), thetas)  # one position per row
        for h in range(Hkv):
            kr = apply_rope(np.asarray(k_hat[b, h, :L], dtype=np.float64), pos, thetas)
            vv = np.asarray(v_hat[b, h, :L], dtype=np.float64)
            for a in range(rep):
                hq = h * rep + a
                out[b, hq] = attend_one(qr[hq], kr, vv, sm_scale)
    return out


def decode_attention_from_packed(q, q_pos, kpacked, vpacked, seq_lens, kcb, vcb, theta_base,
                                 sm_scale=None):
    """Full oracle path: unpack -> dequantise -> explicit RoPE -> dense softmax.

    kpacked/vpacked [B, Hkv, Lmax, nbytes] uint8; kcb/vcb [Hkv, G, R, Nc, g].
    Works per (b, KV head) so memory stays bounded at long context."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, G, R, Nc, g = kcb.shape
    Rv, Ncv = vcb.shape[2], vcb.shape[3]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    thetas = rope_thetas(D, theta_base)
    rep = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue  # nothing to attend: the row stays zero
        pos = np.arange(L)
        qr = apply_rope(q[b], np.full(Hq, int(q_pos[b])), thetas)
        for h in range(Hkv):
            kc = unpack_codes(kpacked[b, h, :L], R, G, Nc)[:, None]  # [L, 1, R, G]
            vc = unpack_codes(vpacked[b, h, :L], Rv, G, Ncv)[:, None]
            kh = dequantize(kc, kcb[h:h + 1])[:, 0]
            vh = dequantize(vc, vcb[h:h + 1])[:, 0]
            kr = apply_rope(kh, pos, thetas)
            for a in range(rep):
                hq = h * rep + a
                out[b, hq] = attend_one(qr[hq], kr, vh, sm_scale)
    return out


# ---------------------------------------------------------------------------
# Reordered forms the pages describe (used to pin the algebra the fast path
# relies on; the dense path above stays the oracle's answer)
# ---------------------------------------------------------------------------


def scores_table_form(q, q_pos, codes, codebook, thetas, sm_scale):
    """Score of one query against coded keys via a query x codebook table
    (review: "What carries the argument": because the blocks commute with R_m,
    query- and codebook-dependent factors are computed once and reused).

    T[j, r, l, p] = conj(q~_p) * z[j, r, l, p], with q~ the query rotated to q_pos
    and z = x + iy the entry's pairs; score_m = scale * sum_{j, r, p}
    Re(T[j, r, code[m, r, j], p] * exp(i m theta_p)).

    q [D]; codes [L, R, G] (one KV head); codebook [G, R, Nc, g]."""
    q = np.asarray(q, dtype=np.float64)
    D = q.shape[0]
    G, R, Nc, g = codebook.shape
    P = g // 2
    qr = apply_rope(q[None], np.array([q_pos]), thetas)[0]
    qz = qr[0::2] + 1j * qr[1::2]  # [D/2]
    cbz = codebook[..., 0::2] + 1j * codebook[..., 1::2]  # [G, R, Nc, P]
    T = np.conj(qz.reshape(G, 1, 1, P)) * cbz  # [G, R, Nc, P]
    L = codes.shape[0]
    m = np.arange(L, dtype=np.float64)
    phase = np.exp(1j * m[:, None] * thetas[None, :]).reshape(L, G, P)  # [L, G, P]
    s = np.zeros(L, dtype=np.float64)
    for j in range(G):
        for r in range(R):
            s += np.sum(np.real(T[j, r, codes[:, r, j], :] * phase[:, j, :]), axis=-1)
    return s * sm_scale


def values_histogram_form(weights, codes, codebook):
    """Value read-out with the weights applied to the codes before the codebook
    (review: "If this is right", fourth bullet): H[j, r, l] = sum_m w_m [code = l],
    out[g*j:g*j+g] = sum_{r, l} H[j, r, l] * codebook[j, r, l].

    weights [L]; codes [L, R, G]; codebook [G, R, Nc, g] -> [G*g]."""
    G, R, Nc, g = codebook.shape
    out = np.zeros((G, g), dtype=np.float64)
    for j in range(G):
        for r in range(R):
            H = np.bincount(codes[:, r, j], weights=weights, minlength=Nc)
            out[j] += H @ codebook[j, r]
    return out.reshape(G * g)


# ---------------------------------------------------------------------------
# Codebook fitting: one EM iteration for one residual round. The abstract says
# the codebook is trained with an Expectation-Maximization algorithm; the review
# ("Assumptions & free parameters") describes it as alternating assignment and
# update in the manner of k-means, stabilised by soft assignment and annealing,
# and ("Referee Report", Significance) notes that the update has a closed form.
# Reading taken: round r is fitted on the residuals the earlier rounds leave
# (greedy, as `encode`); the objective is the squared reconstruction error of
# each group; the annealed soft assignment is a softmax over -distance /
# temperature, and temperature 0 is the hard (nearest-entry) assignment.
# ---------------------------------------------------------------------------


def em_round_residuals(x: np.ndarray, codebook: np.ndarray, round_index: int) -> np.ndarray:
    """Residuals [N, H, G, g] that round `round_index` is fitted on: each group
    reduced greedily by the nearest entry of every earlier round."""
    x = np.asarray(x, dtype=np.float64)
    cb = np.asarray(codebook, dtype=np.float64)
    N, H, D = x.shape
    _, G, R, Nc, g = cb.shape
    e = x.reshape(N, H, G, g).copy()
    for r in range(round_index):
        entries = cb[:, :, r]  # [H, G, Nc, g]
        best = np.argmin(sq_distances(e, entries[None]), axis=-1)  # [N, H, G], first index on ties
        e = e - np.take_along_axis(entries[None], best[..., None, None], axis=-2)[..., 0, :]
    return e


def em_step(x: np.ndarray, codebook: np.ndarray, round_index: int, temperature: float, min_mass: float = 0.0):
    """One EM iteration for round `round_index` of `codebook` [H, G, R, Nc, g].

    E-step: for each residual e (see em_round_residuals) and the round's entries
    c_l, d_l = |e - c_l|^2; responsibilities w_l = exp(-(d_l - min d) / T) / sum
    for T > 0, one-hot on the nearest entry (lowest index on ties) for T = 0.
    M-step: c_l = sum_n w_nl e_n / sum_n w_nl, the minimiser of
    sum_n w_nl |e_n - c_l|^2; an entry whose mass sum_n w_nl is not above
    min_mass keeps its value.
    Returns (entries of the round [H, G, Nc, g], mass [H, G, Nc]), float64."""
    cb = np.asarray(codebook, dtype=np.float64)
    e = em_round_residuals(x, cb, round_index)  # [N, H, G, g]
    entries = cb[:, :, round_index]  # [H, G, Nc, g]
    d = sq_distances(e, entries[None])  # [N, H, G, Nc]
    if temperature > 0:
        w = np.exp(-(d - d.min(axis=-1, keepdims=True)) / temperature)
        w = w / w.sum(axis=-1, keepdims=True)
    else:
        w = np.zeros_like(d)
        np.put_along_axis(w, np.argmin(d, axis=-1)[..., None], 1.0, axis=-1)
    mass = w.sum(axis=0)  # [H, G, Nc]
    sums = np.einsum("nhgl,nhgi->hgli", w, e)  # [H, G, Nc, g]
    new = entries.copy()
    upd = mass > min_mass
    new[upd] = sums[upd] / mass[upd][:, None]
    return new, mass


def reconstruction_error(x: np.ndarray, codebook: np.ndarray) -> float:
    """Mean squared error of the greedy residual encoding: sum over rounds of the
    chosen entries against x, averaged over every scalar."""
    x = np.asarray(x, dtype=np.float64)
    cb = np.asarray(codebook, dtype=np.float64)
    codes, _ = encode(x, cb)
    xh = dequantize(codes, cb)
    return float(np.mean((x - xh) ** 2))


# ---------------------------------------------------------------------------
# The paper's value coder (review, "Assumptions & free parameters": Nc value
# codebook rows, 1024 for 1 bit and 2048 for 2 bits, average bit width Nc/d;
# "Referee Report", minor comment 4: values use binary codes s in {0,1}^Nc,
# keys the index-sharing code). Reading taken: a token's whole value vector
# (all KV heads, d = Hkv * D scalars) is one Nc-bit code s, decoded as
# s^T C = the sum of the codebook rows whose bits are set; bits are stored
# LSB-first, Nc/8 bytes per token.
# ---------------------------------------------------------------------------


def unpack_bits(packed: np.ndarray, n_bits: int) -> np.ndarray:
    """bytes [..., n_bits/8] -> {0, 1} [..., n_bits]; bit i is bit i % 8 of byte i // 8."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.zeros(packed.shape[:-1] + (n_bits,), dtype=np.int64)
    for i in range(n_bits):
        out[..., i] = (packed[..., i // 8] >> (i % 8)) & 1
    return out


def binary_values(packed: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Decoded values s^T C: packed bits [..., Nc/8], rows C [Nc, d] -> [..., d] float64."""
    C = np.asarray(rows, dtype=np.float64)
    s = unpack_bits(packed, C.shape[0]).astype(np.float64)
    return s @ C


def decode_attention_bit_values(q, q_pos, kpacked, vbits, seq_lens, kcb, rows, theta_base, sm_scale=None):
    """Dense oracle with keys from the residual commutative codebook (as
    decode_attention_from_packed) and values from binary codes: vbits
    [B, Lmax, Nc/8] uint8, rows [Nc, Hkv * D]. Query head hq reads KV head
    hq // (Hq // Hkv) and its value slice [h D, (h + 1) D)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, G, R, Nc, g = kcb.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    thetas = rope_thetas(D, theta_base)
    rep = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        pos = np.arange(L)
        qr = apply_rope(q[b], np.full(Hq, int(q_pos[b])), thetas)
        vv = binary_values(vbits[b, :L], rows)  # [L, Hkv * D]
        for h in range(Hkv):
            kc = unpack_codes(kpacked[b, h, :L], R, G, Nc)[:, None]
            kr = apply_rope(dequantize(kc, kcb[h:h + 1])[:, 0], pos, thetas)
            for a in range(rep):
                hq = h * rep + a
                out[b, hq] = attend_one(qr[hq], kr, vv[:, h * D:(h + 1) * D], sm_scale)
    return out


def bit_values_reordered(weights: np.ndarray, packed: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """The reordered value path (review, "If this is right", fourth bullet): the
    weighted sum of the binary codes first, u = sum_m w_m s_m, then one product
    u^T C. weights [L], packed [L, Nc/8], rows [Nc, d] -> [d]."""
    C = np.asarray(rows, dtype=np.float64)
    s = unpack_bits(packed, C.shape[0]).astype(np.float64)
    u = np.asarray(weights, dtype=np.float64) @ s
    return u @ C
