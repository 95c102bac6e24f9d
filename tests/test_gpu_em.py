"""GPU parity of one EM iteration of codebook fitting (commvq_em_step, through
the C ABI) against the oracle's em_step on the same seeded inputs.

Where floating point decides an integer (the greedy choice of earlier rounds,
the nearest entry of the fitted round at temperature 0), the GPU decides in
fp32 and the oracle in fp64. Every vector stays in the input; a decision whose
relative top-2 gap on the oracle's distances is below 1e-4 is a near tie that
the GPU may take either way. Each such (vector, group) is logged, and its
alternatives (every combination of the two nearest entries at its near-tied
rounds) are followed in float64:
- temperature 0: the entries its alternatives can reach are "touched"; their
  mass may differ by the number of touching vectors and their value is not
  compared; every other entry meets the bars below;
- temperature > 0: the first-order change of every entry's weighted mean and
  mass under the worst alternative is added to that entry's bound.
Bars:
- masses: equal at temperature 0 (counts), within 1e-4 relative otherwise;
- updated entries: within half an fp16 ulp plus 1e-4 of the group's largest
  entry (fp32 sums, one rounding to fp16);
- entries at or below min_mass and every other round: bit-identical."""

import numpy as np
import pytest
import torch

from long_context_attention_commvq_amd import api, synth
from oracle import commvq_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TIE_REL = 1e-4


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def near_tie_alternatives(x, cb, r, temperature):
    """Near-tie decisions of the oracle (rounds < r, and round r at temperature
    0). Returns {(n, h, j): [residuals at round r, one per alternative]} for every
    (vector, group) with at least one such decision (the oracle's own path first),
    and for temperature 0 {(n, h, j): set of round-r entries the alternatives pick}."""
    _, gaps = O.encode(x, cb)  # [N, H, R, G]
    last = r + 1 if temperature == 0 else r
    alts, reach = {}, {}
    if last == 0:
        return alts, reach
    _, G, _, Nc, g = cb.shape
    cbd = cb.astype(np.float64)
    for n, h, j in np.argwhere((gaps[:, :, :last] < TIE_REL).any(axis=2)):
        paths = [x[n, h, j * g:(j + 1) * g].astype(np.float64)]
        for rr in range(r):
            d = [O.sq_distances(e, cbd[h, j, rr]) for e in paths]
            nxt = []
            for e, dd in zip(paths, d):
                order = np.argsort(dd, kind="stable")
                dmin = float(dd[order[0]])
                rel = (float(dd[order[1]]) - dmin) / max(dmin, 1e-12 * float(e @ e), 1e-300)
                nxt.append(e - cbd[h, j, rr, order[0]])
                if rel < TIE_REL:
                    nxt.append(e - cbd[h, j, rr, order[1]])
            paths = nxt
        key = (int(n), int(h), int(j))
        alts[key] = paths
        if temperature == 0:
            picks = set()
            for e in paths:
                dd = O.sq_distances(e, cbd[h, j, r])
                order = np.argsort(dd, kind="stable")
                picks.add(int(order[0]))
                dmin = float(dd[order[0]])
                if (float(dd[order[1]]) - dmin) / max(dmin, 1e-12 * float(e @ e), 1e-300) < TIE_REL:
                    picks.add(int(order[1]))
            reach[key] = picks
    return alts, reach


def tie_slack(alts, cb, r, temperature, ref, mass_r):
    """temperature > 0: per entry, the first-order change of its weighted mean
    (|dS - ref dM| / M, per scalar) and of its mass (|dM|) when a near-tie vector
    follows its worst alternative, summed over such vectors."""
    H, G, _, Nc, g = cb.shape
    dval = np.zeros((H, G, Nc, g))
    dmass = np.zeros((H, G, Nc))
    cbd = cb.astype(np.float64)
    for (n, h, j), paths in alts.items():
        ws = []
        for e in paths:
            d = O.sq_distances(e, cbd[h, j, r])
            w = np.exp(-(d - d.min()) / temperature)
            ws.append(w / w.sum())
        w0, e0 = ws[0], paths[0]
        worst_v = np.zeros((Nc, g))
        worst_m = np.zeros(Nc)
        for w, e in zip(ws[1:], paths[1:]):
            dS = w[:, None] * e[None, :] - w0[:, None] * e0[None, :]
            dM = w - w0
            worst_v = np.maximum(worst_v, np.abs(dS - ref[h, j] * dM[:, None]) / np.maximum(mass_r[h, j], 1e-30)[:, None])
            worst_m = np.maximum(worst_m, np.abs(dM))
        dval[h, j] += worst_v
        dmass[h, j] += worst_m
    return dval, dmass


def check_update(got, mass_g, ref, mass_r, cb_old, r, temperature, min_mass, ties=None):
    """got [H, G, R, Nc, g] fp16 entries after the GPU step; ref [H, G, Nc, g],
    mass_r [H, G, Nc] from the oracle; cb_old the entries before; ties the
    near-tie alternatives of near_tie_alternatives (None: there are none)."""
    got = got.astype(np.float64)
    old = cb_old.astype(np.float64)
    H, G, R, Nc, g = cb_old.shape
    for rr in range(R):
        if rr != r:
            assert np.array_equal(got[:, :, rr], old[:, :, rr])
    alts, reach = ties if ties is not None else ({}, {})
    touched = np.zeros((H, G, Nc), dtype=np.int64)
    for (n, h, j), picks in reach.items():
        for l in picks:
            touched[h, j, l] += 1
    if temperature == 0:
        assert np.all(np.abs(mass_g.astype(np.float64) - mass_r) <= touched)
        dval = np.zeros_like(ref)
    else:
        dval, dmass = tie_slack(alts, cb_old, r, temperature, ref, mass_r)
        assert np.all(np.abs(mass_g - mass_r) <= 1e-4 * np.abs(mass_r) + 1e-4 + dmass)
    # kept entries (mass at or below the floor in both) are bit-identical
    kept = (mass_r <= min_mass) & (mass_g <= min_mass) & (touched == 0)
    assert np.array_equal(got[:, :, r][kept], old[:, :, r][kept])
    upd = (mass_r > min_mass) & (touched == 0)
    g_r = got[:, :, r]
    scale = np.abs(ref).max(axis=(2, 3), keepdims=True)  # per (head, group)
    big = np.maximum(np.abs(ref), np.abs(g_r))
    bound = 0.5 * np.spacing(big.astype(np.float16)).astype(np.float64) + 1e-4 * scale + dval
    excess = (np.abs(g_r - ref) / bound)[upd]
    return float(excess.max()) if excess.size else 0.0


def log_ties(tag, ties):
    alts, reach = ties
    if alts:
        some = list(alts)[:4]
        print(f"[{tag}] {len(alts)} near-tie (vector, group) decisions followed both ways, e.g. {some}", flush=True)


@pytest.mark.parametrize("case", [
    dict(H=2, D=128, g=8, Nc=256, R=1, r=0, N=3000, T=0.0),
    dict(H=2, D=128, g=8, Nc=256, R=2, r=1, N=2000, T=0.0),
    dict(H=1, D=64, g=4, Nc=16, R=3, r=2, N=1000, T=0.0, min_mass=20.0),
    dict(H=3, D=48, g=6, Nc=8, R=1, r=0, N=517, T=0.0),        # ragged last tile of 256 vectors
    dict(H=1, D=64, g=16, Nc=64, R=2, r=1, N=700, T=0.0),
    dict(H=2, D=128, g=8, Nc=256, R=1, r=0, N=3000, T=0.5),
    dict(H=1, D=64, g=4, Nc=16, R=2, r=1, N=1000, T=2.0),
    dict(H=1, D=32, g=2, Nc=4, R=1, r=0, N=300, T=100.0),
    dict(H=1, D=128, g=8, Nc=256, R=4, r=3, N=600, T=0.0),      # four rounds of fp32 codebook in LDS
])
def test_em_step_matches_oracle(case):
    H, D, g, Nc, R, r, N, T = (case[k] for k in ("H", "D", "g", "Nc", "R", "r", "N", "T"))
    min_mass = case.get("min_mass", 0.0)
    seed = 4000 + 17 * D + 5 * g + Nc + 3 * R + r + int(T * 10)
    x = synth.kv(seed, N, H, D)
    cb = synth.codebook(seed + 1, H, D, g, Nc, R)
    ties = near_tie_alternatives(x, cb, r, T)
    log_ties(f"em {case}", ties)
    ref, mass_r = O.em_step(x, cb, r, T, min_mass)
    q = api.Quantizer(dev(cb), g)
    out = dev(cb)  # updated out of place; every other round must stay as it was
    new, mass = api.em_step(q, dev(x), r, T, min_mass, new_entries=out, with_mass=True)
    torch.cuda.synchronize()
    worst = check_update(new.cpu().numpy(), mass.cpu().numpy(), ref, mass_r, cb, r, T, min_mass, ties)
    print(f"[em {case}] {x.shape[0]} vectors, max entry error / bound {worst:.3f}", flush=True)
    assert worst <= 1.0
    # in place (the codebook the quantizer holds): the same bar (the fp32 atomics
    # may add in another order, so the bytes need not repeat)
    _, mass2 = api.em_step(q, dev(x), r, T, min_mass, with_mass=True)
    torch.cuda.synchronize()
    assert check_update(q.entries.cpu().numpy(), mass2.cpu().numpy(), ref, mass_r, cb, r, T, min_mass, ties) <= 1.0


def test_em_annealed_iterations_track_the_oracle():
    """Three iterations with a falling temperature, then two hard ones, each
    GPU iteration starting from the GPU's previous codebook and the oracle's
    from the same fp16 entries: every iteration meets the bar."""
    H, D, g, Nc, R = 1, 64, 8, 32, 1
    x = synth.kv(4500, 2000, H, D)
    cb = synth.codebook(4501, H, D, g, Nc, R)
    q = api.Quantizer(dev(cb), g)
    xd = dev(x)
    for it, T in enumerate([4.0, 1.0, 0.25, 0.0, 0.0]):
        start = q.entries.cpu().numpy()
        xs = x
        ties = near_tie_alternatives(xs, start, 0, T)
        log_ties(f"em anneal {it}", ties)
        ref, mass_r = O.em_step(xs, start, 0, T)
        new, mass = api.em_step(q, xd, 0, T, with_mass=True)
        torch.cuda.synchronize()
        worst = check_update(new.cpu().numpy(), mass.cpu().numpy(), ref, mass_r, start, 0, T, 0.0, ties)
        print(f"[em anneal] iteration {it} T={T}: {xs.shape[0]} vectors, max error / bound {worst:.3f}", flush=True)
        assert worst <= 1.0


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_em_full_size_128k_sampled(T):
    """The prefill workload's key tensor (131072 tokens x 8 KV heads, g = 8,
    Nc' = 256), round 0, in one call over every head and group; the oracle
    recomputes three sampled (head, group) slices over all 131072 vectors. At
    temperature 0 the few vectors with near-tie decisions may go either way:
    the entries they touch are checked with their count allowed for."""
    w = synth.WORKLOADS["llama8b_encode128k_b4_2bit"]
    N, H, D, g, Nc = w.context, w.n_kv_heads, w.head_dim, w.group_size, w.n_entries
    x = synth.kv(w.seed + 10, N, H, D, heavy_tail=True)
    cb = synth.codebook(w.seed + 1, H, D, g, Nc, 1)
    q = api.Quantizer(dev(cb), g)
    print(f"[em full size T={T}] N={N} H={H}", flush=True)
    out = dev(cb)
    new, mass = api.em_step(q, dev(x), 0, T, new_entries=out, with_mass=True)
    torch.cuda.synchronize()
    got = new.cpu().numpy().astype(np.float64)
    mass_g = mass.cpu().numpy()
    rng = np.random.default_rng(4600)
    for h, j in [(0, 0), (int(rng.integers(0, H)), int(rng.integers(0, D // g))), (H - 1, D // g - 1)]:
        xs = x[:, h:h + 1, j * g:(j + 1) * g]
        cs = cb[h:h + 1, j:j + 1]
        ref, mass_r = O.em_step(xs, cs, 0, T)
        ref, mass_r = ref[0, 0], mass_r[0, 0]
        gr, mg = got[h, j, 0], mass_g[h, j]
        scale = np.abs(ref).max()
        bound = 0.5 * np.spacing(np.maximum(np.abs(ref), np.abs(gr)).astype(np.float16)).astype(np.float64) + 1e-4 * scale
        if T == 0:
            _, gaps = O.encode(xs, cs)
            d = O.sq_distances(xs.reshape(N, 1, 1, g).astype(np.float64), cs[:, :, 0][None].astype(np.float64))
            ties = np.flatnonzero(gaps[:, 0, 0, 0] < TIE_REL)
            touched = np.zeros(Nc, dtype=np.int64)
            for n in ties:  # the two nearest entries of a near-tie vector may each gain or lose it
                top2 = np.argsort(d[n, 0, 0])[:2]
                touched[top2] += 1
            assert np.all(np.abs(mg - mass_r) <= touched), (h, j)
            clean = (touched == 0) & (mass_r > 0)
            err = (np.abs(gr - ref) / bound)[clean]
            print(f"[em full size T=0] head {h} group {j}: {len(ties)} near-tie vectors, "
                  f"max error / bound over {clean.sum()} untouched entries {err.max():.3f}", flush=True)
            assert err.max() <= 1.0
        else:
            assert np.allclose(mg, mass_r, rtol=1e-4, atol=1e-3)
            err = np.abs(gr - ref) / bound
            print(f"[em full size T={T}] head {h} group {j}: max error / bound {err.max():.3f}", flush=True)
            assert err.max() <= 1.0
