"""commvq_decode_step_noalloc (the decode step for callers that cannot
allocate: its partials live in a static per-GPU scratch array) against
commvq_decode_step with a caller workspace, through the C ABI: the same kernels
run, so outputs and appended records must be identical. Two calls in a row, the
second on a smaller input (the scratch keeps the first call's contents)."""

import math

import numpy as np
import pytest
import torch

from long_context_attention_commvq_amd import _lib, api, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def one_case(seed, B, Hq, Hkv, R, lens, Lmax):
    D, g, Nc = 128, 8, 256
    print(f"[noalloc] seed {seed} B={B} Hq={Hq} Hkv={Hkv} R={R} lens={lens} Lmax={Lmax}", flush=True)
    rng = np.random.default_rng(seed)
    kcb = synth.codebook(seed + 1, Hkv, D, g, Nc, R)
    vcb = synth.codebook(seed + 2, Hkv, D, g, Nc, R)
    kq, vq = api.Quantizer(dev(kcb), g), api.Quantizer(dev(vcb), g)
    bpt = kq.bytes_per_token
    kp = rng.integers(0, 256, size=(B, Hkv, Lmax, bpt), dtype=np.uint8)
    vp = rng.integers(0, 256, size=(B, Hkv, Lmax, bpt), dtype=np.uint8)
    kn = synth.kv(seed + 3, B, Hkv, D)
    vn = synth.kv(seed + 4, B, Hkv, D)
    q = synth.queries(seed + 5, B, Hq, D)
    lens = np.asarray(lens, dtype=np.int32)
    pos = lens - 1  # the new token is the last position of each sequence
    sm = 1.0 / math.sqrt(D)
    rope = _lib.make_rope(500000.0)
    outs, caches = [], []
    for noalloc in (False, True):
        kc, vc = dev(kp), dev(vp)
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        args = (kq.desc, vq.desc, rope, dev(kn), dev(vn), dev(pos), dev(q), dev(pos), kc, vc, dev(lens), B, Hq, Lmax,
                Lmax, sm, out)
        if noalloc:
            _lib.commvq_decode_step_noalloc(*args)
        else:
            ws = api.DecodeWorkspace(kq, vq, B, Hq, Lmax, DEV)
            _lib.commvq_decode_step(*args, ws.buf, ws.nbytes)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        caches.append((kc.cpu().numpy(), vc.cpu().numpy()))
    assert np.all(np.isfinite(outs[0]))
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(caches[0][0], caches[1][0]) and np.array_equal(caches[0][1], caches[1][1])
    # the step did append: the new records differ from the random bytes they replaced somewhere
    assert not np.array_equal(caches[0][0], kp)


def test_noalloc_step_matches_workspace_step_twice_then_smaller():
    one_case(8101, B=2, Hq=32, Hkv=8, R=1, lens=[8000, 5000], Lmax=8192)
    one_case(8102, B=1, Hq=8, Hkv=2, R=2, lens=[1500], Lmax=2048)


def test_noalloc_step_rejects_a_shape_beyond_its_scratch():
    D, g, Nc, R, Hkv = 128, 8, 256, 1, 8
    kcb = synth.codebook(1, Hkv, D, g, Nc, R)
    kq = api.Quantizer(dev(kcb), g)
    B, Hq, Lmax = 64, 32, 131072
    need = _lib.commvq_decode_workspace_bytes(B, Hq, Lmax, kq.desc, kq.desc)
    assert need > _lib.COMMVQ_NOALLOC_SCRATCH_BYTES
    z = torch.zeros(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(_lib.CommvqError) as e:
        _lib.commvq_decode_step_noalloc(kq.desc, kq.desc, _lib.make_rope(500000.0), z, z, z, z, z, z, z, z, B, Hq,
                                        Lmax, Lmax, 0.1, z)
    assert e.value.status == _lib.COMMVQ_ERR_WORKSPACE
