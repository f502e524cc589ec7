"""GPU parity of kvbank_window_advance (memory-key write path) against the
fp64 oracle: departing window rows re-rotated to temporal coordinate 0,
values copied, arriving rows written into the freed ring slots."""
import numpy as np
import pytest

from kvsynth import WORKLOADS, LayerGen, round_bf16
from oracle import rope as orope

import gpu_common as gc

pytestmark = pytest.mark.gpu


def _case(name, dtype, cap_frames, start, n_frames, t_first, with_new=True, seed=0):
    import torch
    import kv_cache_compression_head_amd as kb
    wl = WORKLOADS[name]
    gc.banner(f"window advance {name} {dtype} cap={cap_frames}F start={start} frames={n_frames} t0={t_first}")
    F, H, d = wl.F, wl.H, wl.d
    cap = cap_frames * F
    gen = LayerGen(wl, seed, 0)
    rnd = round_bf16 if dtype == "bf16" else (lambda x: x.astype(np.float32))
    kdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # ring rows: generator keys of successive frames, each at its window coordinate
    ring_k = np.zeros((H, cap, d), np.float32)
    ring_v = np.zeros((H, cap, d), np.float32)
    for j in range(cap_frames):
        slot = ((start + j * F) % cap)
        rows = (slot + np.arange(F)) % cap
        t = t_first + j
        for h in range(H):
            ring_k[h, rows] = rnd(gen._rotate(gen.prerope_keys(h, [j + 1]), [t]).reshape(F, d))
            ring_v[h, rows] = rnd(gen.values(h, [j + 1]))
    n = n_frames * F
    rng = np.random.default_rng(seed + 7)
    new_k = rnd(rng.normal(size=(H, n, d)).astype(np.float32)) if with_new else None
    new_v = rnd(rng.normal(size=(H, n, d)).astype(np.float32)) if with_new else None
    desc = kb.LayerDesc(H=H, d=d, M=1, dtype=kb.KVB_BF16 if dtype == "bf16" else kb.KVB_F32, frame_tokens=F,
                        labels=[0] * H)
    rk, rv = gc.dev(ring_k, kdt), gc.dev(ring_v, kdt)
    ck = torch.empty(H, n, d, dtype=kdt, device="cuda")
    cv = torch.empty(H, n, d, dtype=kdt, device="cuda")
    nk = gc.dev(new_k, kdt) if with_new else None
    nv = gc.dev(new_v, kdt) if with_new else None
    kb.kvbank_window_advance(desc, rk, rv, start, n, t_first, ck, cv, nk, nv)
    torch.cuda.synchronize()
    ref_k, ref_v, ref_rk, ref_rv = orope.window_advance(ring_k, ring_v, start, n, F, t_first, new_k, new_v)
    got_k = ck.float().cpu().numpy().astype(np.float64)
    # values, the arriving rows and every other ring slot: bit for bit
    np.testing.assert_array_equal(cv.float().cpu().numpy(), ref_v)
    np.testing.assert_array_equal(rk.float().cpu().numpy(), ref_rk)
    np.testing.assert_array_equal(rv.float().cpu().numpy(), ref_rv)
    # spatial pairs bit for bit; temporal pairs within one rounding of the exact value
    nt = orope.temporal_pairs(d)
    np.testing.assert_array_equal(got_k[..., 2 * nt:], ref_k[..., 2 * nt:])
    ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    err = np.abs(got_k[..., :2 * nt] - ref_k[..., :2 * nt])
    bound = ulp * np.abs(ref_k[..., :2 * nt]) + ulp * 1e-3 * np.abs(ref_k).max()
    assert np.all(err <= bound), (err.max(), np.argmax(err - bound))
    return got_k, ref_k, gen, wl


@pytest.mark.parametrize("name,dtype", [("tiny", "f32"), ("tiny", "bf16"), ("480p", "bf16")])
def test_window_advance_parity(name, dtype):
    # ring of 6 frames, the 3 oldest leave, the ring wraps inside the block
    _case(name, dtype, 6, 4 * WORKLOADS[name].F + 5, 3, 2)


def test_window_advance_turns_generator_keys_back_to_zero():
    """Departing keys written at coordinate t come back as the generator's
    own coordinate-0 keys, up to two bf16 roundings."""
    got, ref, gen, wl = _case("tiny", "bf16", 4, 0, 2, 3, with_new=False)
    F, d = wl.F, wl.d
    for h in range(wl.H):
        at0 = gen._rotate(gen.prerope_keys(h, [1, 2]), [0, 0]).reshape(2 * F, d)
        np.testing.assert_allclose(got[h], at0, rtol=2 ** -7, atol=2 ** -7 * np.abs(at0).max())


def test_window_advance_coordinate_zero_is_a_copy():
    """A frame already at coordinate 0 leaves the ring unchanged, bit for bit."""
    got, ref, _, _ = _case("tiny", "bf16", 3, 7, 1, 0)
    np.testing.assert_array_equal(got, ref)
