"""GPU parity of forcing_head_profile (Forcing-KV offline head profiling,
section 3.2) against the fp64 oracle."""
import ctypes

import numpy as np
import pytest

from kvsynth import round_bf16
from oracle import forcing as of

import gpu_common as gc

pytestmark = pytest.mark.gpu


def _table(H, seg_cap, per_head):
    import torch
    import kv_cache_compression_head_amd as kb
    arr = (kb.kvb_segment * (H * seg_cap))()
    for h, segs in enumerate(per_head):
        for i, (kp, ln) in enumerate(segs):
            arr[h * seg_cap + i] = kb.kvb_segment(kp, 0, ln, 0)
    raw = np.frombuffer(bytes(arr), dtype=np.uint8).copy()
    return torch.from_numpy(raw).to("cuda"), torch.tensor([len(s) for s in per_head], dtype=torch.int32,
                                                             device="cuda")


@pytest.mark.parametrize("d,F,C,hist_frames,dtype", [(128, 96, 3, 4, "bf16"), (64, 40, 2, 3, "f32"),
                                                     (128, 1560, 3, 12, "bf16")])
def test_head_profile(d, F, C, hist_frames, dtype):
    """Heads whose chunk and transition keys are scaled up draw most of the
    mass there (static); the others spread it (dynamic).  Masses and scores
    against the oracle; labels equal except within 1e-3 of alpha."""
    import torch
    import kv_cache_compression_head_amd as kb
    gc.banner(f"head profile d={d} F={F} C={C} hist={hist_frames} {dtype}")
    H, Lq = 6, C * F
    rng = np.random.default_rng(d + F)
    rnd = round_bf16 if dtype == "bf16" else (lambda x: x.astype(np.float32))
    kdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    et = kb.KVB_BF16 if dtype == "bf16" else kb.KVB_F32
    Q = rnd(rng.normal(size=(H, Lq, d)).astype(np.float32))
    # regions: sink frame, other history (hist_frames - 1 frames), transition frame, chunk
    sizes = [(1, F), (0, (hist_frames - 1) * F), (2, F), (3, Lq)]
    keep, per_head, regions, Ks = [], [], [], []
    for h in range(H):
        boost = [0.3, 0.2, 3.0, 0.5, 0.15, 2.5][h]      # scale of the transition and chunk keys
        segs, reg, kk = [], [], []
        for r, n in sizes:
            k = rng.normal(size=(n, d)).astype(np.float32) * (boost if r in (2, 3) else 0.3)
            k = rnd(k)
            t = gc.dev(k, kdt)
            keep.append(t)
            segs.append((t.data_ptr(), n))
            reg.append(r)
            kk.append((k, r))
        per_head.append(segs)
        regions.append(reg)
        Ks.append(kk)
    seg_cap = 5
    segs_t, nseg_t = _table(H, seg_cap, per_head)
    reg_np = np.zeros((H, seg_cap), np.int32)
    for h in range(H):
        reg_np[h, :4] = regions[h]
    region = torch.from_numpy(reg_np).to("cuda")
    max_len = max(n for _, n in sizes)
    score = torch.empty(H, dtype=torch.float32, device="cuda")
    label = torch.empty(H, dtype=torch.uint8, device="cuda")
    mass = torch.empty(H, 4, dtype=torch.float32, device="cuda")
    kb.forcing_head_profile(H, d, Lq, et, gc.dev(Q, kdt), segs_t, nseg_t, seg_cap, region, max_len, score, label,
                            mass)
    torch.cuda.synchronize()
    sc, lb, ms = score.cpu().numpy(), label.cpu().numpy(), mass.cpu().numpy()
    labels = []
    for h in range(H):
        K = np.concatenate([k for k, _ in Ks[h]]).astype(np.float64)
        rg = np.concatenate([np.full(k.shape[0], r) for k, r in Ks[h]])
        m = of.attention_mass(Q[h].astype(np.float64), K, rg)
        s_ref = of.head_score(m)
        np.testing.assert_allclose(ms[h], m, rtol=5e-3, atol=1e-3 * Lq)
        assert abs(sc[h] - s_ref) < 2e-3, (h, sc[h], s_ref)
        if abs(s_ref - 0.8) > 1e-3:
            assert lb[h] == (kb.KVB_HEAD_STATIC if s_ref > 0.8 else kb.KVB_HEAD_DYNAMIC), (h, lb[h], s_ref)
        labels.append(int(lb[h]))
    gc.banner(f"  scores {np.round(sc, 3).tolist()} labels {labels}")
    assert kb.KVB_HEAD_STATIC in labels and kb.KVB_HEAD_DYNAMIC in labels


def test_head_profile_rejects_a_segment_beyond_max_len():
    """A segment longer than max_len: that head gets score NaN and label
    0xFF, nothing is read past the workspace, the other heads are scored."""
    import torch
    import kv_cache_compression_head_amd as kb
    H, d, Lq = 2, 64, 40
    rng = np.random.default_rng(1)
    Q = torch.from_numpy(rng.normal(size=(H, Lq, d)).astype(np.float32)).to("cuda")
    K0 = torch.from_numpy(rng.normal(size=(30, d)).astype(np.float32)).to("cuda")
    K1 = torch.from_numpy(rng.normal(size=(50, d)).astype(np.float32)).to("cuda")
    segs_t, nseg_t = _table(H, 2, [[(K0.data_ptr(), 30)], [(K1.data_ptr(), 50)]])
    region = torch.tensor([[3, 0], [3, 0]], dtype=torch.int32, device="cuda")
    score = torch.empty(H, dtype=torch.float32, device="cuda")
    label = torch.empty(H, dtype=torch.uint8, device="cuda")
    kb.forcing_head_profile(H, d, Lq, kb.KVB_F32, Q, segs_t, nseg_t, 2, region, 40, score, label)
    torch.cuda.synchronize()
    sc, lb = score.cpu().numpy(), label.cpu().numpy()
    assert lb[0] == kb.KVB_HEAD_STATIC and abs(sc[0] - 1.0) < 1e-6
    assert lb[1] == 0xFF and np.isnan(sc[1])
