"""GPU parity of chunk_attention on ragged segment tables (fp64 oracle)."""
import ctypes

import numpy as np
import pytest

from kvsynth import round_bf16
from oracle.attention import attention as oracle_attention

import gpu_common as gc

pytestmark = pytest.mark.gpu


def _seg_table(H, seg_cap, per_head):
    import torch
    import kv_cache_compression_head_amd as kb
    arr = (kb.kvb_segment * (H * seg_cap))()
    ns = []
    for h, segs in enumerate(per_head):
        for i, (kp, vp, ln) in enumerate(segs):
            arr[h * seg_cap + i] = kb.kvb_segment(kp, vp, ln, 0)
        ns.append(len(segs))
    raw = np.frombuffer(bytes(arr), dtype=np.uint8).copy()
    return torch.from_numpy(raw).to("cuda"), torch.tensor(ns, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("d,Lq,lens,dtype", [
    (128, 300, [[70, 1, 64, 129], [5], [64 * 5]], "bf16"),
    (64, 129, [[33, 31], [1, 2, 3, 4, 5, 200], [640]], "bf16"),
    (128, 4680, [[1560, 9360, 3120, 1560, 4680]], "bf16"),
    (64, 48, [[16, 64, 48], [16, 60, 48]], "f32"),
    (128, 700, [[0], [3000, 17], [], [64]], "bf16"),
])
@pytest.mark.parametrize("ws", ["auto", None])
def test_attention_ragged(d, Lq, lens, dtype, ws):
    """Ragged segment tables; heads with no keys (an empty segment, or none)
    give zeros.  ws "auto": the balanced grid (left-over items cut into a
    main piece and a tail, merged from fp32 partials); None: one work-group
    per item."""
    _attention_case(d, Lq, lens, dtype, ws=ws)


# Segments whose key scales differ by large factors: the running maximum of a
# query moves by far more than 2^8 between tiles (up, then down), so the
# online softmax has to rescale its accumulated numerator and denominator.
# With scales of 40 the later scores exceed the first tile's by far more than
# 2^127 (in the exponent), so weights against the first tile's maximum
# overflow and the kernel must redo the tiles with the running maximum.
@pytest.mark.parametrize("d,Lq,lens,kscale", [
    (128, 300, [[130, 200, 64]], [0.05, 6.0, 0.5]),
    (128, 257, [[64, 64, 70], [10, 300]], [0.1, 3.0, 8.0]),
    (64, 100, [[200, 130]], [0.2, 7.0]),
    (128, 200, [[64, 300], [70, 129, 5]], [0.05, 40.0, 0.3]),
    (64, 90, [[100, 100]], [0.1, 40.0]),
])
def test_attention_rescale(d, Lq, lens, kscale):
    _attention_case(d, Lq, lens, "bf16", kscale)


def _attention_case(d, Lq, lens, dtype, kscale=None, ws="auto", heads=None, ret=False):
    import torch
    import kv_cache_compression_head_amd as kb
    gc.banner(f"attention d={d} Lq={Lq} lens={lens} {dtype} kscale={kscale} ws={ws}")
    rng = np.random.default_rng(d + Lq)
    H = len(lens)
    kdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rnd = (lambda x: round_bf16(x)) if dtype == "bf16" else (lambda x: x.astype(np.float32))
    Q = rnd(rng.normal(size=(H, Lq, d)).astype(np.float32) * 1.5)
    seg_cap = max(len(l) for l in lens) + 1
    keep = []
    per_head = []
    Ks, Vs = [], []
    for h, ls in enumerate(lens):
        segs = []
        kk, vv = [], []
        for i, ln in enumerate(ls):
            ks = 1.5 if kscale is None else kscale[(i + h) % len(kscale)]
            k = rnd(rng.normal(size=(ln, d)).astype(np.float32) * ks)
            v = rnd(rng.normal(size=(ln, d)).astype(np.float32))
            tk, tv = gc.dev(k, kdt), gc.dev(v, kdt)
            keep += [tk, tv]
            segs.append((tk.data_ptr(), tv.data_ptr(), ln))
            kk.append(k)
            vv.append(v)
        per_head.append(segs)
        Ks.append(np.concatenate(kk) if kk else np.zeros((0, d), np.float32))
        Vs.append(np.concatenate(vv) if vv else np.zeros((0, d), np.float32))
    segs_t, nseg_t = _seg_table(H, seg_cap, per_head)
    Qd = gc.dev(Q, kdt)
    O = torch.empty(H, Lq, d, dtype=torch.float32, device="cuda")
    et = kb.KVB_BF16 if dtype == "bf16" else kb.KVB_F32
    kb.chunk_attention(H, d, Lq, et, Qd, segs_t, nseg_t, seg_cap, O, out_f32=True, ws=ws)
    torch.cuda.synchronize()
    On = O.cpu().numpy()
    if ret:
        return On
    tol = (2e-2, 2e-3) if dtype == "bf16" else (1e-4, 1e-5)
    errs = []
    for h in (range(H) if heads is None else heads):
        if Ks[h].shape[0] == 0:   # no keys: the kernels write zeros
            assert np.all(On[h] == 0.0), f"head {h} without keys"
            continue
        ref = oracle_attention(Q[h].astype(np.float64), Ks[h].astype(np.float64), Vs[h].astype(np.float64))
        errs.append(np.abs(On[h] - ref).reshape(-1))
    e = np.concatenate(errs)
    assert e.max() <= tol[0] and e.mean() <= tol[1], (e.max(), e.mean())


def test_attention_bf16_output_dtype():
    import torch
    import kv_cache_compression_head_amd as kb
    rng = np.random.default_rng(7)
    H, Lq, d, L = 2, 200, 128, 333
    Q = round_bf16(rng.normal(size=(H, Lq, d)).astype(np.float32))
    K = round_bf16(rng.normal(size=(H, L, d)).astype(np.float32))
    V = round_bf16(rng.normal(size=(H, L, d)).astype(np.float32))
    tk, tv = gc.dev(K, torch.bfloat16), gc.dev(V, torch.bfloat16)
    per_head = [[(tk[h].data_ptr(), tv[h].data_ptr(), L)] for h in range(H)]
    segs_t, nseg_t = _seg_table(H, 2, per_head)
    O = torch.empty(H, Lq, d, dtype=torch.bfloat16, device="cuda")
    kb.chunk_attention(H, d, Lq, kb.KVB_BF16, gc.dev(Q, torch.bfloat16), segs_t, nseg_t, 2, O)
    torch.cuda.synchronize()
    On = O.float().cpu().numpy()
    for h in range(H):
        ref = oracle_attention(Q[h].astype(np.float64), K[h].astype(np.float64), V[h].astype(np.float64))
        e = np.abs(On[h] - ref)
        assert e.max() <= 2e-2 and e.mean() <= 2e-3


def test_attention_balanced_rounds():
    """More items than slots (8 heads x 33 query tiles = 264 on 256 slots):
    a round of whole items, then the 8 left-over items balanced over every
    work-group; heads of different lengths."""
    lens = [[300 + 97 * h, 64 * h] for h in range(8)]
    _attention_case(128, 8200, lens, "bf16")


def test_attention_balanced_multi_tail():
    """10 heads x 19 query tiles over 6,400 keys (190 items on 256 slots):
    the tails are short enough that each tail work-group takes several items
    of one head.  Three heads against the oracle; every head against the
    one-work-group-per-item grid."""
    lens = [[1560, 3200, 1640] for _ in range(10)]
    _attention_case(128, 4680, lens, "bf16", heads=[0, 5, 9])
    a = _attention_case(128, 4680, lens, "bf16", ret=True)
    b = _attention_case(128, 4680, lens, "bf16", ws=None, ret=True)
    e = np.abs(a - b)
    assert e.max() <= 1e-2 and e.mean() <= 1e-3, (e.max(), e.mean())


def test_attention_balanced_short_items_take_tails():
    """Heads of two lengths, as in the Forcing-KV hybrid layer (6 heads of
    7,800 keys, 6 of 18,720; 228 items on 256 slots): the work-groups whose
    own item is short also take tails of the long heads' items, besides the
    spare work-groups.  Three heads against the oracle; every head against
    the one-work-group-per-item grid."""
    lens = [[1560, 1560, 4680]] * 6 + [[1560, 12480, 4680]] * 6
    _attention_case(128, 4680, lens, "bf16", heads=[0, 6, 11])
    a = _attention_case(128, 4680, lens, "bf16", ret=True)
    b = _attention_case(128, 4680, lens, "bf16", ws=None, ret=True)
    e = np.abs(a - b)
    assert e.max() <= 1e-2 and e.mean() <= 1e-3, (e.max(), e.mean())


def test_attention_whole_items_of_one_length():
    """12 heads of one length x 19 query tiles (228 items on 256 slots, more
    than four fifths): the plan keeps every item whole, so the output equals
    the one-work-group-per-item grid bit for bit; three heads against the
    oracle."""
    lens = [[1560, 640]] * 12
    _attention_case(128, 4680, lens, "bf16", heads=[0, 5, 11])
    a = _attention_case(128, 4680, lens, "bf16", ret=True)
    b = _attention_case(128, 4680, lens, "bf16", ws=None, ret=True)
    assert np.array_equal(a, b)


def test_attention_balanced_d64():
    """d = 64 on the balanced grid, with a ragged tail tile."""
    _attention_case(64, 1000, [[900, 333], [1500], [64, 64, 7]], "bf16")


def test_attention_workspace_size():
    """The workspace covers the left-over items' partials: two pieces of
    8 waves x (2 d/16 + 1) float4 per lane each, plus a flag per item; none
    when the items fill whole rounds (one work-group of 256 queries per
    compute unit)."""
    import kv_cache_compression_head_amd as kb
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for H, d, Lq in [(12, 128, 4680), (10, 128, 4680), (8, 128, 8200), (3, 64, 300), (12, 128, 24480)]:
        items = -(-Lq // 256) * H
        ir = items % cus
        per = 2 * 8 * (2 * (d // 16) + 1) * 64 * 16
        use = ir > 0
        want = -(-ir * 4 // 256) * 256 + ir * per if use else 0
        assert kb.chunk_attention_workspace_size(H, d, Lq, kb.KVB_BF16) == want
    assert kb.chunk_attention_workspace_size(12, 128, 4680, kb.KVB_F32) == 0
