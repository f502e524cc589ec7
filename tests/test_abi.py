"""CPU checks of the C ABI: the library loads, exports every function its
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import kv_cache_compression_head_amd as kb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvbank.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(kb.HEADER_FUNCTIONS)


def test_library_exports_every_declared_symbol():
    lib = kb.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", kb.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(_declared()) <= exported


def test_library_is_built_from_these_sources():
    """The loader refuses a library whose embedded source hash differs from
    the sources beside it; the hash covers every HIP file and the header."""
    from kv_cache_compression_head_amd import build as kbuild
    lib = kb.load_library()
    assert lib.kvb_source_hash().decode() == kbuild.source_hash()
    names = {os.path.basename(f) for f in kbuild.source_files()}
    assert "kvbank.h" in names and all(s in names for s in kbuild.SOURCES)


def test_dynamic_heads_too_wide_for_the_cosine_kernel():
    # 33 fp32 dynamic heads of d = 128 need 33 x 32 16-byte chunks per token (> 1,024)
    import ctypes
    H = 33
    desc = kb.LayerDesc(H=H, d=128, M=0, dtype=kb.KVB_F32, frame_tokens=16, labels=[2] * H, seg_len=16,
                        retention=0.5)
    lib = kb.load_library()
    c = desc.c()
    buf = ctypes.create_string_buffer(4096 + 256)
    p = (ctypes.addressof(buf) + 255) // 256 * 256
    rc = lib.kvbank_score(ctypes.byref(c), None, p, p, 16, None, p, p, p, p, 1 << 40, None)
    assert rc == -2 and b"cosine" in lib.kvb_last_error()


def _desc(**kw):
    base = dict(H=2, d=64, M=64, dtype=kb.KVB_F32, frame_tokens=16, labels=[0, 0])
    base.update(kw)
    return kb.LayerDesc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), -2), (dict(H=0, labels=[]), -2), (dict(H=65, labels=[0] * 65), -2), (dict(dtype=5), -3),
    (dict(M=0), -2), (dict(tau=0.5), -4), (dict(tau=math.nan), -4), (dict(sigma=0.0), -4), (dict(p=-1.0), -4),
    (dict(eps=0.0), -4), (dict(labels=[0, 7]), -4), (dict(labels=[2, 2], seg_len=5), -4),
    (dict(labels=[2, 2], seg_len=4, retention=1.5), -4), (dict(frame_tokens=0), -2),
    (dict(policy=256), -4), (dict(policy=kb.KVB_POL_EVICT_DENSEST | kb.KVB_POL_EVICT_OLDEST), -4),
])
def test_host_validation(kw, code):
    with pytest.raises(kb.KvbError) as e:
        kb.kvbank_workspace_size(_desc(**kw), 48)
    assert e.value.code == code
    assert kb.kvb_last_error()


def test_descriptor_widths():
    """Descriptor rows of 64 and 128 in either precision; 256 ([K; V] at
    d = 128) in bf16 only; any other width is a shape error."""
    for dt in (kb.KVB_F32, kb.KVB_BF16):
        for dx in (64, 128):
            assert kb.kvbank_workspace_size(_desc(dtype=dt, desc_dim=dx), 48) > 0
    assert kb.kvbank_workspace_size(_desc(d=128, dtype=kb.KVB_BF16, desc_dim=256), 48) > 0
    for kw in (dict(dtype=kb.KVB_F32, desc_dim=256), dict(dtype=kb.KVB_BF16, desc_dim=96),
               dict(dtype=kb.KVB_BF16, desc_dim=512)):
        with pytest.raises(kb.KvbError) as e:
            kb.kvbank_workspace_size(_desc(**kw), 48)
        assert e.value.code == -2 and "desc_dim" in kb.kvb_last_error()


def test_negative_N_and_forcing_multiple():
    with pytest.raises(kb.KvbError) as e:
        kb.kvbank_workspace_size(_desc(), -1)
    assert e.value.code == -2
    with pytest.raises(kb.KvbError) as e:
        kb.kvbank_workspace_size(_desc(labels=[1, 1], M=0), 17)
    assert e.value.code == -2


def test_workspace_size_sane():
    b = kb.kvbank_workspace_size(_desc(H=12, d=128, M=9360, dtype=kb.KVB_BF16, frame_tokens=1560, labels=[0] * 12),
                                 23400)
    assert 10e6 < b < 1e9
    assert kb.kvbank_workspace_size(_desc(), 0) >= 0


def _raw(lib_fn, *args):
    return lib_fn(*args)


def test_score_update_attention_reject_before_launch():
    lib = kb.load_library()
    d = _desc().c()
    # workspace too small -> EWORKSPACE, nothing launched
    rc = lib.kvbank_score(ctypes.byref(d), None, 16, 16, 48, None, 16, 16, 16, None, 0, None)
    assert rc == -5
    # misaligned candidate pointer
    rc = lib.kvbank_score(ctypes.byref(d), None, 17, 16, 48, None, 16, 16, 16, 16, 1 << 30, None)
    assert rc == -1
    # update without a layout
    rc = lib.kvbank_update(ctypes.byref(d), None, 16, 16, 16, 48, 16, 16, None, None, 16, 1 << 30, None)
    assert rc == -1
    # attention: bad d, bad seg_cap, and Lq = 0 (valid no-op)
    a = kb.kvb_attn_desc(2, 96, 10, 0, 0.0, 4, 0, 0)
    assert lib.chunk_attention(ctypes.byref(a), 16, 16, 16, 16, None, 0, None) == -2
    a = kb.kvb_attn_desc(2, 64, 10, 0, 0.0, 300, 0, 0)
    assert lib.chunk_attention(ctypes.byref(a), 16, 16, 16, 16, None, 0, None) == -2
    a = kb.kvb_attn_desc(2, 64, 0, 0, 0.0, 4, 0, 0)
    assert lib.chunk_attention(ctypes.byref(a), None, None, None, None, None, 0, None) == 0


def test_struct_layouts_match_the_c_header(tmp_path):
    """ctypes mirrors of the header structs have the C compiler's sizes and offsets."""
    structs = {"kvb_params": kb.kvb_params, "kvb_layer_desc": kb.kvb_layer_desc, "kvb_bank": kb.kvb_bank,
               "kvb_kv_layout": kb.kvb_kv_layout, "kvb_segment": kb.kvb_segment,
               "kvb_update_out": kb.kvb_update_out, "kvb_attn_desc": kb.kvb_attn_desc}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "kvbank.h"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append(f'printf("{name} size %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{name}.{f} %zu\\n", offsetof({name}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "abi.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                         check=True).stdout.splitlines())
    for name, cls in structs.items():
        assert int(got[f"{name} size"]) == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert int(got[f"{name}.{f}"]) == getattr(cls, f).offset, f"{name}.{f}"


def test_window_advance_rejects_before_launch():
    """kvbank_window_advance checks shapes, parameters and pointers on the
    host; n_rows = 0 is a no-op (nothing launched, no pointer read)."""
    lib = kb.load_library()
    d = _desc().c()                      # F = 16
    wa = lib.kvbank_window_advance
    ok = dict(ring_k=16, ring_v=32, cap=64, start=0, n=32, t0=1, base=10000.0, nk=None, nv=None, ck=48, cv=64)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return wa(ctypes.byref(d), a["ring_k"], a["ring_v"], a["cap"], a["start"], a["n"], a["t0"], a["base"],
                  a["nk"], a["nv"], a["ck"], a["cv"], None)
    assert call(n=0, ring_k=None, ring_v=None, ck=None, cv=None) == 0
    assert call(n=24) == -2                 # not a multiple of F
    assert call(n=80) == -2                 # more rows than the ring holds
    assert call(start=64) == -2             # start outside the ring
    assert call(base=1.0) == -4
    assert call(base=math.inf) == -4
    assert call(nk=16) == -1                # new_k without new_v
    assert call(ck=17) == -1                # misaligned
    assert call(cv=None) == -1
    assert kb.kvb_last_error()


def test_head_profile_rejects_before_launch():
    lib = kb.load_library()
    a = kb.kvb_attn_desc(2, 64, 40, 1, 0.0, 4, 1, 0)
    n = ctypes.c_size_t(0)
    assert lib.forcing_head_profile_workspace_size(ctypes.byref(a), 100, ctypes.byref(n)) == 0 and n.value > 0
    prof = lib.forcing_head_profile
    # alpha outside [0, 1]
    assert prof(ctypes.byref(a), 16, 16, 16, 16, 100, ctypes.c_float(1.5), None, 16, 16, 16, n.value, None) == -4
    # workspace too small
    assert prof(ctypes.byref(a), 16, 16, 16, 16, 100, ctypes.c_float(0.8), None, 16, 16, 16, n.value - 1, None) == -5
    # bad d, negative max_len
    b = kb.kvb_attn_desc(2, 96, 40, 1, 0.0, 4, 1, 0)
    assert lib.forcing_head_profile_workspace_size(ctypes.byref(b), 100, ctypes.byref(n)) == -2
    assert lib.forcing_head_profile_workspace_size(ctypes.byref(a), -1, ctypes.byref(n)) == -2


def test_score_layers_rejects_before_launch():
    """kvbank_score_layers takes Forcing-KV layers only, checks the layer
    strides, the item count and the workspace on the host; nlayers = 0 is a
    no-op."""
    lib = kb.load_library()
    F, N = 16, 64
    fk = kb.LayerDesc(H=4, d=64, M=0, dtype=kb.KVB_BF16, frame_tokens=F, labels=[1, 2, 2, 1], seg_len=8,
                      retention=0.5)
    dn = kb.LayerDesc(H=4, d=64, M=32, dtype=kb.KVB_BF16, frame_tokens=F, labels=[0, 2, 2, 1], seg_len=8,
                      retention=0.5)
    n = ctypes.c_size_t(0)
    c = fk.c()
    assert lib.kvbank_score_layers_workspace_size(ctypes.byref(c), 3, N, ctypes.byref(n)) == 0
    assert n.value == (3 * N * 4 + 255) // 256 * 256
    cd = dn.c()
    assert lib.kvbank_score_layers_workspace_size(ctypes.byref(cd), 3, N, ctypes.byref(n)) == -4
    per = dict(fk.__dict__)
    per["policy"] = kb.KVB_POL_FRAME_BOTTOMK
    cf = kb.LayerDesc(**per).c()
    assert lib.kvbank_score_layers_workspace_size(ctypes.byref(cf), 3, N, ctypes.byref(n)) == -4
    sl = lib.kvbank_score_layers
    hs, cs = 4 * N * 64, 4 * 2 * F * 64    # one layer of history keys, of chunk keys
    ws = 1 << 40

    def call(nl=3, hstr=hs, cstr=cs, cl=2 * F, wsb=ws, ck=16, desc=c):
        return sl(ctypes.byref(desc), nl, ck, hstr, 32, cstr, cl, N, 48, 64, 256, wsb, None)
    assert call(nl=0, ck=None) == 0
    assert call(hstr=hs - 8) == -2              # stride shorter than a layer
    assert call(cstr=cs + 4) == -2              # not a 16-byte multiple
    assert call(cl=F - 1) == -2                 # chunk shorter than a frame
    assert call(ck=17) == -1                    # misaligned
    assert call(wsb=16) == -5                   # workspace too small
    assert call(desc=cd) == -4                  # density heads
    assert kb.kvb_last_error()
