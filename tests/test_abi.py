"""CPU-only checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments on the host before any HIP call.

No call here passes validation, so nothing touches a GPU (fake device
addresses are fine: they are compared, never dereferenced).
"""
import ctypes
import os
import re
import subprocess

import pytest

import long_context_exact_ring_amd as ra
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_attn.h")

BASE = 0x7F0000000000  # fake device addresses


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|void|size_t|const char\*)\s+(ring_attn_\w+)\(", txt, re.M)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for must in ("ring_attn_fwd", "ring_attn_merge", "ring_attn_bwd"):
        assert must in names
    assert set(names) == set(ra.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ra.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ra.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(ring_attn_\w+)", out))
    assert set(declared_functions()) <= exported


def _fwd(**kw):
    args = dict(q=BASE, k_blocks=[BASE + 0x10000000 * (j + 1) for j in range(4)],
                v_blocks=[BASE + 0x10000000 * (j + 5) for j in range(4)], n_blocks=4, block_len=256,
                heads=2, kv_heads=1, head_dim=64, causal=1, rank=0, out=BASE + 0x100000000,
                lse=BASE + 0x200000000, stream=0)
    args.update(kw)
    return ra.ring_attn_fwd(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), ra.RA_ERR_INVALID_ARG),
    (dict(out=None), ra.RA_ERR_INVALID_ARG),
    (dict(lse=None), ra.RA_ERR_INVALID_ARG),
    (dict(n_blocks=0), ra.RA_ERR_INVALID_ARG),
    (dict(rank=4), ra.RA_ERR_INVALID_ARG),
    (dict(rank=-1), ra.RA_ERR_INVALID_ARG),
    (dict(block_len=0), ra.RA_ERR_INVALID_ARG),
    (dict(heads=3, kv_heads=2), ra.RA_ERR_INVALID_ARG),
    (dict(kv_heads=0), ra.RA_ERR_INVALID_ARG),
    (dict(head_dim=96), ra.RA_ERR_UNSUPPORTED),
    (dict(head_dim=256), ra.RA_ERR_UNSUPPORTED),
    (dict(block_len=1 << 24, heads=128), ra.RA_ERR_INVALID_ARG),
    (dict(out=BASE + 0x100), ra.RA_ERR_INVALID_ARG),                 # out overlaps q
    (dict(lse=BASE + 0x10000000 * 2 + 64), ra.RA_ERR_INVALID_ARG),   # lse inside K block 1
    (dict(lse=BASE + 0x100000000 + 16), ra.RA_ERR_INVALID_ARG),      # lse overlaps out
])
def test_fwd_rejects_bad_arguments_before_any_hip_call(kw, code):
    assert _fwd(**kw) == code
    assert ra.last_error() != ""


def test_fwd_rejects_null_block_pointer():
    kb = [BASE + 0x10000000 * (j + 1) for j in range(4)]
    kb[2] = None
    assert _fwd(k_blocks=kb) == ra.RA_ERR_INVALID_ARG
    assert "k_blocks[2]" in ra.last_error()


def test_bwd_rejects_overlapping_gradients():
    kb = [BASE + 0x10000000 * (j + 1) for j in range(2)]
    vb = [BASE + 0x10000000 * (j + 5) for j in range(2)]
    dk = [BASE + 0x300000000, BASE + 0x300000000 + 1024]  # overlap each other
    dv = [BASE + 0x400000000, BASE + 0x500000000]
    rc = ra.ring_attn_bwd(BASE, kb, vb, BASE + 0x600000000, BASE + 0x700000000, BASE + 0x800000000, 2, 128,
                          2, 2, 64, 1, 1, BASE + 0x900000000, dk, dv, 0)
    assert rc == ra.RA_ERR_INVALID_ARG
    dk = [BASE + 0x300000000, BASE + 0x380000000]
    rc = ra.ring_attn_bwd(BASE, kb, vb, BASE + 0x600000000, BASE + 0x700000000, BASE + 0x800000000, 2, 128,
                          2, 2, 64, 1, 1, BASE + 0x600000000, dk, dv, 0)   # dq == out (a forward input)
    assert rc == ra.RA_ERR_INVALID_ARG
    rc = ra.ring_attn_bwd_f32(BASE, kb, vb, None, BASE + 0x700000000, BASE + 0x800000000, 2, 128,
                              2, 2, 64, 1, 1, BASE + 0x900000000, dk, dv, 0)
    assert rc == ra.RA_ERR_INVALID_ARG


def test_merge_validation():
    o, l = BASE, BASE + 0x10000000
    ob, lb = BASE + 0x20000000, BASE + 0x30000000
    rows, heads, d = 100, 4, 64
    assert ra.ring_attn_merge(None, l, ob, lb, rows, heads, d, o, l, 0) == ra.RA_ERR_INVALID_ARG
    assert ra.ring_attn_merge(o, l, ob, lb, -1, heads, d, o, l, 0) == ra.RA_ERR_INVALID_ARG
    assert ra.ring_attn_merge(o, l, ob, lb, rows, 0, d, o, l, 0) == ra.RA_ERR_INVALID_ARG
    # partial overlap of the output with an input is rejected (exact aliasing is allowed)
    assert ra.ring_attn_merge(o, l, ob, lb, rows, heads, d, o + 64, BASE + 0x40000000, 0) == ra.RA_ERR_INVALID_ARG
    assert ra.ring_attn_merge(o, l, ob, lb, rows, heads, d, BASE + 0x50000000, l + 4, 0) == ra.RA_ERR_INVALID_ARG
    # rows == 0 is a valid no-op that enqueues nothing
    assert ra.ring_attn_merge(o, l, ob, lb, 0, heads, d, o, l, 0) == ra.RA_OK


@pytest.mark.parametrize("D", [1, 2, 3, 4, 8, 16])
def test_library_schedule_matches_the_oracle_ring(D):
    for r in range(D):
        for causal in (False, True):
            assert ra.ring_attn_schedule(r, D, causal) == oracle.ring_steps(r, D, causal)


def test_schedule_rejects_bad_rank():
    with pytest.raises(ra.RingAttnError):
        ra.ring_attn_schedule(5, 4, False)


def test_workspace_is_two_k_and_two_v_blocks():
    # six resident blocks per host: Q, O, K/V in use, K/V in flight -> staging = 2 x (K + V)
    assert ra.ring_attn_workspace_bytes(8192, 32, 128, 2) == 4 * 8192 * 32 * 128 * 2
    assert ra.ring_attn_workspace_bytes(256, 1, 64, 4) == 4 * 256 * 64 * 4
    assert ra.ring_attn_workspace_bytes(0, 1, 64, 2) == 0


def test_debug_and_profile_toggles():
    assert ra.lib().ring_attn_debug(0, -5) == ra.RA_ERR_INVALID_ARG
    ra.ring_attn_debug(False, 0)
    assert ra.ring_attn_profile_enable(False) == ra.RA_OK
    recs, copy_ms, hidden = ra.ring_attn_profile_read()   # nothing recorded: no HIP call needed
    assert copy_ms == 0.0 and hidden == 0.0 and all(v == (0.0, 0) for v in recs.values())


def test_set_workspace_validation_before_any_hip_call():
    L = ra.lib()
    assert L.ring_attn_set_workspace(None, 4096) == ra.RA_ERR_INVALID_ARG       # size without memory
    assert L.ring_attn_set_workspace(BASE, 0) == ra.RA_ERR_INVALID_ARG          # memory without size
    assert L.ring_attn_set_workspace(BASE + 16, 4096) == ra.RA_ERR_INVALID_ARG  # not 256-byte aligned
    assert b"aligned" in L.ring_attn_last_error()


def test_mfma_rate_validation_before_any_hip_call():
    L = ra.lib()
    out = ctypes.c_double()
    assert L.ring_attn_mfma_rate(0, BASE, ctypes.byref(out), None) == ra.RA_ERR_INVALID_ARG
    assert L.ring_attn_mfma_rate(1 << 25, BASE, ctypes.byref(out), None) == ra.RA_ERR_INVALID_ARG
    assert L.ring_attn_mfma_rate(10, None, ctypes.byref(out), None) == ra.RA_ERR_INVALID_ARG


def test_decode_validation_before_any_hip_call():
    L = ra.lib()
    q, o, l = BASE, BASE + 0x10000000, BASE + 0x20000000
    kb = (ctypes.c_void_p * 2)(BASE + 0x30000000, BASE + 0x40000000)
    vb = (ctypes.c_void_p * 2)(BASE + 0x50000000, BASE + 0x60000000)

    def call(**kw):
        a = dict(q=q, kb=kb, vb=vb, nb=2, c=256, ql=1, hq=8, hkv=2, d=128, pos=511, o=o, l=l)
        a.update(kw)
        return L.ring_attn_decode(a["q"], a["kb"], a["vb"], a["nb"], a["c"], a["ql"], a["hq"], a["hkv"], a["d"],
                                  a["pos"], a["o"], a["l"], None)
    assert call(q=None) == ra.RA_ERR_INVALID_ARG
    assert call(nb=0) == ra.RA_ERR_INVALID_ARG
    assert call(nb=65) == ra.RA_ERR_INVALID_ARG
    assert call(ql=0) == ra.RA_ERR_INVALID_ARG
    assert call(hq=6, hkv=4) == ra.RA_ERR_INVALID_ARG
    assert call(d=96) == ra.RA_ERR_UNSUPPORTED
    assert call(hq=66, hkv=2) == ra.RA_ERR_UNSUPPORTED  # group 33: more than 32 rows even for one query
    assert call(pos=-1) == ra.RA_ERR_INVALID_ARG
    assert call(l=o + 16) == ra.RA_ERR_INVALID_ARG       # lse inside out
    assert call(o=kb[1]) == ra.RA_ERR_INVALID_ARG        # out overlaps a K block


def test_zigzag_rejects_odd_block_len_before_any_hip_call():
    L = ra.lib()
    kb = (ctypes.c_void_p * 2)(BASE + 0x30000000, BASE + 0x40000000)
    vb = (ctypes.c_void_p * 2)(BASE + 0x50000000, BASE + 0x60000000)
    rc = L.ring_attn_fwd_zigzag(BASE, kb, vb, 2, 33, 2, 2, 128, 1, 0, BASE + 0x10000000, BASE + 0x20000000, None)
    assert rc == ra.RA_ERR_INVALID_ARG and b"even" in L.ring_attn_last_error()


def test_ffn_validation_before_any_hip_call():
    L = ra.lib()
    x, w1, w2, y = BASE, BASE + 0x10000000, BASE + 0x20000000, BASE + 0x30000000
    assert L.ring_attn_ffn_blockwise(None, w1, None, w2, None, 8, 128, 256, 0, y, None) == ra.RA_ERR_INVALID_ARG
    assert L.ring_attn_ffn_blockwise(x, w1, None, w2, None, 0, 128, 256, 0, y, None) == ra.RA_ERR_INVALID_ARG
    assert L.ring_attn_ffn_blockwise(x, w1, None, w2, None, 8, 96, 256, 0, y, None) == ra.RA_ERR_UNSUPPORTED
    assert L.ring_attn_ffn_blockwise(x, w1, None, w2, None, 8, 128, 200, 0, y, None) == ra.RA_ERR_UNSUPPORTED
    assert L.ring_attn_ffn_blockwise(x, w1, None, w2, None, 8, 128, 256, -1, y, None) == ra.RA_ERR_INVALID_ARG
    assert L.ring_attn_ffn_blockwise(x, w1, None, w2, None, 8, 128, 256, 0, x + 64, None) == ra.RA_ERR_INVALID_ARG


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError, match="GPU tensor"):
        ra._addr(torch.zeros(4))
