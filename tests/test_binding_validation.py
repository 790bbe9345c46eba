"""Host-side checks of the Python binding (CPU only, no kernel is launched).

The C library sees raw pointers only, so the tensor conveniences must refuse a
tensor whose shape, dtype or device differs from what the C call would read or
write -- before anything is enqueued.  Each case below builds otherwise valid
CPU tensors with one mismatch and expects a ValueError naming that tensor.
(With every tensor valid, the CPU tensors are refused as not being on the GPU.)
"""
import pytest
import torch

import long_context_exact_ring_amd as ra

C, HQ, HKV, D, NB = 64, 4, 2, 64, 3
BF, F32 = torch.bfloat16, torch.float32


def _ring(dtype=BF):
    q = torch.zeros((C, HQ, D), dtype=dtype)
    kb = [torch.zeros((C, HKV, D), dtype=dtype) for _ in range(NB)]
    vb = [torch.zeros((C, HKV, D), dtype=dtype) for _ in range(NB)]
    return q, kb, vb


def test_fwd_valid_cpu_tensors_are_refused_as_not_on_gpu():
    q, kb, vb = _ring()
    with pytest.raises(ValueError, match="GPU tensor"):
        ra.fwd(q, kb, vb, causal=True, rank=1)


@pytest.mark.parametrize("which", ["k_dtype", "v_shape", "v_count", "out_shape", "lse_dtype", "out_dtype"])
def test_fwd_mismatch(which):
    q, kb, vb = _ring()
    out = lse = None
    name = {"k_dtype": "k_blocks[1]", "v_shape": "v_blocks[2]", "v_count": "v_blocks", "out_shape": "out",
            "lse_dtype": "lse", "out_dtype": "out"}[which]
    if which == "k_dtype":
        kb[1] = kb[1].float()
    elif which == "v_shape":
        vb[2] = torch.zeros((C - 1, HKV, D), dtype=BF)
    elif which == "v_count":
        vb = vb[:2]
    elif which == "out_shape":
        out = torch.zeros((C, HQ, D // 2), dtype=F32)
    elif which == "lse_dtype":
        lse = torch.zeros((HQ, C), dtype=BF)
    elif which == "out_dtype":
        out = torch.zeros((C, HQ, D), dtype=BF)
    with pytest.raises(ValueError, match=r"^" + name.replace("[", r"\[").replace("]", r"\]")):
        ra.fwd(q, kb, vb, causal=True, rank=1, out=out, lse=lse)


def test_fwd_f32_query_with_bf16_blocks_is_refused():
    q, kb, vb = _ring()
    with pytest.raises(ValueError, match=r"k_blocks\[0\].*dtype"):
        ra.fwd(q.float(), kb, vb, causal=False, rank=0)


@pytest.mark.parametrize("which", ["out", "dout", "lse", "dq", "dk_count", "dk_shape", "dv_dtype"])
def test_bwd_mismatch(which):
    q, kb, vb = _ring()
    args = dict(out=torch.zeros((C, HQ, D), dtype=F32), dout=torch.zeros((C, HQ, D), dtype=BF),
                lse=torch.zeros((HQ, C), dtype=F32))
    kw = {}
    if which == "out":
        args["out"] = torch.zeros((C, HQ, D), dtype=BF)
    elif which == "dout":
        args["dout"] = torch.zeros((C, HQ, D), dtype=F32)
    elif which == "lse":
        args["lse"] = torch.zeros((C, HQ), dtype=F32)
    elif which == "dq":
        kw["dq"] = torch.zeros((C // 2, HQ, D), dtype=F32)
    elif which == "dk_count":
        kw["dk_blocks"] = [torch.zeros((C, HKV, D), dtype=F32) for _ in range(NB - 1)]
    elif which == "dk_shape":
        kw["dk_blocks"] = [torch.zeros((C, HKV, D), dtype=F32) for _ in range(NB)]
        kw["dk_blocks"][1] = torch.zeros((C, HQ, D), dtype=F32)
    elif which == "dv_dtype":
        kw["dv_blocks"] = [torch.zeros((C, HKV, D), dtype=BF) for _ in range(NB)]
    name = {"out": "out", "dout": "dout", "lse": "lse", "dq": "dq", "dk_count": "dk_blocks",
            "dk_shape": r"dk_blocks\[1\]", "dv_dtype": r"dv_blocks\[0\]"}[which]
    with pytest.raises(ValueError, match=r"^" + name):
        ra.bwd(q, kb, vb, args["out"], args["dout"], args["lse"], causal=True, rank=2, **kw)


def test_decode_mismatch():
    q = torch.zeros((3, HQ, D), dtype=BF)
    kb = [torch.zeros((C, HKV, D), dtype=BF) for _ in range(NB)]
    vb = [torch.zeros((C, HKV, D), dtype=BF) for _ in range(NB)]
    with pytest.raises(ValueError, match=r"^v_blocks\[1\]"):
        ra.decode(q, kb, [vb[0], torch.zeros((C, HKV, D + 64), dtype=BF), vb[2]], q_pos0=C * NB)
    with pytest.raises(ValueError, match=r"^lse"):
        ra.decode(q, kb, vb, q_pos0=C * NB, lse=torch.zeros((3, HQ), dtype=F32))
    with pytest.raises(ValueError, match=r"^q"):
        ra.decode(q.float(), kb, vb, q_pos0=C * NB)


def test_ffn_mismatch():
    x = torch.zeros((32, 128), dtype=BF)
    w1 = torch.zeros((512, 128), dtype=BF)
    w2 = torch.zeros((128, 512), dtype=BF)
    with pytest.raises(ValueError, match=r"^w2"):
        ra.ffn_blockwise(x, w1, w2.t().contiguous())
    with pytest.raises(ValueError, match=r"^b1"):
        ra.ffn_blockwise(x, w1, w2, b1=torch.zeros((128,), dtype=F32))
    with pytest.raises(ValueError, match=r"^y"):
        ra.ffn_blockwise(x, w1, w2, y=torch.zeros((32, 128), dtype=BF))


def test_merge_mismatch():
    o = torch.zeros((C, HQ, D), dtype=F32)
    l = torch.zeros((HQ, C), dtype=F32)
    with pytest.raises(ValueError, match=r"^out_b"):
        ra.merge(o, l, o[:-1].contiguous(), l)
    with pytest.raises(ValueError, match=r"^lse_b"):
        ra.merge(o, l, o, l.t().contiguous())
    with pytest.raises(ValueError, match=r"^out"):
        ra.merge(o, l, o, l, out=torch.zeros((C, HQ, D), dtype=BF))
