"""Python binding of the MI355X ring-attention step library (``libringattn.so``).

Argument marshalling only: every step of the forward, merge and backward runs
in the library's HIP kernels on gfx950.  PyTorch is used for device memory and
streams; tensors are passed by ``data_ptr()`` and the caller's current HIP
stream.  If the shared library has not been built the import of the native
functions fails loudly -- there is no CPU fallback.

The low-level functions carry the C ABI's names and parameters
(``ring_attn_fwd``, ``ring_attn_fwd_f32``, ``ring_attn_merge``,
``ring_attn_bwd``, ``ring_attn_bwd_f32``, ...).  ``fwd``, ``bwd`` and
``merge`` are conveniences that read sizes from tensor shapes, allocate the
outputs and pick the bf16 or fp32 entry point from the input dtype.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libringattn.so")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP, RA_ERR_OOM = range(5)
PROFILE_KINDS = ("fwd_step", "bwd_dkdv", "bwd_dq", "bwd_pre", "merge", "copy", "decode_partial", "decode_merge",
                 "ffn_up", "ffn_down")

EXPORTED = (
    "ring_attn_fwd", "ring_attn_fwd_f32", "ring_attn_merge", "ring_attn_bwd", "ring_attn_bwd_f32",
    "ring_attn_last_error", "ring_attn_workspace_bytes", "ring_attn_profile_enable",
    "ring_attn_profile_read", "ring_attn_shutdown", "ring_attn_schedule", "ring_attn_debug",
    "ring_attn_set_workspace", "ring_attn_mfma_rate", "ring_attn_decode",
    "ring_attn_fwd_zigzag", "ring_attn_bwd_zigzag", "ring_attn_ffn_blockwise", "ring_attn_decode_noalloc",
)
MFMA_RATE_SINK_FLOATS = 1024


class RingAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"ring_attn error {code}: {message}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load ``libringattn.so`` (built by ``long_context_exact_ring_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m long_context_exact_ring_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
    fwd_args = [vp, vp, vp, i, i, i, i, i, i, i, f32p, f32p, vp]
    for name in ("ring_attn_fwd", "ring_attn_fwd_f32", "ring_attn_fwd_zigzag"):
        fn = getattr(L, name)
        fn.argtypes = fwd_args
        fn.restype = i
    bwd_args = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, vp, vp, vp]
    for name in ("ring_attn_bwd", "ring_attn_bwd_f32", "ring_attn_bwd_zigzag"):
        fn = getattr(L, name)
        fn.argtypes = bwd_args
        fn.restype = i
    L.ring_attn_merge.argtypes = [vp, vp, vp, vp, i, i, i, vp, vp, vp]
    L.ring_attn_merge.restype = i
    L.ring_attn_last_error.argtypes = []
    L.ring_attn_last_error.restype = ctypes.c_char_p
    L.ring_attn_workspace_bytes.argtypes = [i, i, i, i]
    L.ring_attn_workspace_bytes.restype = ctypes.c_size_t
    L.ring_attn_set_workspace.argtypes = [vp, ctypes.c_size_t]
    L.ring_attn_set_workspace.restype = i
    for name in ("ring_attn_decode", "ring_attn_decode_noalloc"):
        fn = getattr(L, name)
        fn.argtypes = [vp, vp, vp, i, i, i, i, i, i, ctypes.c_longlong, vp, vp, vp]
        fn.restype = i
    L.ring_attn_ffn_blockwise.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, vp, vp]
    L.ring_attn_ffn_blockwise.restype = i
    L.ring_attn_mfma_rate.argtypes = [i, vp, ctypes.POINTER(ctypes.c_double), vp]
    L.ring_attn_mfma_rate.restype = i
    L.ring_attn_profile_enable.argtypes = [i]
    L.ring_attn_profile_enable.restype = i
    L.ring_attn_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int),
                                         ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    L.ring_attn_profile_read.restype = i
    L.ring_attn_schedule.argtypes = [i, i, i, ctypes.POINTER(ctypes.c_int), i]
    L.ring_attn_schedule.restype = i
    L.ring_attn_debug.argtypes = [i, ctypes.c_longlong]
    L.ring_attn_debug.restype = i
    L.ring_attn_shutdown.argtypes = []
    L.ring_attn_shutdown.restype = None
    _lib = L
    return L


# ------------------------------------------------------------------ marshalling helpers
def _addr(x) -> Optional[int]:
    """Device address of a tensor (or a raw integer address / None).

    The library reads every buffer as a dense row-major array, so a tensor must live
    on the GPU and be contiguous; views with other strides are refused here."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"expected a GPU tensor, got one on {x.device}")
    if not x.is_contiguous():
        raise ValueError(f"expected a contiguous tensor, got strides {tuple(x.stride())} for shape {tuple(x.shape)}")
    return x.data_ptr()


def _ptr_array(xs: Sequence) -> ctypes.Array:
    arr = (ctypes.c_void_p * max(1, len(xs)))()
    for j, x in enumerate(xs):
        arr[j] = _addr(x)
    return arr


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> None:
    if rc != RA_OK:
        msg = lib().ring_attn_last_error()
        raise RingAttnError(rc, msg.decode() if msg else "")


def last_error() -> str:
    msg = lib().ring_attn_last_error()
    return msg.decode() if msg else ""


# ------------------------------------------------------------------ C-ABI mirrors
def ring_attn_fwd(q, k_blocks, v_blocks, n_blocks, block_len, heads, kv_heads, head_dim, causal, rank,
                  out, lse, stream=None) -> int:
    """bf16 forward ring step; returns the C status code (no exception)."""
    return lib().ring_attn_fwd(_addr(q), _ptr_array(k_blocks), _ptr_array(v_blocks), n_blocks, block_len,
                               heads, kv_heads, head_dim, int(bool(causal)), rank, _addr(out), _addr(lse),
                               _stream(stream))


def ring_attn_fwd_f32(q, k_blocks, v_blocks, n_blocks, block_len, heads, kv_heads, head_dim, causal, rank,
                      out, lse, stream=None) -> int:
    return lib().ring_attn_fwd_f32(_addr(q), _ptr_array(k_blocks), _ptr_array(v_blocks), n_blocks,
                                   block_len, heads, kv_heads, head_dim, int(bool(causal)), rank, _addr(out),
                                   _addr(lse), _stream(stream))


def ring_attn_merge(out_a, lse_a, out_b, lse_b, rows, heads, head_dim, out, lse, stream=None) -> int:
    return lib().ring_attn_merge(_addr(out_a), _addr(lse_a), _addr(out_b), _addr(lse_b), rows, heads,
                                 head_dim, _addr(out), _addr(lse), _stream(stream))


def ring_attn_fwd_zigzag(q, k_blocks, v_blocks, n_blocks, block_len, heads, kv_heads, head_dim, causal, rank,
                         out, lse, stream=None) -> int:
    return lib().ring_attn_fwd_zigzag(_addr(q), _ptr_array(k_blocks), _ptr_array(v_blocks), n_blocks, block_len,
                                      heads, kv_heads, head_dim, int(bool(causal)), rank, _addr(out), _addr(lse),
                                      _stream(stream))


def ring_attn_bwd_zigzag(q, k_blocks, v_blocks, out, dout, lse, n_blocks, block_len, heads, kv_heads, head_dim,
                         causal, rank, dq, dk_blocks, dv_blocks, stream=None) -> int:
    return lib().ring_attn_bwd_zigzag(_addr(q), _ptr_array(k_blocks), _ptr_array(v_blocks), _addr(out),
                                      _addr(dout), _addr(lse), n_blocks, block_len, heads, kv_heads, head_dim,
                                      int(bool(causal)), rank, _addr(dq), _ptr_array(dk_blocks),
                                      _ptr_array(dv_blocks), _stream(stream))


def ring_attn_bwd(q, k_blocks, v_blocks, out, dout, lse, n_blocks, block_len, heads, kv_heads, head_dim,
                  causal, rank, dq, dk_blocks, dv_blocks, stream=None) -> int:
    return lib().ring_attn_bwd(_addr(q), _ptr_array(k_blocks), _ptr_array(v_blocks), _addr(out), _addr(dout),
                               _addr(lse), n_blocks, block_len, heads, kv_heads, head_dim, int(bool(causal)),
                               rank, _addr(dq), _ptr_array(dk_blocks), _ptr_array(dv_blocks), _stream(stream))


def ring_attn_bwd_f32(q, k_blocks, v_blocks, out, dout, lse, n_blocks, block_len, heads, kv_heads, head_dim,
                      causal, rank, dq, dk_blocks, dv_blocks, stream=None) -> int:
    return lib().ring_attn_bwd_f32(_addr(q), _ptr_array(k_blocks), _ptr_array(v_blocks), _addr(out),
                                   _addr(dout), _addr(lse), n_blocks, block_len, heads, kv_heads, head_dim,
                                   int(bool(causal)), rank, _addr(dq), _ptr_array(dk_blocks),
                                   _ptr_array(dv_blocks), _stream(stream))


def ring_attn_workspace_bytes(block_len, kv_heads, head_dim, elem_bytes) -> int:
    return lib().ring_attn_workspace_bytes(block_len, kv_heads, head_dim, elem_bytes)


def ring_attn_set_workspace(dev_ptr, nbytes: int) -> None:
    """Use caller-owned device memory (an address or a tensor; None with 0 resets) as K/V staging."""
    _check(lib().ring_attn_set_workspace(_addr(dev_ptr) if dev_ptr is not None else None, int(nbytes)))


def ring_attn_decode(q, k_blocks, v_blocks, n_blocks, block_len, q_len, heads, kv_heads, head_dim, q_pos0, out,
                     lse, stream=None) -> int:
    return lib().ring_attn_decode(_addr(q), _ptr_array(k_blocks), _ptr_array(v_blocks), n_blocks, block_len, q_len,
                                  heads, kv_heads, head_dim, int(q_pos0), _addr(out), _addr(lse), _stream(stream))


def ring_attn_decode_noalloc(q, k_blocks, v_blocks, n_blocks, block_len, q_len, heads, kv_heads, head_dim, q_pos0,
                             out, lse, stream=None) -> int:
    """ring_attn_decode with its partials in the library's fixed device scratch (allocates nothing)."""
    return lib().ring_attn_decode_noalloc(_addr(q), _ptr_array(k_blocks), _ptr_array(v_blocks), n_blocks, block_len,
                                          q_len, heads, kv_heads, head_dim, int(q_pos0), _addr(out), _addr(lse),
                                          _stream(stream))


def ring_attn_ffn_blockwise(x, w1, b1, w2, b2, rows, hidden, ffn, chunk_rows, y, stream=None) -> int:
    return lib().ring_attn_ffn_blockwise(_addr(x), _addr(w1), _addr(b1), _addr(w2), _addr(b2), rows, hidden, ffn,
                                         chunk_rows, _addr(y), _stream(stream))


def ring_attn_mfma_rate(iters: int, sink, stream=None) -> float:
    """Dense bf16 MFMA TFLOP/s of a register-only loop (sink: >= MFMA_RATE_SINK_FLOATS device floats)."""
    out = ctypes.c_double()
    _check(lib().ring_attn_mfma_rate(int(iters), _addr(sink), ctypes.byref(out), _stream(stream)))
    return out.value


def ring_attn_profile_enable(enable: bool) -> int:
    return lib().ring_attn_profile_enable(int(bool(enable)))


def ring_attn_profile_read():
    """Returns ({kind: (ms, count)}, copy_ms, hidden_ms) and resets the records."""
    ms = (ctypes.c_double * len(PROFILE_KINDS))()
    cnt = (ctypes.c_int * len(PROFILE_KINDS))()
    cms, hid = ctypes.c_double(), ctypes.c_double()
    _check(lib().ring_attn_profile_read(ms, cnt, ctypes.byref(cms), ctypes.byref(hid)))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(PROFILE_KINDS)}, cms.value, hid.value


def ring_attn_schedule(rank: int, n_blocks: int, causal: bool) -> List[int]:
    """Block ids of the rounds one rank executes, in ring order (from the library)."""
    n = lib().ring_attn_schedule(rank, n_blocks, int(bool(causal)), None, 0)
    if n < 0:
        _check(-n)
    buf = (ctypes.c_int * max(1, n))()
    m = lib().ring_attn_schedule(rank, n_blocks, int(bool(causal)), buf, n)
    if m < 0:
        _check(-m)
    return list(buf[:m])


def ring_attn_debug(poison: bool, delay_cycles: int = 0) -> None:
    _check(lib().ring_attn_debug(int(bool(poison)), int(delay_cycles)))


def ring_attn_shutdown() -> None:
    lib().ring_attn_shutdown()


# ------------------------------------------------------------------ tensor conveniences
# The conveniences check, on the host and before anything is enqueued, that every
# tensor has exactly the shape, dtype and device the C call will read or write:
# the library only sees raw pointers, so a short or mistyped buffer would be read
# or written past its end on the GPU.
def _expect(t, name: str, shape: Tuple[int, ...], dtype, device) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")


def _expect_blocks(ts: Sequence, name: str, n: int, shape, dtype, device) -> None:
    if len(ts) != n:
        raise ValueError(f"{name}: expected {n} blocks, got {len(ts)}")
    for j, t in enumerate(ts):
        _expect(t, f"{name}[{j}]", shape, dtype, device)


def _dims(q, k_blocks) -> Tuple[int, int, int, int]:
    if q.dim() != 3:
        raise ValueError(f"q: expected [block_len, heads, head_dim], got shape {tuple(q.shape)}")
    if len(k_blocks) < 1:
        raise ValueError("k_blocks: at least one block is needed")
    if k_blocks[0].dim() != 3:
        raise ValueError(f"k_blocks[0]: expected [block_len, kv_heads, head_dim], got shape {tuple(k_blocks[0].shape)}")
    block_len, heads, head_dim = q.shape
    kv_heads = k_blocks[0].shape[1]
    return block_len, heads, kv_heads, head_dim


def _check_ring_inputs(q, k_blocks, v_blocks):
    """Shared checks of fwd/bwd: q [c, Hq, d]; every K/V block [c, Hkv, d] of q's dtype and device."""
    import torch
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"unsupported dtype {q.dtype}")
    c, hq, hkv, d = _dims(q, k_blocks)
    _expect_blocks(k_blocks, "k_blocks", len(k_blocks), (c, hkv, d), q.dtype, q.device)
    _expect_blocks(v_blocks, "v_blocks", len(k_blocks), (c, hkv, d), q.dtype, q.device)
    return c, hq, hkv, d


def fwd(q, k_blocks: List, v_blocks: List, *, causal: bool, rank: int, out=None, lse=None, stream=None,
        zigzag: bool = False):
    """Forward ring step on torch tensors; returns (out fp32 [c,Hq,d], lse fp32 [Hq,c]).

    zigzag=True selects the load-balanced layout (block b holds chunks b and 2D-1-b; bf16 only)."""
    import torch
    c, hq, hkv, d = _check_ring_inputs(q, k_blocks, v_blocks)
    if out is None:
        out = torch.empty((c, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((hq, c), dtype=torch.float32, device=q.device)
    _expect(out, "out", (c, hq, d), torch.float32, q.device)
    _expect(lse, "lse", (hq, c), torch.float32, q.device)
    fn = ring_attn_fwd if q.dtype == torch.bfloat16 else ring_attn_fwd_f32
    if zigzag:
        if q.dtype != torch.bfloat16:
            raise TypeError("the zig-zag layout takes bf16 inputs")
        fn = ring_attn_fwd_zigzag
    _check(fn(q, k_blocks, v_blocks, len(k_blocks), c, hq, hkv, d, causal, rank, out, lse, stream))
    return out, lse


def bwd(q, k_blocks: List, v_blocks: List, out, dout, lse, *, causal: bool, rank: int, dq=None,
        dk_blocks=None, dv_blocks=None, stream=None, zigzag: bool = False):
    """Backward ring step; dk/dv blocks are accumulated into (zero-initialised if not given)."""
    import torch
    c, hq, hkv, d = _check_ring_inputs(q, k_blocks, v_blocks)
    _expect(out, "out", (c, hq, d), torch.float32, q.device)
    _expect(dout, "dout", (c, hq, d), q.dtype, q.device)
    _expect(lse, "lse", (hq, c), torch.float32, q.device)
    if dq is None:
        dq = torch.empty((c, hq, d), dtype=torch.float32, device=q.device)
    if dk_blocks is None:
        dk_blocks = [torch.zeros((c, hkv, d), dtype=torch.float32, device=q.device) for _ in k_blocks]
    if dv_blocks is None:
        dv_blocks = [torch.zeros((c, hkv, d), dtype=torch.float32, device=q.device) for _ in k_blocks]
    _expect(dq, "dq", (c, hq, d), torch.float32, q.device)
    _expect_blocks(dk_blocks, "dk_blocks", len(k_blocks), (c, hkv, d), torch.float32, q.device)
    _expect_blocks(dv_blocks, "dv_blocks", len(k_blocks), (c, hkv, d), torch.float32, q.device)
    fn = ring_attn_bwd if q.dtype == torch.bfloat16 else ring_attn_bwd_f32
    if zigzag:
        if q.dtype != torch.bfloat16:
            raise TypeError("the zig-zag layout takes bf16 inputs")
        fn = ring_attn_bwd_zigzag
    _check(fn(q, k_blocks, v_blocks, out, dout, lse, len(k_blocks), c, hq, hkv, d, causal, rank, dq,
              dk_blocks, dv_blocks, stream))
    return dq, dk_blocks, dv_blocks


def decode(q, k_blocks: List, v_blocks: List, *, q_pos0: int, out=None, lse=None, stream=None):
    """Decode step: q [q_len, Hq, d] bf16 against every block; returns (out, lse)."""
    import torch
    if q.dim() != 3:
        raise ValueError(f"q: expected [q_len, heads, head_dim], got shape {tuple(q.shape)}")
    _expect(q, "q", tuple(q.shape), torch.bfloat16, q.device)
    q_len, hq, d = q.shape
    if len(k_blocks) < 1 or k_blocks[0].dim() != 3:
        raise ValueError("k_blocks: expected at least one [block_len, kv_heads, head_dim] block")
    block_len, hkv = k_blocks[0].shape[0], k_blocks[0].shape[1]
    _expect_blocks(k_blocks, "k_blocks", len(k_blocks), (block_len, hkv, d), torch.bfloat16, q.device)
    _expect_blocks(v_blocks, "v_blocks", len(k_blocks), (block_len, hkv, d), torch.bfloat16, q.device)
    if out is None:
        out = torch.empty((q_len, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((hq, q_len), dtype=torch.float32, device=q.device)
    _expect(out, "out", (q_len, hq, d), torch.float32, q.device)
    _expect(lse, "lse", (hq, q_len), torch.float32, q.device)
    _check(ring_attn_decode(q, k_blocks, v_blocks, len(k_blocks), block_len, q_len, hq, hkv, d, q_pos0, out, lse,
                            stream))
    return out, lse


def ffn_blockwise(x, w1, w2, *, b1=None, b2=None, chunk_rows: int = 0, y=None, stream=None):
    """y = GELU(x W1^T + b1) W2^T + b2 over row chunks; x [rows, hidden] bf16, weights [out, in] bf16."""
    import torch
    if x.dim() != 2 or w1.dim() != 2:
        raise ValueError("x and w1 must be 2-D ([rows, hidden] and [ffn, hidden])")
    rows, hidden = x.shape
    ffn = w1.shape[0]
    _expect(x, "x", (rows, hidden), torch.bfloat16, x.device)
    _expect(w1, "w1", (ffn, hidden), torch.bfloat16, x.device)
    _expect(w2, "w2", (hidden, ffn), torch.bfloat16, x.device)
    if b1 is not None:
        _expect(b1, "b1", (ffn,), torch.float32, x.device)
    if b2 is not None:
        _expect(b2, "b2", (hidden,), torch.float32, x.device)
    if y is None:
        y = torch.empty((rows, hidden), dtype=torch.float32, device=x.device)
    _expect(y, "y", (rows, hidden), torch.float32, x.device)
    _check(ring_attn_ffn_blockwise(x, w1, b1, w2, b2, rows, hidden, ffn, chunk_rows, y, stream))
    return y


def merge(out_a, lse_a, out_b, lse_b, *, out=None, lse=None, stream=None):
    import torch
    if out_a.dim() != 3:
        raise ValueError(f"out_a: expected [rows, heads, head_dim], got shape {tuple(out_a.shape)}")
    rows, heads, head_dim = out_a.shape
    dev = out_a.device
    _expect(out_a, "out_a", (rows, heads, head_dim), torch.float32, dev)
    _expect(out_b, "out_b", (rows, heads, head_dim), torch.float32, dev)
    _expect(lse_a, "lse_a", (heads, rows), torch.float32, dev)
    _expect(lse_b, "lse_b", (heads, rows), torch.float32, dev)
    if out is None:
        out = torch.empty_like(out_a)
    if lse is None:
        lse = torch.empty_like(lse_a)
    _expect(out, "out", (rows, heads, head_dim), torch.float32, dev)
    _expect(lse, "lse", (heads, rows), torch.float32, dev)
    _check(ring_attn_merge(out_a, lse_a, out_b, lse_b, rows, heads, head_dim, out, lse, stream))
    return out, lse
