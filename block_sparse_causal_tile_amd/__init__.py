"""Python binding of the MALA HIP library (``libmala.so``, C ABI in include/mala.h).

Argument marshalling only: every step of MassAlloc Attention runs in the HIP
kernels behind the C ABI. PyTorch supplies device memory and the stream.
There is no CPU fallback: if the library is missing or fails to load, using
any entry point raises.

Entry points mirror the C names: ``mala_fwd``, ``mala_bwd``, ``mala_decode``
(+ workspace-size queries and ``mala_error_string``) and the operator-fidelity
instrumentation ``mala_omitted_mass``, ``mala_sq_err_heads``,
``mala_slot_histogram`` and ``mala_rademacher``. Tensors are BSHD
``[batch, seq, heads, head_dim]`` contiguous CUDA tensors of one dtype
(bfloat16 or float32), with the softmax scale already folded into q.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MalaError", "MalaProblem", "lib_path", "load", "make_problem",
    "mala_fwd", "mala_bwd", "mala_decode", "mala_bwd_workspace_size",
    "mala_decode_workspace_size", "mala_error_string", "STAT_NAMES", "mala_omitted_mass",
    "mala_sq_err_heads", "mala_slot_histogram", "mala_rademacher", "mala_decode_paged",
    "mala_fwd_varlen", "mala_fwd_latent", "mala_decode_latent", "mala_bwd_latent",
    "mala_bwd_latent_workspace_size", "mala_decode_noalloc",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmala.so"

MALA_OK = 0
MALA_EINVAL = -1
MALA_EUNSUPPORTED = -2
MALA_EWORKSPACE = -3
MALA_EHIP = -4
MALA_ETOOLARGE = -5
MALA_NOALLOC_SCRATCH_BYTES = 64 << 20  # the device scratch behind mala_decode_noalloc
MALA_BF16 = 0
MALA_FP32 = 1
STAT_NAMES = ("legal_tiles", "retained_tiles", "post_score_slots", "loaded_tiles")

EXPORTED_SYMBOLS = ("mala_fwd", "mala_bwd", "mala_bwd_workspace_size", "mala_decode",
                    "mala_decode_workspace_size", "mala_error_string", "mala_omitted_mass",
                    "mala_sq_err_heads", "mala_slot_histogram", "mala_rademacher",
                    "mala_decode_paged", "mala_fwd_varlen", "mala_fwd_latent",
                    "mala_decode_latent", "mala_bwd_latent", "mala_bwd_latent_workspace_size",
                    "mala_decode_noalloc")


class MalaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {mala_error_string(status)} (status {status})")
        self.status = status


class MalaProblem(ctypes.Structure):
    """Mirror of ``mala_problem`` in include/mala.h."""
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("heads_q", ctypes.c_int64),
        ("heads_kv", ctypes.c_int64),
        ("seqlen_q", ctypes.c_int64),
        ("seqlen_k", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("block_q", ctypes.c_int32),
        ("block_k", ctypes.c_int32),
        ("tau", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("causal_offset", ctypes.c_int64),
    ]


_lib = None


def lib_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load():
    """Load libmala.so (built in-tree by ``block_sparse_causal_tile_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_sparse_causal_tile_amd.build` "
            "(MALA has no CPU fallback)")
    lib = ctypes.CDLL(path)
    p_prob = ctypes.POINTER(MalaProblem)
    vp = ctypes.c_void_p
    lib.mala_fwd.argtypes = [p_prob, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mala_fwd.restype = ctypes.c_int
    lib.mala_bwd_workspace_size.argtypes = [p_prob]
    lib.mala_bwd_workspace_size.restype = ctypes.c_size_t
    lib.mala_bwd.argtypes = [p_prob, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                             vp, vp, vp, vp]
    lib.mala_bwd.restype = ctypes.c_int
    lib.mala_decode_workspace_size.argtypes = [p_prob, ctypes.c_int]
    lib.mala_decode_workspace_size.restype = ctypes.c_size_t
    lib.mala_decode.argtypes = [p_prob, vp, vp, vp, vp, vp, ctypes.c_int, vp, ctypes.c_size_t,
                                vp, vp, vp]
    lib.mala_decode.restype = ctypes.c_int
    lib.mala_decode_noalloc.argtypes = [p_prob, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp]
    lib.mala_decode_noalloc.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.mala_fwd_varlen.argtypes = [p_prob, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, vp]
    lib.mala_fwd_varlen.restype = ctypes.c_int
    lib.mala_fwd_latent.argtypes = [p_prob, vp, vp, i64, vp, vp, vp, vp, vp]
    lib.mala_fwd_latent.restype = ctypes.c_int
    lib.mala_decode_latent.argtypes = [p_prob, vp, vp, i64, vp, vp, ctypes.c_int, vp, ctypes.c_size_t,
                                       vp, vp, vp]
    lib.mala_decode_latent.restype = ctypes.c_int
    lib.mala_bwd_latent_workspace_size.argtypes = [p_prob]
    lib.mala_bwd_latent_workspace_size.restype = ctypes.c_size_t
    lib.mala_bwd_latent.argtypes = [p_prob, vp, vp, i64, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp, vp, vp]
    lib.mala_bwd_latent.restype = ctypes.c_int
    lib.mala_decode_paged.argtypes = [p_prob, vp, vp, vp, vp, vp, i64, ctypes.c_int32, ctypes.c_int32,
                                      vp, vp, ctypes.c_int, vp, ctypes.c_size_t, vp, vp, vp]
    lib.mala_decode_paged.restype = ctypes.c_int
    lib.mala_omitted_mass.argtypes = [vp, vp, vp, i64, vp]
    lib.mala_omitted_mass.restype = ctypes.c_int
    lib.mala_sq_err_heads.argtypes = [vp, vp, i64, i64, i64, i64, ctypes.c_int32, vp, vp, vp]
    lib.mala_sq_err_heads.restype = ctypes.c_int
    lib.mala_slot_histogram.argtypes = [p_prob, vp, vp, vp]
    lib.mala_slot_histogram.restype = ctypes.c_int
    lib.mala_rademacher.argtypes = [vp, i64, ctypes.c_int32, ctypes.c_uint64, vp]
    lib.mala_rademacher.restype = ctypes.c_int
    lib.mala_error_string.argtypes = [ctypes.c_int]
    lib.mala_error_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def mala_error_string(status: int) -> str:
    return load().mala_error_string(int(status)).decode()


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return MALA_BF16
    if dt == torch.float32:
        return MALA_FP32
    raise TypeError(f"MALA supports bfloat16 and float32 tensors, got {dt}")


def make_problem(q: torch.Tensor, k: torch.Tensor, tau: float, block_q: int, block_k: int,
                 causal_offset: int | None = None) -> MalaProblem:
    """Problem descriptor from BSHD q [B, Nq, Hq, d] and k [B, Nk, Hkv, d];
    causal_offset defaults to Nk - Nq (bottom-right alignment)."""
    B, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    off = nk - nq if causal_offset is None else int(causal_offset)
    return MalaProblem(B, hq, hkv, nq, nk, d, int(block_q), int(block_k), float(tau),
                       _dtype_code(q.dtype), off)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("MALA tensors must be on a CUDA (HIP) device")
        if not t.is_contiguous():
            raise ValueError("MALA tensors must be contiguous (BSHD)")


def _expect(t, name, shape=None, dtype=None):
    """Shape / dtype check of one tensor argument before it reaches the
    kernels: a buffer smaller than the problem implies would be read or
    written out of bounds on the device."""
    if t is None:
        return
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")


def _expect_stats(stats):
    if stats is not None and (stats.dtype != torch.int64 or stats.numel() < 4):
        raise ValueError("stats: expected an int64 tensor of at least 4 elements")


def _expect_bshd(q, k, v, name_k="k", name_v="v", same_width=True):
    """q [B, Nq, Hq, d] and k, v [B, Nk, Hkv, d] of q's dtype."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be BSHD [batch, seq, heads, head_dim]")
    if k.shape[0] != q.shape[0] or (same_width and k.shape[3] != q.shape[3]):
        raise ValueError(f"{name_k}: shape {tuple(k.shape)} does not fit q {tuple(q.shape)}")
    _expect(k, name_k, dtype=q.dtype)
    if v is not None:
        _expect(v, name_v, shape=k.shape, dtype=q.dtype)


def _expect_mask(tile_mask, B, hq, nq, nk, bq, bk):
    _expect(tile_mask, "tile_mask", shape=(B, hq, num_blocks(nq, bq), num_blocks(nk, bk)), dtype=torch.uint8)


def _expect_decode_mask(tile_mask, B, hq, nk, bk):
    _expect(tile_mask, "tile_mask", shape=(B, hq, num_blocks(nk, bk)), dtype=torch.uint8)


def _decode_z(q, z):
    """z of a decode of q [B, N_q, Hq, d]: [B, Hq, N_q] float32, or [B, Hq]
    for a single token (allocated here when None)."""
    B, nq, hq, _ = q.shape
    shape = (B, hq) if nq == 1 else (B, hq, nq)
    if z is None:
        return torch.empty(shape, device=q.device, dtype=torch.float32)
    if nq == 1 and tuple(z.shape) == (B, hq, 1):
        shape = (B, hq, 1)
    _expect(z, "z", shape=shape, dtype=torch.float32)
    return z


def _raise(st, what):
    if st != MALA_OK:
        raise MalaError(st, what)


def mala_fwd(q, k, v, tau: float, block_q: int, block_k: int, causal_offset=None, o=None,
             z=None, stats=None, tile_mask=None, stream=None):
    """MALA forward. Returns (o [B, Nq, Hq, d], z [B, Hq, Nq] float32).
    ``stats`` (int64[4]) is added to; ``tile_mask`` (uint8 [B, Hq, nQB, nKB])
    receives 1/0 for legal tiles."""
    lib = load()
    _expect_bshd(q, k, v)
    prob = make_problem(q, k, tau, block_q, block_k, causal_offset)
    if o is None:
        o = torch.empty_like(q)
    if z is None:
        z = torch.empty((q.shape[0], q.shape[2], q.shape[1]), device=q.device, dtype=torch.float32)
    B, nq, hq, _ = q.shape
    _expect(o, "o", shape=q.shape, dtype=q.dtype)
    _expect(z, "z", shape=(B, hq, nq), dtype=torch.float32)
    _expect_stats(stats)
    _expect_mask(tile_mask, B, hq, nq, k.shape[1], block_q, block_k)
    _check(q, k, v, o, z, stats, tile_mask)
    st = lib.mala_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(z),
                      _ptr(stats), _ptr(tile_mask), _stream(stream))
    _raise(st, "mala_fwd")
    return o, z


def mala_fwd_latent(q, kv, d_v: int, tau: float, block_q: int, block_k: int, causal_offset=None,
                    o=None, z=None, stats=None, tile_mask=None, stream=None):
    """MALA forward on latent (MLA-shaped) attention: q [B, Nq, Hq, d_qk],
    kv [B, Nk, 1, d_qk]; the value is kv[..., :d_v]. Returns
    (o [B, Nq, Hq, d_v], z [B, Hq, Nq] float32)."""
    lib = load()
    _expect_bshd(q, kv, None, name_k="kv")
    prob = make_problem(q, kv, tau, block_q, block_k, causal_offset)
    if o is None:
        o = torch.empty(q.shape[:3] + (int(d_v),), device=q.device, dtype=q.dtype)
    if z is None:
        z = torch.empty((q.shape[0], q.shape[2], q.shape[1]), device=q.device, dtype=torch.float32)
    B, nq, hq, _ = q.shape
    _expect(o, "o", shape=q.shape[:3] + (int(d_v),), dtype=q.dtype)
    _expect(z, "z", shape=(B, hq, nq), dtype=torch.float32)
    _expect_stats(stats)
    _expect_mask(tile_mask, B, hq, nq, kv.shape[1], block_q, block_k)
    _check(q, kv, o, z, stats, tile_mask)
    st = lib.mala_fwd_latent(ctypes.byref(prob), _ptr(q), _ptr(kv), int(d_v), _ptr(o), _ptr(z),
                             _ptr(stats), _ptr(tile_mask), _stream(stream))
    _raise(st, "mala_fwd_latent")
    return o, z


def mala_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    tau: float, block_q: int, block_k: int, o=None, z=None, stats=None, tile_mask=None,
                    stream=None):
    """MALA forward over packed sequences: q [total_q, Hq, d], k, v
    [total_k, Hkv, d]; cu_seqlens_* int32 [B + 1]. Per-sequence bottom-right
    causal alignment. Returns (o [total_q, Hq, d], z [Hq, total_q] float32)."""
    lib = load()
    total_q, hq, d = q.shape
    total_k, hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1 or cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens_q / cu_seqlens_k must be int32 [B + 1]")
    prob = MalaProblem(B, hq, hkv, int(max_seqlen_q), int(max_seqlen_k), d, int(block_q), int(block_k),
                       float(tau), _dtype_code(q.dtype), 0)
    o = torch.empty_like(q) if o is None else o
    if z is None:
        z = torch.empty((hq, total_q), device=q.device, dtype=torch.float32)
    if k.dim() != 3 or k.shape[2] != d:
        raise ValueError(f"k: expected [total_k, Hkv, {d}], got {tuple(k.shape)}")
    _expect(k, "k", dtype=q.dtype)
    _expect(v, "v", shape=k.shape, dtype=q.dtype)
    _expect(o, "o", shape=q.shape, dtype=q.dtype)
    _expect(z, "z", shape=(hq, total_q), dtype=torch.float32)
    _expect_stats(stats)
    _expect_mask(tile_mask, B, hq, int(max_seqlen_q), int(max_seqlen_k), block_q, block_k)
    _check(q, k, v, cu_seqlens_q, cu_seqlens_k, o, z, stats, tile_mask)
    st = lib.mala_fwd_varlen(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                             _ptr(cu_seqlens_k), total_q, total_k, _ptr(o), _ptr(z), _ptr(stats),
                             _ptr(tile_mask), _stream(stream))
    _raise(st, "mala_fwd_varlen")
    return o, z


def mala_bwd_workspace_size(prob: MalaProblem) -> int:
    return int(load().mala_bwd_workspace_size(ctypes.byref(prob)))


def mala_bwd(q, k, v, o, dout, z, tau: float, block_q: int, block_k: int, causal_offset=None,
             dq=None, dk=None, dv=None, workspace=None, stats=None, tile_mask=None, tile_mask_dq=None,
             stream=None):
    """MALA backward. Returns (dq, dk, dv); dk/dv are summed over each KV
    group's query heads. ``tile_mask`` receives the key-major pass's
    decisions, ``tile_mask_dq`` the query-major dQ pass's own."""
    lib = load()
    _expect_bshd(q, k, v)
    prob = make_problem(q, k, tau, block_q, block_k, causal_offset)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = mala_bwd_workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q.device, dtype=torch.uint8)
    B, nq, hq, _ = q.shape
    for t, n in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _expect(t, n, shape=q.shape, dtype=q.dtype)
    _expect(dk, "dk", shape=k.shape, dtype=q.dtype)
    _expect(dv, "dv", shape=k.shape, dtype=q.dtype)
    _expect(z, "z", shape=(B, hq, nq), dtype=torch.float32)
    _expect_stats(stats)
    _expect_mask(tile_mask, B, hq, nq, k.shape[1], block_q, block_k)
    _expect_mask(tile_mask_dq, B, hq, nq, k.shape[1], block_q, block_k)
    _check(q, k, v, o, dout, z, dq, dk, dv, workspace, stats, tile_mask, tile_mask_dq)
    st = lib.mala_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(z),
                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                      workspace.numel() * workspace.element_size(), _ptr(stats), _ptr(tile_mask),
                      _ptr(tile_mask_dq), _stream(stream))
    _raise(st, "mala_bwd")
    return dq, dk, dv


def mala_decode_workspace_size(prob: MalaProblem, num_splits: int) -> int:
    return int(load().mala_decode_workspace_size(ctypes.byref(prob), int(num_splits)))


def mala_decode(q, k_cache, v_cache, tau: float, block_k: int, num_splits: int = 1, o=None,
                z=None, workspace=None, stats=None, tile_mask=None, stream=None):
    """MALA decode of a short query: q [B, N_q, Hq, d] holds the N_q newest
    tokens (N_q = 1: single-token decode), caches [B, Nk, Hkv, d]. Returns
    (o [B, N_q, Hq, d], z [B, Hq, N_q] float32; [B, Hq] when N_q = 1)."""
    lib = load()
    _expect_bshd(q, k_cache, v_cache, "k_cache", "v_cache")
    prob = make_problem(q, k_cache, tau, 1, block_k, k_cache.shape[1] - q.shape[1])
    o = torch.empty_like(q) if o is None else o
    z = _decode_z(q, z)
    need = mala_decode_workspace_size(prob, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q.device, dtype=torch.uint8)
    B, _, hq, _ = q.shape
    _expect(o, "o", shape=q.shape, dtype=q.dtype)
    _expect_stats(stats)
    _expect_decode_mask(tile_mask, B, hq, k_cache.shape[1], block_k)
    _check(q, k_cache, v_cache, o, z, workspace, stats, tile_mask)
    st = lib.mala_decode(ctypes.byref(prob), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o),
                         _ptr(z), int(num_splits), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _ptr(stats),
                         _ptr(tile_mask), _stream(stream))
    _raise(st, "mala_decode")
    return o, z


def mala_decode_noalloc(q, k_cache, v_cache, tau: float, block_k: int, num_splits: int = 1, o=None, z=None,
                        stats=None, tile_mask=None, stream=None):
    """``mala_decode`` without a workspace: the split partials live in the
    library's per-device scratch array (``MALA_NOALLOC_SCRATCH_BYTES``), so
    the C call allocates nothing - for callers under graph capture or in
    loops that must not allocate (pass ``o`` and ``z`` to allocate nothing
    here either). Calls that overlap on one GPU race on the scratch. Raises
    MalaError(MALA_ETOOLARGE) when the partials exceed the scratch."""
    lib = load()
    _expect_bshd(q, k_cache, v_cache, "k_cache", "v_cache")
    prob = make_problem(q, k_cache, tau, 1, block_k, k_cache.shape[1] - q.shape[1])
    o = torch.empty_like(q) if o is None else o
    z = _decode_z(q, z)
    B, _, hq, _ = q.shape
    _expect(o, "o", shape=q.shape, dtype=q.dtype)
    _expect_stats(stats)
    _expect_decode_mask(tile_mask, B, hq, k_cache.shape[1], block_k)
    _check(q, k_cache, v_cache, o, z, stats, tile_mask)
    st = lib.mala_decode_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(z),
                                 int(num_splits), _ptr(stats), _ptr(tile_mask), _stream(stream))
    _raise(st, "mala_decode_noalloc")
    return o, z


def mala_bwd_latent_workspace_size(prob: MalaProblem) -> int:
    return int(load().mala_bwd_latent_workspace_size(ctypes.byref(prob)))


def mala_bwd_latent(q, kv, d_v: int, o, dout, z, tau: float, block_q: int, block_k: int, causal_offset=None,
                    dq=None, dkv=None, workspace=None, stats=None, tile_mask=None, tile_mask_dq=None,
                    stream=None):
    """MALA backward on latent (MLA-shaped) attention: q [B, Nq, Hq, d_qk],
    kv [B, Nk, 1, d_qk], o and dout [B, Nq, Hq, d_v], z [B, Hq, Nq]. Returns
    (dq [B, Nq, Hq, d_qk], dkv [B, Nk, 1, d_qk]); dkv = dK + [dV, 0] summed
    over the query heads."""
    lib = load()
    _expect_bshd(q, kv, None, name_k="kv")
    prob = make_problem(q, kv, tau, block_q, block_k, causal_offset)
    dq = torch.empty_like(q) if dq is None else dq
    dkv = torch.empty_like(kv) if dkv is None else dkv
    need = mala_bwd_latent_workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q.device, dtype=torch.uint8)
    B, nq, hq, _ = q.shape
    for t, n in ((o, "o"), (dout, "dout")):
        _expect(t, n, shape=q.shape[:3] + (int(d_v),), dtype=q.dtype)
    _expect(dq, "dq", shape=q.shape, dtype=q.dtype)
    _expect(dkv, "dkv", shape=kv.shape, dtype=q.dtype)
    _expect(z, "z", shape=(B, hq, nq), dtype=torch.float32)
    _expect_stats(stats)
    _expect_mask(tile_mask, B, hq, nq, kv.shape[1], block_q, block_k)
    _expect_mask(tile_mask_dq, B, hq, nq, kv.shape[1], block_q, block_k)
    _check(q, kv, o, dout, z, dq, dkv, workspace, stats, tile_mask, tile_mask_dq)
    st = lib.mala_bwd_latent(ctypes.byref(prob), _ptr(q), _ptr(kv), int(d_v), _ptr(o), _ptr(dout), _ptr(z),
                             _ptr(dq), _ptr(dkv), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _ptr(stats), _ptr(tile_mask), _ptr(tile_mask_dq), _stream(stream))
    _raise(st, "mala_bwd_latent")
    return dq, dkv


def mala_decode_latent(q, kv_cache, d_v: int, tau: float, block_k: int, num_splits: int = 1, o=None,
                       z=None, workspace=None, stats=None, tile_mask=None, stream=None):
    """Single-token MALA decode on latent (MLA-shaped) attention: q [B, 1, Hq, d_qk],
    kv_cache [B, Nk, 1, d_qk]; the value is kv_cache[..., :d_v]. Returns
    (o [B, 1, Hq, d_v], z [B, Hq] float32)."""
    lib = load()
    _expect_bshd(q, kv_cache, None, name_k="kv_cache")
    prob = make_problem(q, kv_cache, tau, 1, block_k, kv_cache.shape[1] - 1)
    if o is None:
        o = torch.empty(q.shape[:3] + (int(d_v),), device=q.device, dtype=q.dtype)
    if z is None:
        z = torch.empty((q.shape[0], q.shape[2]), device=q.device, dtype=torch.float32)
    need = mala_decode_workspace_size(prob, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q.device, dtype=torch.uint8)
    B, _, hq, _ = q.shape
    _expect(o, "o", shape=q.shape[:3] + (int(d_v),), dtype=q.dtype)
    _expect(z, "z", shape=(B, hq), dtype=torch.float32)
    _expect_stats(stats)
    _expect_decode_mask(tile_mask, B, hq, kv_cache.shape[1], block_k)
    _check(q, kv_cache, o, z, workspace, stats, tile_mask)
    st = lib.mala_decode_latent(ctypes.byref(prob), _ptr(q), _ptr(kv_cache), int(d_v), _ptr(o),
                                _ptr(z), int(num_splits), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _ptr(stats),
                                _ptr(tile_mask), _stream(stream))
    _raise(st, "mala_decode_latent")
    return o, z


def mala_decode_paged(q, k_pages, v_pages, block_table, seq_lens, tau: float, block_k: int,
                      num_splits: int = 1, o=None, z=None, workspace=None, stats=None, tile_mask=None,
                      stream=None):
    """MALA decode of a short query over a paged cache: q [B, N_q, Hq, d]
    (the N_q newest tokens of each sequence); k_pages, v_pages [num_pages,
    page_size, Hkv, d]; block_table int32 [B, max_pages]; seq_lens int32 [B].
    Returns (o [B, N_q, Hq, d], z [B, Hq, N_q]; [B, Hq] when N_q = 1)."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, N_q, Hq, d]")
    B, nq, hq, d = q.shape
    num_pages, page_size, hkv, _ = k_pages.shape
    max_pages = block_table.shape[1]
    cap = max_pages * page_size
    prob = MalaProblem(B, hq, hkv, nq, cap, d, 1, int(block_k), float(tau), _dtype_code(q.dtype), cap - nq)
    o = torch.empty_like(q) if o is None else o
    z = _decode_z(q, z)
    need = mala_decode_workspace_size(prob, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q.device, dtype=torch.uint8)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if k_pages.dim() != 4 or k_pages.shape[3] != d:
        raise ValueError("k_pages must be [num_pages, page_size, Hkv, d]")
    _expect(k_pages, "k_pages", dtype=q.dtype)
    _expect(v_pages, "v_pages", shape=k_pages.shape, dtype=q.dtype)
    _expect(block_table, "block_table", shape=(B, max_pages))
    _expect(seq_lens, "seq_lens", shape=(B,))
    _expect(o, "o", shape=q.shape, dtype=q.dtype)
    _expect_stats(stats)
    _expect_decode_mask(tile_mask, B, hq, cap, block_k)
    _check(q, k_pages, v_pages, block_table, seq_lens, o, z, workspace, stats, tile_mask)
    st = lib.mala_decode_paged(ctypes.byref(prob), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                               _ptr(seq_lens), num_pages, page_size, max_pages, _ptr(o), _ptr(z),
                               int(num_splits), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _ptr(stats), _ptr(tile_mask), _stream(stream))
    _raise(st, "mala_decode_paged")
    return o, z


def mala_omitted_mass(z_screened, z_reference, out=None, stream=None):
    """Per-row omitted mass 1 - exp(z_screened - z_reference) (float32, same
    shape as the inputs)."""
    lib = load()
    if z_screened.shape != z_reference.shape or z_screened.dtype != torch.float32 \
            or z_reference.dtype != torch.float32:
        raise ValueError("z_screened and z_reference must be float32 tensors of one shape")
    out = torch.empty_like(z_screened) if out is None else out
    _check(z_screened, z_reference, out)
    st = lib.mala_omitted_mass(_ptr(z_screened), _ptr(z_reference), _ptr(out), z_screened.numel(),
                               _stream(stream))
    _raise(st, "mala_omitted_mass")
    return out


def mala_sq_err_heads(x, ref, stream=None):
    """Per-(batch, head) float64 sums of (x - ref)^2 and ref^2 for BSHD x, ref.
    Returns (sq_diff, sq_ref), each [batch, heads]."""
    lib = load()
    if x.shape != ref.shape or x.dtype != ref.dtype or x.dim() != 4:
        raise ValueError("x and ref must be BSHD tensors of one shape and dtype")
    B, n, h, d = x.shape
    sd = torch.empty((B, h), device=x.device, dtype=torch.float64)
    sr = torch.empty((B, h), device=x.device, dtype=torch.float64)
    _check(x, ref, sd, sr)
    st = lib.mala_sq_err_heads(_ptr(x), _ptr(ref), B, n, h, d, _dtype_code(x.dtype), _ptr(sd), _ptr(sr),
                               _stream(stream))
    _raise(st, "mala_sq_err_heads")
    return sd, sr


def mala_slot_histogram(tile_mask, seqlen_q: int, seqlen_k: int, block_q: int, block_k: int,
                        heads_kv: int | None = None, hist=None, stream=None):
    """Histogram over query rows of the number of retained tiles in the row's
    query block (post-score slots per query = index * block_k), from a tile
    mask [B, Hq, nQB, nKB] of mala_fwd or mala_bwd. Returns int64 [nKB + 1]
    (``hist``, if given, is added to)."""
    lib = load()
    B, hq, nqb, nkb = tile_mask.shape
    prob = MalaProblem(B, hq, hq if heads_kv is None else heads_kv, int(seqlen_q), int(seqlen_k), 1,
                       int(block_q), int(block_k), 0.0, MALA_BF16, int(seqlen_k) - int(seqlen_q))
    if hist is None:
        hist = torch.zeros(nkb + 1, device=tile_mask.device, dtype=torch.int64)
    if tile_mask.dtype != torch.uint8 or nqb != num_blocks(seqlen_q, block_q) \
            or nkb != num_blocks(seqlen_k, block_k) or hist.numel() < nkb + 1:
        raise ValueError("tile_mask must be uint8 [B, Hq, ceil(Nq/Bq), ceil(Nk/Bk)], hist int64 [nKB+1]")
    _check(tile_mask, hist)
    st = lib.mala_slot_histogram(ctypes.byref(prob), _ptr(tile_mask), _ptr(hist), _stream(stream))
    _raise(st, "mala_slot_histogram")
    return hist


def mala_rademacher(shape, seed: int, dtype=torch.bfloat16, device="cuda", out=None, stream=None):
    """Deterministic +-1 tensor: element i (row-major) is -1 iff the top bit of
    SplitMix64 output i for ``seed`` is set."""
    lib = load()
    out = torch.empty(shape, device=device, dtype=dtype) if out is None else out
    _check(out)
    st = lib.mala_rademacher(_ptr(out), out.numel(), _dtype_code(out.dtype),
                             ctypes.c_uint64(int(seed) & ((1 << 64) - 1)), _stream(stream))
    _raise(st, "mala_rademacher")
    return out


def num_blocks(n: int, b: int) -> int:
    return (n + b - 1) // b


def new_tile_mask(batch, heads_q, seqlen_q, seqlen_k, block_q, block_k, device):
    """A debug mask buffer prefilled with 255 (= not a legal tile)."""
    return torch.full((batch, heads_q, num_blocks(seqlen_q, block_q), num_blocks(seqlen_k, block_k)),
                      255, dtype=torch.uint8, device=device)


def new_stats(device):
    return torch.zeros(4, dtype=torch.int64, device=device)

