"""The C ABI library loads, exports what include/mala.h declares, and its
host-side validation returns the documented status codes (no kernel is
launched by any call here, so no GPU is needed)."""

import ctypes
import os
import re

import pytest

import block_sparse_causal_tile_amd as mala

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mala.lib_path()):
        from block_sparse_causal_tile_amd import build
        build.build()
    return mala.load()


def declared_functions():
    with open(os.path.join(ROOT, "include", "mala.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(mala_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"mala_fwd", "mala_bwd", "mala_decode", "mala_error_string",
                          "mala_bwd_workspace_size", "mala_decode_workspace_size"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(mala.EXPORTED_SYMBOLS) <= set(names)


def test_problem_struct_layout():
    assert ctypes.sizeof(mala.MalaProblem) == 72
    assert mala.MalaProblem.causal_offset.offset == 64
    assert mala.MalaProblem.tau.offset == 56


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first


def prob(**kw):
    base = dict(batch=1, heads_q=4, heads_kv=2, seqlen_q=128, seqlen_k=128, head_dim=128,
                block_q=64, block_k=64, tau=0.05, dtype=0, causal_offset=0)
    base.update(kw)
    return mala.MalaProblem(**base)


def fwd(lib, p, ptr=FAKE):
    return lib.mala_fwd(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, None, None, None)


@pytest.mark.parametrize("kw", [
    dict(heads_q=3), dict(tau=-0.1), dict(tau=float("nan")), dict(tau=float("inf")),
    dict(causal_offset=-1), dict(seqlen_q=129), dict(causal_offset=1), dict(batch=0),
    dict(head_dim=0), dict(block_q=0), dict(heads_q=1 << 18, heads_kv=1 << 18),  # row > 2^24 elements
])
def test_fwd_invalid(lib, kw):
    assert fwd(lib, prob(**kw)) == mala.MALA_EINVAL


def test_fwd_null_and_misaligned(lib):
    assert fwd(lib, prob(), ptr=None) == mala.MALA_EINVAL
    assert fwd(lib, prob(), ptr=ctypes.c_void_p((1 << 20) + 2)) == mala.MALA_EINVAL


@pytest.mark.parametrize("kw", [dict(head_dim=96), dict(block_q=32), dict(block_k=256),
                                dict(dtype=7)])
def test_fwd_unsupported(lib, kw):
    assert fwd(lib, prob(**kw)) == mala.MALA_EUNSUPPORTED


def test_workspace_queries(lib):
    p = prob()
    rows = 1 * 4 * 128
    up = lambda x: (x + 255) // 256 * 256
    # three fp32 row values (rows padded to a multiple of 128), 1024 partial
    # maxima of |dO|, the scale, dO as 16-bit values
    assert lib.mala_bwd_workspace_size(ctypes.byref(p)) == up(rows * 3 * 4) + 4096 + 256 + up(rows * 128 * 2)
    assert lib.mala_bwd_workspace_size(ctypes.byref(prob(heads_q=3))) == 0
    d = prob(seqlen_q=1, causal_offset=127, block_q=1, block_k=64)
    assert lib.mala_decode_workspace_size(ctypes.byref(d), 2) == 1 * 4 * 2 * 128 * 4 + 256
    assert lib.mala_decode_workspace_size(ctypes.byref(d), 0) == 0
    d4 = prob(seqlen_q=4, causal_offset=124, block_q=1, block_k=64)  # partials of every token
    assert lib.mala_decode_workspace_size(ctypes.byref(d4), 2) == 1 * 4 * 4 * 2 * 128 * 4 + 256


def test_bwd_workspace_too_small(lib):
    p = prob()
    args = [ctypes.byref(p)] + [FAKE] * 9 + [FAKE, ctypes.c_size_t(16), None, None, None, None]
    assert lib.mala_bwd(*args) == mala.MALA_EWORKSPACE
    args[10] = None
    args[11] = ctypes.c_size_t(1 << 30)
    assert lib.mala_bwd(*args) == mala.MALA_EWORKSPACE


def test_decode_invalid(lib):
    ws = ctypes.c_size_t(1 << 30)
    good = prob(seqlen_q=1, causal_offset=127, block_q=1, block_k=64)
    call = lambda p, s: lib.mala_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, s, FAKE,
                                        ws, None, None, None)
    assert call(prob(seqlen_q=2, causal_offset=127), 1) == mala.MALA_EINVAL   # offset must be N_k - N_q
    assert call(prob(seqlen_q=1, causal_offset=100), 1) == mala.MALA_EINVAL
    assert call(prob(seqlen_q=17, causal_offset=111), 1) == mala.MALA_EINVAL  # at most 16 tokens
    # 2 heads per KV group x 9 tokens > the 16 columns of one matrix-core op
    assert call(prob(seqlen_q=9, causal_offset=119), 1) == mala.MALA_EUNSUPPORTED
    assert call(good, 0) == mala.MALA_EINVAL
    assert call(good, 3) == mala.MALA_EINVAL  # only 2 tiles
    assert call(prob(seqlen_q=1, causal_offset=127, block_k=64, head_dim=64), 1) == \
        mala.MALA_EUNSUPPORTED


def test_decode_latent_validation(lib):
    ws = ctypes.c_size_t(1 << 30)

    def call(p, s=1, dv=512, ptr=FAKE, wsb=ws):
        return lib.mala_decode_latent(ctypes.byref(p), ptr, ptr, dv, ptr, ptr, s, FAKE, wsb,
                                      None, None, None)
    ok = dict(heads_q=16, heads_kv=1, head_dim=576, seqlen_q=1, seqlen_k=256, causal_offset=255,
              block_q=1, block_k=64)
    assert call(prob(**dict(ok, heads_kv=2))) == mala.MALA_EINVAL      # one cached row
    assert call(prob(**ok), dv=0) == mala.MALA_EINVAL
    assert call(prob(**ok), dv=584) == mala.MALA_EINVAL                # wider than the row
    assert call(prob(**ok), dv=508) == mala.MALA_EINVAL                # not a multiple of 8
    assert call(prob(**ok), ptr=None) == mala.MALA_EINVAL
    assert call(prob(**dict(ok, seqlen_q=2, causal_offset=254))) == mala.MALA_EINVAL
    assert call(prob(**dict(ok, causal_offset=100))) == mala.MALA_EINVAL
    assert call(prob(**ok), s=0) == mala.MALA_EINVAL
    assert call(prob(**ok), s=5) == mala.MALA_EINVAL                   # only 4 tiles
    assert call(prob(**ok), wsb=ctypes.c_size_t(16)) == mala.MALA_EWORKSPACE
    # well-formed but not compiled: other widths, tiles, head counts or dtype
    assert call(prob(**ok), dv=256) == mala.MALA_EUNSUPPORTED
    assert call(prob(**dict(ok, block_k=128))) == mala.MALA_EUNSUPPORTED
    assert call(prob(**dict(ok, heads_q=8))) == mala.MALA_EUNSUPPORTED
    assert call(prob(**dict(ok, dtype=1))) == mala.MALA_EUNSUPPORTED


def test_bwd_latent_validation(lib):
    ws = ctypes.c_size_t(1 << 34)

    def call(p, dv=512, ptr=FAKE, wsb=ws):
        return lib.mala_bwd_latent(ctypes.byref(p), ptr, ptr, dv, ptr, ptr, ptr, ptr, ptr, FAKE, wsb,
                                   None, None, None, None)
    ok = dict(heads_q=16, heads_kv=1, head_dim=576, seqlen_q=256, seqlen_k=256)
    assert call(prob(**dict(ok, heads_kv=2))) == mala.MALA_EINVAL      # one cached row
    assert call(prob(**ok), dv=0) == mala.MALA_EINVAL
    assert call(prob(**ok), dv=584) == mala.MALA_EINVAL
    assert call(prob(**ok), dv=508) == mala.MALA_EINVAL
    assert call(prob(**ok), ptr=None) == mala.MALA_EINVAL
    assert call(prob(**dict(ok, causal_offset=1))) == mala.MALA_EINVAL
    assert call(prob(**ok), wsb=ctypes.c_size_t(16)) == mala.MALA_EWORKSPACE
    assert call(prob(**ok), dv=256) == mala.MALA_EUNSUPPORTED
    assert call(prob(**dict(ok, block_q=128))) == mala.MALA_EUNSUPPORTED
    assert call(prob(**dict(ok, dtype=1))) == mala.MALA_EUNSUPPORTED
    # workspace: D_q, then one fp32 partial of dKV per head group
    p = prob(**ok)
    rows = 16 * 256
    assert lib.mala_bwd_latent_workspace_size(ctypes.byref(p)) >= rows * 4 + 256 * 576 * 4
    assert lib.mala_bwd_latent_workspace_size(ctypes.byref(prob(**dict(ok, heads_kv=2)))) == 0


def test_error_strings(lib):
    for st in (0, -1, -2, -3, -4, 5):
        assert mala.mala_error_string(st).startswith("MALA")


def test_fidelity_validation(lib):
    i64 = ctypes.c_int64
    assert lib.mala_omitted_mass(FAKE, FAKE, FAKE, i64(0), None) == mala.MALA_EINVAL
    assert lib.mala_omitted_mass(None, FAKE, FAKE, i64(8), None) == mala.MALA_EINVAL
    assert lib.mala_sq_err_heads(FAKE, FAKE, i64(1), i64(0), i64(1), i64(8), 0, FAKE, FAKE,
                                 None) == mala.MALA_EINVAL
    assert lib.mala_sq_err_heads(FAKE, FAKE, i64(1), i64(4), i64(1), i64(8), 9, FAKE, FAKE,
                                 None) == mala.MALA_EUNSUPPORTED
    assert lib.mala_slot_histogram(ctypes.byref(prob(heads_q=3)), FAKE, FAKE, None) == mala.MALA_EINVAL
    assert lib.mala_slot_histogram(ctypes.byref(prob()), None, FAKE, None) == mala.MALA_EINVAL
    assert lib.mala_rademacher(FAKE, i64(-1), 0, ctypes.c_uint64(1), None) == mala.MALA_EINVAL
    assert lib.mala_rademacher(FAKE, i64(16), 5, ctypes.c_uint64(1), None) == mala.MALA_EUNSUPPORTED
    assert lib.mala_rademacher(ctypes.c_void_p((1 << 20) + 4), i64(16), 0, ctypes.c_uint64(1),
                               None) == mala.MALA_EINVAL


def test_decode_paged_validation(lib):
    P, maxp = 16, 8
    cap = P * maxp
    dp = prob(seqlen_q=1, seqlen_k=cap, causal_offset=cap - 1, block_k=64)
    ws = ctypes.c_size_t(1 << 20)
    i64, i32 = ctypes.c_int64, ctypes.c_int32

    def call(p=dp, table=FAKE, lens=FAKE, pages=16, page=P, mp=maxp, splits=1):
        return lib.mala_decode_paged(ctypes.byref(p), FAKE, FAKE, FAKE, table, lens, i64(pages), i32(page),
                                     i32(mp), FAKE, FAKE, splits, FAKE, ws, None, None, None)

    assert call(table=None) == mala.MALA_EINVAL
    assert call(lens=ctypes.c_void_p((1 << 20) + 2)) == mala.MALA_EINVAL
    assert call(page=24) == mala.MALA_EINVAL                   # not a power of two
    assert call(page=8) == mala.MALA_EINVAL                    # below 16
    assert call(mp=4) == mala.MALA_EINVAL                      # seqlen_k != capacity
    assert call(pages=0) == mala.MALA_EINVAL
    assert call(splits=3) == mala.MALA_EINVAL                  # > ceil(128 / 64)
    assert call(p=prob(seqlen_q=2, seqlen_k=cap, causal_offset=cap - 1)) == mala.MALA_EINVAL
    assert call(p=prob(seqlen_q=9, seqlen_k=cap, causal_offset=cap - 9)) == mala.MALA_EUNSUPPORTED
    bad = prob(seqlen_q=1, seqlen_k=cap, causal_offset=cap - 1, block_k=32)
    assert call(p=bad) == mala.MALA_EUNSUPPORTED


def test_fwd_varlen_validation(lib):
    i64 = ctypes.c_int64

    def call(p=None, cu=FAKE, tq=100, tk=100):
        p = p or prob()
        return lib.mala_fwd_varlen(ctypes.byref(p), FAKE, FAKE, FAKE, cu, FAKE, i64(tq), i64(tk), FAKE, FAKE,
                                   None, None, None)

    assert call(cu=None) == mala.MALA_EINVAL
    assert call(cu=ctypes.c_void_p((1 << 20) + 2)) == mala.MALA_EINVAL
    assert call(tq=0) == mala.MALA_EINVAL
    assert call(p=prob(causal_offset=3, seqlen_k=256)) == mala.MALA_EINVAL
    assert call(p=prob(heads_q=3)) == mala.MALA_EINVAL
    assert call(p=prob(dtype=1)) == mala.MALA_EUNSUPPORTED
    assert call(p=prob(head_dim=96)) == mala.MALA_EUNSUPPORTED


def test_fwd_latent_validation(lib):
    def call(p, dv=512, ptr=FAKE):
        return lib.mala_fwd_latent(ctypes.byref(p), ptr, ptr, dv, ptr, ptr, None, None, None)
    ok = dict(heads_q=16, heads_kv=1, head_dim=576)
    assert call(prob(**dict(ok, heads_kv=2, heads_q=16))) == mala.MALA_EINVAL  # one cached row
    assert call(prob(**ok), dv=0) == mala.MALA_EINVAL
    assert call(prob(**ok), dv=580) == mala.MALA_EINVAL   # wider than the row
    assert call(prob(**ok), dv=500) == mala.MALA_EINVAL   # not a multiple of 8
    assert call(prob(**ok), ptr=None) == mala.MALA_EINVAL
    assert call(prob(**dict(ok, tau=-1.0))) == mala.MALA_EINVAL
    # well-formed but not compiled: other widths, tiles or dtype
    assert call(prob(**ok), dv=256) == mala.MALA_EUNSUPPORTED
    assert call(prob(**dict(ok, head_dim=128)), dv=128) == mala.MALA_EUNSUPPORTED
    assert call(prob(**dict(ok, block_q=128))) == mala.MALA_EUNSUPPORTED
    assert call(prob(**dict(ok, dtype=1))) == mala.MALA_EUNSUPPORTED
