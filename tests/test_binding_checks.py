"""Host-side argument checks of the Python binding: every wrapper compares
the shapes and dtypes of its tensors with the problem built from q and k
before anything reaches the library, and refuses host tensors (there is no
CPU path). CPU tensors only; no kernel is launched."""

import os

import pytest
import torch

import block_sparse_causal_tile_amd as mala

B, NQ, HQ, HKV, D = 1, 128, 4, 2, 64


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(mala.lib_path()):
        from block_sparse_causal_tile_amd import build
        build.build()
    return mala.load()


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def qkv(nk=NQ):
    return bf(B, NQ, HQ, D), bf(B, nk, HKV, D), bf(B, nk, HKV, D)


def test_host_tensors_are_refused():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="CUDA"):
        mala.mala_fwd(q, k, v, 0.05, 64, 64)
    with pytest.raises(ValueError, match="CUDA"):
        mala.mala_bwd(q, k, v, q, q, torch.zeros(B, HQ, NQ), 0.05, 64, 64)
    with pytest.raises(ValueError, match="CUDA"):
        mala.mala_decode(bf(B, 1, HQ, D), k, v, 0.05, 64)


@pytest.mark.parametrize("name,kw,match", [
    ("v rows", dict(v=bf(B, NQ - 1, HKV, D)), "v: expected shape"),
    ("v heads", dict(v=bf(B, NQ, HKV + 1, D)), "v: expected shape"),
    ("v dtype", dict(v=torch.zeros(B, NQ, HKV, D)), "v: expected dtype"),
    ("k dtype", dict(k=torch.zeros(B, NQ, HKV, D)), "k: expected dtype"),
    ("k width", dict(k=bf(B, NQ, HKV, D + 8), v=bf(B, NQ, HKV, D + 8)), "does not fit q"),
    ("o shape", dict(o=bf(B, NQ, HQ, D - 8)), "o: expected shape"),
    ("z dtype", dict(z=torch.zeros(B, HQ, NQ, dtype=torch.float64)), "z: expected dtype"),
    ("z shape", dict(z=torch.zeros(B, NQ, HQ)), "z: expected shape"),
    ("stats dtype", dict(stats=torch.zeros(4, dtype=torch.int32)), "stats"),
    ("stats size", dict(stats=torch.zeros(3, dtype=torch.int64)), "stats"),
    ("mask blocks", dict(tile_mask=torch.zeros(B, HQ, 4, 4, dtype=torch.uint8)), "tile_mask"),
    ("mask dtype", dict(tile_mask=torch.zeros(B, HQ, 2, 2, dtype=torch.int32)), "tile_mask"),
])
def test_fwd_argument_checks(name, kw, match):
    q, k, v = qkv()
    args = dict(q=q, k=k, v=v)
    args.update({n: kw[n] for n in ("q", "k", "v") if n in kw})
    rest = {n: t for n, t in kw.items() if n not in ("q", "k", "v")}
    with pytest.raises(ValueError, match=match):
        mala.mala_fwd(args["q"], args["k"], args["v"], 0.05, 64, 64, **rest)


@pytest.mark.parametrize("name,kw,match", [
    ("dout dtype", dict(dout=torch.zeros(B, NQ, HQ, D)), "dout: expected dtype"),
    ("dout rows", dict(dout=bf(B, NQ - 64, HQ, D)), "dout: expected shape"),
    ("o heads", dict(o=bf(B, NQ, HQ - 1, D)), "o: expected shape"),
    ("dq shape", dict(dq=bf(B, NQ, HKV, D)), "dq: expected shape"),
    ("dk shape", dict(dk=bf(B, NQ, HQ, D)), "dk: expected shape"),
    ("dv dtype", dict(dv=torch.zeros(B, NQ, HKV, D)), "dv: expected dtype"),
    ("z dtype", dict(z=bf(B, HQ, NQ)), "z: expected dtype"),
    ("dq mask", dict(tile_mask_dq=torch.zeros(B, HQ, 2, 3, dtype=torch.uint8)), "tile_mask"),
])
def test_bwd_argument_checks(name, kw, match):
    q, k, v = qkv()
    a = dict(o=bf(B, NQ, HQ, D), dout=bf(B, NQ, HQ, D), z=torch.zeros(B, HQ, NQ))
    a.update({n: kw[n] for n in ("o", "dout", "z") if n in kw})
    rest = {n: t for n, t in kw.items() if n not in ("o", "dout", "z")}
    with pytest.raises(ValueError, match=match):
        mala.mala_bwd(q, k, v, a["o"], a["dout"], a["z"], 0.05, 64, 64, **rest)


@pytest.mark.parametrize("name,q,kw,match", [
    ("cache heads", bf(B, 1, HQ, D), dict(v_cache=bf(B, NQ, HKV + 2, D)), "v_cache: expected shape"),
    ("cache dtype", bf(B, 1, HQ, D), dict(k_cache=torch.zeros(B, NQ, HKV, D)), "k_cache: expected dtype"),
    ("o shape", bf(B, 2, HQ, D), dict(o=bf(B, 1, HQ, D)), "o: expected shape"),
    ("mask tiles", bf(B, 1, HQ, D), dict(tile_mask=torch.zeros(B, HQ, 3, dtype=torch.uint8)), "tile_mask"),
])
def test_decode_argument_checks(name, q, kw, match):
    _, k, v = qkv()
    caches = dict(k_cache=k, v_cache=v)
    caches.update({n: kw[n] for n in ("k_cache", "v_cache") if n in kw})
    rest = {n: t for n, t in kw.items() if n not in ("k_cache", "v_cache")}
    with pytest.raises(ValueError, match=match):
        mala.mala_decode(q, caches["k_cache"], caches["v_cache"], 0.05, 64, **rest)
