"""Parity helpers: compare HIP results with the CPU oracle.

Test infrastructure. The oracle is run on exact host copies of the device
inputs. Where a tile's block margin lies within ``BAND`` (natural log) of the
threshold, either decision is accepted; in the forward pass such a tile
changes the running state of the later tiles of its query block, so the
oracle enumerates every admissible decision sequence of the block
(``oracle.forward_block_branches``) and the HIP result must coincide with one
of them: identical decisions on every tile, values within tolerance of that
branch. No oracle input or expected value is taken from the HIP side; the
HIP mask only selects which oracle branch is compared.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle

BAND = 1e-3
# bf16 outputs: max-abs 2e-2 and relative L2 1e-2; fp32 quantities: max-abs 1e-4
TOL_BF16_ABS = 2e-2
TOL_BF16_REL = 1e-2
TOL_FP32_ABS = 1e-4


def host64(t):
    return t.detach().to("cpu").double().numpy()


@dataclass
class FwdReport:
    blocks: int = 0
    tiles: int = 0
    inband_tiles: int = 0
    branch_blocks: int = 0
    mismatched_blocks: list = field(default_factory=list)
    max_abs_o: float = 0.0
    max_abs_z: float = 0.0
    rel_l2_o: float = 0.0
    max_ref_o: float = 0.0
    _num: float = 0.0
    _den: float = 0.0

    def finish(self):
        self.rel_l2_o = math.sqrt(self._num / self._den) if self._den > 0 else 0.0
        return self


def forward_parity(q, k, v, tau, block_q, block_k, offset, o_gpu, z_gpu, mask_gpu, blocks=None,
                   band=BAND):
    """Compare a HIP forward (o, z, tile mask) with the oracle on ``blocks``
    (iterable of (b, h, i); all blocks if None). Inputs are device or host
    tensors; the oracle sees their exact values in float64."""
    q64, k64, v64 = host64(q), host64(k), host64(v)
    og, zg, mg = host64(o_gpu), host64(z_gpu), mask_gpu.detach().cpu().numpy()
    B, nq, hq, _ = q64.shape
    nk, hkv = k64.shape[1], k64.shape[2]
    nqb = oracle.num_blocks(nq, block_q)
    if blocks is None:
        blocks = [(b, h, i) for b in range(B) for h in range(hq) for i in range(nqb)]
    rep = FwdReport()
    for (b, h, i) in blocks:
        g = oracle.kv_head(h, hq, hkv)
        rows, lastv, L, tiles = oracle.prefill_block_args(i, block_q, block_k, nq, nk, offset)
        branches = oracle.forward_block_branches(q64[b, rows, h], k64[b, :, g], v64[b, :, g],
                                                 lastv, L, tiles, tau, block_k, band=band)
        rep.blocks += 1
        rep.tiles += len(tiles)
        if len(branches) > 1:
            rep.branch_blocks += 1
        gpu_dec = {j: int(mg[b, h, i, j]) for j in tiles}
        match = [br for br in branches if br.decision == gpu_dec]
        if not match:
            rep.mismatched_blocks.append(((b, h, i), {j: (gpu_dec[j], branches[0].decision[j],
                                                          branches[0].margin[j])
                                                      for j in tiles
                                                      if gpu_dec[j] != branches[0].decision[j]}))
            continue
        br = match[0]
        rep.inband_tiles += sum(1 for j in tiles if abs(br.margin[j]) < band)
        d_o = og[b, rows, h] - br.o
        rep.max_abs_o = max(rep.max_abs_o, float(np.abs(d_o).max()))
        rep.max_ref_o = max(rep.max_ref_o, float(np.abs(br.o).max()))
        rep.max_abs_z = max(rep.max_abs_z, float(np.abs(zg[b, h, rows] - br.z).max()))
        rep._num += float((d_o ** 2).sum())
        rep._den += float((br.o ** 2).sum())
    return rep.finish()


def assert_forward(rep: FwdReport, fp32: bool):
    """bf16: max-abs within 2e-2 relative to max(1, max |o_ref|) (for outputs
    of magnitude above 1 the bf16 rounding of o alone reaches |o| 2^-8) and
    relative L2 within 1e-2; fp32: max-abs within 1e-4."""
    assert not rep.mismatched_blocks, f"tile decisions differ outside the band: {rep.mismatched_blocks[:3]}"
    if fp32:
        assert rep.max_abs_o <= TOL_FP32_ABS, rep
    else:
        scale = max(1.0, rep.max_ref_o)
        assert rep.max_abs_o <= TOL_BF16_ABS * scale, rep
        assert rep.rel_l2_o <= TOL_BF16_REL, rep
    assert rep.max_abs_z <= TOL_FP32_ABS, rep


def sample_blocks(B, hq, nqb, n, seed=0, always=()):
    """A reproducible sample of (b, h, i) query blocks: the heaviest and the
    lightest block plus ``n`` random ones."""
    rng = np.random.default_rng(seed)
    out = {(0, 0, nqb - 1), (B - 1, hq - 1, 0), *always}
    while len(out) < n + 2:
        out.add((int(rng.integers(B)), int(rng.integers(hq)), int(rng.integers(nqb))))
    return sorted(out)


def to_dev(*ts, device="cuda"):
    return [None if t is None else t.to(device) for t in ts]


def legal_tile_count(B, hq, nq, nk, bq, bk, off):
    n = 0
    for i in range(oracle.num_blocks(nq, bq)):
        last = min((i + 1) * bq, nq) - 1 + off
        n += last // bk + 1
    return B * hq * n


def fresh_mask(B, hq, nq, nk, bq, bk, device="cuda"):
    return torch.full((B, hq, oracle.num_blocks(nq, bq), oracle.num_blocks(nk, bk)), 255,
                      dtype=torch.uint8, device=device)


def matched_forward(q, k, v, tau, block_q, block_k, offset, mask_gpu, band=BAND, blocks=None):
    """Oracle forward assembled from, for every block, the branch whose
    decisions equal the HIP forward's (see module doc). Returns (o, z, ok)
    as float64 arrays; rows of unmatched or unsampled blocks are NaN."""
    q64, k64, v64 = host64(q), host64(k), host64(v)
    mg = mask_gpu.detach().cpu().numpy()
    B, nq, hq, _ = q64.shape
    nk, hkv, dv = k64.shape[1], k64.shape[2], v64.shape[3]
    nqb = oracle.num_blocks(nq, block_q)
    o = np.full((B, nq, hq, dv), np.nan)
    z = np.full((B, hq, nq), np.nan)
    ok = True
    if blocks is None:
        blocks = [(b, h, i) for b in range(B) for h in range(hq) for i in range(nqb)]
    for (b, h, i) in blocks:
        g = oracle.kv_head(h, hq, hkv)
        rows, lastv, L, tiles = oracle.prefill_block_args(i, block_q, block_k, nq, nk, offset)
        brs = oracle.forward_block_branches(q64[b, rows, h], k64[b, :, g], v64[b, :, g], lastv, L,
                                            tiles, tau, block_k, band=band)
        dec = {j: int(mg[b, h, i, j]) for j in tiles}
        m = [br for br in brs if br.decision == dec]
        if not m:
            ok = False
            continue
        o[b, rows, h] = m[0].o
        z[b, h, rows] = m[0].z
    return o, z, ok


@dataclass
class BwdReport:
    tiles: int = 0
    inband_tiles: int = 0
    outband_mismatch: list = field(default_factory=list)
    err: dict = field(default_factory=dict)


def close_bf16(x, ref, name, rep, rows_mask=None):
    """bf16 tolerance for a tensor: max |x - ref| <= 2e-2 * max(1, max |ref|)
    and ||x - ref|| / ||ref|| <= 1e-2.

    The max-abs bound is taken relative to the tensor's scale once that
    exceeds 1: a bf16 value near 2^e is only representable to 2^(e-8), so
    gradients of magnitude ~30 cannot be stored within an absolute 2e-2."""
    if rows_mask is not None:
        x, ref = x[rows_mask], ref[rows_mask]
    if not d_size(x):
        rep.err[name] = {"empty": True}
        return True
    d = np.abs(x - ref)
    scale = max(1.0, float(np.abs(ref).max()))
    rel = float(np.linalg.norm(d.ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))
    rep.err[name] = {"max_abs": float(d.max()), "ref_max": float(np.abs(ref).max()),
                     "max_abs_over_scale": float(d.max()) / scale, "rel_l2": rel}
    return float(d.max()) <= TOL_BF16_ABS * scale and rel <= TOL_BF16_REL


def d_size(x):
    return x.size


def backward_parity(q, k, v, do, tau, block_q, block_k, offset, o_ref, z_ref, dq, dk, dv, mask_gpu,
                    key_blocks=None, query_blocks=None, band=BAND):
    """Compare a HIP backward with the oracle backward run on the oracle's
    own forward (o_ref, z_ref, from ``matched_forward``). The backward's O and
    z inputs are the tensors a forward delivers, so the oracle's O is rounded
    to the dtype of the HIP tensors (bf16, round-to-nearest-even) and its z
    to float32 before they enter D = rowsum(dO * O) and P = exp(S - z): the
    oracle models the interface, and no HIP value enters it. Backward
    decisions do not cascade, so each in-band tile simply contributes the HIP
    side's choice: its oracle contribution is added or removed accordingly."""
    q64, k64, v64, do64 = host64(q), host64(k), host64(v), host64(do)
    o_ref = torch.from_numpy(np.ascontiguousarray(o_ref)).to(q.dtype).double().numpy()
    z_ref = np.asarray(z_ref).astype(np.float32).astype(np.float64)
    mg = mask_gpu.detach().cpu().numpy()
    rep = BwdReport()
    out = {}
    runs = []
    if key_blocks is not None or query_blocks is None:
        runs.append(("kv", dict(key_blocks=key_blocks)))
    if query_blocks is not None:
        runs.append(("q", dict(query_blocks=set(query_blocks))))
    for kind, kw in runs:
        r = oracle.mala_backward(q64, k64, v64, o_ref, do64, z_ref, tau, block_q, block_k,
                                 causal_offset=offset, band=band, **kw)
        legal = r["mask"] != 255
        rep.tiles += int(legal.sum())
        diff = legal & (r["mask"] != mg)
        inb = np.abs(r["margin"]) < band
        bad = diff & ~inb
        if bad.any():
            rep.outband_mismatch += [tuple(x) for x in np.argwhere(bad)[:5]]
        rep.inband_tiles += int((legal & inb).sum())
        dq_e, dk_e, dv_e = r["dq"].copy(), r["dk"].copy(), r["dv"].copy()
        B, nq, hq, _ = q64.shape
        hkv = k64.shape[2]
        nk = k64.shape[1]
        for (b, h, i, j, ret, gq, gk, gv) in r["band_tiles"]:
            want = int(mg[b, h, i, j])
            if want == ret:
                continue
            sgn = 1.0 if want else -1.0
            rows = np.arange(i * block_q, min((i + 1) * block_q, nq))
            ks, ke = j * block_k, min((j + 1) * block_k, nk)
            g = oracle.kv_head(h, hq, hkv)
            dq_e[b, rows, h] += sgn * gq
            dk_e[b, ks:ke, g] += sgn * gk
            dv_e[b, ks:ke, g] += sgn * gv
        out[kind] = (dq_e, dk_e, dv_e, r)
    return rep, out


@dataclass
class DecReport:
    rows: int = 0
    tiles: int = 0
    inband_tiles: int = 0
    mismatched: list = field(default_factory=list)
    max_abs_o: float = 0.0
    max_abs_z: float = 0.0
    rel_l2_o: float = 0.0
    _num: float = 0.0
    _den: float = 0.0


def decode_parity(q, k, v, tau, block_k, num_splits, o_gpu, z_gpu, mask_gpu, rows=None, band=BAND):
    """Compare a HIP split-KV decode with the oracle on (b, h) rows. Each
    split is an independent online run, so each split's decisions must match
    one admissible oracle branch of that split."""
    B, _, hq, _ = q.shape
    hkv = k.shape[2]
    og, zg = host64(o_gpu), host64(z_gpu)
    mg = mask_gpu.detach().cpu().numpy()
    if rows is None:
        rows = [(b, h) for b in range(B) for h in range(hq)]
    rep = DecReport()
    cache = {}
    for (b, h) in rows:
        g = oracle.kv_head(h, hq, hkv)
        if (b, g) not in cache:
            cache = {(b, g): (host64(k[b, :, g]), host64(v[b, :, g]))}
        kk, vv = cache[(b, g)]
        qrow = host64(q[b, 0, h])
        per_split = oracle.decode_row_branches(qrow, kk, vv, tau, block_k, num_splits, band=band)
        parts = []
        rep.rows += 1
        for brs in per_split:
            tiles = sorted(brs[0].decision)
            rep.tiles += len(tiles)
            dec = {j: int(mg[b, h, j]) for j in tiles}
            m = [br for br in brs if br.decision == dec]
            if not m:
                rep.mismatched.append(((b, h), {j: (dec[j], brs[0].decision[j], brs[0].margin[j])
                                                for j in tiles if dec[j] != brs[0].decision[j]}))
                parts = None
                break
            rep.inband_tiles += sum(1 for j in tiles if abs(m[0].margin[j]) < band)
            parts.append((m[0].o[0], m[0].z[0]))
        if parts is None:
            continue
        o_ref, z_ref = oracle.combine_splits(parts)
        d = og[b, 0, h] - o_ref
        rep.max_abs_o = max(rep.max_abs_o, float(np.abs(d).max()))
        rep.max_abs_z = max(rep.max_abs_z, abs(float(zg[b, h]) - float(z_ref)))
        rep._num += float((d ** 2).sum())
        rep._den += float((o_ref ** 2).sum())
    rep.rel_l2_o = math.sqrt(rep._num / rep._den) if rep._den > 0 else 0.0
    return rep


def paged_decode_parity(q, k_pages, v_pages, block_table, seq_lens, page_size, tau, block_k, num_splits,
                        o_gpu, z_gpu, mask_gpu, band=BAND):
    """``decode_parity`` for a paged cache: each sequence's keys are gathered
    on the host through the block table (plain indexing) and compared as a
    contiguous cache of N_k(b) keys; splits with an empty tile range hold no
    keys and leave the combine; a sequence without keys must give o = 0,
    z = -inf."""
    B, _, hq, _ = q.shape
    hkv = k_pages.shape[2]
    kp, vp = host64(k_pages), host64(v_pages)
    table, lens = block_table.cpu().numpy(), seq_lens.cpu().numpy()
    og, zg = host64(o_gpu), host64(z_gpu)
    mg = mask_gpu.detach().cpu().numpy()
    rep = DecReport()
    for b in range(B):
        nk = int(lens[b])
        if nk == 0:
            assert (og[b] == 0).all() and np.isneginf(zg[b]).all(), "empty sequence must give o = 0, z = -inf"
            continue
        keys = np.arange(nk)
        pages, rows = table[b, keys // page_size], keys % page_size
        T = oracle.num_blocks(nk, block_k)
        assert (mg[b, :, T:] == 255).all(), "tiles past a sequence's end must stay untouched"
        for h in range(hq):
            g = oracle.kv_head(h, hq, hkv)
            with np.errstate(divide="ignore", invalid="ignore"):
                per_split = oracle.decode_row_branches(host64(q[b, 0, h]), kp[pages, rows, g], vp[pages, rows, g],
                                                       tau, block_k, num_splits, band=band)
            parts = []
            rep.rows += 1
            for (lo, hi), brs in zip(oracle.split_ranges(T, num_splits), per_split):
                if hi == lo:
                    continue
                tiles = sorted(brs[0].decision)
                rep.tiles += len(tiles)
                dec = {j: int(mg[b, h, j]) for j in tiles}
                m = [br for br in brs if br.decision == dec]
                if not m:
                    rep.mismatched.append(((b, h), {j: (dec[j], brs[0].decision[j], brs[0].margin[j])
                                                    for j in tiles if dec[j] != brs[0].decision[j]}))
                    parts = None
                    break
                rep.inband_tiles += sum(1 for j in tiles if abs(m[0].margin[j]) < band)
                parts.append((m[0].o[0], m[0].z[0]))
            if parts is None:
                continue
            o_ref, z_ref = oracle.combine_splits(parts)
            d = og[b, 0, h] - o_ref
            rep.max_abs_o = max(rep.max_abs_o, float(np.abs(d).max()))
            rep.max_abs_z = max(rep.max_abs_z, abs(float(zg[b, h]) - float(z_ref)))
            rep._num += float((d ** 2).sum())
            rep._den += float((o_ref ** 2).sum())
    rep.rel_l2_o = math.sqrt(rep._num / rep._den) if rep._den > 0 else 0.0
    return rep


def assert_decode(rep: DecReport):
    assert not rep.mismatched, f"decode decisions differ outside the band: {rep.mismatched[:3]}"
    assert rep.max_abs_o <= TOL_BF16_ABS, rep
    assert rep.rel_l2_o <= TOL_BF16_REL, rep
    assert rep.max_abs_z <= TOL_FP32_ABS, rep


# ---------------------------------------------------------------------------
# latent (MLA-shaped) backward: the value is the first 512 columns of the
# cached row, and the row's gradient is dK + [dV, 0]
# ---------------------------------------------------------------------------
LATENT_DV = 512


def run_latent_pass(mala, q, kv, do, tau, off=None):
    B, nq, hq, _ = q.shape
    nk = kv.shape[1]
    off = nk - nq if off is None else off
    mf = fresh_mask(B, hq, nq, nk, 64, 64)
    mb = fresh_mask(B, hq, nq, nk, 64, 64)
    sb = torch.zeros(4, dtype=torch.int64, device="cuda")
    print(f"mala_fwd_latent + mala_bwd_latent B={B} nq={nq} nk={nk} hq={hq} tau={tau} off={off}", flush=True)
    o, z = mala.mala_fwd_latent(q, kv, LATENT_DV, tau, 64, 64, causal_offset=off, tile_mask=mf)
    dq, dkv = mala.mala_bwd_latent(q, kv, LATENT_DV, o, do, z, tau, 64, 64, causal_offset=off, stats=sb, tile_mask=mb)
    torch.cuda.synchronize()
    return dict(o=o, z=z, dq=dq, dkv=dkv, mf=mf, mb=mb, sb=sb, off=off)


def check_latent_backward(q, kv, do, tau, r, key_blocks=None, query_blocks=None, fwd_blocks=None):
    off = r["off"]
    v = kv[..., :LATENT_DV]
    o_ref, z_ref, ok = matched_forward(q, kv, v, tau, 64, 64, off, r["mf"], blocks=fwd_blocks)
    assert ok, "forward decisions differ outside the band"
    B, nq, hq, _ = q.shape
    nk = kv.shape[1]
    rep, out = backward_parity(q, kv, v, do, tau, 64, 64, off, o_ref, z_ref, r["dq"], r["dkv"], r["dkv"],
                               r["mb"], key_blocks=key_blocks, query_blocks=query_blocks)
    assert not rep.outband_mismatch, rep.outband_mismatch
    dq, dkv = host64(r["dq"]), host64(r["dkv"])
    good = True
    if "kv" in out:
        dq_e, dk_e, dv_e, _ = out["kv"]
        dkv_e = dk_e.copy()
        dkv_e[..., :LATENT_DV] += dv_e
        sel = np.ones(dkv.shape, bool)
        if key_blocks is not None:
            sel[:] = False
            for (b, _, j) in key_blocks:
                sel[b, j * 64:(j + 1) * 64] = True
        good &= close_bf16(dkv, dkv_e, "dkv", rep, rows_mask=sel)
        if key_blocks is None and query_blocks is None:
            good &= close_bf16(dq, dq_e, "dq", rep)
    if "q" in out:
        sel = np.zeros(dq.shape, bool)
        for i in query_blocks:
            sel[:, i * 64:(i + 1) * 64] = True
        good &= close_bf16(dq, out["q"][0], "dq", rep, rows_mask=sel)
    print(rep)
    assert good, rep.err
    return rep
