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
# bf16 outputs: every element within 2e-2 plus half a bf16 unit in the last
# place of its magnitude, and relative L2 within 1e-2; fp32 quantities:
# max-abs 1e-4
TOL_BF16_ABS = 2e-2
TOL_BF16_REL = 1e-2
TOL_FP32_ABS = 1e-4


def host64(t):
    return t.detach().to("cpu").double().numpy()


def bf16_half_ulp(a):
    """Half a unit in the last place of a bf16 number of magnitude ``a``
    (8 significant bits): 2^(e - 8) for 2^e <= |a| < 2^(e + 1), 0 at 0. This
    is the largest error that storing an exact value in bf16 can make."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (e - 8).astype(np.int64)), 0.0)


def bf16_elem_bound(x, ref):
    """Per-element bound for a bf16 result ``x`` against ``ref``:
    2e-2 + half an ulp at max(|x|, |ref|) (the ulp of the stored value's
    binade, whichever side of a power of two the rounding lands)."""
    return TOL_BF16_ABS + bf16_half_ulp(np.maximum(np.abs(x), np.abs(ref)))


@dataclass
class ElemErr:
    """Worst element of a bf16 comparison: |x - ref| over its bound."""
    max_abs: float = 0.0
    ratio: float = 0.0      # max over elements of |x - ref| / bound (pass: <= 1)
    at_delta: float = 0.0   # |x - ref| at that element
    at_ref: float = 0.0     # |ref| at that element
    at_index: tuple = ()

    def add(self, x, ref, where=()):
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if not x.size:
            return
        d = np.abs(x - ref)
        self.max_abs = max(self.max_abs, float(d.max()))
        r = d / bf16_elem_bound(x, ref)
        k = int(np.argmax(r))
        if float(r.flat[k]) > self.ratio:
            self.ratio = float(r.flat[k])
            self.at_delta = float(d.flat[k])
            self.at_ref = float(abs(ref.flat[k]))
            self.at_index = tuple(where) + tuple(int(v) for v in np.unravel_index(k, d.shape))


def bf16_close(x, ref, rel_tol=TOL_BF16_REL):
    """(ok, report) for a whole bf16 tensor: every element within
    ``bf16_elem_bound`` and relative L2 within ``rel_tol``. A reference that
    is exactly zero everywhere has no relative error (dK and dQ of rows that
    see a single key: dS = P (dP - D) vanishes); the element bound alone
    applies to it."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    e = ElemErr()
    e.add(x, ref)
    nref = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm((x - ref).ravel()) / nref) if nref > 0 else 0.0
    rep = {"max_abs": e.max_abs, "worst_ratio": e.ratio, "worst_delta": e.at_delta,
           "worst_ref": e.at_ref, "worst_index": e.at_index, "rel_l2": rel}
    return e.ratio <= 1.0 and rel <= rel_tol, rep


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
    err_o: ElemErr = field(default_factory=ElemErr)
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
        rep.err_o.add(og[b, rows, h], br.o, where=(b, h, i))
        rep.max_abs_o = max(rep.max_abs_o, float(np.abs(d_o).max()))
        rep.max_ref_o = max(rep.max_ref_o, float(np.abs(br.o).max()))
        rep.max_abs_z = max(rep.max_abs_z, float(np.abs(zg[b, h, rows] - br.z).max()))
        rep._num += float((d_o ** 2).sum())
        rep._den += float((br.o ** 2).sum())
    return rep.finish()


def assert_forward(rep: FwdReport, fp32: bool):
    """bf16: every element of o within 2e-2 plus half a bf16 ulp of its
    magnitude, and relative L2 within 1e-2; fp32: max-abs within 1e-4.
    z (fp32) within 1e-4 either way."""
    assert not rep.mismatched_blocks, f"tile decisions differ outside the band: {rep.mismatched_blocks[:3]}"
    if fp32:
        assert rep.max_abs_o <= TOL_FP32_ABS, rep
    else:
        assert rep.err_o.ratio <= 1.0, rep
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


def v_copies_from_mask(mask, block_q, bf16=True):
    """V tiles a bf16 forward copies, from its tile mask: a workgroup covers
    128 query rows, i.e. one 128-row decision block or two 64-row ones that
    share one copy of V_j, made when either retains tile j. (fp32: one block
    per workgroup, one copy per retained tile.)"""
    m = np.asarray(mask) == 1
    if not bf16 or block_q == 128:
        return int(m.sum())
    B, hq, nqb, nkb = m.shape
    if nqb % 2:
        m = np.concatenate([m, np.zeros((B, hq, 1, nkb), bool)], axis=2)
    return int((m[:, :, 0::2] | m[:, :, 1::2]).sum())


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
    """bf16 tolerance for a tensor: every element within 2e-2 plus half a
    bf16 ulp of its magnitude (``bf16_elem_bound``), and
    ||x - ref|| / ||ref|| <= 1e-2. The worst element (its error, |ref| and
    index) goes into ``rep.err[name]``."""
    if rows_mask is not None:
        x, ref = x[rows_mask], ref[rows_mask]
    if not d_size(x):
        rep.err[name] = {"empty": True}
        return True
    ok, r = bf16_close(x, ref)
    rep.err[name] = r
    return ok


def d_size(x):
    return x.size


def as_forward_tensors(q, o_ref, z_ref):
    """The oracle forward's o and z as a forward delivers them - o in q's
    dtype (round to nearest even), z float32 - on q's device, to be handed to
    the HIP backward. Rows the oracle did not compute (NaN in sampled runs)
    become o = 0, z = +inf: every tile of such a row is then skipped and its
    P is 0. The tensors flow from the oracle into the HIP call, never back."""
    o = np.nan_to_num(np.asarray(o_ref, dtype=np.float64), nan=0.0)
    z = np.asarray(z_ref, dtype=np.float64)
    z = np.where(np.isnan(z), np.inf, z)
    return (torch.from_numpy(np.ascontiguousarray(o)).to(q.dtype).to(q.device),
            torch.from_numpy(np.ascontiguousarray(z)).float().to(q.device))


def oracle_backward_runs(q, k, v, do, tau, block_q, block_k, offset, o_ref, z_ref, key_blocks=None,
                         query_blocks=None, band=BAND):
    """The oracle backward on the oracle's own forward (o_ref, z_ref, from
    ``matched_forward``), rounded to the tensors a forward delivers: O to the
    dtype of q (bf16, round to nearest even), z to float32 - exactly the
    values ``as_forward_tensors`` hands the HIP backward. Returns a list of
    (kind, oracle result) for the key-block run ("kv") and/or the
    query-block run ("q")."""
    q64, k64, v64, do64 = host64(q), host64(k), host64(v), host64(do)
    o_ref = torch.from_numpy(np.ascontiguousarray(o_ref)).to(q.dtype).double().numpy()
    z_ref = np.asarray(z_ref).astype(np.float32).astype(np.float64)
    runs = []
    if key_blocks is not None or query_blocks is None:
        runs.append(("kv", dict(key_blocks=key_blocks)))
    if query_blocks is not None:
        runs.append(("q", dict(query_blocks=set(query_blocks))))
    return [(kind, oracle.mala_backward(q64, k64, v64, o_ref, do64, z_ref, tau, block_q, block_k,
                                        causal_offset=offset, band=band, **kw)) for kind, kw in runs]


def backward_parity(q, k, v, do, tau, block_q, block_k, offset, o_ref, z_ref, dq, dk, dv, mask_gpu,
                    key_blocks=None, query_blocks=None, band=BAND, runs=None):
    """Compare a HIP backward's decisions with the oracle backward (see
    ``oracle_backward_runs``; pass ``runs`` to reuse one) and assemble the
    oracle gradients that go with the HIP decisions. Backward decisions do
    not cascade, so each in-band tile simply contributes the HIP side's
    choice: its oracle contribution is added or removed accordingly."""
    if runs is None:
        runs = oracle_backward_runs(q, k, v, do, tau, block_q, block_k, offset, o_ref, z_ref,
                                    key_blocks=key_blocks, query_blocks=query_blocks, band=band)
    B, nq, hq, _ = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    mg = mask_gpu.detach().cpu().numpy()
    rep = BwdReport()
    out = {}
    for kind, r in runs:
        legal = r["mask"] != 255
        rep.tiles += int(legal.sum())
        diff = legal & (r["mask"] != mg)
        inb = np.abs(r["margin"]) < band
        bad = diff & ~inb
        if bad.any():
            rep.outband_mismatch += [tuple(x) for x in np.argwhere(bad)[:5]]
        rep.inband_tiles += int((legal & inb).sum())
        dq_e, dk_e, dv_e = r["dq"].copy(), r["dk"].copy(), r["dv"].copy()
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


def rel_l2_only(x, ref, name, rep, rows_mask=None):
    """End-to-end check of one gradient (HIP forward -> HIP backward against
    oracle forward -> oracle backward): relative L2 within 1e-2. The worst
    element against the per-element bound is recorded, not asserted: the
    two forwards' O differ by their own rounding, which moves
    D = rowsum(dO * O) and, through dS, every gradient element."""
    if rows_mask is not None:
        x, ref = x[rows_mask], ref[rows_mask]
    if not d_size(x):
        rep.err[name] = {"empty": True}
        return True
    ok, r = bf16_close(x, ref)
    rep.err[name] = r
    return r["rel_l2"] <= TOL_BF16_REL


def compare_gradients(rep, out, grads, block_q, block_k, key_blocks=None, query_blocks=None, strict=True,
                      latent_dv=None):
    """Compare HIP gradients with the oracle ones of ``backward_parity``'s
    ``out`` on the rows the oracle computed completely: every row when
    nothing was sampled; the rows of the sampled key blocks (dK, dV) and
    query blocks (dQ) otherwise. ``grads`` = (dq, dk, dv) host arrays, or
    (dq, dkv) with ``latent_dv`` = d_v for the latent cache (its row gradient
    is dK + [dV, 0]). ``strict``: per-element bound plus relative L2
    (``close_bf16``); else relative L2 only (``rel_l2_only``)."""
    check = close_bf16 if strict else rel_l2_only
    good = True
    if latent_dv is not None:
        dq, dkv = grads
    else:
        dq, dk, dv = grads
    if "kv" in out:
        dq_e, dk_e, dv_e, _ = out["kv"]
        if latent_dv is not None:
            dkv_e = dk_e.copy()
            dkv_e[..., :latent_dv] += dv_e
            sel = None
            if key_blocks is not None:
                sel = np.zeros(dkv.shape, bool)
                for (b, g, j) in key_blocks:
                    sel[b, j * block_k:(j + 1) * block_k, g] = True
            good &= check(dkv, dkv_e, "dkv", rep, rows_mask=sel)
        else:
            sel = None
            if key_blocks is not None:
                sel = np.zeros(dk.shape, bool)
                for (b, g, j) in key_blocks:
                    sel[b, j * block_k:(j + 1) * block_k, g] = True
            good &= check(dk, dk_e, "dk", rep, rows_mask=sel)
            good &= check(dv, dv_e, "dv", rep, rows_mask=sel)
        if key_blocks is None and query_blocks is None:
            good &= check(dq, dq_e, "dq", rep)
    if "q" in out:
        sel = np.zeros(dq.shape, bool)
        for i in query_blocks:
            sel[:, i * block_q:(i + 1) * block_q] = True
        good &= check(dq, out["q"][0], "dq", rep, rows_mask=sel)
    return good


def check_backward(run_hip_bwd, q, k, v, do, tau, block_q, block_k, offset, mask_fwd, e2e=None,
                   key_blocks=None, query_blocks=None, fwd_blocks=None, latent_dv=None):
    """Backward parity in two parts.

    1. Kernel parity (strict): the HIP backward run on the oracle forward's
       o and z (``as_forward_tensors``) against the oracle backward on the
       same values: decisions equal outside the band, every gradient element
       within 2e-2 plus half a bf16 ulp, relative L2 within 1e-2; and the
       query-major dQ pass's own decisions equal the key-major pass's bit
       for bit, in-band tiles included (one decision per tile).
       ``run_hip_bwd(o, z)`` launches it and returns (grads..., tile_mask,
       tile_mask_dq, stats) with device tensors.
    2. End to end, if ``e2e`` = (grads..., tile_mask) of the HIP backward run
       on the HIP forward's o and z: decisions equal outside the band (the
       two z differ by float32 rounding only), relative L2 within 1e-2.

    ``mask_fwd`` is the HIP forward's tile mask; it selects the oracle
    forward branch (``matched_forward``). Returns (strict report, e2e report
    or None, strict HIP outputs)."""
    o_ref, z_ref, ok = matched_forward(q, k, v, tau, block_q, block_k, offset, mask_fwd, blocks=fwd_blocks)
    assert ok, "forward decisions differ outside the band"
    o_t, z_t = as_forward_tensors(q, o_ref, z_ref)
    res = run_hip_bwd(o_t, z_t)
    torch.cuda.synchronize()
    *g_iso, mask_iso, mask_dq, stats_iso = res
    assert torch.equal(mask_iso, mask_dq), "the dQ pass took other decisions than the key-major pass"
    assert int((mask_iso != 255).sum()) == int((mask_dq != 255).sum())
    runs = oracle_backward_runs(q, k, v, do, tau, block_q, block_k, offset, o_ref, z_ref,
                                key_blocks=key_blocks, query_blocks=query_blocks)
    rep, out = backward_parity(q, k, v, do, tau, block_q, block_k, offset, o_ref, z_ref,
                               *((g_iso[0], g_iso[1], g_iso[1]) if latent_dv is not None else g_iso),
                               mask_iso, key_blocks=key_blocks, query_blocks=query_blocks, runs=runs)
    assert not rep.outband_mismatch, rep.outband_mismatch
    good = compare_gradients(rep, out, [host64(t) for t in g_iso], block_q, block_k, key_blocks, query_blocks,
                             strict=True, latent_dv=latent_dv)
    print("backward on the oracle forward:", rep, flush=True)
    assert good, rep.err
    rep2 = None
    if e2e is not None:
        *g_e2e, mask_e2e = e2e
        rep2, out2 = backward_parity(q, k, v, do, tau, block_q, block_k, offset, o_ref, z_ref,
                                     *((g_e2e[0], g_e2e[1], g_e2e[1]) if latent_dv is not None else g_e2e),
                                     mask_e2e, key_blocks=key_blocks, query_blocks=query_blocks, runs=runs)
        assert not rep2.outband_mismatch, rep2.outband_mismatch
        good2 = compare_gradients(rep2, out2, [host64(t) for t in g_e2e], block_q, block_k, key_blocks,
                                  query_blocks, strict=False, latent_dv=latent_dv)
        print("end to end:", rep2, flush=True)
        assert good2, rep2.err
    return rep, rep2, res


@dataclass
class DecReport:
    rows: int = 0
    tiles: int = 0
    inband_tiles: int = 0
    mismatched: list = field(default_factory=list)
    max_abs_o: float = 0.0
    max_abs_z: float = 0.0
    rel_l2_o: float = 0.0
    err_o: ElemErr = field(default_factory=ElemErr)
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
        rep.err_o.add(og[b, 0, h], o_ref, where=(b, h))
        rep.max_abs_o = max(rep.max_abs_o, float(np.abs(d).max()))
        rep.max_abs_z = max(rep.max_abs_z, abs(float(zg[b, h]) - float(z_ref)))
        rep._num += float((d ** 2).sum())
        rep._den += float((o_ref ** 2).sum())
    rep.rel_l2_o = math.sqrt(rep._num / rep._den) if rep._den > 0 else 0.0
    return rep


def decode_short_parity(q, k, v, tau, block_k, num_splits, o_gpu, z_gpu, mask_gpu, seq_lens=None, heads=None,
                        band=BAND):
    """Compare a HIP decode of a short query (q [B, N_q, Hq, d], the newest
    N_q tokens; caches [B, N_k, Hkv, d], of which sequence b uses the first
    seq_lens[b] rows when given) with the oracle per (b, h). The N_q rows of
    a head are one query block: each split's decisions must match one
    admissible oracle branch of that split (``decode_block_branches``),
    then every row's combined output is compared element by element. Rows
    at a negative position must give o = 0, z = -inf."""
    B, nq, hq, _ = q.shape
    hkv = k.shape[2]
    og, zg = host64(o_gpu), host64(z_gpu)
    if zg.ndim == 2:
        zg = zg[:, :, None]
    mg = mask_gpu.detach().cpu().numpy()
    lens = None if seq_lens is None else np.asarray(seq_lens.cpu() if torch.is_tensor(seq_lens) else seq_lens)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(hq)]
    rep = DecReport()
    cache = {}
    for (b, h) in heads:
        nk = k.shape[1] if lens is None else int(lens[b])
        pos = nk - nq + np.arange(nq)
        for r in np.nonzero(pos < 0)[0]:
            assert (og[b, r, h] == 0).all() and np.isneginf(zg[b, h, r]), "a row without keys must give o = 0, z = -inf"
        rows = np.nonzero(pos >= 0)[0]
        if nk == 0 or rows.size == 0:
            continue
        T = oracle.num_blocks(nk, block_k)
        assert (mg[b, h, T:] == 255).all(), "tiles past a sequence's end must stay untouched"
        g = oracle.kv_head(h, hq, hkv)
        if (b, g) not in cache:
            cache = {(b, g): (host64(k[b, :nk, g]), host64(v[b, :nk, g]))}
        kk, vv = cache[(b, g)]
        per_split = oracle.decode_block_branches(host64(q[b, rows, h]), kk, vv, pos[rows], tau, block_k,
                                                 num_splits, band=band)
        rep.rows += int(rows.size)
        results = []
        for brs in per_split:
            tiles = sorted(brs[0].decision)
            rep.tiles += len(tiles)
            dec = {j: int(mg[b, h, j]) for j in tiles}
            m = [br for br in brs if br.decision == dec]
            if not m:
                rep.mismatched.append(((b, h), {j: (dec[j], brs[0].decision[j], brs[0].margin[j])
                                                for j in tiles if dec[j] != brs[0].decision[j]}))
                results = None
                break
            rep.inband_tiles += sum(1 for j in tiles if abs(m[0].margin[j]) < band)
            results.append(m[0])
        if results is None:
            continue
        o_ref, z_ref = oracle.combine_split_rows(results, rows.size)
        for i, r in enumerate(rows):
            d = og[b, r, h] - o_ref[i]
            rep.err_o.add(og[b, r, h], o_ref[i], where=(b, int(r), h))
            rep.max_abs_o = max(rep.max_abs_o, float(np.abs(d).max()))
            rep.max_abs_z = max(rep.max_abs_z, abs(float(zg[b, h, r]) - float(z_ref[i])))
            rep._num += float((d ** 2).sum())
            rep._den += float((o_ref[i] ** 2).sum())
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
            rep.err_o.add(og[b, 0, h], o_ref, where=(b, h))
            rep.max_abs_o = max(rep.max_abs_o, float(np.abs(d).max()))
            rep.max_abs_z = max(rep.max_abs_z, abs(float(zg[b, h]) - float(z_ref)))
            rep._num += float((d ** 2).sum())
            rep._den += float((o_ref ** 2).sum())
    rep.rel_l2_o = math.sqrt(rep._num / rep._den) if rep._den > 0 else 0.0
    return rep


def assert_decode(rep: DecReport):
    """Decisions as the module doc; o per element within 2e-2 plus half a
    bf16 ulp and relative L2 within 1e-2; z within 1e-4."""
    assert not rep.mismatched, f"decode decisions differ outside the band: {rep.mismatched[:3]}"
    assert rep.err_o.ratio <= 1.0, rep
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
    mq = fresh_mask(B, hq, nq, nk, 64, 64)
    sb = torch.zeros(4, dtype=torch.int64, device="cuda")
    print(f"mala_fwd_latent + mala_bwd_latent B={B} nq={nq} nk={nk} hq={hq} tau={tau} off={off}", flush=True)
    o, z = mala.mala_fwd_latent(q, kv, LATENT_DV, tau, 64, 64, causal_offset=off, tile_mask=mf)
    dq, dkv = mala.mala_bwd_latent(q, kv, LATENT_DV, o, do, z, tau, 64, 64, causal_offset=off, stats=sb, tile_mask=mb,
                                   tile_mask_dq=mq)
    torch.cuda.synchronize()
    assert torch.equal(mb, mq), "the dQ pass took other decisions than the key-major pass"
    return dict(o=o, z=z, dq=dq, dkv=dkv, mf=mf, mb=mb, sb=sb, off=off)


def check_latent_backward(mala, q, kv, do, tau, r, key_blocks=None, query_blocks=None, fwd_blocks=None):
    """``check_backward`` for the latent cache: strict kernel parity of
    mala_bwd_latent on the oracle forward's o and z, and the end-to-end run
    ``r`` of ``run_latent_pass`` by relative L2."""
    off = r["off"]
    v = kv[..., :LATENT_DV]
    B, nq, hq, _ = q.shape
    nk = kv.shape[1]

    def run(o, z):
        mb = fresh_mask(B, hq, nq, nk, 64, 64)
        mq = fresh_mask(B, hq, nq, nk, 64, 64)
        sb = torch.zeros(4, dtype=torch.int64, device="cuda")
        print(f"mala_bwd_latent on the oracle forward B={B} nq={nq} nk={nk} hq={hq} tau={tau} off={off}",
              flush=True)
        dq, dkv = mala.mala_bwd_latent(q, kv, LATENT_DV, o, do, z, tau, 64, 64, causal_offset=off, stats=sb,
                                       tile_mask=mb, tile_mask_dq=mq)
        return dq, dkv, mb, mq, sb

    rep, rep2, res = check_backward(run, q, kv, v, do, tau, 64, 64, off, r["mf"], e2e=(r["dq"], r["dkv"], r["mb"]),
                                    key_blocks=key_blocks, query_blocks=query_blocks, fwd_blocks=fwd_blocks,
                                    latent_dv=LATENT_DV)
    return rep
