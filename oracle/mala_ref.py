"""Plain fp64 CPU oracle for MassAlloc Attention (MALA).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code, tables or helpers with the HIP
library in ``block_sparse_causal_tile_amd``; the only module both sides use is
``workloads`` (seeded input generators, which hold none of the method's
arithmetic).

Everything here is written from the MALA paper page ("MassAlloc Attention: Let
Attention Allocate Its Own Compute"), in numpy float64, one tile at a time and
in the visiting order the page prescribes. Citations name the page's section:

* problem setup, the contribution scale tau / L_q and L_q itself: section 2
  (the paragraphs before "Online Sparse Softmax");
* forward rule (running m, l over retained tiles, log-domain block test,
  empty-state rule, diagonal-first traversal, finalization z = m + log l):
  "Online Sparse Softmax" and "Fused forward execution";
* backward rule (test against the finalized z, key-major traversal,
  P = exp(S - z), standard dV/dP/dS/dQ/dK): "Offline Sparse Probability" and
  "Fused backward execution";
* split-KV decoding and the normalizer-aware combine: the paragraph on
  split-KV decoding and "Fused decoding execution";
* slots per query, omitted mass, relative L2: the allocation-metric paragraph
  and the operator-fidelity paragraphs of the experiments.

The dense brute force (``dense_attention`` and its gradient) follows the
"teaching reference" of the attention tutorial page (Atlas "Attention",
section "One masked attention row"): mask logits first, softmax, weights @ V.

The displayed equations of the MALA page were lost in extraction; the readings
used here (written out in each docstring) are

* R1  Z_q^(t) = sum_{k in R_q^(t)} exp(s_qk) = exp(m_q) * l_q
* R2  r_qj^(t) = max_{k in J_j, legal} exp(s_qk) / Z_q^(t)
* R3  forward skip  <=>  for every relevant row q of the block:
      rowmax_q(S_ij) - (m_q + log l_q) < log tau - log L_q
      (a tie retains; l_q = 0 gives +inf, i.e. retain)
* R4  backward skip <=>  for every legal (q, k) of the tile:
      S_qk - z_q < log tau - log L_q
* R5  P = exp(S - z)
* R6  z_q = m_q + log l_q = log Z_{R,q}

Parity pins for every public function live in ``tests/test_oracle_*.py``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "dense_attention",
    "dense_attention_backward",
    "forward_block",
    "forward_block_branches",
    "forward_block_from_scratch",
    "mala_forward",
    "mala_forward_varlen",
    "mala_forward_latent",
    "mala_backward",
    "mala_backward_latent",
    "mala_decode_latent",
    "mala_decode",
    "mala_decode_paged",
    "mala_decode_short",
    "decode_row_branches",
    "decode_block_branches",
    "num_blocks",
    "kv_head",
    "omitted_mass",
    "slot_histogram",
    "sq_err_heads",
    "splitmix64",
    "rademacher",
    "rel_l2",
]


# ---------------------------------------------------------------------------
# small helpers (shape bookkeeping only)
# ---------------------------------------------------------------------------

def num_blocks(n: int, b: int) -> int:
    """Number of blocks of size ``b`` covering ``n`` positions (last may be ragged)."""
    return (n + b - 1) // b


def kv_head(h: int, heads_q: int, heads_kv: int) -> int:
    """Grouped-query attention: query head h reads KV head h // (H_q / H_kv)
    (contiguous grouping, tutorial page section "MHA -> MQA -> GQA")."""
    return h // (heads_q // heads_kv)


def _as64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: exact upcast of its values
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _log_thr(tau: float, L: np.ndarray) -> np.ndarray:
    """log(tau / L_q) = log tau - log L_q (MALA page, section 2).

    tau = 0 is the FullAttn limit of the page ("as tau -> 0 the skip
    conditions vanish"), represented by a threshold of -inf."""
    L = np.asarray(L, dtype=np.float64)
    if tau == 0.0:
        return np.full(L.shape, -np.inf)
    return math.log(tau) - np.log(L)


# ---------------------------------------------------------------------------
# dense brute force (the FullAttn definition)
# ---------------------------------------------------------------------------

def _dense_probs(qh: np.ndarray, kh: np.ndarray, off: int):
    """Masked causal softmax of one head: returns (P, z) with P[q, k] the
    attention weight and z[q] = log sum_k exp(s_qk) over visible keys."""
    nq, nk = qh.shape[0], kh.shape[0]
    s = qh @ kh.T
    visible = np.arange(nk)[None, :] <= (np.arange(nq) + off)[:, None]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    zsum = e.sum(axis=1)
    return e / zsum[:, None], m + np.log(zsum), visible


def dense_attention(q, k, v, causal_offset: int | None = None):
    """Dense causal softmax attention (FullAttn), fp64.

    q: [B, Nq, Hq, d] (softmax scale already folded into q, as on the MALA
    page), k, v: [B, Nk, Hkv, d]. Query row q sees keys k <= q + off with
    off = Nk - Nq by default. Returns (o [B, Nq, Hq, dv], z [B, Hq, Nq])."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, nq, hq, _ = q.shape
    nk, hkv, dv = k.shape[1], k.shape[2], v.shape[3]
    off = nk - nq if causal_offset is None else causal_offset
    o = np.zeros((B, nq, hq, dv))
    z = np.zeros((B, hq, nq))
    for b in range(B):
        for h in range(hq):
            g = kv_head(h, hq, hkv)
            p, zz, _ = _dense_probs(q[b, :, h], k[b, :, g], off)
            o[b, :, h] = p @ v[b, :, g]
            z[b, h] = zz
    return o, z


def dense_attention_backward(q, k, v, do, causal_offset: int | None = None):
    """Gradient of dense causal attention w.r.t. q, k, v for upstream dO.

    Standard softmax backward: dV = P^T dO, dP = dO V^T,
    dS = P * (dP - rowsum(P * dP)), dQ = dS K, dK = dS^T Q; dK and dV of a
    KV head are summed over the query heads of its group."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, nq, hq, _ = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    off = nk - nq if causal_offset is None else causal_offset
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(hq):
            g = kv_head(h, hq, hkv)
            p, _, _ = _dense_probs(q[b, :, h], k[b, :, g], off)
            dp = do[b, :, h] @ v[b, :, g].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dv[b, :, g] += p.T @ do[b, :, h]
            dq[b, :, h] = ds @ k[b, :, g]
            dk[b, :, g] += ds.T @ q[b, :, h]
    return dq, dk, dv


# ---------------------------------------------------------------------------
# forward: online sparse softmax of one query block
# ---------------------------------------------------------------------------

@dataclass
class BlockResult:
    o: np.ndarray                 # [rows, dv] normalized output
    z: np.ndarray                 # [rows] final log-normalizer
    decision: dict = field(default_factory=dict)   # tile j -> 1 retained / 0 skipped
    margin: dict = field(default_factory=dict)     # tile j -> block log-margin M_ij
    inband: list = field(default_factory=list)     # tiles with |M_ij| < band, visit order
    forced: dict = field(default_factory=dict)


def forward_block(qi, k, v, last_visible, L, tiles, tau: float, block_k: int,
                  forced: dict | None = None, band: float = 0.0) -> BlockResult:
    """Algorithm 1 of the MALA page for one query block.

    qi: [r, d] query rows of the block (valid rows only); k, v: [Nk, d] of the
    block's KV head; last_visible[r]: largest key index row q may see
    (q + off in prefill); L[r]: L_q, the number of causally visible keys used
    in the threshold tau / L_q; tiles: key-block indices in visiting order
    (prefill: the diagonal block first, then descending).

    State per row: running max m, shifted sum l, unnormalized output acc,
    all over retained tiles only ("Online Sparse Softmax"). For every tile:

    1. score discovery S = Q_i K_j^T, causally masked entries -inf;
    2. relevant rows: those with at least one legal key in the tile;
    3. row margin = rowmax - (m + log l) - (log tau - log L_q), or +inf while
       l = 0 (empty state); block margin M = max over relevant rows;
    4. skip iff M < 0 (R3); a tie retains;
    5. a retained tile applies the standard online-softmax update to every
       row with a legal key in it; rows without one, and all rows of a
       skipped tile, keep m, l, acc unchanged.

    Finally o = acc / l and z = m + log l (R6). ``forced`` maps tile -> 0/1
    and overrides step 4 for that tile (used only to enumerate both outcomes
    of in-band tiles, see ``forward_block_branches``); ``band`` > 0 records
    tiles with finite |M| < band in ``inband``.
    """
    qi, k, v = _as64(qi), _as64(k), _as64(v)
    forced = forced or {}
    r, nk, dv = qi.shape[0], k.shape[0], v.shape[1]
    last_visible = np.asarray(last_visible)
    thr = _log_thr(tau, L)
    m = np.full(r, -np.inf)
    l = np.zeros(r)
    acc = np.zeros((r, dv))
    res = BlockResult(o=None, z=None, forced=dict(forced))
    for j in tiles:
        ks, ke = j * block_k, min((j + 1) * block_k, nk)
        keys = np.arange(ks, ke)
        legal = keys[None, :] <= last_visible[:, None]
        s = np.where(legal, qi @ k[ks:ke].T, -np.inf)
        relevant = legal.any(axis=1)
        if not relevant.any():
            continue  # not a legal tile for this block
        rowmax = s.max(axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
            row_margin = np.where(l > 0, rowmax - lse - thr, np.inf)
        M = float(row_margin[relevant].max())
        res.margin[j] = M
        if band > 0 and math.isfinite(M) and abs(M) < band:
            res.inband.append(j)
        retain = int(M >= 0.0)
        if j in forced:
            retain = int(forced[j])
        res.decision[j] = retain
        if not retain:
            continue
        upd = relevant
        m_new = np.where(upd, np.maximum(m, rowmax), m)
        with np.errstate(invalid="ignore"):
            c = np.where(upd & (l > 0), np.exp(m - m_new), np.where(upd, 0.0, 1.0))
        with np.errstate(invalid="ignore"):
            p = np.where(legal & upd[:, None], np.exp(s - m_new[:, None]), 0.0)
        l = l * c + p.sum(axis=1)
        acc = acc * c[:, None] + p @ v[ks:ke]
        m = m_new
    res.o = acc / l[:, None]
    res.z = m + np.log(l)
    return res


def forward_block_branches(qi, k, v, last_visible, L, tiles, tau, block_k,
                           band: float, max_branches: int = 64):
    """Every admissible outcome of ``forward_block`` when tiles whose block
    margin lies within ``band`` of the threshold may go either way.

    A tile decided differently inside the band changes the running state of
    the later tiles of the same block, so each in-band tile splits the run in
    two. Branches are produced by rerunning the block with the in-band
    decisions pinned; all decisions outside the band follow the rule."""
    out = []

    def walk(forced):
        if len(out) >= max_branches:
            raise RuntimeError("too many in-band tiles in one block")
        res = forward_block(qi, k, v, last_visible, L, tiles, tau, block_k,
                            forced=forced, band=band)
        free = [j for j in res.inband if j not in forced]
        if not free:
            out.append(res)
            return
        j = free[0]
        walk({**forced, j: res.decision[j]})
        walk({**forced, j: 1 - res.decision[j]})

    walk({})
    return out


def forward_block_from_scratch(qi, k, v, last_visible, L, tiles, tau, block_k):
    """Second, independent formulation of the forward rule (pins R1/R2).

    Instead of a running (m, l), keep the retained key set R_q of every row
    and, at each test, recompute Z_q = sum_{k in R_q} exp(s_qk) directly and
    the ratio r_qj = max_{legal k in J_j} exp(s_qk) / Z_q (r = +inf while
    R_q is empty). The tile is skipped iff r_qj < tau / L_q for every
    relevant row. Linear domain, no rescaling: only for small scores.
    Returns (o, z, decision dict)."""
    qi, k, v = _as64(qi), _as64(k), _as64(v)
    r, nk = qi.shape[0], k.shape[0]
    s_all = qi @ k.T
    last_visible = np.asarray(last_visible)
    L = np.asarray(L, dtype=np.float64)
    retained = [[] for _ in range(r)]
    decision = {}
    for j in tiles:
        keys = list(range(j * block_k, min((j + 1) * block_k, nk)))
        skip_all = True
        any_relevant = False
        for row in range(r):
            legal = [kk for kk in keys if kk <= last_visible[row]]
            if not legal:
                continue
            any_relevant = True
            zq = sum(math.exp(s_all[row, kk]) for kk in retained[row])
            top = max(math.exp(s_all[row, kk]) for kk in legal)
            ratio = math.inf if zq == 0.0 else top / zq
            if not (ratio < tau / L[row]):
                skip_all = False
        if not any_relevant:
            continue
        decision[j] = 0 if skip_all else 1
        if decision[j]:
            for row in range(r):
                retained[row] += [kk for kk in keys if kk <= last_visible[row]]
    o = np.zeros((r, v.shape[1]))
    z = np.zeros(r)
    for row in range(r):
        w = np.array([math.exp(s_all[row, kk]) for kk in retained[row]])
        zq = w.sum()
        o[row] = (w[:, None] * v[retained[row]]).sum(axis=0) / zq
        z[row] = math.log(zq)
    return o, z, decision


# ---------------------------------------------------------------------------
# forward over a whole problem
# ---------------------------------------------------------------------------

def _block_rows(i: int, block_q: int, nq: int) -> np.ndarray:
    return np.arange(i * block_q, min((i + 1) * block_q, nq))


def prefill_block_args(i: int, block_q: int, block_k: int, nq: int, nk: int, off: int):
    """Rows, last visible key, L_q and tile visiting order of query block i:
    the highest legal key block (the diagonal) first, then descending
    ("Fused forward execution")."""
    rows = _block_rows(i, block_q, nq)
    last_visible = np.minimum(rows + off, nk - 1)
    L = rows + off + 1
    jmax = int(last_visible.max()) // block_k
    return rows, last_visible, L, list(range(jmax, -1, -1))


def mala_forward(q, k, v, tau: float, block_q: int, block_k: int,
                 causal_offset: int | None = None, blocks=None):
    """MALA forward over [B, Nq, Hq, d] queries and [B, Nk, Hkv, d] keys/values.

    Query blocks are independent ("Algorithm 1 parallelizes over query
    blocks"), so the oracle simply runs ``forward_block`` for each
    (b, h, i). ``blocks``, if given, is an iterable of (b, h, i) to compute
    (sampling); other rows are left as NaN.

    Returns dict with o [B, Nq, Hq, dv], z [B, Hq, Nq], mask and margin
    [B, Hq, nQB, nKB] (mask 1 retained, 0 skipped, 255 not a legal tile;
    margin NaN where not legal)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, nq, hq, _ = q.shape
    nk, hkv, dv = k.shape[1], k.shape[2], v.shape[3]
    off = nk - nq if causal_offset is None else causal_offset
    nqb, nkb = num_blocks(nq, block_q), num_blocks(nk, block_k)
    o = np.full((B, nq, hq, dv), np.nan)
    z = np.full((B, hq, nq), np.nan)
    mask = np.full((B, hq, nqb, nkb), 255, dtype=np.uint8)
    margin = np.full((B, hq, nqb, nkb), np.nan)
    if blocks is None:
        blocks = [(b, h, i) for b in range(B) for h in range(hq) for i in range(nqb)]
    for (b, h, i) in blocks:
        g = kv_head(h, hq, hkv)
        rows, lastv, L, tiles = prefill_block_args(i, block_q, block_k, nq, nk, off)
        res = forward_block(q[b, rows, h], k[b, :, g], v[b, :, g], lastv, L, tiles,
                            tau, block_k)
        o[b, rows, h] = res.o
        z[b, h, rows] = res.z
        for j, dcs in res.decision.items():
            mask[b, h, i, j] = dcs
            margin[b, h, i, j] = res.margin[j]
    return {"o": o, "z": z, "mask": mask, "margin": margin, "offset": off}


def mala_forward_latent(q, kv, d_v: int, tau: float, block_q: int, block_k: int,
                        causal_offset: int | None = None, blocks=None):
    """MALA forward on latent (MLA-shaped) attention: q [B, Nq, Hq, d_qk]
    and one cached row per position kv [B, Nk, 1, d_qk], whose first d_v
    columns are the latent that serves as the value.

    The attention tutorial page (section "MLA: compress the cached
    representation") describes this absorbed form: the key expansion is
    folded into the query, so queries score the cached latent (plus its
    decoupled positional part) directly, and the value expansion is moved
    after the weighted sum, so the value read per position is the latent
    itself. MALA's rule is shape-agnostic (the page's per-slot accounting
    counts 2 h d_v post-score FLOPs), so this is ``mala_forward`` with
    k = kv and v = kv[..., :d_v]."""
    kv = _as64(kv)
    return mala_forward(q, kv, kv[..., :d_v], tau, block_q, block_k,
                        causal_offset=causal_offset, blocks=blocks)


def mala_forward_varlen(q, k, v, cu_q, cu_k, tau: float, block_q: int, block_k: int):
    """MALA forward over packed sequences: q [total_q, Hq, d], k, v
    [total_k, Hkv, d]; sequence b owns rows [cu_q[b], cu_q[b+1]) of q and
    [cu_k[b], cu_k[b+1]) of k, v. Each sequence runs ``mala_forward`` on its
    own rows with bottom-right alignment (offset N_k(b) - N_q(b)); rows that
    see no key (offset < 0) are defined as o = 0, z = -inf. Returns dict with
    o [total_q, Hq, dv], z [Hq, total_q], mask / margin
    [B, Hq, max nQB, max nKB] (255 / NaN outside each sequence's tiles)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    cu_q, cu_k = np.asarray(cu_q, dtype=np.int64), np.asarray(cu_k, dtype=np.int64)
    B = len(cu_q) - 1
    hq, dv = q.shape[1], v.shape[2]
    nqs, nks = np.diff(cu_q), np.diff(cu_k)
    nqb = num_blocks(int(nqs.max()), block_q) if B else 0
    nkb = num_blocks(int(max(nks.max(), 1)), block_k) if B else 0
    o = np.zeros((q.shape[0], hq, dv))
    z = np.full((hq, q.shape[0]), -np.inf)
    mask = np.full((B, hq, nqb, nkb), 255, dtype=np.uint8)
    margin = np.full((B, hq, nqb, nkb), np.nan)
    for b in range(B):
        nq, nk = int(nqs[b]), int(nks[b])
        if nq == 0:
            continue
        qs, ks = int(cu_q[b]), int(cu_k[b])
        with np.errstate(divide="ignore", invalid="ignore"):  # rows without keys
            r = mala_forward(q[None, qs:qs + nq], k[None, ks:ks + nk], v[None, ks:ks + nk], tau,
                             block_q, block_k, causal_offset=nk - nq)
        seen = np.arange(nq) + (nk - nq) >= 0          # rows with at least one key
        ob = np.where(seen[:, None, None], r["o"][0], 0.0)
        zb = np.where(seen[None, :], r["z"][0], -np.inf)
        o[qs:qs + nq] = ob
        z[:, qs:qs + nq] = zb
        mb, gb = r["mask"][0], r["margin"][0]
        mask[b, :, :mb.shape[1], :mb.shape[2]] = mb
        margin[b, :, :mb.shape[1], :mb.shape[2]] = gb
    return {"o": o, "z": z, "mask": mask, "margin": margin}


# ---------------------------------------------------------------------------
# backward: offline sparse probability
# ---------------------------------------------------------------------------

def backward_tile_grads(qi, kj, vj, doi, Di, zi, legal):
    """Post-score work of one retained backward tile ("Offline Sparse
    Probability"): P = exp(S - z) (R5), dV_j = P^T dO_i, dP = dO_i V_j^T,
    dS = P * (dP - D_i), dQ_i = dS K_j, dK_j = dS^T Q_i.
    Returns (dq_i, dk_j, dv_j) contributions of this tile."""
    s = qi @ kj.T
    p = np.where(legal, np.exp(np.where(legal, s, 0.0) - zi[:, None]), 0.0)
    dp = doi @ vj.T
    ds = p * (dp - Di[:, None])
    return ds @ kj, ds.T @ qi, p.T @ doi


def mala_backward(q, k, v, o, do, z, tau: float, block_q: int, block_k: int,
                  causal_offset: int | None = None, band: float = 0.0,
                  key_blocks=None, query_blocks=None):
    """MALA backward ("Offline Sparse Probability", "Fused backward execution").

    Inputs as in ``mala_forward`` plus the forward output o, the upstream
    gradient do [B, Nq, Hq, dv] and the finalized log-normalizer z
    [B, Hq, Nq]. D_q = sum_d dO_qd O_qd (the standard softmax-backward row
    term, computed from the given o).

    Key-major: for each key block j and each query block i from the diagonal
    upward, recompute S = Q_i K_j^T, form the tile margin
    M' = max over legal (q, k) of S_qk - z_q - (log tau - log L_q) (R4), and
    run ``backward_tile_grads`` iff M' >= 0. Decisions use only the final z,
    so they do not depend on visiting order.

    ``band`` > 0 additionally returns, for every legal tile with finite
    |M'| < band, its (b, h, i, j, decision, dq_i, dk_j, dv_j) so a caller can
    account for either outcome of such a tile. ``key_blocks``, if given,
    restricts the computation to an iterable of (b, g, j) with g the KV head
    (sampling): dk/dv rows of other blocks and dq are then partial.
    ``query_blocks``, if given, is a set of query-block indices i: only
    tiles of those blocks are visited (their dq rows are then complete).

    Returns dict with dq, dk, dv, mask/margin [B, Hq, nQB, nKB], D, band_tiles.
    """
    q, k, v, o, do, z = (_as64(t) for t in (q, k, v, o, do, z))
    B, nq, hq, _ = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    off = nk - nq if causal_offset is None else causal_offset
    nqb, nkb = num_blocks(nq, block_q), num_blocks(nk, block_k)
    D = (do * o).sum(axis=-1)                       # [B, Nq, Hq]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    mask = np.full((B, hq, nqb, nkb), 255, dtype=np.uint8)
    margin = np.full((B, hq, nqb, nkb), np.nan)
    band_tiles = []
    group = hq // hkv
    if key_blocks is None:
        key_blocks = [(b, g, j) for b in range(B) for g in range(hkv) for j in range(nkb)]
    for (b, g, j) in key_blocks:
        ks, ke = j * block_k, min((j + 1) * block_k, nk)
        keys = np.arange(ks, ke)
        kj, vj = k[b, ks:ke, g], v[b, ks:ke, g]
        i0 = max(0, ks - off) // block_q
        for h in range(g * group, (g + 1) * group):
            for i in range(i0, nqb):
                if query_blocks is not None and i not in query_blocks:
                    continue
                rows = _block_rows(i, block_q, nq)
                legal = keys[None, :] <= (rows + off)[:, None]
                if not legal.any():
                    continue
                qi, doi = q[b, rows, h], do[b, rows, h]
                zi, Di = z[b, h, rows], D[b, rows, h]
                thr = _log_thr(tau, rows + off + 1)
                s = qi @ kj.T
                with np.errstate(invalid="ignore"):
                    t = np.where(legal, s - zi[:, None] - thr[:, None], -np.inf)
                M = float(t.max())
                margin[b, h, i, j] = M
                retain = int(M >= 0.0)
                mask[b, h, i, j] = retain
                inband = band > 0 and math.isfinite(M) and abs(M) < band
                if retain or inband:
                    gq, gk, gv = backward_tile_grads(qi, kj, vj, doi, Di, zi, legal)
                    if inband:
                        band_tiles.append((b, h, i, j, retain, gq, gk, gv))
                    if retain:
                        dq[b, rows, h] += gq
                        dk[b, ks:ke, g] += gk
                        dv[b, ks:ke, g] += gv
    return {"dq": dq, "dk": dk, "dv": dv, "mask": mask, "margin": margin,
            "D": D, "band_tiles": band_tiles, "offset": off}


def mala_backward_latent(q, kv, d_v: int, o, do, z, tau: float, block_q: int, block_k: int,
                         causal_offset: int | None = None, **kw):
    """MALA backward on latent (MLA-shaped) attention: q [B, Nq, Hq, d_qk],
    one cached row per position kv [B, Nk, 1, d_qk] whose first d_v columns
    are the value (absorbed form, attention tutorial page, section "MLA:
    compress the cached representation"), o and do [B, Nq, Hq, d_v].

    The rule is ``mala_backward``'s with k = kv and v = kv[..., :d_v]. The
    cached row feeds both the scores and the value, so its gradient is the
    sum of the two paths: dkv = dk + [dv, 0] (dv padded with zeros over the
    d_qk - d_v positional columns). Returns ``mala_backward``'s dict plus
    ``dkv`` [B, Nk, 1, d_qk]."""
    kv = _as64(kv)
    r = mala_backward(q, kv, kv[..., :d_v], o, do, z, tau, block_q, block_k,
                      causal_offset=causal_offset, **kw)
    dkv = r["dk"].copy()
    dkv[..., :d_v] += r["dv"]
    r["dkv"] = dkv
    return r


# ---------------------------------------------------------------------------
# decode with split-KV
# ---------------------------------------------------------------------------

def split_ranges(num_tiles: int, num_splits: int):
    """Split s owns key tiles [floor(s T / S), floor((s + 1) T / S)): contiguous,
    near-equal ranges of whole tiles (the page leaves the partition open)."""
    return [((s * num_tiles) // num_splits, ((s + 1) * num_tiles) // num_splits)
            for s in range(num_splits)]


def decode_row_branches(qrow, k, v, tau, block_k, num_splits, band=0.0,
                        max_branches=64):
    """One decode query row against the whole cache of its KV head.

    Each split starts from an empty state (m = -inf, l = 0), visits its own
    tiles from the most recent one downward and tests them against its own
    partial normalizer, while L = N_k (the full causal context, counting the
    current token) stays in the threshold. Returns, per split, the list of
    admissible ``BlockResult`` outcomes (one unless ``band`` > 0 and an
    in-band tile occurs)."""
    nk = k.shape[0]
    T = num_blocks(nk, block_k)
    out = []
    for lo, hi in split_ranges(T, num_splits):
        args = (qrow[None, :], k, v, np.array([nk - 1]), np.array([nk]),
                list(range(hi - 1, lo - 1, -1)), tau, block_k)
        if band > 0:
            out.append(forward_block_branches(*args, band=band, max_branches=max_branches))
        else:
            out.append([forward_block(*args)])
    return out


def decode_block_branches(qblock, k, v, last_visible, tau, block_k, num_splits, band=0.0,
                          max_branches=64):
    """A short decoding query - the rows of one head, each at its own
    position - against the whole cache of its KV head ("Fused decoding
    execution": the forward rule with a short query and a longer KV
    sequence). The rows form one query block: they share every tile
    decision, each keeps its own running state, and row q sees keys up to
    last_visible[q] with L_q = last_visible[q] + 1 (a single row at the end
    of the cache gives L_0 = N_k). Each split starts from an empty state and
    visits its own tiles from the most recent one downward, as in
    ``decode_row_branches``. Returns, per split, the list of admissible
    ``BlockResult`` outcomes (one unless ``band`` > 0 and an in-band tile
    occurs)."""
    nk = k.shape[0]
    T = num_blocks(nk, block_k)
    last_visible = np.asarray(last_visible)
    out = []
    for lo, hi in split_ranges(T, num_splits):
        args = (qblock, k, v, last_visible, last_visible + 1, list(range(hi - 1, lo - 1, -1)), tau, block_k)
        with np.errstate(divide="ignore", invalid="ignore"):  # rows without keys in a split: l = 0
            if band > 0:
                out.append(forward_block_branches(*args, band=band, max_branches=max_branches))
            else:
                out.append([forward_block(*args)])
    return out


def combine_split_rows(results, nrows):
    """Per-row normalizer-aware combine of split results (``BlockResult`` with
    o [rows, dv] and z [rows]). A row that holds no key in a split (l = 0
    there, so z = -inf) takes no part in that row's combine; a row with no
    key in any split gets o = 0, z = -inf. Returns (o [rows, dv], z [rows])."""
    dv = results[0].o.shape[1]
    o = np.zeros((nrows, dv))
    z = np.full(nrows, -np.inf)
    for r in range(nrows):
        parts = [(res.o[r], res.z[r]) for res in results if np.isfinite(res.z[r])]
        if parts:
            o[r], z[r] = combine_splits(parts)
    return o, z


def mala_decode_short(q, k, v, tau: float, block_k: int, num_splits: int = 1, seq_lens=None,
                      heads=None):
    """MALA decode of a short query: q [B, Nq, Hq, d] holds the Nq newest
    tokens of each sequence, caches k, v [B, Nk, Hkv, d] (or the first
    seq_lens[b] rows of them for sequence b). Token t of sequence b sits at
    position N_k(b) - Nq + t and sees the keys up to it, so L_q counts its
    full causal context; the Nq rows of a head form one query block
    (``decode_block_branches``), split into ``num_splits`` contiguous tile
    ranges of that sequence's T_b tiles and combined per row. Rows at a
    negative position (N_k(b) < Nq) have no keys: o = 0, z = -inf. With
    Nq = 1 this is ``mala_decode``. ``heads`` optionally restricts the
    computation to an iterable of (b, h). Returns dict with o [B, Nq, Hq, dv],
    z [B, Hq, Nq], mask and margin [B, Hq, T] (T = tiles of the full cache;
    255 / NaN past a sequence's last tile)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, nq, hq, _ = q.shape
    nk_cap, hkv, dv = k.shape[1], k.shape[2], v.shape[3]
    T_cap = num_blocks(nk_cap, block_k)
    o = np.zeros((B, nq, hq, dv))
    z = np.full((B, hq, nq), -np.inf)
    mask = np.full((B, hq, T_cap), 255, dtype=np.uint8)
    margin = np.full((B, hq, T_cap), np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(hq)]
    for (b, h) in heads:
        nk = nk_cap if seq_lens is None else int(seq_lens[b])
        pos = nk - nq + np.arange(nq)
        rows = np.nonzero(pos >= 0)[0]
        if nk == 0 or rows.size == 0:
            continue
        g = kv_head(h, hq, hkv)
        per_split = decode_block_branches(q[b, rows, h], k[b, :nk, g], v[b, :nk, g], pos[rows], tau,
                                          block_k, num_splits)
        results = []
        for (res,) in per_split:
            results.append(res)
            for j, dcs in res.decision.items():
                mask[b, h, j] = dcs
                margin[b, h, j] = res.margin[j]
        o_rows, z_rows = combine_split_rows(results, rows.size)
        o[b, rows, h] = o_rows
        z[b, h, rows] = z_rows
    return {"o": o, "z": z, "mask": mask, "margin": margin}


def combine_splits(parts):
    """Normalizer-aware reduction of split partials (o_s, z_s):
    z = log sum_s exp(z_s), o = sum_s exp(z_s - z) o_s (the block-combination
    rule of the tutorial page's FlashAttention section)."""
    zs = np.array([p[1] for p in parts])
    zmax = zs.max()
    w = np.exp(zs - zmax)
    z = zmax + np.log(w.sum())
    o = sum(np.exp(zs[s] - z) * parts[s][0] for s in range(len(parts)))
    return o, z


def mala_decode(q, k, v, tau: float, block_k: int, num_splits: int = 1, rows=None):
    """Single-token MALA decode: q [B, 1, Hq, d], caches k, v [B, Nk, Hkv, d].

    The forward rule with N_q = 1 and L_0 = N_k ("Fused decoding execution"),
    optionally over ``num_splits`` contiguous tile ranges combined by
    ``combine_splits``. ``rows`` optionally restricts to an iterable of
    (b, h). Returns dict with o [B, Hq, dv], z [B, Hq] and the per-tile
    decisions mask [B, Hq, T] (1 retained, 0 skipped; each tile belongs to
    exactly one split)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, _, hq, _ = q.shape
    nk, hkv, dv = k.shape[1], k.shape[2], v.shape[3]
    T = num_blocks(nk, block_k)
    o = np.full((B, hq, dv), np.nan)
    z = np.full((B, hq), np.nan)
    mask = np.full((B, hq, T), 255, dtype=np.uint8)
    margin = np.full((B, hq, T), np.nan)
    if rows is None:
        rows = [(b, h) for b in range(B) for h in range(hq)]
    for (b, h) in rows:
        g = kv_head(h, hq, hkv)
        per_split = decode_row_branches(q[b, 0, h], k[b, :, g], v[b, :, g], tau,
                                        block_k, num_splits)
        parts = []
        for (res,) in per_split:
            parts.append((res.o[0], res.z[0]))
            for j, dcs in res.decision.items():
                mask[b, h, j] = dcs
                margin[b, h, j] = res.margin[j]
        o[b, h], z[b, h] = combine_splits(parts)
    return {"o": o, "z": z, "mask": mask, "margin": margin}


def mala_decode_latent(q, kv, d_v: int, tau: float, block_k: int, num_splits: int = 1, rows=None):
    """Single-token MALA decode on latent (MLA-shaped) attention: q [B, 1, Hq, d_qk]
    and one cached row per position kv [B, Nk, 1, d_qk]; the value is the
    latent, the first d_v columns of the row (absorbed form, attention
    tutorial page, section "MLA: compress the cached representation").
    The decode rule ("Fused decoding execution" and the split-KV paragraph)
    does not depend on the shapes, so this is ``mala_decode`` with k = kv and
    v = kv[..., :d_v]."""
    kv = _as64(kv)
    return mala_decode(q, kv, kv[..., :d_v], tau, block_k, num_splits=num_splits, rows=rows)


def mala_decode_paged(q, k_pages, v_pages, block_table, seq_lens, page_size: int, tau: float,
                      block_k: int, num_splits: int = 1):
    """Single-token MALA decode over a paged cache with per-sequence lengths.

    Sequence b's keys are gathered in order, key k from row k % page_size of
    page block_table[b, k // page_size]; then the decode rule runs on them
    exactly as in ``mala_decode`` with L_0 = N_k(b) = seq_lens[b] and the
    split partition over that sequence's own T_b tiles. A split whose tile
    range is empty holds no keys and is left out of the combine; a sequence
    with no keys gets o = 0, z = -inf. Returns dict with o [B, Hq, dv],
    z [B, Hq], mask [B, Hq, T_cap] (255 past a sequence's last tile) and
    margin, T_cap = ceil(max_pages * page_size / block_k)."""
    q, kp, vp = _as64(q), _as64(k_pages), _as64(v_pages)
    table, lens = np.asarray(block_table), np.asarray(seq_lens)
    B, _, hq, _ = q.shape
    hkv, dv = kp.shape[2], vp.shape[3]
    t_cap = num_blocks(table.shape[1] * page_size, block_k)
    o = np.zeros((B, hq, dv))
    z = np.full((B, hq), -np.inf)
    mask = np.full((B, hq, t_cap), 255, dtype=np.uint8)
    margin = np.full((B, hq, t_cap), np.nan)
    for b in range(B):
        nk = int(lens[b])
        if nk == 0:
            continue
        keys = np.arange(nk)
        pages = table[b, keys // page_size]
        rows = keys % page_size
        for h in range(hq):
            g = kv_head(h, hq, hkv)
            kseq, vseq = kp[pages, rows, g], vp[pages, rows, g]
            with np.errstate(divide="ignore", invalid="ignore"):  # empty splits: l = 0
                per_split = decode_row_branches(q[b, 0, h], kseq, vseq, tau, block_k, num_splits)
            parts = []
            for (lo, hi), (res,) in zip(split_ranges(num_blocks(nk, block_k), num_splits), per_split):
                if hi > lo:
                    parts.append((res.o[0], res.z[0]))
                for j, dcs in res.decision.items():
                    mask[b, h, j] = dcs
                    margin[b, h, j] = res.margin[j]
            o[b, h], z[b, h] = combine_splits(parts)
    return {"o": o, "z": z, "mask": mask, "margin": margin}


# ---------------------------------------------------------------------------
# reported quantities
# ---------------------------------------------------------------------------

def omitted_mass(z_screened, z_reference):
    """1 - exp(z_screened - z_reference): dense-softmax mass of the positions
    the screened operator left out (MALA page, experiments)."""
    return 1.0 - np.exp(_as64(z_screened) - _as64(z_reference))


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 (MALA page, operator fidelity)."""
    x, ref = _as64(x), _as64(ref)
    return float(np.linalg.norm((x - ref).ravel()) / np.linalg.norm(ref.ravel()))


def post_score_slots(mask, block_q: int, block_k: int, nq: int) -> int:
    """Post-score key slots of a prefill mask [B, Hq, nQB, nKB]: every
    retained tile gives B_k slots to each valid row of its query block (the
    page's allocation metric)."""
    mask = np.asarray(mask)
    total = 0
    nqb = mask.shape[2]
    for i in range(nqb):
        rows = min((i + 1) * block_q, nq) - i * block_q
        total += int((mask[:, :, i, :] == 1).sum()) * block_k * rows
    return total



def slot_histogram(mask, block_q: int, nq: int) -> np.ndarray:
    """Histogram of post-score key slots per query (MALA page, allocation
    metric as recorded per query in its fidelity study) from a tile mask
    [B, Hq, nQB, nKB]: for each query block, c = number of retained tiles in
    its mask row; each valid query row of the block counts once in bin c (its
    post-score slots are c * B_k). Returns int64 [nKB + 1]."""
    mask = np.asarray(mask)
    B, H, nqb, nkb = mask.shape
    hist = np.zeros(nkb + 1, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                c = int((mask[b, h, i] == 1).sum())
                hist[c] += min((i + 1) * block_q, nq) - i * block_q
    return hist


def sq_err_heads(x, ref):
    """Per (batch, head) sums of (x - ref)^2 and ref^2 over a BSHD tensor's
    [seq, head_dim] slice (the pieces of the per-head relative L2 error of the
    page's operator-fidelity study). Returns two float64 arrays [B, H]."""
    x, ref = _as64(x), _as64(ref)
    d = x - ref
    return (d * d).sum(axis=(1, 3)), (ref * ref).sum(axis=(1, 3))


_SM_GAMMA = np.uint64(0x9E3779B97F4A7C15)


def splitmix64(seed: int, n: int) -> np.ndarray:
    """Outputs 0..n-1 of SplitMix64 (Steele, Lea and Flood, 2014) seeded with
    ``seed``: the state advances by the golden gamma 0x9E3779B97F4A7C15 per
    output and each output is the published mixing function of the state, so
    output i mixes seed + (i + 1) * gamma (arithmetic mod 2^64)."""
    i = np.arange(1, n + 1, dtype=np.uint64)
    z = np.uint64(seed & ((1 << 64) - 1)) + i * _SM_GAMMA
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def rademacher(n: int, seed: int) -> np.ndarray:
    """Deterministic Rademacher probe (the page drives its backward fidelity
    comparison with one): -1 where the top bit of SplitMix64 output i is set,
    +1 elsewhere."""
    return np.where(splitmix64(seed, n) >> np.uint64(63), -1.0, 1.0)