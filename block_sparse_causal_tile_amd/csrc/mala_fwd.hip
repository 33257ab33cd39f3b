// MALA forward / prefill kernels for gfx950.
//
// One workgroup owns one (batch, query head, query block I_i) work item and
// walks the legal key blocks J_j from the diagonal downward (MALA page,
// "Fused forward execution"). For each tile it
//   1. has K_j copied from HBM straight into a swizzled LDS tile,
//   2. computes S^T = K_j Q_i^T on the matrix cores (bf16 in, fp32 out),
//   3. takes each row's maximum over its legal keys and evaluates the
//      log-domain block test against the running (m, l) of that row
//      ("Online Sparse Softmax"): retain iff some relevant row has
//      rowmax - (m + log l) >= log tau - log L_q, l = 0 meaning +inf,
//   4. ORs the per-wave votes through LDS into one workgroup-uniform flag,
//   5. only for a retained tile: copies V_j into LDS, applies the
//      online-softmax update while the copy lands, and accumulates P V_j on
//      the matrix cores, reading V^T with the LDS transpose loads.
// A skipped tile never touches V. The final O / l and z = m + log l are the
// only writes (plus the optional debug mask and counters).
//
// Layout of the work inside a workgroup: B_q / 32 waves, each wave owns 32
// query rows. Scores are computed transposed (keys x rows) so that every
// lane holds a single query row: row statistics are per-lane scalars and
// the rescale of the output accumulator is a per-lane multiply.
#include <math.h>

#include "mala_common.hpp"

namespace mala {
namespace {

// Key row fed to A-row x of the score MFMA: bits 2 and 3 of x swapped. With
// this order, accumulator registers 8a..8a+7 of lane half hh hold the eight
// consecutive keys 16a + 8hh + 0..7 - the k-slot order the PV MFMA expects
// for its B operand, so P goes from score registers to the PV MFMA without
// any data movement.
__device__ __forceinline__ int key_perm(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Per key tile j (diagonal first, then descending):
//   S_j = K_j Q^T on the matrix cores (K_j in LDS) -> row maxima and the
//   block test -> wave votes -> barrier -> if retained, the V_j copy into
//   LDS is issued, then K_{j-1}'s -> the online-softmax update of a retained
//   tile (it needs only S_j) overlaps both copies -> wait, barrier -> P V_j.
// K and V tiles move straight from HBM into LDS (no register staging), so
// the only long-lived registers are Q, the scores and the accumulator, and
// several workgroups fit on a CU to cover each other's waits.
template <int D, int BQ, int BK, int SUB, bool VARLEN>
__global__ void __launch_bounds__(BQ * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(FwdParams a) {
  constexpr int NW = BQ / 32;
  // The workgroup covers BQ query rows; decisions are taken per query block
  // of SUB rows (SUB = B_q of the problem, BQ / SUB blocks per workgroup, each
  // with its own waves, votes, statistics and mask entries). Blocks that
  // share a workgroup share its K and V tiles and barriers; V is copied when
  // any of them retains the tile.
  constexpr int HALVES = BQ / SUB;
  constexpr int WPH = SUB / 32;
  static_assert(BQ % SUB == 0 && SUB % 32 == 0, "decision blocks split the workgroup by waves");
  constexpr int KSTEPS = D / 16;  // score MFMA steps over head_dim
  constexpr int MB = BK / 32;     // 32-key blocks per tile
  constexpr int EB = D / 32;      // 32-dim blocks of the output
  constexpr int PSTEPS = BK / 16; // PV MFMA steps over keys
  constexpr int KT = BK * D;      // elements of a K or V tile

  __shared__ __attribute__((aligned(1024))) uint16_t sK[KT];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[KT];
  __shared__ int sVote[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int l32 = lane & 31;

  // Heaviest work first: query blocks from the last (longest causal row) to
  // the first. Workgroups go to the 8 XCDs round-robin by index, so each XCD
  // is given its own share of the (batch, head) pairs - whole KV groups when
  // they divide evenly - and the K/V tiles it re-reads stay in its L2.
  // (Packed sequences differ in length, so whole heads per XCD would leave
  // XCDs idle; there the items simply go round-robin, and the query blocks
  // are counted from each sequence's own end, so every sequence's heaviest
  // blocks - a short chunk after a long cached context included - come
  // first rather than those of the longest sequence alone.)
  const int BH = a.batch * a.heads_q;
  const int nx = (!VARLEN && BH % 8 == 0) ? 8 : 1;
  const int xcd = blockIdx.x % nx, slot = blockIdx.x / nx, h_per = BH / nx;
  const int nqb_w = (a.seqlen_q + BQ - 1) / BQ;  // workgroup blocks per (batch, head)
  int i = nqb_w - 1 - slot / h_per;
  const int bh = xcd * h_per + slot % h_per;
  const int b = bh / a.heads_q;
  const int h = bh % a.heads_q;
  const int g = h / (a.heads_q / a.heads_kv);

  // the sequence: lengths, causal offset and first rows of q/o and k/v
  int n_q = a.seqlen_q, n_k = a.seqlen_k, off = a.offset;
  size_t q_start = (size_t)b * a.seqlen_q, k_start = (size_t)b * a.seqlen_k;
  size_t z_row0 = ((size_t)b * a.heads_q + h) * a.seqlen_q;
  if (VARLEN) {
    // packed sequences, bounds clamped to the packed tensors; bottom-right
    // causal alignment per sequence (offset N_k - N_q; rows before the first
    // key see nothing and come out as o = 0, z = -inf)
    const int qs = min(max(a.cu_q[b], 0), a.total_q), qe = min(max(a.cu_q[b + 1], qs), a.total_q);
    const int ks = min(max(a.cu_k[b], 0), a.total_k), ke = min(max(a.cu_k[b + 1], ks), a.total_k);
    n_q = min(qe - qs, a.seqlen_q);
    n_k = min(ke - ks, a.seqlen_k);
    off = n_k - n_q;
    q_start = qs;
    k_start = ks;
    z_row0 = (size_t)h * a.total_q + qs;
    i = (n_q + BQ - 1) / BQ - 1 - slot / h_per;  // the (slot / h_per)-th block from the end
    if (i < 0) return;  // the sequence has fewer blocks (uniform)
  }

  const int row0 = i * BQ;
  const int valid_rows = min(BQ, n_q - row0);
  const int last_key = row0 + valid_rows - 1 + off;  // last key the workgroup sees
  const int jmax = last_key >= 0 ? last_key / BK : -1;
  const bool ragged_rows = valid_rows < BQ;
  // the decision blocks: highest legal tile of each (-1: no rows or no keys)
  int jmax_h[HALVES], rows_h[HALVES];
#pragma unroll
  for (int x = 0; x < HALVES; ++x) {
    rows_h[x] = min(max(n_q - (row0 + x * SUB), 0), SUB);
    const int lk = row0 + x * SUB + rows_h[x] - 1 + off;
    jmax_h[x] = (rows_h[x] > 0 && lk >= 0) ? lk / BK : -1;
  }
  const int hf = wave / WPH;  // this wave's decision block

  const int row = row0 + wave * 32 + l32;
  const bool row_valid = row < n_q;
  const int row_lim = row_valid ? row + off : -1;  // last visible key
  // log(tau / L_q) with L_q = q + offset + 1
  const float thr = a.log_tau - __logf((float)(row + off + 1));

  const size_t q_rs = (size_t)a.heads_q * D;   // elements between sequence rows
  const size_t kv_rs = (size_t)a.heads_kv * D;
  const uint16_t* kbase = (const uint16_t*)a.k + (k_start * a.heads_kv + g) * D;
  const uint16_t* vbase = (const uint16_t*)a.v + (k_start * a.heads_kv + g) * D;
  const size_t qo_off = (q_start * a.heads_q + h) * D + (size_t)row * q_rs;

  // Q row fragment, the B operand of the score MFMA (8 dims per step).
  u32x4_t qf[KSTEPS];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + qo_off;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qf[kk] = row_valid ? ld16(qrow + 16 * kk + 8 * hh) : zero16();
  }
  // Per-lane LDS offsets (elements), fixed for the whole loop: the score
  // operand of key row 32 mb + key_perm(l32) at dims 16 kk + 8 hh, and the
  // two transposing reads of the PV operand (tile_col8 layout).
  int koff[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) koff[kk] = tile_idx<D>(key_perm(l32), 16 * kk + 8 * hh);
  int voff_lo[EB], voff_hi[EB];
  {
    const int grp = lane >> 4, y = lane & 15;
    const int rl = 8 * (grp >> 1) + (y >> 2);
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      const int col = 32 * e + 16 * (grp & 1) + 4 * (y & 3);
      voff_lo[e] = tile_idx<D>(rl, col);
      voff_hi[e] = tile_idx<D>(rl + 4, col);
    }
  }
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

  f32x16_t acc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) acc[e] = f32x16_t{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  int n_retained = 0;
  int n_vcopy = 0;  // V tiles copied by the workgroup (some block retained)

  // ---- the steps of one tile, used in software-pipelined order below -------
  // score discovery S^T = K Q^T from the K tile in LDS
  auto score = [&](f32x16_t* sc) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) sc[mb] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        sc[mb] = mfma32(*reinterpret_cast<const u32x4_t*>(&sK[32 * mb * D + koff[kk]]), qf[kk], sc[mb]);
    interleave_ds_mfma<KSTEPS * MB, 1>();
  };
  // causal mask, row maxima and the block test; the barrier inside also
  // marks every wave done reading the K and V tiles in LDS
  float mx = -INFINITY;
  bool relevant = false;
  bool retain_any = false;  // some block of the workgroup retains the tile
  auto decide = [&](int j, f32x16_t* sc) -> bool {
    const bool need_mask = ragged_rows || (j * BK + BK - 1 > row0 + off);
    mx = -INFINITY;
    if (need_mask) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * BK + 32 * mb + key_perm(acc_row(r, hh));
          if (key > row_lim) sc[mb][r] = -INFINITY;
          mx = fmaxf(mx, sc[mb][r]);
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[mb][r]);
    }
    mx = wave_max_halves(mx);
    relevant = mx > -INFINITY;  // row has a legal key in this tile
    float margin = -INFINITY;
    if (relevant) margin = (l_run > 0.f) ? (mx - m_run - test_log(l_run) - thr) : INFINITY;
    const bool vote = __ballot(margin >= 0.f) != 0ull;
    if (lane == 0) sVote[wave] = vote ? 1 : 0;
    __syncthreads();  // votes visible; every wave is done reading K and V
    bool retain = false;
    retain_any = false;
#pragma unroll
    for (int x = 0; x < HALVES; ++x) {
      bool r = false;
#pragma unroll
      for (int w = x * WPH; w < (x + 1) * WPH; ++w) r |= sVote[w] != 0;
      retain_any |= r;
      if (x == hf) retain = r;
      if (tid == 0 && a.tile_mask && j <= jmax_h[x])
        a.tile_mask[(((size_t)b * a.heads_q + h) * a.nqb + i * HALVES + x) * a.nkb + j] = r ? 1 : 0;
    }
    return retain;
  };
  // online-softmax update of a retained tile; P packed as the PV B operand
  u32x4_t pf[PSTEPS];
  auto update = [&](const f32x16_t* sc) {
    // m is the row's reference, not always its running maximum: it moves
    // only on the row's first legal tile or when the tile's maximum exceeds
    // it by more than 8 / log2(e) (a factor 2^8 in probability), so most
    // tiles skip the rescale. P = 2^((S - m) log2 e) then stays below 2^8,
    // and l is the sum relative to m, so m + log l = log Z as before (the
    // test and z use only that sum).
    const bool grow = relevant && (mx - m_run) * kLog2e > 8.f;
    const float m_new = grow ? mx : m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e) : 1.f;
    if (__ballot(grow) != 0ull) {  // rescale only when some row's reference moved
#pragma unroll
      for (int e = 0; e < EB; ++e) acc[e] *= alpha;
    }
    // a row with no legal key in the tile has every score at -inf; shifting
    // it by +inf instead of m_new (which may still be -inf) sends each of its
    // exponentials to exp2(-inf) = 0 without a per-entry select
    const float msc = relevant ? m_new * kLog2e : INFINITY;
    float rs = 0.f;
#pragma unroll
    for (int c = 0; c < PSTEPS; ++c) {
      float p[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float sv = sc[c >> 1][8 * (c & 1) + x];
        p[x] = __builtin_amdgcn_exp2f(fmaf(sv, kLog2e, -msc));
        rs += p[x];
      }
      pf[c] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])};
    }
    rs = wave_sum_halves(rs);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    ++n_retained;
  };
  // O^T += V^T P^T from the V tile in LDS (transposing reads)
  auto pv = [&]() {
#pragma unroll
    for (int c = 0; c < PSTEPS; ++c)
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&sV[16 * c * D + voff_lo[e]]);
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&sV[16 * c * D + voff_hi[e]]);
        const u32x2_t x = __builtin_bit_cast(u32x2_t, lo), y = __builtin_bit_cast(u32x2_t, hi);
        acc[e] = mfma32(u32x4_t{x[0], x[1], y[0], y[1]}, pf[c], acc[e]);
      }
  };

  // ---- the walk over the key tiles, diagonal first --------------------------
  // With 64-key tiles it is software-pipelined: tile j's decision and
  // softmax update come one step before its P V, and the score discovery of
  // tile j - 1 runs beside that P V - one run of independent MFMAs per step
  // (S_{j-1} and P_j V_j), then the VALU work of tile j - 1 (mask, test,
  // update) while V_{j-1} and K_{j-2} land in LDS.
  f32x16_t s[MB];
  bool retain = false;
  if constexpr (BK == 64) {
    // Copies per wave for one tile (the waves split a tile's copy).
    constexpr int CI = TileCopy<D, BK, NW>::CI;
    // Per tile: the decision (its barrier also frees the K and V tiles),
    // then the copy of K_{j-1} and, for a retained tile, of V_j - K first,
    // so that waiting for K leaves V in flight; the softmax update overlaps
    // both copies, the score discovery of tile j-1 overlaps the V copy, and
    // V_j is awaited only right before P V_j.
    TileCopy<D, BK, NW> cp;
    cp.init(kv_rs, wave, lane);
    if (jmax >= 0) {
      cp.copy(sK, kbase, kv_rs, jmax * BK, n_k, wave, lane);
      wait_vmcnt<0>();
      __syncthreads();
      score(s);
    }
    for (int j = jmax; j >= 0; --j) {
      retain = decide(j, s);
      const bool any = retain_any;
      n_vcopy += any ? 1 : 0;
      if (j > 0) cp.copy(sK, kbase, kv_rs, (j - 1) * BK, n_k, wave, lane);
      if (any) cp.copy(sV, vbase, kv_rs, j * BK, n_k, wave, lane);
      if (retain) update(s);
      if (j > 0) {
        if (any) wait_vmcnt<CI>(); else wait_vmcnt<0>();  // K_{j-1} landed; V_j may fly
        lds_barrier();
        score(s);  // S_{j-1}
      }
      if (any) {
        wait_vmcnt<0>();  // V_j landed
        lds_barrier();
        if (retain) pv();
      }
    }
  } else {
    // 128-key tiles: the scores alone fill 64 registers, too many to hold a
    // second tile's beside P; the steps of a tile run in sequence (the
    // builtin copies measured faster here than the inline-assembly ones)
    TileCopy<D, BK, NW, true> cp;
    cp.init(kv_rs, wave, lane);
    if (jmax >= 0) cp.copy(sK, kbase, kv_rs, jmax * BK, n_k, wave, lane);
    wait_vmcnt<0>();
    __syncthreads();
    for (int j = jmax; j >= 0; --j) {
      score(s);
      retain = decide(j, s);
      n_vcopy += retain_any ? 1 : 0;
      if (retain_any) cp.copy(sV, vbase, kv_rs, j * BK, n_k, wave, lane);
      if (j > 0) cp.copy(sK, kbase, kv_rs, (j - 1) * BK, n_k, wave, lane);
      if (retain) update(s);
      wait_vmcnt<0>();
      __syncthreads();  // V_j and K_{j-1} are in LDS
      if (retain) pv();
    }
  }

  // ---- finalize: O = acc / l, z = m + log l ---------------------------------
  if (row_valid) {
    // a row that saw no key (possible only in packed sequences with
    // N_k < N_q) has l = 0: o = 0, z = -inf
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* orow = (uint16_t*)a.o + qo_off;
#pragma unroll
    for (int e = 0; e < EB; ++e)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = 32 * e + 8 * rq + 4 * hh;
        u32x2_t w = {pack_bf16x2(acc[e][4 * rq] * inv, acc[e][4 * rq + 1] * inv),
                     pack_bf16x2(acc[e][4 * rq + 2] * inv, acc[e][4 * rq + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(orow + d) = w;
      }
    if (hh == 0) a.z[z_row0 + row] = l_run > 0.f ? m_run + __logf(l_run) : -INFINITY;
  }
  // counters per decision block, from the block's first wave; V copies
  // once per workgroup (a tile's V is copied once when any of the
  // workgroup's blocks retains it)
  if (lane == 0 && wave % WPH == 0 && a.stats) {
    atomicAdd(&a.stats[0], (unsigned long long)(jmax_h[hf] + 1));
    atomicAdd(&a.stats[1], (unsigned long long)n_retained);
    atomicAdd(&a.stats[2], (unsigned long long)n_retained * BK * rows_h[hf]);
    if (wave == 0) atomicAdd(&a.stats[3], (unsigned long long)n_vcopy);
  }
}

// fp32 path: plain fp32 SIMT arithmetic, 4 threads per query row (each
// scores a quarter of the tile's keys and accumulates a quarter of the
// output dims). Same traversal, test and update as the bf16 kernel.
template <int D, int BQ, int BK>
__global__ void __launch_bounds__(BQ * 4) fwd_fp32_kernel(FwdParams a) {
  constexpr int NT = BQ * 4;
  constexpr int KPT = BK / 4;
  constexpr int DPT = D / 4;
  constexpr int KS = D + 1;  // padded LDS row of K
  constexpr int PS = BK + 1; // padded LDS row of P
  constexpr int KP_WORDS = (BK * KS > BQ * PS) ? BK * KS : BQ * PS;
  __shared__ float sKP[KP_WORDS];  // K tile while scoring, then P
  __shared__ float sV[BK * D];
  __shared__ int sVote;

  const int tid = threadIdx.x;
  const int sub = tid & 3;
  const int r = tid >> 2;

  const int BH = a.batch * a.heads_q;
  const int i = a.nqb - 1 - (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int b = bh / a.heads_q;
  const int h = bh % a.heads_q;
  const int g = h / (a.heads_q / a.heads_kv);

  const int row0 = i * BQ;
  const int valid_rows = min(BQ, a.seqlen_q - row0);
  const int jmax = (row0 + valid_rows - 1 + a.offset) / BK;
  const int row = row0 + r;
  const bool row_valid = row < a.seqlen_q;
  const int row_lim = row_valid ? row + a.offset : -1;
  const float thr = a.log_tau - logf((float)(row + a.offset + 1));

  const size_t q_rs = (size_t)a.heads_q * D;
  const size_t kv_rs = (size_t)a.heads_kv * D;
  const float* kbase = (const float*)a.k + ((size_t)b * a.seqlen_k * a.heads_kv + g) * D;
  const float* vbase = (const float*)a.v + ((size_t)b * a.seqlen_k * a.heads_kv + g) * D;
  const size_t qo_off = ((size_t)b * a.seqlen_q * a.heads_q + h) * D + (size_t)row * q_rs;

  // my quarter of the query row: dims sub * DPT .. sub * DPT + DPT - 1
  float qv[DPT];
#pragma unroll
  for (int x = 0; x < DPT; ++x) qv[x] = row_valid ? ((const float*)a.q)[qo_off + sub * DPT + x] : 0.f;
  float o[DPT];
#pragma unroll
  for (int x = 0; x < DPT; ++x) o[x] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  int n_retained = 0;

  for (int j = jmax; j >= 0; --j) {
    __syncthreads();
    for (int e = tid; e < BK * D; e += NT) {
      const int kr = e / D, d = e % D;
      const int key = j * BK + kr;
      sKP[kr * KS + d] = key < a.seqlen_k ? kbase[(size_t)key * kv_rs + d] : 0.f;
    }
    if (tid == 0) sVote = 0;
    __syncthreads();
    // scores: each thread forms partial dot products over its quarter of the
    // dims for 16 keys at a time; the four quarters are summed across the
    // row's threads and thread `sub` keeps keys 16 c + 4 sub + 0..3.
    float s[KPT];
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < BK / 16; ++c) {
      float part[16];
#pragma unroll
      for (int kx = 0; kx < 16; ++kx) {
        const float* krow = &sKP[(16 * c + kx) * KS + sub * DPT];
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < DPT; ++x) acc = fmaf(qv[x], krow[x], acc);
        part[kx] = acc;
      }
#pragma unroll
      for (int kx = 0; kx < 16; ++kx) {
        part[kx] += __shfl_xor(part[kx], 1);
        part[kx] += __shfl_xor(part[kx], 2);
      }
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int kr = 16 * c + 4 * sub + y;
        const float sv = (j * BK + kr <= row_lim) ? part[4 * sub + y] : -INFINITY;
        s[4 * c + y] = sv;
        mx = fmaxf(mx, sv);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    const bool relevant = mx > -INFINITY;
    float margin = -INFINITY;
    if (relevant) margin = (l_run > 0.f) ? (mx - m_run - logf(l_run) - thr) : INFINITY;
    if (margin >= 0.f) sVote = 1;
    __syncthreads();
    const bool retain = sVote != 0;
    if (tid == 0 && a.tile_mask)
      a.tile_mask[(((size_t)b * a.heads_q + h) * a.nqb + i) * a.nkb + j] = retain ? 1 : 0;
    if (!retain) continue;
    // sKP now becomes the P tile; every thread has finished reading K above.
    for (int e = tid; e < BK * D; e += NT) {
      const int kr = e / D, d = e % D;
      const int key = j * BK + kr;
      sV[kr * D + d] = key < a.seqlen_k ? vbase[(size_t)key * kv_rs + d] : 0.f;
    }
    const float m_new = relevant ? fmaxf(m_run, mx) : m_run;
    const float alpha = relevant ? expf(m_run - m_new) : 1.f;
    float rs = 0.f;
#pragma unroll
    for (int x = 0; x < KPT; ++x) {
      const float p = relevant ? expf(s[x] - m_new) : 0.f;
      rs += p;
      sKP[r * PS + 16 * (x >> 2) + 4 * sub + (x & 3)] = p;
    }
    rs += __shfl_xor(rs, 1);
    rs += __shfl_xor(rs, 2);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < DPT; ++x) {
      const int d = sub * DPT + x;
      float acc = o[x] * alpha;
      for (int kr = 0; kr < BK; ++kr) acc = fmaf(sKP[r * PS + kr], sV[kr * D + d], acc);
      o[x] = acc;
    }
    ++n_retained;
  }

  if (row_valid) {
    float* orow = (float*)a.o + qo_off;
#pragma unroll
    for (int x = 0; x < DPT; ++x) orow[sub * DPT + x] = o[x] / l_run;
    if (sub == 0) a.z[((size_t)b * a.heads_q + h) * a.seqlen_q + row] = m_run + logf(l_run);
  }
  if (tid == 0 && a.stats) {
    atomicAdd(&a.stats[0], (unsigned long long)(jmax + 1));
    atomicAdd(&a.stats[1], (unsigned long long)n_retained);
    atomicAdd(&a.stats[2], (unsigned long long)n_retained * BK * valid_rows);
    atomicAdd(&a.stats[3], (unsigned long long)n_retained);
  }
}

template <int D, int BQ, int BK, int SUB>
hipError_t run_fwd(const mala_problem& p, const FwdParams& a, hipStream_t s) {
  if (p.dtype == MALA_BF16) {
    const dim3 grid((unsigned)(a.batch * a.heads_q * ((a.seqlen_q + BQ - 1) / BQ)));
    if (a.cu_q)
      hipLaunchKernelGGL((fwd_bf16_kernel<D, BQ, BK, SUB, true>), grid, dim3(BQ * 2), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<D, BQ, BK, SUB, false>), grid, dim3(BQ * 2), 0, s, a);
  } else {
    const dim3 grid((unsigned)(a.batch * a.heads_q * a.nqb));
    hipLaunchKernelGGL((fwd_fp32_kernel<D, SUB, BK>), grid, dim3(SUB * 4), 0, s, a);
  }
  return hipGetLastError();
}

// bf16: a workgroup always covers 128 query rows (four waves), i.e. one
// 128-row decision block or two 64-row ones; fp32: one block per workgroup.
template <int D>
hipError_t run_fwd_d(const mala_problem& p, const FwdParams& a, hipStream_t s, bool* ok) {
  *ok = true;
  if (p.block_q == 64 && p.block_k == 64) return run_fwd<D, 128, 64, 64>(p, a, s);
  if (p.block_q == 64 && p.block_k == 128) return run_fwd<D, 128, 128, 64>(p, a, s);
  if (p.block_q == 128 && p.block_k == 64) return run_fwd<D, 128, 64, 128>(p, a, s);
  if (p.block_q == 128 && p.block_k == 128) return run_fwd<D, 128, 128, 128>(p, a, s);
  *ok = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_fwd(const mala_problem& p, const FwdParams& a, hipStream_t s, bool* supported) {
  *supported = false;
  if (p.dtype != MALA_BF16 && p.dtype != MALA_FP32) return hipSuccess;
  if (p.head_dim == 64) return run_fwd_d<64>(p, a, s, supported);
  if (p.head_dim == 128) return run_fwd_d<128>(p, a, s, supported);
  return hipSuccess;
}

}  // namespace mala
