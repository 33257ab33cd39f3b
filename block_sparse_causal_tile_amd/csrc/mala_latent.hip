// MALA forward on latent (MLA-shaped) attention for gfx950.
//
// Every query head scores one shared cached row per position,
// kv_s = [c_s, r_s] (d_qk = 576: a 512-wide latent c_s and a 64-wide
// positional part r_s), and the value is the latent itself, v_s = c_s - the
// absorbed form of multi-head latent attention on the attention tutorial
// page (section "MLA: compress the cached representation"). The rule is
// MALA's, unchanged (MALA page, "Online Sparse Softmax" and "Fused forward
// execution"): every legal tile gets score discovery, the log-domain block
// test against the running (m, l), and only a retained tile gets the
// softmax update and the P V accumulation. Because V is part of the cached
// row, the K tile already in LDS serves as V_j; what a skipped tile saves is
// the exponentials and the P V contraction (2 d_v FLOPs per slot, the page's
// per-slot accounting).
//
// Work item: (batch, query head, 64-row query block I_i), tiles of 64 keys
// visited diagonal first, then descending. A workgroup has eight waves
// (two per SIMD) and the whole 160 KB LDS of a CU:
//  * two 64 x 576 K tiles (the next one is copied HBM -> LDS while the
//    current one is used), a 64 x 64 bf16 P tile and per-row exchange
//    slots;
//  * score discovery: wave w computes S^T for keys 32 (w % 2) .. +31 and
//    rows 16 (w / 2) .. +15 on 16x16x32 MFMAs, its sixteen query rows held
//    in registers as the B operand (A = K rows from LDS), so each lane owns
//    one query row: the half-tile row max is a per-lane value and the two
//    halves of a row meet through LDS;
//  * the test is evaluated per half (the block margin is the max of the
//    halves' margins, so the OR of the half votes is the block vote);
//  * a retained tile: the owners of each row rebuild its m, l, P (bf16 into
//    the P tile), and every wave accumulates O^T for its 64 value columns of
//    all 64 rows on 32x32x16 MFMAs (A = V^T by LDS transpose loads from the
//    K tile, B = P^T rows from the P tile).
// Three barriers per tile: copy landed, votes, P published.
#include <math.h>

#include "mala_latent_tiles.hpp"

namespace mala {
namespace {

using namespace latent;

constexpr int LNW = 8;
constexpr int LNT = 64 * LNW;

__device__ __forceinline__ void lk_copy(uint16_t* tile, const uint16_t* base, size_t rs, int k0, int n,
                                        int wave, int lane) {
  lk_copy_w<LNW>(tile, base, rs, k0, n, wave, lane);
}

struct LatentShared {
  float rmax[2][LBQ];  // half-tile row maxima (per key half)
  float rsum[2][LBQ];  // half-tile row sums of P
  float alpha[LBQ];    // rescale of the output rows
  float inv_l[LBQ];    // 1 / l at the end
  int vote[LNW];
};

__global__ void __launch_bounds__(LNT, 1) fwd_latent_kernel(FwdParams a, int n_chunks) {
  __shared__ __attribute__((aligned(16))) uint16_t sK0[LTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[LTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sP[LBQ * LBK];
  __shared__ LatentShared sh;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, x = lane & 15;  // 16x16 layout: lane group, row within the group
  const int hh = lane >> 5, l32 = lane & 31; // 32x32 layout
  const int rg = wave >> 1, kh = wave & 1;   // score role: row group (16 rows), key half (32 keys)

  // work item: chunks of H_q items (one (b, i), every head) dealt to the
  // XCDs round-robin, so the heads that read the same K tiles run together
  // on one XCD and share its L2; heaviest (last) query blocks first
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int chunk = (slot / a.heads_q) * 8 + xcd;
  if (chunk >= n_chunks) return;
  const int h = slot % a.heads_q;
  const int b = chunk % a.batch;
  const int i = a.nqb - 1 - chunk / a.batch;
  const int q0 = i * LBQ;
  const int off = a.offset;
  const int row_hi = min(q0 + LBQ, a.seqlen_q) - 1;  // last valid row of the block
  const int jmax = (row_hi + off) / LBK;

  const size_t q_rs = (size_t)a.heads_q * LQK;
  const size_t kv_rs = LQK;  // one KV head
  const uint16_t* const kvb = (const uint16_t*)a.k + (size_t)b * a.seqlen_k * kv_rs;

  // this lane's query row (score role) and its test threshold log tau - log L_q
  const int qrow = q0 + 16 * rg + x;
  const bool qvalid = qrow < a.seqlen_q;
  const float thr = a.log_tau - __logf((float)(qrow + off + 1));
  u32x4_t qf[LKC];
  {
    const int rows = min(max(a.seqlen_q - q0, 0), LBQ);
    const rsrc_t rq = make_rsrc((const uint16_t*)a.q + ((size_t)b * a.seqlen_q + q0) * q_rs + (size_t)h * LQK,
                                (uint32_t)rows * (uint32_t)q_rs * 2u);
#pragma unroll
    for (int kk = 0; kk < LKC; ++kk)
      qf[kk] = buf_ld16(rq, (uint32_t)((16 * rg + x) * q_rs + 32 * kk + 8 * g16) * 2u);
  }

  f32x16_t acc[2][2];  // O^T for value columns 64 wave + 32 db, rows 32 rb
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[db][rb] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  int n_retained = 0;

  // one tile: K_j in `cur`; the copy of K_{j-1} goes to `nxt`
  auto step = [&](int j, const uint16_t* cur, uint16_t* nxt) {
    const int k0 = j * LBK;
    wait_vmcnt<0>();
    __syncthreads();  // K_j landed; every wave is done with tile j + 1 (P, exchange slots, nxt)
    if (j > 0) lk_copy(nxt, kvb, kv_rs, k0 - LBK, a.seqlen_k, wave, lane);

    // ---- score discovery: s[kb][r] = S[row qrow][key k0 + 32 kh + 16 kb + 4 g16 + r]
    f32x4_t s[2];
    mfma_run_begin();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4_t{};
      const int krow = 32 * kh + 16 * kb + x;
#pragma unroll
      for (int kk = 0; kk < LKC; ++kk)
        s[kb] = mfma16(lds_ld16(&cur[lk_idx(krow, 32 * kk + 8 * g16)]), qf[kk], s[kb]);
    }
    mfma_run_end();
    // causal mask and rows past N_q
    if (k0 + LBK - 1 > q0 + off || q0 + LBQ > a.seqlen_q) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 32 * kh + 16 * kb + 4 * g16 + r;
          if (!(qvalid && key <= qrow + off)) s[kb][r] = -INFINITY;
        }
    }
    float mh = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mh = wave_max_halves(row_pair_max(mh));  // this half's row max (all four groups agree)
    // half vote: the block margin is the max over the halves' margins
    float margin = -INFINITY;
    if (mh > -INFINITY) margin = (l_run > 0.f) ? (mh - m_run - test_log(l_run) - thr) : INFINITY;
    const bool wave_vote = __ballot(margin >= 0.f) != 0ull;
    if (g16 == 0) sh.rmax[kh][16 * rg + x] = mh;
    if (lane == 0) sh.vote[wave] = wave_vote ? 1 : 0;
    lds_barrier();  // the copy of K_{j-1} stays in flight
    bool retain = false;
#pragma unroll
    for (int w = 0; w < LNW; ++w) retain |= sh.vote[w] != 0;
    if (tid == 0 && a.tile_mask)
      a.tile_mask[(((size_t)b * a.heads_q + h) * a.nqb + i) * a.nkb + j] = retain ? 1 : 0;
    if (!retain) return;
    ++n_retained;

    // ---- owners of each row: m, l, P --------------------------------------
    const float mx = fmaxf(mh, sh.rmax[kh ^ 1][16 * rg + x]);
    const bool relevant = mx > -INFINITY;
    const float m_new = relevant ? fmaxf(m_run, mx) : m_run;
    const float alpha = relevant ? __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e) : 1.f;
    const float msc = m_new * kLog2e;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = relevant ? __builtin_amdgcn_exp2f(fmaf(s[kb][r], kLog2e, -msc)) : 0.f;
        rs += p[r];
      }
      const u32x2_t pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      *reinterpret_cast<u32x2_t*>(&sP[lp_idx(16 * rg + x, 32 * kh + 16 * kb + 4 * g16)]) = pk;
    }
    rs = wave_sum_halves(row_pair_sum(rs));
    if (g16 == 0) {
      sh.rsum[kh][16 * rg + x] = rs;
      if (kh == 0) sh.alpha[16 * rg + x] = alpha;
    }
    lds_barrier();  // P, row sums and rescales published
    l_run = l_run * alpha + (sh.rsum[0][16 * rg + x] + sh.rsum[1][16 * rg + x]);
    m_run = m_new;

    // ---- every wave: O^T[64 wave .. +63][0 .. 63] = alpha O^T + V^T P^T ---
    const float al0 = sh.alpha[l32], al1 = sh.alpha[32 + l32];
    if (__ballot(al0 != 1.f || al1 != 1.f) != 0ull) {
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        acc[db][0] *= al0;
        acc[db][1] *= al1;
      }
    }
    mfma_run_begin();
#pragma unroll
    for (int ks = 0; ks < LBK / 16; ++ks) {
      u32x4_t pb[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) pb[rb] = lds_ld16(&sP[lp_idx(32 * rb + l32, 16 * ks + 8 * hh)]);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        // lane l receives V[key 16 ks + 8 hh + t][d 64 wave + 32 db + l % 32], t = 0..7
        const int grp = lane >> 4, y = lane & 15;
        const int krow = 16 * ks + 8 * (grp >> 1) + (y >> 2);
        const int col = 64 * wave + 32 * db + 16 * (grp & 1) + 4 * (y & 3);
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)&cur[lk_idx(krow, col)]);
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)&cur[lk_idx(krow + 4, col)]);
        const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo), hw = __builtin_bit_cast(u32x2_t, hi);
        const u32x4_t va = {lw[0], lw[1], hw[0], hw[1]};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) acc[db][rb] = mfma32(va, pb[rb], acc[db][rb]);
      }
    }
    mfma_run_end();
  };

  if (jmax >= 0) lk_copy(sK0, kvb, kv_rs, jmax * LBK, a.seqlen_k, wave, lane);
  // tiles alternate between the two K buffers: jmax in sK0, jmax - 1 in sK1, ...
  for (int j = jmax; j >= 0; j -= 2) {
    step(j, sK0, sK1);
    if (j - 1 >= 0) step(j - 1, sK1, sK0);
  }

  // ---- finalize: O = acc / l, z = m + log l -----------------------------------
  __syncthreads();
  if (kh == 0 && g16 == 0) sh.inv_l[16 * rg + x] = l_run > 0.f ? 1.f / l_run : 0.f;
  if (kh == 0 && g16 == 0 && qvalid)
    a.z[((size_t)b * a.heads_q + h) * a.seqlen_q + qrow] = m_run + __logf(l_run);
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = q0 + 32 * rb + l32;
    if (row >= a.seqlen_q) continue;
    const float inv = sh.inv_l[32 * rb + l32];
    uint16_t* orow = (uint16_t*)a.o + ((size_t)b * a.seqlen_q + row) * a.heads_q * LV + (size_t)h * LV;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = 64 * wave + 32 * db + 8 * rq + 4 * hh;
        const u32x2_t w = {pack_bf16x2(acc[db][rb][4 * rq] * inv, acc[db][rb][4 * rq + 1] * inv),
                           pack_bf16x2(acc[db][rb][4 * rq + 2] * inv, acc[db][rb][4 * rq + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(orow + d) = w;
      }
  }
  if (tid == 0 && a.stats) {
    const int rows = row_hi - q0 + 1;
    atomicAdd(&a.stats[0], (unsigned long long)(jmax + 1));
    atomicAdd(&a.stats[1], (unsigned long long)n_retained);
    atomicAdd(&a.stats[2], (unsigned long long)n_retained * LBK * rows);
    atomicAdd(&a.stats[3], (unsigned long long)n_retained);
  }
}


// ---------------------------------------------------------------------------
// Latent decode with split-KV (MALA page, split-KV paragraph and "Fused
// decoding execution"; the cached row and absorbed value as above).
//
// Work item: (batch, split, group of 16 query heads). The 16 heads are the
// 16-wide dimension of the MFMAs, so one workgroup scores a 64-key tile for
// all of them at once and reads each cached row once per head group. The
// split's tiles are visited from the most recent one down; each split
// starts from fresh state (m = -inf, l = 0) and tests every head against
// that partial normalizer with L_0 = N_k. A head that does not retain a
// tile keeps its state and contributes P = 0 to the shared P V contraction,
// which leaves its accumulator bit-for-bit unchanged; a tile no head
// retains skips the contraction. Four waves (one per SIMD) and two K tiles
// in LDS: the next tile is copied HBM -> LDS while the current one is used.
//  * scores: wave w computes S^T for keys 16 w .. 16 w + 15 of the tile and
//    the 16 heads (A = K rows from LDS, B = the heads' query rows held in
//    registers); each lane owns head (lane % 16), and every lane keeps that
//    head's (m, l), so all waves take the same decisions;
//  * values: wave w accumulates O^T for value columns 128 w .. 128 w + 127
//    (A = V^T by LDS transpose loads from the K tile, B = P^T rows).
// The workload is bound by reading the cache (1152 bytes per key);
// arithmetic is about 2 (d_qk + d_v) FLOPs per key and head.
// ---------------------------------------------------------------------------
constexpr int DHG = 16;  // query heads per workgroup
constexpr int DNW = 4;
constexpr int DNT = 64 * DNW;
constexpr int DVW = LV / DNW;  // value columns per wave (128)

// P tile: 16 heads x 64 keys bf16, 16-byte units XORed with head % 8.
__device__ __forceinline__ int dp_idx(int head, int key) {
  return head * LBK + ((((key >> 3) ^ (head & 7))) << 3) + (key & 7);
}

struct DecodeLatentShared {
  float rmax[DNW][DHG];  // per-wave tile maxima of each head
  float rsum[DNW][DHG];  // per-wave row sums of P
  float inv_l[DHG];
};

__global__ void __launch_bounds__(DNT, 1) decode_latent_kernel(DecodeParams a, int n_hg, int n_items) {
  __shared__ __attribute__((aligned(16))) uint16_t sK0[LTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[LTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sP[DHG * LBK];
  __shared__ DecodeLatentShared sh;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, x = lane & 15;  // 16x16 layout: lane group, head (score) / column (value)

  // head groups of one (batch, split) are consecutive on one XCD, so the
  // workgroups that read the same K tiles share that XCD's L2
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int item = (slot / n_hg) * 8 + xcd;
  if (item >= n_items) return;
  const int hg = slot % n_hg;
  const int s = item % a.num_splits;
  const int b = item / a.num_splits;
  const int h = hg * DHG + x;  // this lane's head
  const int n_k = a.seqlen_k;
  const int lo = (int)(((long long)s * a.num_tiles) / a.num_splits);
  const int hi = (int)(((long long)(s + 1) * a.num_tiles) / a.num_splits);
  const float thr = a.log_tau - __logf((float)n_k);  // log tau - log L_0, L_0 = N_k

  const uint16_t* const kvb = (const uint16_t*)a.k + (size_t)b * n_k * LQK;
  u32x4_t qf[LKC];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)b * a.heads_q + h) * LQK + 8 * g16;
#pragma unroll
    for (int kk = 0; kk < LKC; ++kk) qf[kk] = ld16(qrow + 32 * kk);
  }
  f32x4_t acc[DVW / 16];  // O^T[128 wave + 16 db + 4 g16 + r][head x]
#pragma unroll
  for (int db = 0; db < DVW / 16; ++db) acc[db] = f32x4_t{};
  float m_run = -INFINITY, l_run = 0.f;
  unsigned long long n_ret = 0, n_vtile = 0;

  auto step = [&](int j, const uint16_t* cur, uint16_t* nxt) {
    const int k0 = j * LBK;
    wait_vmcnt<0>();
    __syncthreads();  // K_j landed; every wave is done with tile j + 1 (P, exchange slots, nxt)
    if (j > lo) lk_copy_w<DNW>(nxt, kvb, LQK, k0 - LBK, n_k, wave, lane);

    // ---- scores: sv[r] = S[head x][key k0 + 16 wave + 4 g16 + r] ------------
    f32x4_t sv = f32x4_t{};
    mfma_run_begin();
#pragma unroll
    for (int kb = 0; kb < LKC; kb += 6) {
      u32x4_t kf[6];
#pragma unroll
      for (int t = 0; t < 6; ++t) kf[t] = lds_ld16(&cur[lk_idx(16 * wave + x, 32 * (kb + t) + 8 * g16)]);
#pragma unroll
      for (int t = 0; t < 6; ++t) sv = mfma16(kf[t], qf[kb + t], sv);
    }
    mfma_run_end();
    if (k0 + LBK > n_k) {  // the last tile: keys past N_k
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (k0 + 16 * wave + 4 * g16 + r >= n_k) sv[r] = -INFINITY;
    }
    float mw = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mw = wave_max_halves(row_pair_max(mw));
    if (g16 == 0) sh.rmax[wave][x] = mw;
    lds_barrier();  // the copy of K_{j-1} stays in flight
    const float mx = fmaxf(fmaxf(sh.rmax[0][x], sh.rmax[1][x]), fmaxf(sh.rmax[2][x], sh.rmax[3][x]));
    // per-head test against this split's partial normalizer (l = 0: +inf)
    const float margin = (l_run > 0.f) ? (mx - m_run - test_log(l_run) - thr) : INFINITY;
    const bool ret = mx > -INFINITY && margin >= 0.f;
    const unsigned retmask = (unsigned)(__ballot(ret) & 0xffffull);  // bit x: head x (same in every wave)
    if (wave == 0 && g16 == 0 && a.tile_mask)
      a.tile_mask[((size_t)b * a.heads_q + h) * a.num_tiles + j] = ret ? 1 : 0;
    if (retmask == 0) return;
    n_ret += __builtin_popcount(retmask);
    ++n_vtile;

    // ---- retained heads: m, l, P; the others contribute P = 0 ---------------
    const float m_new = ret ? fmaxf(m_run, mx) : m_run;
    const float alpha = ret ? __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e) : 1.f;
    const float msc = ret ? m_new * kLog2e : INFINITY;
    float p[4], rs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(sv[r], kLog2e, -msc));
      rs += p[r];
    }
    const u32x2_t pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    *reinterpret_cast<u32x2_t*>(&sP[dp_idx(x, 16 * wave + 4 * g16)]) = pk;
    rs = wave_sum_halves(row_pair_sum(rs));
    if (g16 == 0) sh.rsum[wave][x] = rs;
    lds_barrier();  // P and row sums published
    l_run = l_run * alpha + ((sh.rsum[0][x] + sh.rsum[1][x]) + (sh.rsum[2][x] + sh.rsum[3][x]));
    m_run = m_new;

    // ---- O^T[128 wave .. +127][heads] = alpha O^T + V^T P^T -----------------
    if (__ballot(alpha != 1.f) != 0ull) {
#pragma unroll
      for (int db = 0; db < DVW / 16; ++db) acc[db] *= alpha;
    }
    mfma_run_begin();
#pragma unroll
    for (int ks = 0; ks < LBK / 32; ++ks) {
      const u32x4_t pb = lds_ld16(&sP[dp_idx(x, 32 * ks + 8 * g16)]);
#pragma unroll
      for (int dh = 0; dh < DVW / 16; dh += 4) {
        // lane l receives V[key 32 ks + 8 g16 + t][d 128 wave + 16 db + l % 16], t = 0..7
        u32x4_t va[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int krow = 32 * ks + 8 * g16 + (x >> 2);
          const int col = DVW * wave + 16 * (dh + t) + 4 * (x & 3);
          const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)&cur[lk_idx(krow, col)]);
          const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)&cur[lk_idx(krow + 4, col)]);
          const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo4), hw = __builtin_bit_cast(u32x2_t, hi4);
          va[t] = u32x4_t{lw[0], lw[1], hw[0], hw[1]};
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[dh + t] = mfma16(va[t], pb, acc[dh + t]);
      }
    }
    mfma_run_end();
  };

  lk_copy_w<DNW>(sK0, kvb, LQK, (hi - 1) * LBK, n_k, wave, lane);
  // tiles alternate between the two K buffers: hi - 1 in sK0, hi - 2 in sK1, ...
  for (int j = hi - 1; j >= lo; j -= 2) {
    step(j, sK0, sK1);
    if (j - 1 >= lo) step(j - 1, sK1, sK0);
  }

  // ---- the split's partial: o_s = O / l (fp32), z_s = m + log l -------------
  const size_t pi = ((size_t)b * a.heads_q + h) * a.num_splits + s;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int db = 0; db < DVW / 16; ++db)
    *reinterpret_cast<f32x4_t*>(a.part_o + pi * LV + DVW * wave + 16 * db + 4 * g16) = acc[db] * inv;
  if (wave == 0 && g16 == 0) a.part_z[pi] = l_run > 0.f ? m_run + __logf(l_run) : -INFINITY;
  if (tid == 0 && a.stats) {
    atomicAdd(&a.stats[0], (unsigned long long)(hi - lo) * DHG);
    atomicAdd(&a.stats[1], n_ret);
    atomicAdd(&a.stats[2], n_ret * LBK);
    atomicAdd(&a.stats[3], n_vtile);
  }
}


// ---------------------------------------------------------------------------
// Latent decode for many heads (H_q a multiple of 64): the same rule, one
// workgroup per (batch, split, group of 64 query heads), each wave owning 16
// heads over all 64 keys of the tile. A head's tile maximum, test, softmax
// state and P stay inside its wave, so the only workgroup barrier per tile
// is the one that hands over the K tile, and each cached row is copied into
// LDS once per 64 heads.
//  * scores: four 16-key chains of 16x16x32 MFMAs per wave (A = K rows from
//    LDS, read one chunk ahead; B = the wave's 16 query rows in registers);
//  * values: O^T for all 512 value columns of the wave's heads (32
//    accumulators of 16 columns, A = V^T by LDS transpose loads from the K
//    tile, read one block ahead; B = P^T rows from the wave's own P tile).
// ---------------------------------------------------------------------------
constexpr int WHG = 64;  // query heads per workgroup of the wide kernel

__global__ void __launch_bounds__(DNT, 1) decode_latent_wide_kernel(DecodeParams a, int n_hg, int n_items) {
  __shared__ __attribute__((aligned(16))) uint16_t sK0[LTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[LTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sPw[DNW][DHG * LBK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, x = lane & 15;

  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int item = (slot / n_hg) * 8 + xcd;
  if (item >= n_items) return;
  const int hg = slot % n_hg;
  const int s = item % a.num_splits;
  const int b = item / a.num_splits;
  const int h = hg * WHG + DHG * wave + x;  // this lane's head
  const int n_k = a.seqlen_k;
  const int lo = (int)(((long long)s * a.num_tiles) / a.num_splits);
  const int hi = (int)(((long long)(s + 1) * a.num_tiles) / a.num_splits);
  const float thr = a.log_tau - __logf((float)n_k);  // log tau - log L_0, L_0 = N_k
  uint16_t* const sP = sPw[wave];

  const uint16_t* const kvb = (const uint16_t*)a.k + (size_t)b * n_k * LQK;
  u32x4_t qf[LKC];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)b * a.heads_q + h) * LQK + 8 * g16;
#pragma unroll
    for (int kk = 0; kk < LKC; ++kk) qf[kk] = ld16(qrow + 32 * kk);
  }
  f32x4_t acc[LV / 16];  // O^T[16 db + 4 g16 + r][head x]
#pragma unroll
  for (int db = 0; db < LV / 16; ++db) acc[db] = f32x4_t{};
  float m_run = -INFINITY, l_run = 0.f;
  unsigned long long n_ret = 0, n_vtile = 0;

  auto step = [&](int j, const uint16_t* cur, uint16_t* nxt) {
    const int k0 = j * LBK;
    wait_vmcnt<0>();
    __syncthreads();  // K_j landed; every wave is done with tile j + 1 (nxt)
    if (j > lo) lk_copy_w<DNW>(nxt, kvb, LQK, k0 - LBK, n_k, wave, lane);

    // ---- scores: sv[kb][r] = S[head x][key k0 + 16 kb + 4 g16 + r] ----------
    f32x4_t sv[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sv[kb] = f32x4_t{};
    mfma_run_begin();
    {
      u32x4_t a0[4], a1[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) a0[kb] = lds_ld16(&cur[lk_idx(16 * kb + x, 8 * g16)]);
#pragma unroll
      for (int kk = 0; kk < LKC; ++kk) {
        u32x4_t* ca = (kk & 1) ? a1 : a0;
        u32x4_t* na = (kk & 1) ? a0 : a1;
        if (kk + 1 < LKC) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) na[kb] = lds_ld16(&cur[lk_idx(16 * kb + x, 32 * (kk + 1) + 8 * g16)]);
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sv[kb] = mfma16(ca[kb], qf[kk], sv[kb]);
      }
    }
    mfma_run_end();
    if (k0 + LBK > n_k) {  // the last tile: keys past N_k
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (k0 + 16 * kb + 4 * g16 + r >= n_k) sv[kb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mx = fmaxf(mx, fmaxf(fmaxf(sv[kb][0], sv[kb][1]), fmaxf(sv[kb][2], sv[kb][3])));
    mx = wave_max_halves(row_pair_max(mx));  // head x's tile maximum (every lane group agrees)
    // per-head test against this split's partial normalizer (l = 0: +inf)
    const float margin = (l_run > 0.f) ? (mx - m_run - test_log(l_run) - thr) : INFINITY;
    const bool ret = mx > -INFINITY && margin >= 0.f;
    const unsigned retmask = (unsigned)(__ballot(ret) & 0xffffull);
    if (g16 == 0 && a.tile_mask) a.tile_mask[((size_t)b * a.heads_q + h) * a.num_tiles + j] = ret ? 1 : 0;
    if (retmask == 0) return;  // this wave's heads all skip the tile
    n_ret += __builtin_popcount(retmask);
    ++n_vtile;

    // ---- retained heads: m, l, P (wave-local); the others contribute P = 0 ---
    const float m_new = ret ? fmaxf(m_run, mx) : m_run;
    const float alpha = ret ? __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e) : 1.f;
    const float msc = ret ? m_new * kLog2e : INFINITY;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f(fmaf(sv[kb][r], kLog2e, -msc));
        rs += p[r];
      }
      *reinterpret_cast<u32x2_t*>(&sP[dp_idx(x, 16 * kb + 4 * g16)]) =
          u32x2_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    }
    rs = wave_sum_halves(row_pair_sum(rs));
    l_run = l_run * alpha + rs;
    m_run = m_new;
    __builtin_amdgcn_wave_barrier();  // P written by each lane is read by others below: keep LDS order
    if (__ballot(alpha != 1.f) != 0ull) {
#pragma unroll
      for (int db = 0; db < LV / 16; ++db) acc[db] *= alpha;
    }

    // ---- O^T[512 columns][heads] += V^T P^T ---------------------------------
    mfma_run_begin();
#pragma unroll
    for (int ks = 0; ks < LBK / 32; ++ks) {
      const u32x4_t pb = lds_ld16(&sP[dp_idx(x, 32 * ks + 8 * g16)]);
      u32x4_t va[2];
      va[0] = lds_tr8(cur, 32 * ks, 0, lane, LkIdx{});
#pragma unroll
      for (int db = 0; db < LV / 16; ++db) {
        if (db + 1 < LV / 16) va[(db + 1) & 1] = lds_tr8(cur, 32 * ks, 16 * (db + 1), lane, LkIdx{});
        acc[db] = mfma16(va[db & 1], pb, acc[db]);
      }
    }
    mfma_run_end();
  };

  lk_copy_w<DNW>(sK0, kvb, LQK, (hi - 1) * LBK, n_k, wave, lane);
  for (int j = hi - 1; j >= lo; j -= 2) {
    step(j, sK0, sK1);
    if (j - 1 >= lo) step(j - 1, sK1, sK0);
  }

  // ---- the split's partial: o_s = O / l (fp32), z_s = m + log l -------------
  const size_t pi = ((size_t)b * a.heads_q + h) * a.num_splits + s;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int db = 0; db < LV / 16; ++db)
    *reinterpret_cast<f32x4_t*>(a.part_o + pi * LV + 16 * db + 4 * g16) = acc[db] * inv;
  if (g16 == 0) a.part_z[pi] = l_run > 0.f ? m_run + __logf(l_run) : -INFINITY;
  if (lane == 0 && a.stats) {
    atomicAdd(&a.stats[0], (unsigned long long)(hi - lo) * DHG);
    atomicAdd(&a.stats[1], n_ret);
    atomicAdd(&a.stats[2], n_ret * LBK);
    atomicAdd(&a.stats[3], n_vtile);
  }
}

}  // namespace

hipError_t launch_fwd_latent(const mala_problem& p, const FwdParams& a, int d_v, hipStream_t s,
                             bool* supported) {
  *supported = p.dtype == MALA_BF16 && p.head_dim == LQK && d_v == LV && p.heads_kv == 1 &&
               p.block_q == LBQ && p.block_k == LBK;
  if (!*supported) return hipSuccess;
  const int n_chunks = a.batch * a.nqb;
  const int grid = (n_chunks + 7) / 8 * 8 * a.heads_q;
  hipLaunchKernelGGL(fwd_latent_kernel, dim3((unsigned)grid), dim3(LNT), 0, s, a, n_chunks);
  return hipGetLastError();
}

hipError_t launch_decode_latent(const mala_problem& p, const DecodeParams& a, int d_v, hipStream_t s,
                                bool* supported) {
  *supported = p.dtype == MALA_BF16 && p.head_dim == LQK && d_v == LV && p.heads_kv == 1 &&
               p.block_k == LBK && p.heads_q % DHG == 0;
  if (!*supported) return hipSuccess;
  const int n_items = a.batch * a.num_splits;
  if (a.heads_q % WHG == 0) {
    const int n_hg = a.heads_q / WHG;
    const int grid = (n_items + 7) / 8 * 8 * n_hg;
    hipLaunchKernelGGL(decode_latent_wide_kernel, dim3((unsigned)grid), dim3(DNT), 0, s, a, n_hg, n_items);
  } else {
    const int n_hg = a.heads_q / DHG;
    const int grid = (n_items + 7) / 8 * 8 * n_hg;
    hipLaunchKernelGGL(decode_latent_kernel, dim3((unsigned)grid), dim3(DNT), 0, s, a, n_hg, n_items);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(a, LV, s);
}

}  // namespace mala
