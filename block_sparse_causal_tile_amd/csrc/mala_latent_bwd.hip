// MALA backward on latent (MLA-shaped) attention for gfx950.
//
// The cached row kv_s (d_qk = 576) is both the key and, through its first
// d_v = 512 columns, the value (absorbed form of multi-head latent attention,
// attention tutorial page, section "MLA: compress the cached
// representation"). The rule is MALA's backward, unchanged (MALA page,
// "Offline Sparse Probability" and "Fused backward execution"): every legal
// tile (query block i, key block j, head h) recomputes S = Q_i K_j^T and is
// retained iff some legal entry has S_qk - z_q >= log tau - log L_q; a
// retained tile rebuilds P = exp(S - z), dP = dO_i V_j^T, dS = P (dP - D)
// and contributes dQ_i += dS K_j, dK_j += dS^T Q_i, dV_j += P^T dO_i. The
// row's gradient is the sum of its two uses: dKV_j = dK_j + [dV_j, 0], summed
// over every query head (one cached row per position).
//
// Three deterministic launches (no atomics on gradients):
//  * bwd_latent_prep_kernel: D_q = sum_d dO_qd O_qd (fp32).
//  * bwd_latent_dkv_kernel (key-major): a workgroup owns key block j of one
//    batch row and a group of query heads; K_j stays in registers (each
//    wave holds 16 keys x 576 as MFMA operands, the first 512 columns being
//    V_j), and for every (head, query block from the diagonal up) the Q_i
//    tile is copied into LDS, S^T = K_j Q_i^T is scored and tested, and only
//    a retained tile copies dO_i and forms dP^T, P^T and dS^T. dKV_j
//    accumulates dS^T Q_i + P^T dO_i in registers (64 keys x 576, 72
//    accumulators per lane over eight waves). Each head group writes an fp32
//    partial; bwd_latent_reduce_kernel sums them in a fixed order into bf16.
//  * bwd_latent_dq_kernel (query-major): a workgroup owns query block i of
//    one head, with Q_i and dO_i held in registers, K tiles streamed through
//    LDS (double buffered, as in the forward); it repeats the test with the
//    same arithmetic and forms dQ_i^T += K_j^T dS^T.
// Both roles score S^T on the same 16x16x32 MFMA with A = K rows and B = Q
// rows over the same 18 chunks of 32 columns in the same order, and test
// S - (z + log tau - log L_q) >= 0 entry by entry with the same float
// offset, so their decisions agree bit for bit.
#include <math.h>

#include <type_traits>

#include "mala_latent_tiles.hpp"

namespace mala {
namespace {

using namespace latent;

constexpr int DTILE = LBQ * LV; // bf16 elements per dO tile

// dO tile: 64 rows x 512 bf16, 1024-byte rows; within each aligned group of
// sixteen 16-byte units the unit index is XORed with a permutation of the
// row's low four bits (b3 b1 b0 b2). Sixteen rows read at one column land on
// sixteen different units (dP operands), and the transposing reads of four
// consecutive rows x 16 columns land on four different unit pairs.
__device__ __forceinline__ int ldo_swz(int row) {
  return ((row & 3) << 1) | ((row >> 2) & 1) | (row & 8);
}
__device__ __forceinline__ int ldo_idx(int row, int col) {
  const int u = col >> 3;
  return row * LV + (((u & ~15) | ((u & 15) ^ ldo_swz(row & 15))) << 3) + (col & 7);
}

// Copy dO rows r0 .. r0 + 63 (clamped to n - 1) into a dO tile with NW waves;
// instruction n fills tile row n (64 units).
template <int NW>
__device__ __forceinline__ void ldo_copy_w(uint16_t* tile, const uint16_t* base, size_t rs, int r0, int n,
                                           int wave, int lane) {
  static_assert(LBQ % NW == 0, "copy instructions split evenly over the waves");
#pragma unroll
  for (int c = 0; c < LBQ / NW; ++c) {
    const int row = wave + c * NW;
    const int lu = (lane & ~15) | ((lane & 15) ^ ldo_swz(row & 15));
    const int grow = min(r0 + row, n - 1);
    lds_dma16_ordered(base + (size_t)grow * rs + lu * 8, tile + row * LV);
  }
}

struct LdoIdx {
  __device__ int operator()(int r, int c) const { return ldo_idx(r, c); }
};

// z + log tau - log L_q of a valid row: S_qk - this >= 0 retains.
__device__ __forceinline__ float latent_test_offset(const BwdParams& a, float z, int q) {
  return z + (a.log_tau - __logf((float)(q + a.offset + 1)));
}

// ---------------------------------------------------------------------------
// D_q = sum_d dO_qd O_qd: one wave per (batch, row, head), 8 columns per lane
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_latent_prep_kernel(BwdParams a) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long rows = (long long)a.batch * a.seqlen_q * a.heads_q;
  if (r >= rows) return;
  const u32x4_t x = ld16((const uint16_t*)a.dout + r * LV + 8 * lane);
  const u32x4_t y = ld16((const uint16_t*)a.o + r * LV + 8 * lane);
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) acc += bf16_lo(x[t]) * bf16_lo(y[t]) + bf16_hi(x[t]) * bf16_hi(y[t]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (lane == 0) {
    const int h = (int)(r % a.heads_q);
    const long long bq = r / a.heads_q;
    const int q = (int)(bq % a.seqlen_q);
    const int b = (int)(bq / a.seqlen_q);
    a.delta[((size_t)b * a.heads_q + h) * a.seqlen_q + q] = acc;
  }
}

// ---------------------------------------------------------------------------
// key-major role: partial dKV_j of one head group
// ---------------------------------------------------------------------------
constexpr int KNW = 8;
constexpr int KNT = 64 * KNW;

struct DkvShared {
  int vote[KNW];
};

__global__ void __launch_bounds__(KNT, 1) bwd_latent_dkv_kernel(BwdParams a, int hpi, int n_hg, float* part) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[LTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[DTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sP[LBQ * LBK];
  __shared__ __attribute__((aligned(16))) uint16_t sdS[LBQ * LBK];
  __shared__ __attribute__((aligned(16))) float sZ[2][LBQ];  // z of the rows, by pair parity
  __shared__ __attribute__((aligned(16))) float sD[2][LBQ];  // D of the rows, by pair parity
  __shared__ DkvShared sh;

  const int tid = threadIdx.x, lane0 = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3;   // scores: keys 16 kg .. 16 kg + 15
  const int rh = wave >> 2;  // scores: query rows 32 rh .. 32 rh + 31
  const int kh = wave & 1;   // accumulators: keys 32 kh .. 32 kh + 31
  const int cq = wave >> 1;  // accumulators: columns 144 cq .. 144 cq + 143

  // work item: heaviest key blocks (most query blocks above them) first
  const int per_j = a.batch * n_hg;
  const int j = blockIdx.x / per_j;
  const int b = (blockIdx.x % per_j) / n_hg;
  const int hg = blockIdx.x % n_hg;
  const int k0 = j * LBK;
  // query blocks with a legal entry for this key block: from the diagonal
  // block up, less a ragged last block that ends before the key block starts
  int i0 = max(0, k0 - a.offset) / LBQ;
  if (i0 < a.nqb && k0 > min(i0 * LBQ + LBQ, a.seqlen_q) - 1 + a.offset) ++i0;
  const int per_head = a.nqb - i0;
  const int n_pairs = per_head > 0 ? hpi * per_head : 0;

  // K_j (and V_j, its first 512 columns) as the A operand: lane holds key
  // 16 kg + x, columns 32 kk + 8 g16 .. + 7
  u32x4_t kf[LKC];
  {
    const int g16 = lane0 >> 4, x = lane0 & 15;
    const int key = min(k0 + 16 * kg + x, a.seqlen_k - 1);
    const uint16_t* kr = (const uint16_t*)a.k + ((size_t)b * a.seqlen_k + key) * LQK + 8 * g16;
#pragma unroll
    for (int kk = 0; kk < LKC; ++kk) kf[kk] = ld16(kr + 32 * kk);
  }
  f32x4_t acc[2][9];  // dKV[key 32 kh + 16 kq + 4 g16 + r][column 144 cq + 16 db + x]
#pragma unroll
  for (int kq = 0; kq < 2; ++kq)
#pragma unroll
    for (int db = 0; db < 9; ++db) acc[kq][db] = f32x4_t{};
  unsigned long long n_legal = 0, n_ret = 0, n_slots = 0;

  const size_t q_rs = (size_t)a.heads_q * LQK, do_rs = (size_t)a.heads_q * LV;
  const uint16_t* const qb = (const uint16_t*)a.q + (size_t)b * a.seqlen_q * q_rs;
  const uint16_t* const ob = (const uint16_t*)a.dout + (size_t)b * a.seqlen_q * do_rs;
  // Software pipeline over the (head, query block) pairs: the copy of Q_i
  // for the next pair is issued as soon as every wave is done reading the
  // current Q tile (after the test of a skipped tile, after dS^T Q_i of a
  // retained one), and the copy of dO_i is issued as soon as Q_i has landed,
  // so it overlaps score discovery; a skipped tile leaves that copy unused.
  auto pair_head = [&](int p) { return hg * hpi + p / per_head; };
  auto pair_block = [&](int p) { return i0 + p % per_head; };
  // z and D of a pair's 64 rows, copied HBM -> LDS one pair ahead by the
  // first two waves (the wait for the next Q tile covers them)
  auto load_rows = [&](int p, int ln) {
    if (wave < 2) {
      const int q = min(pair_block(p) * LBQ + ln, a.seqlen_q - 1);
      const size_t zo = ((size_t)b * a.heads_q + pair_head(p)) * a.seqlen_q + q;
      const float* src = wave == 0 ? a.z : a.delta;
      float* dst = wave == 0 ? sZ[p & 1] : sD[p & 1];
      lds_dma4_ordered(src + zo, dst);
    }
  };
  if (n_pairs > 0) {
    load_rows(0, lane0);
    lk_copy_w<KNW, false, true>(sQ, qb + (size_t)pair_head(0) * LQK, q_rs, pair_block(0) * LBQ, a.seqlen_q, wave, lane0);
  }
  for (int p = 0; p < n_pairs; ++p) {
    const int h = pair_head(p);
    const int i = pair_block(p);
    const int q0 = i * LBQ;
    // the lane index is re-derived per pair, so the copy and LDS addresses
    // are recomputed (a few VALU ops) instead of held across the loop, where
    // they would push the K operands and the accumulators out of registers
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    const int g16 = lane >> 4, x = lane & 15;
    wait_vmcnt<0>();
    __syncthreads();  // Q_i and the row state landed; the previous pair's readers of sdO, sP, sdS, votes are done
    const float* const rz = sZ[p & 1];
    const float* const rd = sD[p & 1];
    if (p + 1 < n_pairs) load_rows(p + 1, lane);
    ldo_copy_w<KNW>(sdO, ob + (size_t)h * LV, do_rs, q0, a.seqlen_q, wave, lane);

    // ---- S^T[key 16 kg + 4 g16 + r][row 32 rh + 16 rb + x] -------------------
    f32x4_t s[2] = {f32x4_t{}, f32x4_t{}};
    mfma_run_begin();
#pragma unroll
    for (int kk = 0; kk < LKC; ++kk)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        s[rb] = mfma16(kf[kk], lds_ld16(&sQ[lk_idx<false>(32 * rh + 16 * rb + x, 32 * kk + 8 * g16)]), s[rb]);
    mfma_run_end();
    const bool masked = k0 + LBK - 1 > q0 + a.offset || q0 + LBQ > a.seqlen_q || k0 + LBK > a.seqlen_k;
    if (masked) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = q0 + 32 * rh + 16 * rb + x, key = k0 + 16 * kg + 4 * g16 + r;
          if (!(key <= q + a.offset && q < a.seqlen_q && key < a.seqlen_k)) s[rb][r] = -INFINITY;
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = 32 * rh + 16 * rb + x, q = q0 + row;
      const float zt = q < a.seqlen_q ? latent_test_offset(a, rz[row], q) : INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmaxf(m, s[rb][r] - zt);
    }
    const bool wave_vote = __ballot(m >= 0.f) != 0ull;
    if (lane == 0) sh.vote[wave] = wave_vote ? 1 : 0;
    lds_barrier();  // votes published; every wave is done reading sQ for the scores
    bool retain = false;
#pragma unroll
    for (int w = 0; w < KNW; ++w) retain |= sh.vote[w] != 0;
    ++n_legal;
    if (tid == 0 && a.tile_mask)
      a.tile_mask[(((size_t)b * a.heads_q + h) * a.nqb + i) * a.nkb + j] = retain ? 1 : 0;
    if (!retain) {
      if (p + 1 < n_pairs)
        lk_copy_w<KNW, false, true>(sQ, qb + (size_t)pair_head(p + 1) * LQK, q_rs, pair_block(p + 1) * LBQ, a.seqlen_q, wave,
                       lane);
      continue;
    }
    ++n_ret;
    n_slots += (unsigned long long)LBK * min(LBQ, a.seqlen_q - q0);

    // ---- retained: dP^T, P^T, dS^T ------------------------------------------------
    float pv[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = 32 * rh + 16 * rb + x;
      const float nzl = q0 + row < a.seqlen_q ? -rz[row] * kLog2e : -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[rb][r] = __builtin_amdgcn_exp2f(fmaf(s[rb][r], kLog2e, nzl));
    }
    wait_vmcnt<0>();
    __syncthreads();  // dO_i landed
    f32x4_t dp[2] = {f32x4_t{}, f32x4_t{}};
    mfma_run_begin();
#pragma unroll
    for (int kk = 0; kk < LVC; ++kk)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        dp[rb] = mfma16(kf[kk], lds_ld16(&sdO[ldo_idx(32 * rh + 16 * rb + x, 32 * kk + 8 * g16)]), dp[rb]);
    mfma_run_end();
    // P and dS enter the contractions as bf16 pairs (rounded value +
    // rounding residual), so the gradients see them to about 16 bits. The
    // tiles sP, sdS hold the rounded words of all 64 rows for a first pass of
    // both contractions, then the residual words for a second; between the
    // passes a wave keeps only its packed residuals.
    uint32_t res_p[2][2], res_d[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float ds[4];
      const int row = 32 * rh + 16 * rb + x, key = 16 * kg + 4 * g16;
      const float del = q0 + row < a.seqlen_q ? rd[row] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) ds[r] = pv[rb][r] * (dp[rb][r] - del);
      const uint32_t p0 = pack_bf16x2(pv[rb][0], pv[rb][1]), p1 = pack_bf16x2(pv[rb][2], pv[rb][3]);
      const uint32_t d0 = pack_bf16x2(ds[0], ds[1]), d1 = pack_bf16x2(ds[2], ds[3]);
      *reinterpret_cast<u32x2_t*>(&sP[lp_idx(row, key)]) = u32x2_t{p0, p1};
      *reinterpret_cast<u32x2_t*>(&sdS[lp_idx(row, key)]) = u32x2_t{d0, d1};
      res_p[rb][0] = pack_bf16x2_residual(pv[rb][0], pv[rb][1], p0);
      res_p[rb][1] = pack_bf16x2_residual(pv[rb][2], pv[rb][3], p1);
      res_d[rb][0] = pack_bf16x2_residual(ds[0], ds[1], d0);
      res_d[rb][1] = pack_bf16x2_residual(ds[2], ds[3], d1);
    }
    lds_barrier();  // rounded P^T and dS^T published

    // ---- dKV[32 kh .. +31][144 cq .. +143] += dS^T Q_i, then + P^T dO_i -------
    // (two 16-key groups per wave share every Q_i / dO_i fragment read from
    // LDS, which halves those reads per MFMA against one group per wave)
    // (a scheduling barrier every six MFMAs bounds how far ahead of their
    // MFMAs the compiler issues the operand reads: the registers are at the
    // limit, and the K fragments spill more without it)
    mfma_run_begin();
#pragma unroll
    for (int ks = 0; ks < LBQ / 32; ++ks) {
      const u32x4_t ads0 = lds_tr8(sdS, 32 * ks, 32 * kh, lane, LpIdx{});
      const u32x4_t ads1 = lds_tr8(sdS, 32 * ks, 32 * kh + 16, lane, LpIdx{});
#pragma unroll
      for (int db = 0; db < 9; ++db) {
        const u32x4_t bq = lds_tr8(sQ, 32 * ks, 144 * cq + 16 * db, lane, LkIdxT<false>{});
        acc[0][db] = mfma16(ads0, bq, acc[0][db]);
        acc[1][db] = mfma16(ads1, bq, acc[1][db]);
        if (db % 3 == 2) __builtin_amdgcn_sched_barrier(0);
      }
    }
    mfma_run_end();
    // the value path covers columns below 512: all 9 blocks of the first
    // three column quarters, the first 5 of the last
    auto value_path = [&](int ln, auto nb) {
      mfma_run_begin();
#pragma unroll
      for (int ks = 0; ks < LBQ / 32; ++ks) {
        const u32x4_t ap0 = lds_tr8(sP, 32 * ks, 32 * kh, ln, LpIdx{});
        const u32x4_t ap1 = lds_tr8(sP, 32 * ks, 32 * kh + 16, ln, LpIdx{});
#pragma unroll
        for (int db = 0; db < decltype(nb)::value; ++db) {
          const u32x4_t bo = lds_tr8(sdO, 32 * ks, 144 * cq + 16 * db, ln, LdoIdx{});
          acc[0][db] = mfma16(ap0, bo, acc[0][db]);
          acc[1][db] = mfma16(ap1, bo, acc[1][db]);
          if (db % 3 == 2) __builtin_amdgcn_sched_barrier(0);
        }
      }
      mfma_run_end();
    };
    if (cq < 3)
      value_path(lane, std::integral_constant<int, 9>{});
    else
      value_path(lane, std::integral_constant<int, (LV - 432) / 16>{});
    lds_barrier();  // every wave is done reading the rounded words

    // ---- the same contractions on the residual words ----------------------------
    // (the lane index is re-derived so the read addresses are recomputed
    // rather than held across the first pass)
    int lane2 = lane0;
    asm volatile("" : "+v"(lane2));
    {
      const int g16b = lane2 >> 4, xb = lane2 & 15;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = 32 * rh + 16 * rb + xb, key = 16 * kg + 4 * g16b;
        *reinterpret_cast<u32x2_t*>(&sP[lp_idx(row, key)]) = u32x2_t{res_p[rb][0], res_p[rb][1]};
        *reinterpret_cast<u32x2_t*>(&sdS[lp_idx(row, key)]) = u32x2_t{res_d[rb][0], res_d[rb][1]};
      }
    }
    lds_barrier();  // residual words published
    mfma_run_begin();
#pragma unroll
    for (int ks = 0; ks < LBQ / 32; ++ks) {
      const u32x4_t ads0 = lds_tr8(sdS, 32 * ks, 32 * kh, lane2, LpIdx{});
      const u32x4_t ads1 = lds_tr8(sdS, 32 * ks, 32 * kh + 16, lane2, LpIdx{});
#pragma unroll
      for (int db = 0; db < 9; ++db) {
        const u32x4_t bq = lds_tr8(sQ, 32 * ks, 144 * cq + 16 * db, lane2, LkIdxT<false>{});
        acc[0][db] = mfma16(ads0, bq, acc[0][db]);
        acc[1][db] = mfma16(ads1, bq, acc[1][db]);
        if (db % 3 == 2) __builtin_amdgcn_sched_barrier(0);
      }
    }
    mfma_run_end();
    if (p + 1 < n_pairs) {
      lds_barrier();  // every wave is done reading sQ
      lk_copy_w<KNW, false, true>(sQ, qb + (size_t)pair_head(p + 1) * LQK, q_rs, pair_block(p + 1) * LBQ, a.seqlen_q, wave,
                     lane2);
    }
    if (cq < 3)
      value_path(lane2, std::integral_constant<int, 9>{});
    else
      value_path(lane2, std::integral_constant<int, (LV - 432) / 16>{});
  }

  // ---- this head group's partial dKV_j (fp32) ------------------------------------
  const int g16 = lane0 >> 4, x = lane0 & 15;
  float* pb = part + ((size_t)hg * a.batch + b) * a.seqlen_k * LQK;
#pragma unroll
  for (int kq = 0; kq < 2; ++kq)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k0 + 32 * kh + 16 * kq + 4 * g16 + r;
      if (key >= a.seqlen_k) continue;
#pragma unroll
      for (int db = 0; db < 9; ++db) pb[(size_t)key * LQK + 144 * cq + 16 * db + x] = acc[kq][db][r];
    }
  if (tid == 0 && a.stats) {
    atomicAdd(&a.stats[0], n_legal);
    atomicAdd(&a.stats[1], n_ret);
    atomicAdd(&a.stats[2], n_slots);
    atomicAdd(&a.stats[3], n_ret);
  }
}

// dKV = sum over head groups of the partials, in group order; 8 columns per thread.
__global__ void __launch_bounds__(256) bwd_latent_reduce_kernel(BwdParams a, int n_hg, const float* part) {
  const long long n = (long long)a.batch * a.seqlen_k * (LQK / 8);
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const size_t stride = (size_t)a.batch * a.seqlen_k * LQK;
  const float* src = part + t * 8;
  f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(src), s1 = *reinterpret_cast<const f32x4_t*>(src + 4);
  for (int g = 1; g < n_hg; ++g) {
    s0 += *reinterpret_cast<const f32x4_t*>(src + g * stride);
    s1 += *reinterpret_cast<const f32x4_t*>(src + g * stride + 4);
  }
  st16((uint16_t*)a.dk + t * 8, u32x4_t{pack_bf16x2(s0[0], s0[1]), pack_bf16x2(s0[2], s0[3]),
                                        pack_bf16x2(s1[0], s1[1]), pack_bf16x2(s1[2], s1[3])});
}

// ---------------------------------------------------------------------------
// query-major role: dQ_i of one head
// ---------------------------------------------------------------------------
constexpr int QNW = 4;
constexpr int QNT = 64 * QNW;
constexpr int QDB = LQK / 16 / QNW;  // 16-column blocks of dQ per wave (9)

struct DqShared {
  int vote[QNW];
};

__global__ void __launch_bounds__(QNT, 1) bwd_latent_dq_kernel(BwdParams a, int n_chunks) {
  __shared__ __attribute__((aligned(16))) uint16_t sK0[LTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[LTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sdS[LBQ * LBK];
  __shared__ DqShared sh;

  const int tid = threadIdx.x, lane0 = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane0 >> 4, x = lane0 & 15;

  // work item: chunks of H_q items (one (b, i), every head) dealt to the
  // XCDs round-robin, heaviest (last) query blocks first, as in the forward
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int chunk = (slot / a.heads_q) * 8 + xcd;
  if (chunk >= n_chunks) return;
  const int h = slot % a.heads_q;
  const int b = chunk % a.batch;
  const int i = a.nqb - 1 - chunk / a.batch;
  const int q0 = i * LBQ;
  const int off = a.offset;
  const int row_hi = min(q0 + LBQ, a.seqlen_q) - 1;
  const int jmax = (row_hi + off) / LBK;

  const size_t q_rs = (size_t)a.heads_q * LQK, do_rs = (size_t)a.heads_q * LV;
  const uint16_t* const kvb = (const uint16_t*)a.k + (size_t)b * a.seqlen_k * LQK;

  // this lane's query row (scores), its test offset, -z log2(e) and D
  const int qrow = q0 + 16 * wave + x;
  const bool qvalid = qrow < a.seqlen_q;
  float zt, nzl, del;
  {
    const size_t zo = ((size_t)b * a.heads_q + h) * a.seqlen_q;
    const float z = qvalid ? a.z[zo + qrow] : INFINITY;
    zt = qvalid ? latent_test_offset(a, z, qrow) : INFINITY;
    nzl = -z * kLog2e;
    del = qvalid ? a.delta[zo + qrow] : 0.f;
  }
  u32x4_t qf[LKC], dof[LVC];
  {
    const int rows = min(max(a.seqlen_q - q0, 0), LBQ);
    const rsrc_t rq = make_rsrc((const uint16_t*)a.q + ((size_t)b * a.seqlen_q + q0) * q_rs + (size_t)h * LQK,
                                (uint32_t)rows * (uint32_t)q_rs * 2u);
    const rsrc_t ro = make_rsrc((const uint16_t*)a.dout + ((size_t)b * a.seqlen_q + q0) * do_rs + (size_t)h * LV,
                                (uint32_t)rows * (uint32_t)do_rs * 2u);
#pragma unroll
    for (int kk = 0; kk < LKC; ++kk)
      qf[kk] = buf_ld16(rq, (uint32_t)((16 * wave + x) * q_rs + 32 * kk + 8 * g16) * 2u);
#pragma unroll
    for (int kk = 0; kk < LVC; ++kk)
      dof[kk] = buf_ld16(ro, (uint32_t)((16 * wave + x) * do_rs + 32 * kk + 8 * g16) * 2u);
  }
  f32x4_t acc[QDB][4];  // dQ^T[column 144 wave + 16 db + 4 g16 + r][row 16 rb + x]
#pragma unroll
  for (int db = 0; db < QDB; ++db)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[db][rb] = f32x4_t{};

  // one tile: K_j in `cur`; the copy of K_{j-1} goes to `nxt`
  // Four chains of MFMAs over 64 keys, A = K rows of the tile, B = this
  // wave's 16 rows in registers; the next chunk's four K fragments are read
  // while the current chunk's MFMAs issue (one wave per SIMD: the wave's own
  // reads are all that can hide the LDS latency).
  auto score4 = [&](const uint16_t* cur, const u32x4_t* bf, auto nk, f32x4_t* acc4, int x, int g16) {
    u32x4_t a0[4], a1[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) a0[kb] = lds_ld16(&cur[lk_idx<false>(16 * kb + x, 8 * g16)]);
#pragma unroll
    for (int kk = 0; kk < decltype(nk)::value; ++kk) {
      u32x4_t* ca = (kk & 1) ? a1 : a0;
      u32x4_t* na = (kk & 1) ? a0 : a1;
      if (kk + 1 < decltype(nk)::value) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) na[kb] = lds_ld16(&cur[lk_idx<false>(16 * kb + x, 32 * (kk + 1) + 8 * g16)]);
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc4[kb] = mfma16(ca[kb], bf[kk], acc4[kb]);
    }
  };

  auto step = [&](int j, const uint16_t* cur, uint16_t* nxt) {
    const int k0 = j * LBK;
    // the lane index is re-derived per tile, so the copy and LDS addresses
    // are recomputed (a few VALU ops) instead of held across the loop, which
    // leaves registers for the LDS reads in flight
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    const int g16 = lane >> 4, x = lane & 15;
    wait_vmcnt<0>();
    __syncthreads();  // K_j landed; every wave is done with tile j + 1 (dS tile, votes, nxt)
    if (j > 0) lk_copy_w<QNW, false, true>(nxt, kvb, LQK, k0 - LBK, a.seqlen_k, wave, lane);

    // ---- S^T[key 16 kb + 4 g16 + r][row qrow] ---------------------------------------
    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb] = f32x4_t{};
    mfma_run_begin();
    score4(cur, qf, std::integral_constant<int, LKC>{}, s, x, g16);
    mfma_run_end();
    if (k0 + LBK - 1 > q0 + off || q0 + LBQ > a.seqlen_q) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 16 * kb + 4 * g16 + r;
          if (!(qvalid && key <= qrow + off)) s[kb][r] = -INFINITY;
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmaxf(m, s[kb][r] - zt);
    const bool wave_vote = __ballot(m >= 0.f) != 0ull;
    if (lane == 0) sh.vote[wave] = wave_vote ? 1 : 0;
    lds_barrier();  // the copy of K_{j-1} stays in flight
    bool retain = false;
#pragma unroll
    for (int w = 0; w < QNW; ++w) retain |= sh.vote[w] != 0;
    if (a.tile_mask_dq && tid == 0)  // this pass's own decision
      a.tile_mask_dq[(((size_t)b * a.heads_q + h) * a.nqb + i) * a.nkb + j] = retain ? 1 : 0;
    if (!retain) return;

    // ---- dP^T, P, dS^T into the dS tile -------------------------------------------
    f32x4_t dp[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) dp[kb] = f32x4_t{};
    mfma_run_begin();
    score4(cur, dof, std::integral_constant<int, LVC>{}, dp, x, g16);
    mfma_run_end();
    // dS enters dQ as a bf16 pair (rounded value + rounding residual). The
    // 64 x 64 dS tile takes one 32-key half at a time: its keys' rounded
    // values in columns 0..31, their residuals in columns 32..63.
    float dsv[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[kb][r], kLog2e, nzl));
        dsv[kb][r] = pr * (dp[kb][r] - del);
      }
#pragma unroll
    for (int ks = 0; ks < LBK / 32; ++ks) {
      if (ks > 0) lds_barrier();  // every wave is done reading the previous half
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float* d = dsv[2 * ks + c];
        const uint32_t d0 = pack_bf16x2(d[0], d[1]), d1 = pack_bf16x2(d[2], d[3]);
        *reinterpret_cast<u32x2_t*>(&sdS[lp_idx(16 * wave + x, 16 * c + 4 * g16)]) = u32x2_t{d0, d1};
        *reinterpret_cast<u32x2_t*>(&sdS[lp_idx(16 * wave + x, 32 + 16 * c + 4 * g16)]) =
            u32x2_t{pack_bf16x2_residual(d[0], d[1], d0), pack_bf16x2_residual(d[2], d[3], d1)};
      }
      lds_barrier();  // this half's dS pairs published

      // ---- dQ^T[144 wave .. +143][rows] += K_j^T dS^T over keys 32 ks .. +31 ----
      mfma_run_begin();
      u32x4_t bds[4], bdr[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        bds[rb] = lds_ld16(&sdS[lp_idx(16 * rb + x, 8 * g16)]);
        bdr[rb] = lds_ld16(&sdS[lp_idx(16 * rb + x, 32 + 8 * g16)]);
      }
      // K^T fragment of the next 16 columns read while this one's MFMAs issue
      u32x4_t ak[2];
      ak[0] = lds_tr8(cur, 32 * ks, 144 * wave, lane, LkIdxT<false>{});
#pragma unroll
      for (int db = 0; db < QDB; ++db) {
        if (db + 1 < QDB) ak[(db + 1) & 1] = lds_tr8(cur, 32 * ks, 144 * wave + 16 * (db + 1), lane, LkIdxT<false>{});
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) acc[db][rb] = mfma16(ak[db & 1], bds[rb], acc[db][rb]);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) acc[db][rb] = mfma16(ak[db & 1], bdr[rb], acc[db][rb]);
      }
      mfma_run_end();
    }
  };

  if (jmax >= 0) lk_copy_w<QNW, false, true>(sK0, kvb, LQK, jmax * LBK, a.seqlen_k, wave, lane0);
  for (int j = jmax; j >= 0; j -= 2) {
    step(j, sK0, sK1);
    if (j - 1 >= 0) step(j - 1, sK1, sK0);
  }

  // ---- dQ rows (bf16) ------------------------------------------------------------
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = q0 + 16 * rb + x;
    if (row >= a.seqlen_q) continue;
    uint16_t* dqr = (uint16_t*)a.dq + ((size_t)b * a.seqlen_q + row) * q_rs + (size_t)h * LQK;
#pragma unroll
    for (int db = 0; db < QDB; ++db) {
      const f32x4_t v = acc[db][rb];
      *reinterpret_cast<u32x2_t*>(dqr + 144 * wave + 16 * db + 4 * g16) =
          u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
}

}  // namespace

// Query heads per key-major work item: the largest divisor of H_q that
// still gives at least 512 items (two per CU), so the fp32 partials stay
// few while the grid fills the chip.
int latent_bwd_heads_per_item(const mala_problem& p) {
  const long long nkb = (p.seqlen_k + LBK - 1) / LBK;
  int best = 1;
  for (int d = 1; d <= p.heads_q; ++d)
    if (p.heads_q % d == 0 && p.batch * nkb * (p.heads_q / d) >= 512) best = d;
  return best;
}

hipError_t launch_bwd_latent(const mala_problem& p, const BwdParams& a, int d_v, float* part, hipStream_t s,
                             bool* supported) {
  *supported = p.dtype == MALA_BF16 && p.head_dim == LQK && d_v == LV && p.heads_kv == 1 &&
               p.block_q == LBQ && p.block_k == LBK;
  if (!*supported) return hipSuccess;
  const long long rows = (long long)a.batch * a.seqlen_q * a.heads_q;
  hipLaunchKernelGGL(bwd_latent_prep_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
  const int hpi = latent_bwd_heads_per_item(p);
  const int n_hg = a.heads_q / hpi;
  hipLaunchKernelGGL(bwd_latent_dkv_kernel, dim3((unsigned)(a.nkb * a.batch * n_hg)), dim3(KNT), 0, s, a, hpi,
                     n_hg, part);
  const long long n8 = (long long)a.batch * a.seqlen_k * (LQK / 8);
  hipLaunchKernelGGL(bwd_latent_reduce_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, a, n_hg,
                     (const float*)part);
  const int n_chunks = a.batch * a.nqb;
  const int grid = (n_chunks + 7) / 8 * 8 * a.heads_q;
  hipLaunchKernelGGL(bwd_latent_dq_kernel, dim3((unsigned)grid), dim3(QNT), 0, s, a, n_chunks);
  return hipGetLastError();
}

}  // namespace mala
