// MALA backward kernels for gfx950 (MALA page, "Offline Sparse Probability"
// and "Fused backward execution").
//
//  bwd_absmax: partial maxima of |dO| (one per workgroup).
//  bwd_prep: D_q = sum_d dO_qd O_qd (fp32), one 16-lane group per
//            (batch, row, head), and the fp16 copy dO 2^s_o, the power of
//            two s_o putting max |dO| into [2^14, 2^15).
//  bwd_main: one launch, two roles over 64 x 64 tiles, no atomics:
//    * key-major (the page's traversal): a workgroup owns key block J_j of
//      one KV head, keeps K_j, V_j on chip and accumulates dK_j, dV_j over the
//      group's query heads and the query blocks I_i from the diagonal
//      upward. Per tile it recomputes S = Q_i K_j^T, tests every legal entry
//      against the saved normalizer (retain iff some S_qk - z_q >=
//      log tau - log L_q), and only for a retained tile loads dO_i and runs
//      P = exp(S - z), dP = dO V^T, dS = P (dP - D), dV += P^T dO,
//      dK += dS^T Q. dP and dV run on fp16 operands (dO 2^s_o, V_j 2^s_v,
//      P), dK on dS as a bf16 pair.
//    * query-major: a workgroup owns two query blocks of one query head,
//      keeps their Q, dO in registers, visits the legal key blocks, recomputes
//      the transposed scores and the same test (bit-identical decisions, see
//      dq_item) and, for retained tiles, loads V_j and accumulates
//      dQ_i += dS K_j in registers. dQ is written once: the result is
//      deterministic.
//  Decisions use only the finalized z, so the two roles need no ordering.
//
// Four waves split a tile 2 x 2 (32 keys x 32 rows each). Transposed MFMA
// operands (Q^T, dO^T, K^T) are read straight from the row-major LDS tiles
// with the LDS transpose loads. The key-major role fetches its tiles with
// buffer loads whose range check zero-fills rows past the end of a
// sequence; the query-major role copies K and V tiles HBM -> LDS directly
// (rows past the end repeat the last row: finite values whose scores are
// masked, so their P and dS are 0).
#include <math.h>

#include <algorithm>

#include "mala_common.hpp"

namespace mala {
namespace {

constexpr int BQ = 64;
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int PREP_NB = 2048;  // workgroups of bwd_prep (grid-stride over the rows)

// fp16 operands of the key-major role's dP = dO V^T and dV += P^T dO.
// Every bf16 value is an fp16 value times a power of two as long as the
// scaled value stays in fp16's normal range (bf16 has 8 significant bits,
// fp16 11), so dO and V enter as x 2^s exactly, with s chosen per tensor
// (dO) or per tile (V) to bring the largest |x| into [2^14, 2^15); only
// values below 2^-28 of that maximum lose bits. P in [0, 1] is rounded to
// fp16 directly: 2^-11 relative instead of bf16's 2^-8.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x16_t mfma32h(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}
// Two floats -> two fp16 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
// A bf16 pair word -> the fp16 pair word of its values times 2^s.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, int s) {
  return pack_f16x2(__builtin_amdgcn_ldexpf(bf16_lo(w), s), __builtin_amdgcn_ldexpf(bf16_hi(w), s));
}
// The exponent s with max|x| 2^s in [2^14, 2^15), from the bf16 bits of
// max|x| (all zeros or subnormal: the scale of the smallest normal).
__device__ __forceinline__ int half_scale(unsigned m) { return 141 - max((int)(m >> 7), 1); }
// Largest |x| of the bf16 pair word w as bf16 bits (|x| orders as its bits).
__device__ __forceinline__ unsigned abs_bits_max(unsigned m, uint32_t w) {
  return max(m, max(w & 0x7fffu, (w >> 16) & 0x7fffu));
}

// Partial maxima of |dO| over the n bf16 values of dO (n a multiple of 8),
// one per workgroup, as bf16 bits: kBwdMaxParts workgroups.
__global__ void __launch_bounds__(256) bwd_absmax_kernel(const uint16_t* x, long long n, unsigned* part) {
  const long long n8 = n / 8;
  unsigned m = 0;
  const long long step = (long long)gridDim.x * 256;
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * step < n8; i += 4 * step) {
    u32x4_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = ld16(x + 8 * (i + u * step));
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) m = abs_bits_max(m, w[u][t]);
  }
  for (; i < n8; i += step) {
    const u32x4_t w = ld16(x + 8 * i);
#pragma unroll
    for (int t = 0; t < 4; ++t) m = abs_bits_max(m, w[t]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, o));
  __shared__ unsigned wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
}

// A-row x of a 32-row MFMA block reads row row_perm(x): bits 2 and 3
// swapped, so accumulator registers 8a..8a+7 of lane half hh hold the
// consecutive rows 16a + 8hh + 0..7 - the k-slot order of an MFMA that
// contracts over those rows.
__device__ __forceinline__ int row_perm(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Test offset of query row q with normalizer z: S_qk is retained-worthy iff
// S_qk - (z + log tau - log L_q) >= 0, L_q = q + offset + 1. Computed once
// per row here; both roles read the stored float, so their tests compare
// the same numbers.
__device__ __forceinline__ float test_offset(const BwdParams& a, float z, int q) {
  return z + (a.log_tau - __logf((float)(q + a.offset + 1)));
}

// The row state of every query row - -z_q log2(e), the test offset and
// D_q, rows past N_q padded with a row that is never retained (offset +inf,
// P = 0, D = 0) - and the fp16 copy dO 2^s_o that the key-major role reads
// (s_o from the partial maxima; workgroup 0 stores it for that role).
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams a, int D) {
  static_assert(kBwdMaxParts % 256 == 0, "partial maxima split evenly over the threads");
  __shared__ unsigned wm[4];
  int s_o;
  {
    unsigned mo = 0;
#pragma unroll
    for (int u = 0; u < kBwdMaxParts / 256; ++u) mo = max(mo, a.absmax[threadIdx.x + 256 * u]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mo = max(mo, (unsigned)__shfl_xor((int)mo, o));
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mo;
    __syncthreads();
    s_o = half_scale(max(max(wm[0], wm[1]), max(wm[2], wm[3])));
    if (blockIdx.x == 0 && threadIdx.x == 0) a.do_scale[0] = s_o;
  }
  const long long rows = (long long)a.batch * a.seqlen_q * a.heads_q;
  const int sub = threadIdx.x & 15;
  for (long long r = (long long)blockIdx.x * 16 + (threadIdx.x >> 4); r < rows; r += (long long)gridDim.x * 16) {
    const int h = (int)(r % a.heads_q);
    const long long bq = r / a.heads_q;
    const int q = (int)(bq % a.seqlen_q);
    const int b = (int)(bq / a.seqlen_q);
    float acc = 0.f;
    if (sub * 8 < D) {
      const size_t off = (size_t)r * D + sub * 8;
      const u32x4_t x = ld16((const uint16_t*)a.dout + off);
      const u32x4_t y = ld16((const uint16_t*)a.o + off);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc += bf16_lo(x[t]) * bf16_lo(y[t]) + bf16_hi(x[t]) * bf16_hi(y[t]);
      st16(a.do16 + off, u32x4_t{bf16x2_to_f16x2(x[0], s_o), bf16x2_to_f16x2(x[1], s_o),
                                  bf16x2_to_f16x2(x[2], s_o), bf16x2_to_f16x2(x[3], s_o)});
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 1);
    if (sub == 0) {
      const size_t bh = (size_t)b * a.heads_q + h;
      const float z = a.z[bh * a.seqlen_q + q];
      float* const rs = a.rowst + bh * 3 * a.rp;
      rs[q] = -z * kLog2e;
      rs[a.rp + q] = test_offset(a, z, q);
      rs[2 * a.rp + q] = acc;
    }
  }
  const int pad = a.rp - a.seqlen_q;
  const long long npad = (long long)a.batch * a.heads_q * pad;
  for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < npad; t += (long long)gridDim.x * 256) {
    float* const rs = a.rowst + (size_t)(t / pad) * 3 * a.rp;
    const int q = a.seqlen_q + (int)(t % pad);
    rs[q] = -INFINITY;
    rs[a.rp + q] = INFINITY;
    rs[2 * a.rp + q] = 0.f;
  }
}

struct Shared {
  // row state of the key-major role's query block: [0] -z_q log2(e)
  // (P = 2^(S log2(e) - z_q log2(e))), [1] the test offset, [2] D_q
  float rst[3][BQ] __attribute__((aligned(16)));
  int vote[4];
  unsigned vmax[4];
};


// Does the tile (query block at q0, key block at k0) hold an illegal entry?
__device__ __forceinline__ bool tile_has_masked(const BwdParams& a, int q0, int k0) {
  return k0 + BK - 1 > q0 + a.offset || q0 + BQ > a.seqlen_q;
}

// ---------------------------------------------------------------------------
// key-major role: dK_j, dV_j
//   S = Q_i K_j^T per wave over 32 rows x 32 keys with Q rows permuted
//   (row_perm), so lane l holds key l % 32 and accumulator registers
//   8 hb .. 8 hb + 7 hold rows 16 hb + 8 (l / 32) + 0..7: packed P and dS
//   are the A operands of dV += P^T dO and dK += dS^T Q as they stand.
// ---------------------------------------------------------------------------
template <int D>
__device__ void dkdv_item(const BwdParams& a, uint16_t* smem, Shared& sh, int j, int bg) {
  constexpr int EB = D / 32;
  constexpr int KS = D / 16;
  constexpr int TILE = 64 * D;
  uint16_t* const sQ = smem;
  uint16_t* const sdO = smem + TILE;
  uint16_t* const sK = smem + 2 * TILE;
  uint16_t* const sV = smem + 3 * TILE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int wk = wave & 1, wr = wave >> 1;

  const int b = bg / a.heads_kv;
  const int g = bg % a.heads_kv;
  const int group = a.heads_q / a.heads_kv;
  const int k0 = j * BK;
  const int i0 = max(0, k0 - a.offset) / BQ;

  const int q_rs = a.heads_q * D, kv_rs = a.heads_kv * D;
  const size_t kvoff = ((size_t)b * a.seqlen_k * a.heads_kv + g) * D;
  const uint16_t* const qb = (const uint16_t*)a.q + (size_t)b * a.seqlen_q * q_rs;
  const uint16_t* const ob = a.do16 + (size_t)b * a.seqlen_q * q_rs;  // dO 2^s_o, fp16
  const int s_o = a.do_scale[0];
  int s_v;
  {
    TileRegs<D, NT> t;
    t.load((const uint16_t*)a.k + kvoff, kv_rs, k0, a.seqlen_k, tid);
    t.store(sK, tid);
    t.load((const uint16_t*)a.v + kvoff, kv_rs, k0, a.seqlen_k, tid);
    // V_j enters dP = dO V^T as the fp16 tile V_j 2^s_v, s_v from its own maximum
    unsigned vm = 0;
#pragma unroll
    for (int c = 0; c < TileRegs<D, NT>::PER_T; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) vm = abs_bits_max(vm, t.r[c][w]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) vm = max(vm, (unsigned)__shfl_xor((int)vm, o));
    if (lane == 0) sh.vmax[wave] = vm;
    __syncthreads();
    s_v = half_scale(max(max(sh.vmax[0], sh.vmax[1]), max(sh.vmax[2], sh.vmax[3])));
#pragma unroll
    for (int c = 0; c < TileRegs<D, NT>::PER_T; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) t.r[c][w] = bf16x2_to_f16x2(t.r[c][w], s_v);
    t.store(sV, tid);
  }

  f32x16_t dv_acc[EB], dk_acc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) dv_acc[e] = dk_acc[e] = f32x16_t{};
  unsigned long long n_legal = 0, n_ret = 0, n_slots = 0;

  // (head, query block) pairs of this item, in order; the next pair's Q tile
  // and row state (thread t < 192 holding row t % 64 of array t / 64) are
  // prefetched into registers while the current pair runs
  const int per_head = a.nqb - i0;
  const int n_pairs = per_head > 0 ? group * per_head : 0;
  TileRegs<D, NT> qn;
  float rn;
  int nh = g * group, ni = i0;
  auto prefetch = [&](int hq, int i) {
    qn.load(qb + (size_t)hq * D, q_rs, i * BQ, a.seqlen_q, tid);
    if (tid < 3 * BQ) rn = a.rowst[(((size_t)b * a.heads_q + hq) * 3 + (tid >> 6)) * a.rp + i * BQ + (tid & 63)];
  };
  if (n_pairs > 0) prefetch(nh, ni);
  const int qr = 32 * wr + row_perm(l32), kr = 32 * wk + l32;
  bool reuse = false;  // the previous pair ran retained work (sQ, sdO, row state read after its vote)
  for (int p = 0; p < n_pairs; ++p) {
    const int hq = nh, i = ni, q0 = i * BQ;
    // the previous pair's readers of sQ, sdO and the row state are done: a
    // skipped pair's readers all came before its vote barrier
    if (reuse) __syncthreads();
    reuse = false;
    qn.store(sQ, tid);
    if (tid < 3 * BQ) (&sh.rst[0][0])[tid] = rn;
    if (p + 1 < n_pairs) {
      if (++ni == a.nqb) {
        ni = i0;
        ++nh;
      }
      prefetch(nh, ni);
    }
    // a ragged last query block may end before the key block starts
    if (k0 > min(q0 + BQ, a.seqlen_q) - 1 + a.offset) continue;
    __syncthreads();

    mfma_run_begin();
    f32x16_t s = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      s = mfma32(tile_row8<D>(sQ, qr, 16 * kk + 8 * hh), tile_row8<D>(sK, kr, 16 * kk + 8 * hh), s);
    interleave_ds_mfma<KS, 2>();
    mfma_run_end();
    // mask; vote iff some legal S_qk - (z_q + log tau - log L_q) >= 0
    if (tile_has_masked(a, q0, k0)) {
      const int key = k0 + kr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 32 * wr + 16 * (r >> 3) + 8 * hh + (r & 7);
        if (!(key <= q + a.offset && q < a.seqlen_q)) s[r] = -INFINITY;
      }
    }
    const f32x4_t* zt4 = reinterpret_cast<const f32x4_t*>(sh.rst[1]) + 8 * wr + 2 * hh;
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4_t zt = zt4[4 * (c >> 1) + (c & 1)];  // rows 16 hb + 8 hh + 4 (c & 1) + 0..3
#pragma unroll
      for (int t = 0; t < 4; ++t) m = fmaxf(m, s[4 * c + t] - zt[t]);
    }
    const bool wave_vote = __ballot(m >= 0.f) != 0ull;
    if (lane == 0) sh.vote[wave] = wave_vote ? 1 : 0;
    __syncthreads();
    const bool retain = (sh.vote[0] | sh.vote[1] | sh.vote[2] | sh.vote[3]) != 0;
    ++n_legal;
    if (tid == 0 && a.tile_mask)
      a.tile_mask[(((size_t)b * a.heads_q + hq) * a.nqb + i) * a.nkb + j] = retain ? 1 : 0;
    if (!retain) continue;
    reuse = true;
    ++n_ret;
    n_slots += (unsigned long long)BK * min(BQ, a.seqlen_q - q0);

    // retained: dO_i (its load overlaps P = exp(S - z))
    TileRegs<D, NT> ot;
    ot.load(ob + (size_t)hq * D, q_rs, q0, a.seqlen_q, tid);
    __builtin_amdgcn_sched_barrier(0);  // keep P between the load and its use
    float pv[16];
    {
      const f32x4_t* nz4 = reinterpret_cast<const f32x4_t*>(sh.rst[0]) + 8 * wr + 2 * hh;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4_t nz = nz4[4 * (c >> 1) + (c & 1)];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          pv[4 * c + t] = __builtin_amdgcn_exp2f(fmaf(s[4 * c + t], kLog2e, nz[t]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    ot.store(sdO, tid);
    __syncthreads();
    mfma_run_begin();
    f32x16_t dp = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      dp = mfma32h(tile_row8<D>(sdO, qr, 16 * kk + 8 * hh), tile_row8<D>(sV, kr, 16 * kk + 8 * hh), dp);
    interleave_ds_mfma<KS, 2>();
    mfma_run_end();
    // dP = dP' 2^-(s_o + s_v) (exact). P enters dV as fp16 (11 bits), dS
    // enters dK as a bf16 pair (rounded value + rounding residual), so dK
    // sees dS to about 16 bits rather than bf16's 8
    u32x4_t pa[2], dsa[2], dsr[2];
    {
      const f32x4_t* d4 = reinterpret_cast<const f32x4_t*>(sh.rst[2]) + 8 * wr + 2 * hh;
      float ds[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4_t dl = d4[4 * (c >> 1) + (c & 1)];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          ds[4 * c + t] = pv[4 * c + t] * (__builtin_amdgcn_ldexpf(dp[4 * c + t], -(s_o + s_v)) - dl[t]);
      }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float* p2 = &pv[8 * hb + 2 * t];
          const float* d2 = &ds[8 * hb + 2 * t];
          pa[hb][t] = pack_f16x2(p2[0], p2[1]);
          dsa[hb][t] = pack_bf16x2(d2[0], d2[1]);
          dsr[hb][t] = pack_bf16x2_residual(d2[0], d2[1], dsa[hb][t]);
        }
      }
    }
    mfma_run_begin();
    // dV_j 2^s_o += P^T dO_i 2^s_o, dK_j += dS^T Q_i over this wave's 32
    // rows: each operand fragment is read once, the dS fragment serves the
    // rounded and the residual term, and consecutive MFMAs write different
    // accumulators
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      u32x4_t ocol[EB], qcol[EB];
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        ocol[e] = tile_col8<D>(sdO, 32 * wr + 16 * hb, 32 * e, lane);
        qcol[e] = tile_col8<D>(sQ, 32 * wr + 16 * hb, 32 * e, lane);
      }
#pragma unroll
      for (int e = 0; e < EB; ++e) dv_acc[e] = mfma32h(pa[hb], ocol[e], dv_acc[e]);
#pragma unroll
      for (int e = 0; e < EB; ++e) dk_acc[e] = mfma32(dsa[hb], qcol[e], dk_acc[e]);
#pragma unroll
      for (int e = 0; e < EB; ++e) dk_acc[e] = mfma32(dsr[hb], qcol[e], dk_acc[e]);
    }
    mfma_run_end();
  }

  // ---- sum the two row halves in LDS (fp32) and store bf16 rows ---------------
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [2][64 keys][D] fp32 = 4 tiles of bf16
  for (int pass = 0; pass < 2; ++pass) {
    if (wr == pass) {
#pragma unroll
      for (int e = 0; e < EB; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * wk + acc_row(r, hh), d = 32 * e + l32;
          float* pk = &red[key * D + d];
          float* pv = &red[64 * D + key * D + d];
          *pk = pass ? *pk + dk_acc[e][r] : dk_acc[e][r];
          const float dvr = __builtin_amdgcn_ldexpf(dv_acc[e][r], -s_o);
          *pv = pass ? *pv + dvr : dvr;
        }
    }
    __syncthreads();
  }
  uint16_t* dkbase = (uint16_t*)a.dk + kvoff;
  uint16_t* dvbase = (uint16_t*)a.dv + kvoff;
  for (int c = tid; c < 2 * 64 * (D / 8); c += NT) {
    const int which = c / (64 * (D / 8)), cc = c % (64 * (D / 8));
    const int key = cc / (D / 8), d0 = (cc % (D / 8)) * 8;
    if (k0 + key >= a.seqlen_k) continue;
    const float* src = &red[which * 64 * D + key * D + d0];
    const u32x4_t w = {pack_bf16x2(src[0], src[1]), pack_bf16x2(src[2], src[3]),
                       pack_bf16x2(src[4], src[5]), pack_bf16x2(src[6], src[7])};
    st16((which ? dvbase : dkbase) + (size_t)(k0 + key) * kv_rs + d0, w);
  }
  if (tid == 0 && a.stats) {
    atomicAdd(&a.stats[0], n_legal);
    atomicAdd(&a.stats[1], n_ret);
    atomicAdd(&a.stats[2], n_slots);
    atomicAdd(&a.stats[3], n_ret);
  }
}

// ---------------------------------------------------------------------------
// query-major role: dQ for 128 query rows = two query blocks I_i
//   One wave per 32 rows, all 64 keys of a tile: the transposed score tile
//   S^T = K_j Q^T with K rows permuted (row_perm), so lane l owns query row
//   l % 32 (its z, D and test offset are lane scalars) and accumulator
//   registers 8 hb .. 8 hb + 7 of 32-key block mb hold keys
//   32 mb + 16 hb + 8 (l / 32) + 0..7: packed dS is the A operand of
//   dQ += dS K as it stands, and each wave owns whole dQ rows. Q and dO stay
//   in registers as the B operands of S^T and dP^T. The two query blocks
//   (waves 0-1 and 2-3) vote separately; V_j is loaded when either retains
//   and used by the block(s) that do. The matrix core's dot products do not
//   depend on which operand is A (checked on the device), so every S and dP
//   entry, and with them every decision, is bit-identical to the key-major
//   role's: a block retains the tile iff max_k S_qk - offset_q >= 0 for some
//   of its rows, which equals that role's test entry by entry because
//   rounding the difference preserves its sign (fp32 denormals are kept).
// ---------------------------------------------------------------------------
template <int D>
__device__ void dq_item(const BwdParams& a, uint16_t* smem, Shared& sh, int isb, int bh) {
  constexpr int EB = D / 32;
  constexpr int KS = D / 16;
  constexpr int TILE = 64 * D;
  constexpr int RW = 128;  // query rows of the item
  // K_j in smem + (j & 1) TILE
  uint16_t* const sV = smem + 2 * TILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  const int half = wave >> 1;  // which query block of the item

  const int b = bh / a.heads_q;
  const int hq = bh % a.heads_q;
  const int g = hq / (a.heads_q / a.heads_kv);
  const int q0 = isb * RW;
  const int q0h = q0 + 64 * half;  // this wave's query block
  const int jmax = (min(q0 + RW, a.seqlen_q) - 1 + a.offset) / BK;

  const int q_rs = a.heads_q * D, kv_rs = a.heads_kv * D;
  const size_t qoff = ((size_t)b * a.seqlen_q * a.heads_q + hq) * D;
  const size_t kvoff = ((size_t)b * a.seqlen_k * a.heads_kv + g) * D;
  const int q = q0 + 32 * wave + l32;  // this lane's query row
  // row state of this lane's row (q < rp: the arrays are padded)
  const float* const rsb = a.rowst + (size_t)bh * 3 * a.rp;
  const float nzl = rsb[q], zt = rsb[a.rp + q], del = rsb[2 * a.rp + q];
  u32x4_t qf[KS], of[KS];
  {
    const int rows = min(max(a.seqlen_q - q0, 0), RW);
    const rsrc_t rq = make_rsrc((const uint16_t*)a.q + qoff + (size_t)q0 * q_rs, (uint32_t)rows * q_rs * 2u);
    const rsrc_t ro = make_rsrc((const uint16_t*)a.dout + qoff + (size_t)q0 * q_rs, (uint32_t)rows * q_rs * 2u);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint32_t off = (uint32_t)((32 * wave + l32) * q_rs + 16 * kk + 8 * hh) * 2u;
      qf[kk] = buf_ld16(rq, off);
      of[kk] = buf_ld16(ro, off);
    }
  }

  f32x16_t dq[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) dq[e] = f32x16_t{};
  // K tiles go HBM -> LDS directly, double-buffered (the copy of K_{j+1}
  // overlaps tile j); V_j is copied only for a retained tile, beside P
  const uint16_t* const kbase = (const uint16_t*)a.k + kvoff;
  const uint16_t* const vbase = (const uint16_t*)a.v + kvoff;
  TileCopy<D, BK, 4> cp;
  cp.init(kv_rs, wave, lane);
  cp.copy(smem, kbase, kv_rs, 0, a.seqlen_k, wave, lane);
  for (int j = 0; j <= jmax; ++j) {
    const int k0 = j * BK;
    const uint16_t* const sK = smem + (j & 1) * TILE;
    wait_vmcnt<0>();  // this wave's share of K_j landed
    __syncthreads();  // K_j visible; the previous tile's readers of the other K buffer and of sV are done
    if (j < jmax) cp.copy(smem + ((j + 1) & 1) * TILE, kbase, kv_rs, k0 + BK, a.seqlen_k, wave, lane);
    f32x16_t st[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) st[mb] = f32x16_t{};
    mfma_run_begin();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        st[mb] = mfma32(tile_row8<D>(sK, 32 * mb + row_perm(l32), 16 * kk + 8 * hh), qf[kk], st[mb]);
    interleave_ds_mfma<2 * KS, 1>();
    mfma_run_end();
    if (tile_has_masked(a, q0h, k0)) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * hh + (r & 7);
          if (!(key <= q + a.offset && q < a.seqlen_q)) st[mb][r] = -INFINITY;
        }
    }
    float mx = st[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[mb][r]);
    const bool wave_vote = __ballot(mx - zt >= 0.f) != 0ull;
    if (lane == 0) sh.vote[wave] = wave_vote ? 1 : 0;
    lds_barrier();  // votes visible (the copy of K_{j+1} stays in flight)
    const bool ret0 = (sh.vote[0] | sh.vote[1]) != 0, ret1 = (sh.vote[2] | sh.vote[3]) != 0;
    const bool retain = half ? ret1 : ret0;
    if (a.tile_mask_dq && tid == 0) {
      // this pass's own decisions, for legal tiles of each of its blocks
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int qb0 = q0 + 64 * x;
        if (qb0 < a.seqlen_q && j <= (min(qb0 + BQ, a.seqlen_q) - 1 + a.offset) / BK)
          a.tile_mask_dq[(((size_t)b * a.heads_q + hq) * a.nqb + 2 * isb + x) * a.nkb + j] = (x ? ret1 : ret0) ? 1 : 0;
      }
    }
    if (!(ret0 || ret1)) continue;
    // V_j for the block(s) that retain (its copy overlaps P = exp(S - z))
    cp.copy(sV, vbase, kv_rs, k0, a.seqlen_k, wave, lane);
    float pv[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pv[mb][r] = __builtin_amdgcn_exp2f(fmaf(st[mb][r], kLog2e, nzl));
    wait_vmcnt<0>();  // V_j landed (and K_{j+1}, issued before it)
    lds_barrier();
    if (!retain) continue;  // wave-uniform: the other block retained this tile
    f32x16_t dpt[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) dpt[mb] = f32x16_t{};
    mfma_run_begin();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        dpt[mb] = mfma32(tile_row8<D>(sV, 32 * mb + row_perm(l32), 16 * kk + 8 * hh), of[kk], dpt[mb]);
    interleave_ds_mfma<2 * KS, 1>();
    mfma_run_begin();
    // dQ (this wave's 32 rows) += dS K_j over the tile's 64 keys, dS as a
    // bf16 pair (rounded value + residual) like the key-major role's
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float ds[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) ds[t] = pv[mb][8 * hb + t] * (dpt[mb][8 * hb + t] - del);
        u32x4_t dsa, dsr;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          dsa[t] = pack_bf16x2(ds[2 * t], ds[2 * t + 1]);
          dsr[t] = pack_bf16x2_residual(ds[2 * t], ds[2 * t + 1], dsa[t]);
        }
        u32x4_t kcol[EB];
#pragma unroll
        for (int e = 0; e < EB; ++e) kcol[e] = tile_col8<D>(sK, 32 * mb + 16 * hb, 32 * e, lane);
#pragma unroll
        for (int e = 0; e < EB; ++e) dq[e] = mfma32(dsa, kcol[e], dq[e]);
#pragma unroll
        for (int e = 0; e < EB; ++e) dq[e] = mfma32(dsr, kcol[e], dq[e]);
      }
    }
    mfma_run_end();
  }

  // ---- dQ: rows through LDS (fp32) for coalesced bf16 16-byte stores --------
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // 128 x D fp32 over the four tiles
#pragma unroll
  for (int e = 0; e < EB; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(32 * wave + acc_row(r, hh)) * D + 32 * e + l32] = dq[e][r];
  __syncthreads();
  uint16_t* dqbase = (uint16_t*)a.dq + qoff;
  for (int c = tid; c < RW * (D / 8); c += NT) {
    const int row = c / (D / 8), d0 = (c % (D / 8)) * 8;
    if (q0 + row >= a.seqlen_q) continue;
    const float* src = &red[row * D + d0];
    const u32x4_t w = {pack_bf16x2(src[0], src[1]), pack_bf16x2(src[2], src[3]),
                       pack_bf16x2(src[4], src[5]), pack_bf16x2(src[6], src[7])};
    st16(dqbase + (size_t)(q0 + row) * q_rs + d0, w);
  }
}

// One grid, both roles. Workgroups are handed to the 8 XCDs round-robin by
// index, so the index is split as (slot, xcd) and each XCD gets the items of
// its own share of the KV heads (and of their query heads): the K/V and
// Q/dO tiles an XCD keeps re-reading stay in its L2. Within an XCD the two
// roles alternate, each list heaviest first (key-major: key block 0 first;
// query-major: the last query block first); the longer list finishes.
template <int D>
__global__ void __launch_bounds__(NT, 2) bwd_main_kernel(BwdParams a, int n_kv, int n_q) {
  constexpr int TILE = 64 * D;
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];
  __shared__ Shared sh;
  const int BG = a.batch * a.heads_kv, BH = a.batch * a.heads_q;
  const int nx = (BG % 8 == 0) ? 8 : 1;  // XCD split only when the heads divide evenly
  const int xcd = blockIdx.x % nx, slot = blockIdx.x / nx;
  const int g_per = BG / nx, h_per = BH / nx;      // heads owned per XCD
  const int n1 = n_kv / nx, n2 = n_q / nx;         // items per XCD
  const int both = 2 * min(n1, n2);
  int role, r;
  if (slot < both) {
    role = slot & 1;
    r = slot >> 1;
  } else {
    role = n1 > n2 ? 0 : 1;
    r = min(n1, n2) + (slot - both);
  }
  if (role == 0)
    dkdv_item<D>(a, smem, sh, r / g_per, xcd * g_per + r % g_per);
  else
    dq_item<D>(a, smem, sh, (a.seqlen_q + 127) / 128 - 1 - r / h_per, xcd * h_per + r % h_per);
}

}  // namespace

hipError_t launch_bwd(const mala_problem& p, const BwdParams& a, hipStream_t s, bool* supported) {
  *supported = p.dtype == MALA_BF16 && p.block_q == BQ && p.block_k == BK &&
               (p.head_dim == 64 || p.head_dim == 128);
  if (!*supported) return hipSuccess;
  const int D = (int)p.head_dim;
  const long long rows = (long long)a.batch * a.seqlen_q * a.heads_q;
  hipLaunchKernelGGL(bwd_absmax_kernel, dim3(kBwdMaxParts), dim3(256), 0, s, (const uint16_t*)a.dout, rows * D,
                     a.absmax);
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)std::min<long long>((rows + 15) / 16, PREP_NB)), dim3(256), 0,
                     s, a, D);
  const int n_kv = a.batch * a.heads_kv * a.nkb;
  const int n_q = a.batch * a.heads_q * (int)((a.seqlen_q + 127) / 128);  // 128-row dQ items
  const dim3 grid((unsigned)(n_kv + n_q));
  if (D == 64)
    hipLaunchKernelGGL(bwd_main_kernel<64>, grid, dim3(NT), 0, s, a, n_kv, n_q);
  else
    hipLaunchKernelGGL(bwd_main_kernel<128>, grid, dim3(NT), 0, s, a, n_kv, n_q);
  return hipGetLastError();
}

}  // namespace mala
