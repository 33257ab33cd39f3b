// MALA backward kernels for gfx950 (MALA page, "Offline Sparse Probability"
// and "Fused backward execution").
//
//  bwd_prep:     D_q = sum_d dO_qd O_qd (fp32) and zeroing of the fp32 dQ
//                accumulator - one 16-lane group per (batch, row, head).
//  bwd_main:     key-major. One workgroup owns a key block J_j of one KV
//                head and keeps K_j, V_j and its dK_j, dV_j accumulators on
//                chip; for each query head of the group and each query block
//                I_i from the diagonal upward it recomputes S = Q_i K_j^T,
//                tests every legal entry against the saved normalizer
//                (retain iff some S_qk - z_q >= log tau - log L_q) and, only
//                for a retained tile, loads dO_i and runs P = exp(S - z),
//                dP = dO V^T, dS = P (dP - D), dV += P^T dO, dK += dS^T Q and
//                dQ += dS K (fp32 atomics into the workspace accumulator).
//  bwd_finalize: fp32 dQ accumulator -> bf16 dQ.
//
// Tiles are 64 x 64. Four waves split a tile 2 x 2 (32 keys x 32 rows
// each); each wave keeps partial dK/dV for its 32 keys, and the two waves
// sharing keys are summed once at the end of the work item.
#include <math.h>

#include "mala_common.hpp"

namespace mala {
namespace {

constexpr int BQ = 64;
constexpr int BK = 64;
constexpr int NT = 256;

// Row fed to A-row x of a 32-row MFMA block: bits 2 and 3 swapped, so that
// accumulator registers 8a..8a+7 of lane half hh hold the consecutive rows
// 16a + 8hh + 0..7 (the k-slot order of a following MFMA that contracts over
// those rows).
__device__ __forceinline__ int row_perm(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}
__device__ __forceinline__ int r_swz(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int t_swz(int d) { return (d & 7) ^ ((d >> 3) & 7); }

// Row-major [64][D] bf16 tile, 16-byte units XOR-swizzled by row.
template <int D>
__device__ __forceinline__ int rm_idx(int row, int unit) {
  return row * D + ((unit ^ r_swz(row)) * 8);
}
// Transposed [D][64] bf16 tile (64 = rows or keys), 16-byte units swizzled by d.
__device__ __forceinline__ int tr_idx(int d, int unit) { return d * 64 + ((unit ^ t_swz(d)) * 8); }

// Four rows x eight dims of a BSHD tensor (rows r0..r0+3, dims d0..d0+7)
// loaded as 4 x 16 bytes; rows outside [0, n) read as zero.
__device__ __forceinline__ void load_group(u32x4_t w[4], const uint16_t* base, size_t rs, int r0,
                                           int n, int d0) {
#pragma unroll
  for (int x = 0; x < 4; ++x)
    w[x] = (r0 + x < n) ? ld16(base + (size_t)(r0 + x) * rs + d0) : zero16();
}

template <int D>
__device__ __forceinline__ void store_group_rm(uint16_t* s, const u32x4_t w[4], int r0, int d0) {
#pragma unroll
  for (int x = 0; x < 4; ++x) st16(&s[rm_idx<D>(r0 + x, d0 / 8)], w[x]);
}

// Same group written transposed: element (row, d) goes to [d][row].
__device__ __forceinline__ void store_group_tr(uint16_t* s, const u32x4_t w[4], int r0, int d0) {
  const int unit = r0 >> 3, half = r0 & 7;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int d = d0 + 2 * p;
    u32x2_t lo = {__byte_perm(w[0][p], w[1][p], 0x5410), __byte_perm(w[2][p], w[3][p], 0x5410)};
    u32x2_t hi = {__byte_perm(w[0][p], w[1][p], 0x7632), __byte_perm(w[2][p], w[3][p], 0x7632)};
    *reinterpret_cast<u32x2_t*>(&s[tr_idx(d, unit) + half]) = lo;
    *reinterpret_cast<u32x2_t*>(&s[tr_idx(d + 1, unit) + half]) = hi;
  }
}

__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams a, int D) {
  // 16 lanes per (b, row, head); each lane covers 8 consecutive dims (D = 128)
  // or the first 8 lanes do (D = 64).
  const long long rows = (long long)a.batch * a.seqlen_q * a.heads_q;
  const long long r = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (r >= rows) return;
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
    f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4_t*>(a.dq_accum + off) = zero;
    *reinterpret_cast<f32x4_t*>(a.dq_accum + off + 4) = zero;
  }
  acc += __shfl_xor(acc, 8);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 1);
  if (sub == 0) a.delta[((size_t)b * a.heads_q + h) * a.seqlen_q + q] = acc;
}

__global__ void __launch_bounds__(256) bwd_finalize_kernel(BwdParams a, long long n8) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  const f32x4_t x = *reinterpret_cast<const f32x4_t*>(a.dq_accum + t * 8);
  const f32x4_t y = *reinterpret_cast<const f32x4_t*>(a.dq_accum + t * 8 + 4);
  u32x4_t w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]),
               pack_bf16x2(y[2], y[3])};
  st16((uint16_t*)a.dq + t * 8, w);
}

template <int D>
__global__ void __launch_bounds__(NT) bwd_main_kernel(BwdParams a) {
  constexpr int KSTEPS = D / 16;        // MFMA steps over head_dim
  constexpr int EB = D / 32;            // 32-dim blocks
  constexpr int GROUPS = 64 * D / 32;   // 4 x 8 groups per 64 x D tile
  constexpr int TILE = 64 * D;          // bf16 elements per 64 x D tile
  constexpr int DS_STRIDE = BK + 8;     // padded row of the dS tile
  constexpr int EBW = EB / 2;           // dQ d-blocks per wave

  // one LDS block, carved explicitly so the end-of-item reduction can reuse it
  __shared__ __attribute__((aligned(16))) uint16_t smem[5 * TILE + BQ * DS_STRIDE];
  uint16_t* const sQ = smem;
  uint16_t* const sQt = smem + TILE;
  uint16_t* const sdO = smem + 2 * TILE;
  uint16_t* const sdOt = smem + 3 * TILE;
  uint16_t* const sKt = smem + 4 * TILE;
  uint16_t* const sdS = smem + 5 * TILE;
  __shared__ float sZ[BQ];
  __shared__ float sZT[BQ];
  __shared__ float sDel[BQ];
  __shared__ int sVote[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int wk = wave & 1;   // key half of the tile owned by this wave
  const int wr = wave >> 1;  // row half of the tile owned by this wave

  // Heaviest work first: key block 0 is seen by every query block.
  const int BG = a.batch * a.heads_kv;
  const int j = (int)(blockIdx.x / BG);
  const int bg = blockIdx.x % BG;
  const int b = bg / a.heads_kv;
  const int g = bg % a.heads_kv;
  const int group = a.heads_q / a.heads_kv;
  const int k0 = j * BK;
  const int i0 = max(0, k0 - a.offset) / BQ;

  const size_t q_rs = (size_t)a.heads_q * D;
  const size_t kv_rs = (size_t)a.heads_kv * D;
  const uint16_t* kbase = (const uint16_t*)a.k + ((size_t)b * a.seqlen_k * a.heads_kv + g) * D;
  const uint16_t* vbase = (const uint16_t*)a.v + ((size_t)b * a.seqlen_k * a.heads_kv + g) * D;

  // K_j and V_j fragments (B operands: lane = key, 8 dims per step).
  const int mykey = k0 + 32 * wk + l32;
  u32x4_t kf[KSTEPS], vf[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const bool ok = mykey < a.seqlen_k;
    kf[kk] = ok ? ld16(kbase + (size_t)mykey * kv_rs + 16 * kk + 8 * hh) : zero16();
    vf[kk] = ok ? ld16(vbase + (size_t)mykey * kv_rs + 16 * kk + 8 * hh) : zero16();
  }
  // K_j transposed into LDS for the dQ contraction.
  for (int gi = tid; gi < GROUPS; gi += NT) {
    const int d0 = 8 * (gi % (D / 8)), r0 = 4 * (gi / (D / 8));
    u32x4_t w[4];
    load_group(w, kbase, kv_rs, k0 + r0, a.seqlen_k, d0);
    store_group_tr(sKt, w, r0, d0);
  }

  f32x16_t dv_acc[EB], dk_acc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    dv_acc[e] = f32x16_t{};
    dk_acc[e] = f32x16_t{};
  }
  unsigned long long n_legal = 0, n_ret = 0, n_slots = 0;

  for (int hq = g * group; hq < (g + 1) * group; ++hq) {
    const uint16_t* qbase = (const uint16_t*)a.q + ((size_t)b * a.seqlen_q * a.heads_q + hq) * D;
    const uint16_t* dobase =
        (const uint16_t*)a.dout + ((size_t)b * a.seqlen_q * a.heads_q + hq) * D;
    const float* zrow = a.z + ((size_t)b * a.heads_q + hq) * a.seqlen_q;
    const float* delrow = a.delta + ((size_t)b * a.heads_q + hq) * a.seqlen_q;
    for (int i = i0; i < a.nqb; ++i) {
      const int q0 = i * BQ;
      // a ragged last query block may end before the key block starts
      if (k0 > min(q0 + BQ, a.seqlen_q) - 1 + a.offset) continue;
      __syncthreads();  // previous tile's LDS readers are done
      // ---- Q_i (row-major), z and the test offset z + thr per row -------------
      u32x4_t qg[4];
      const bool has_group = tid < GROUPS;
      const int gd0 = 8 * (tid % (D / 8)), gr0 = 4 * (tid / (D / 8));
      if (has_group) {
        load_group(qg, qbase, q_rs, q0 + gr0, a.seqlen_q, gd0);
        store_group_rm<D>(sQ, qg, gr0, gd0);
      }
      if (tid < BQ) {
        const int q = q0 + tid;
        const bool ok = q < a.seqlen_q;
        const float z = ok ? zrow[q] : INFINITY;
        const float thr = a.log_tau - __logf((float)(q + a.offset + 1));
        sZ[tid] = z;
        sZT[tid] = ok ? z + thr : INFINITY;
      }
      __syncthreads();

      // ---- score discovery S = Q_i K_j^T on this wave's 32 x 32 sub-tile ----
      f32x16_t s = f32x16_t{};
      {
        const int qr = 32 * wr + row_perm(l32);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const u32x4_t af = *reinterpret_cast<const u32x4_t*>(&sQ[rm_idx<D>(qr, 2 * kk + hh)]);
          s = mfma32(af, kf[kk], s);
        }
      }
      // legal entries: key <= row + offset and row < N_q (row index of
      // register r: 32 wr + row_perm(acc_row(r, hh)))
      const bool diag = k0 + BK - 1 > q0 + a.offset || q0 + BQ > a.seqlen_q;
      bool vote = false;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = 32 * wr + row_perm(acc_row(r, hh));
        const bool legal = !diag || (mykey <= q0 + lr + a.offset && q0 + lr < a.seqlen_q);
        if (!legal) s[r] = -INFINITY;
        vote |= (s[r] - sZT[lr]) >= 0.f;
      }
      const bool wave_vote = __ballot(vote) != 0ull;
      if (lane == 0) sVote[wave] = wave_vote ? 1 : 0;
      __syncthreads();
      const bool retain = (sVote[0] | sVote[1] | sVote[2] | sVote[3]) != 0;
      ++n_legal;
      if (tid == 0 && a.tile_mask)
        a.tile_mask[(((size_t)b * a.heads_q + hq) * a.nqb + i) * a.nkb + j] = retain ? 1 : 0;
      if (!retain) continue;
      ++n_ret;
      n_slots += (unsigned long long)BK * min(BQ, a.seqlen_q - q0);

      // ---- retained: dO_i (both layouts), Q_i^T and D_i ------------------------
      if (has_group) {
        store_group_tr(sQt, qg, gr0, gd0);
        u32x4_t og[4];
        load_group(og, dobase, q_rs, q0 + gr0, a.seqlen_q, gd0);
        store_group_rm<D>(sdO, og, gr0, gd0);
        store_group_tr(sdOt, og, gr0, gd0);
      }
      if (tid < BQ) {
        const int q = q0 + tid;
        sDel[tid] = q < a.seqlen_q ? delrow[q] : 0.f;
      }
      __syncthreads();

      // dP = dO_i V_j^T (same sub-tile and layout as S)
      f32x16_t dp = f32x16_t{};
      {
        const int qr = 32 * wr + row_perm(l32);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const u32x4_t af = *reinterpret_cast<const u32x4_t*>(&sdO[rm_idx<D>(qr, 2 * kk + hh)]);
          dp = mfma32(af, vf[kk], dp);
        }
      }
      // P = exp(S - z), dS = P (dP - D); packed as A operands over rows
      u32x4_t pa[2], dsa[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float p[8], ds[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int r = 8 * hb + t;
          const int lr = 32 * wr + row_perm(acc_row(r, hh));
          p[t] = __builtin_amdgcn_exp2f((s[r] - sZ[lr]) * kLog2e);
          ds[t] = p[t] * (dp[r] - sDel[lr]);
        }
        pa[hb] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                         pack_bf16x2(p[6], p[7])};
        dsa[hb] = u32x4_t{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]),
                          pack_bf16x2(ds[4], ds[5]), pack_bf16x2(ds[6], ds[7])};
        // dS (bf16) into LDS, row-major [row][key], for the dQ contraction
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int lr = 32 * wr + 16 * hb + 8 * hh + t;
          const uint32_t w = (t & 1) ? (dsa[hb][t >> 1] >> 16) : (dsa[hb][t >> 1] & 0xffffu);
          sdS[lr * DS_STRIDE + 32 * wk + l32] = (uint16_t)w;
        }
      }
      // dV_j += P^T dO_i and dK_j += dS^T Q_i over this wave's 32 rows
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int unit = 4 * wr + 2 * hb + hh;
#pragma unroll
        for (int e = 0; e < EB; ++e) {
          const int d = 32 * e + l32;
          const u32x4_t bo = *reinterpret_cast<const u32x4_t*>(&sdOt[tr_idx(d, unit)]);
          const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(&sQt[tr_idx(d, unit)]);
          dv_acc[e] = mfma32(pa[hb], bo, dv_acc[e]);
          dk_acc[e] = mfma32(dsa[hb], bq, dk_acc[e]);
        }
      }
      __syncthreads();  // dS tile complete
      // dQ_i += dS K_j: wave covers rows 32 wr.., d-blocks EBW * wk ..
      {
        f32x16_t dq[EBW];
#pragma unroll
        for (int e = 0; e < EBW; ++e) dq[e] = f32x16_t{};
        const int qr = 32 * wr + l32;
#pragma unroll
        for (int c = 0; c < BK / 16; ++c) {
          const u32x4_t af = *reinterpret_cast<const u32x4_t*>(&sdS[qr * DS_STRIDE + 16 * c + 8 * hh]);
#pragma unroll
          for (int e = 0; e < EBW; ++e) {
            const int d = 32 * (EBW * wk + e) + l32;
            const u32x4_t bk = *reinterpret_cast<const u32x4_t*>(&sKt[tr_idx(d, 2 * c + hh)]);
            dq[e] = mfma32(af, bk, dq[e]);
          }
        }
        // dQ^T layout: lane holds column d of 16 rows
#pragma unroll
        for (int e = 0; e < EBW; ++e) {
          const int d = 32 * (EBW * wk + e) + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = q0 + 32 * wr + acc_row(r, hh);
            if (q < a.seqlen_q)
              atomicAdd(&a.dq_accum[(((size_t)b * a.seqlen_q + q) * a.heads_q + hq) * D + d], dq[e][r]);
          }
        }
      }
    }
  }

  // ---- sum the two row halves of dK_j / dV_j and store -----------------------
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // the tiles are dead now
  static_assert(5 * TILE * 2 >= 2 * 2 * 32 * D * 4, "reduction buffer");
  // layout: [wk][dk|dv][e][r][lane]
  if (wr == 1) {
#pragma unroll
    for (int e = 0; e < EB; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[(((wk * 2 + 0) * EB + e) * 16 + r) * 64 + lane] = dk_acc[e][r];
        red[(((wk * 2 + 1) * EB + e) * 16 + r) * 64 + lane] = dv_acc[e][r];
      }
  }
  __syncthreads();
  if (wr == 0) {
    uint16_t* dkbase = (uint16_t*)a.dk + ((size_t)b * a.seqlen_k * a.heads_kv + g) * D;
    uint16_t* dvbase = (uint16_t*)a.dv + ((size_t)b * a.seqlen_k * a.heads_kv + g) * D;
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      const int d = 32 * e + l32;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        // accumulator rows are keys 32 wk + acc_row(r, hh); column d
        const float k0v = dk_acc[e][r] + red[(((wk * 2 + 0) * EB + e) * 16 + r) * 64 + lane];
        const float k1v = dk_acc[e][r + 1] + red[(((wk * 2 + 0) * EB + e) * 16 + r + 1) * 64 + lane];
        const float v0v = dv_acc[e][r] + red[(((wk * 2 + 1) * EB + e) * 16 + r) * 64 + lane];
        const float v1v = dv_acc[e][r + 1] + red[(((wk * 2 + 1) * EB + e) * 16 + r + 1) * 64 + lane];
        const int key0 = k0 + 32 * wk + acc_row(r, hh);
        const uint32_t kw = pack_bf16x2(k0v, k1v), vw = pack_bf16x2(v0v, v1v);
        if (key0 < a.seqlen_k) {
          dkbase[(size_t)key0 * kv_rs + d] = (uint16_t)(kw & 0xffffu);
          dvbase[(size_t)key0 * kv_rs + d] = (uint16_t)(vw & 0xffffu);
        }
        if (key0 + 1 < a.seqlen_k) {
          dkbase[(size_t)(key0 + 1) * kv_rs + d] = (uint16_t)(kw >> 16);
          dvbase[(size_t)(key0 + 1) * kv_rs + d] = (uint16_t)(vw >> 16);
        }
      }
    }
  }
  if (tid == 0 && a.stats) {
    atomicAdd(&a.stats[0], n_legal);
    atomicAdd(&a.stats[1], n_ret);
    atomicAdd(&a.stats[2], n_slots);
    atomicAdd(&a.stats[3], n_ret);
  }
}

}  // namespace

hipError_t launch_bwd(const mala_problem& p, const BwdParams& a, hipStream_t s, bool* supported) {
  *supported = p.dtype == MALA_BF16 && p.block_q == BQ && p.block_k == BK &&
               (p.head_dim == 64 || p.head_dim == 128);
  if (!*supported) return hipSuccess;
  const int D = (int)p.head_dim;
  const long long rows = (long long)a.batch * a.seqlen_q * a.heads_q;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, a, D);
  const dim3 grid((unsigned)(a.batch * a.heads_kv * a.nkb));
  if (D == 64)
    hipLaunchKernelGGL(bwd_main_kernel<64>, grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_main_kernel<128>, grid, dim3(NT), 0, s, a);
  const long long n8 = rows * D / 8;
  hipLaunchKernelGGL(bwd_finalize_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, a, n8);
  return hipGetLastError();
}

}  // namespace mala
