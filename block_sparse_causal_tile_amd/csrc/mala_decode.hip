// MALA decode with split-KV for gfx950 (MALA page, split-KV paragraph and
// "Fused decoding execution": the forward rule with a short query against a
// longer KV sequence).
//
// decode_split: one workgroup per (batch, KV head, split), W = B_k / 64
//   waves, wave w owning keys 64 w .. 64 w + 63 of every tile of the split.
//   The G query heads of the KV group (GQA: K and V are read once for the
//   whole group), times the N_q tokens of a short query, are the columns of
//   the matrix-core ops (G N_q <= 16), so the whole group is scored at once.
//   Token t of N_q sits at position N_k - N_q + t and sees the keys up to
//   it; the N_q rows of a head form one query block (one decision per
//   tile, each row with its own running state and L = position + 1, which
//   is L_0 = N_k for a single token). The split walks its key tiles from
//   the most recent one down; per tile
//     1. S^T = K_tile q^T on 16x16x32 MFMAs, K rows loaded from HBM straight
//        into MFMA operand registers (the next tile's rows are requested
//        before this tile is scored, so they stream in during its work);
//     2. each row's tile maximum: lane reduction, then across the waves
//        through LDS, together with the waves' P sums of the previous tile,
//        so every wave holds the same (m, l) of every row;
//     3. the per-row test against the split's partial normalizer:
//        rowmax - (m + log l) >= log tau - log L (l = 0 counts as +inf),
//        taken by the rows with a key in the tile; a head retains the tile
//        iff one of its rows passes;
//     4. only if some head retains: V_tile is copied HBM -> LDS (each wave
//        its own 64 rows), the retaining heads' state is rescaled, P is
//        formed in the score registers (0 for the other rows, which keep
//        their state bit for bit) and O^T += V^T P^T runs on the matrix
//        cores with V^T read by LDS transpose loads. A tile no head retains
//        never touches V.
//   The waves' partial outputs are summed through LDS at the end and the
//   split writes its normalized partial output and log-normalizer.
// decode_combine: normalizer-aware merge of each row's split partials,
//   z = log sum_s exp(z_s), o = sum_s exp(z_s - z) o_s; a split in which a
//   row has no key (z_s = -inf) drops out of that row's merge.
//
// Paged caches (PAGED = true): K/V rows live in pages of page_size tokens,
// sequence b's key k in page block_table[b][k / page_size] at row
// k % page_size, and every sequence has its own length N_k(b) (so its own
// positions N_k(b) - N_q + t and its own number of tiles T_b, cut into the
// same num_splits ranges). A split whose range is empty (T_b < num_splits)
// has no keys: it writes o_s = 0, z_s = -inf and drops out of the combine;
// so does a row at a negative position (N_k(b) < N_q). Lengths are
// clamped to the table's capacity and page ids to the pool, so malformed
// tables cannot send a load out of bounds.
//
// The workload is bound by HBM bandwidth (K always, V when retained); the
// arithmetic rides on the matrix cores so that the vector ALU does little
// more than the softmax, and several workgroups per CU keep the loads of
// two tiles in flight.
#include <math.h>

#include "mala_common.hpp"

namespace mala {
namespace {

constexpr int DD = 128;       // head_dim
constexpr int WK = 64;        // keys per wave per tile
constexpr int OSTRIDE = 132;  // floats per head row of the final O reduction (padded)

// Row kb * 16 + x of a wave's 64 keys fed to A-row x of score block kb:
// the keys of 32-key step c = kb / 2 are interleaved so that lane l's four
// accumulator registers of blocks 2c and 2c + 1 hold the eight consecutive
// keys 32 c + 8 (l / 16) + 0..7 - the k-slots of the P V MFMA's B operand.
__device__ __forceinline__ int score_key(int kb, int x) {
  return 32 * (kb >> 1) + 8 * (x >> 2) + 4 * (kb & 1) + (x & 3);
}

// A operand of a 16x16x32 MFMA running down a column of a row-major
// DD-wide bf16 tile (tile_idx layout): lane l receives
// T[rowbase + 8 (l / 16) + t][colbase + l % 16], t = 0..7, read with two LDS
// transpose loads (lane y of each 16-lane group addresses row
// rowbase + 8 (l / 16) + y / 4, +4 for the second load, at column
// colbase + 4 (y % 4)).
__device__ __forceinline__ u32x4_t tile_col8_16(const uint16_t* s, int rowbase, int colbase, int lane) {
  const int grp = lane >> 4, y = lane & 15;
  const int row = rowbase + 8 * grp + (y >> 2);
  const int col = colbase + 4 * (y & 3);
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&s[tile_idx<DD>(row, col)]));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&s[tile_idx<DD>(row + 4, col)]));
  const u32x2_t a = __builtin_bit_cast(u32x2_t, lo), b = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}

template <int BK, bool PAGED>
__global__ void __launch_bounds__(BK) __attribute__((amdgpu_waves_per_eu(2)))
decode_split_kernel(DecodeParams a, int G) {
  constexpr int W = BK / WK;  // waves per workgroup
  __shared__ __attribute__((aligned(1024))) uint16_t sV[W][WK * DD];
  // exchange slots of the heads' tile maxima and the waves' P sums, by tile
  // parity: a wave writes tile t's slots only after the barrier of tile
  // t + 1, which every wave passes after reading tile t + 2's (same parity)
  __shared__ float sMax[2][W][16];
  __shared__ float sSum[2][W][16];
  __shared__ float sFin[2][16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, x = lane & 15;  // lane group; column (head, token)
  const int s = blockIdx.x % a.num_splits;
  const int bg = blockIdx.x / a.num_splits;
  const int g = bg % a.heads_kv;
  const int b = bg / a.heads_kv;
  const int nq = a.nq;
  // column x = head gl of the group, token tq of the short query
  const bool col_ok = x < G * nq;
  const int gl = col_ok ? x / nq : 0, tq = col_ok ? x % nq : 0;

  int n_k = a.seqlen_k;
  if (PAGED) n_k = min(max(a.seq_lens[b], 0), a.max_pages * a.page_size);
  const int n_tiles = PAGED ? (n_k + BK - 1) / BK : a.num_tiles;
  const int lo = (int)(((long long)s * n_tiles) / a.num_splits);
  const int hi = (int)(((long long)(s + 1) * n_tiles) / a.num_splits);
  // this column's token position (keys up to it are visible) and
  // log tau - log L, L = position + 1 (L_0 = N_k for a single token)
  const int pos = n_k - nq + tq;
  const float thr = a.log_tau - __logf((float)max(pos + 1, 1));

  const size_t kv_rs = (size_t)a.heads_kv * DD;
  const size_t seq_off = PAGED ? 0 : (size_t)b * a.seqlen_k * kv_rs;
  const uint16_t* const kbase = (const uint16_t*)a.k + seq_off + (size_t)g * DD;
  const uint16_t* const vbase = (const uint16_t*)a.v + seq_off + (size_t)g * DD;
  const int* const table = PAGED ? a.block_table + (size_t)b * a.max_pages : nullptr;
  const int seq_pages = PAGED ? (n_k + a.page_size - 1) / a.page_size : 0;

  // Element offset of key k's row, k clamped to the last key of the
  // sequence (a wave whose 64 keys straddle the end reads that row for the
  // keys past it: finite data the mask sets aside). Paged: pid holds the
  // page ids of the wave's 64 keys (at most four pages; a 64-key window
  // never straddles a page boundary it does not contain).
  auto row_off = [&](int k, const int* pid) -> size_t {
    k = min(k, n_k - 1);
    if (!PAGED) return (size_t)k * kv_rs;
    const int pi = (k & (WK - 1)) / a.page_size;  // page of k within the wave's window
    const int id = pi == 0 ? pid[0] : pi == 1 ? pid[1] : pi == 2 ? pid[2] : pid[3];
    return ((size_t)id * a.page_size + (k & (a.page_size - 1))) * kv_rs;
  };
  // Paged: request the page ids of tile t's window for this wave (lanes
  // 0..3; taken with readlane a step later, so the table read overlaps a
  // whole tile of work).
  auto request_pages = [&](int t) -> int {
    int id = 0;
    if (PAGED && t >= lo) {
      const int pi = (t * BK + WK * w) / a.page_size + lane;
      if (lane < 4 && lane * a.page_size < WK && pi < seq_pages)
        id = (int)min(max((long long)table[pi], 0ll), a.num_pages - 1);
    }
    return id;
  };
  auto take_pages = [&](int id, int* pid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) pid[i] = PAGED ? __builtin_amdgcn_readlane(id, i) : 0;
  };

  // q^T as the B operand of the score MFMAs: column x = (head g G + gl,
  // token tq), the k-slots of step ks are dims 32 (l / 16) + 8 ks + 0..7
  // (the K rows are read with the same dim order, so each lane reads 64
  // contiguous bytes).
  u32x4_t qf[4];
  {
    const uint16_t* qr =
        (const uint16_t*)a.q + (((size_t)b * nq + tq) * a.heads_q + g * G + gl) * DD + 32 * g16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = col_ok ? ld16(qr + 8 * ks) : zero16();
  }

  f32x4_t acc[DD / 16];  // O^T[dim 16 db + 4 g16 + r][column x] over this wave's keys
#pragma unroll
  for (int db = 0; db < DD / 16; ++db) acc[db] = f32x4_t{};
  // softmax state of column x (the same in every wave); l_part: this wave's
  // P sum of the last retained tile, added to l at the next exchange
  float m_run = -INFINITY, l_run = 0.f, l_part = 0.f;
  unsigned long long n_ret = 0, n_vload = 0;

  // K rows of tile t for this wave, as score MFMA A operands
  auto load_k = [&](int t, const int* pid, u32x4_t* kf) {
    const int k0 = t * BK + WK * w;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint16_t* row = kbase + row_off(k0 + score_key(kb, x), pid) + 32 * g16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[4 * kb + ks] = ld16(row + 8 * ks);
    }
  };
  // V rows of tile t for this wave, HBM -> LDS in the tile_idx layout:
  // instruction n fills rows 4 n .. 4 n + 3 (1 KB); lane p fetches the
  // 16-byte unit the swizzle places at physical slot p
  auto copy_v = [&](int t, const int* pid, uint16_t* dst) {
    const int k0 = t * BK + WK * w;
    const int pr = lane >> 4, pu = lane & 15;
#pragma unroll
    for (int n = 0; n < WK / 4; ++n) {
      const int row = 4 * n + pr;
      const int lu = pu ^ tile_swz<DD>(row);
      lds_dma16(vbase + row_off(k0 + row, pid) + lu * 8, lds_address(dst + n * 512));
    }
  };

  int pid_cur[4] = {0, 0, 0, 0}, pid_nxt[4] = {0, 0, 0, 0};  // page ids of tiles t and t - 1
  int id_req = request_pages(hi - 1);

  // one tile: K rows of t in kf (requested one step ago); once the score
  // MFMAs have taken them, kf receives tile t - 1's rows
  u32x4_t kf[16];
  auto step = [&](int t) {
    const int k0 = t * BK + WK * w;
    wait_vmcnt<0>();  // K rows of t (and the page ids of t - 1) landed
    // ---- S^T for this wave's 64 keys x the group's heads -------------------------
    f32x4_t sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[kb] = f32x4_t{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sc[kb] = mfma16(kf[4 * kb + ks], qf[ks], sc[kb]);
#pragma unroll
    for (int i = 0; i < 4; ++i) pid_cur[i] = pid_nxt[i];
    if (t - 1 >= lo) {
      take_pages(id_req, pid_nxt);
      load_k(t - 1, pid_nxt, kf);
      id_req = request_pages(t - 2);
    }
    if (k0 + WK > n_k - nq + 1) {  // keys past a column's position (or past N_k) score -inf
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (k0 + 32 * (kb >> 1) + 8 * g16 + 4 * (kb & 1) + r > pos) sc[kb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = wave_max_halves(row_pair_max(mx));
    // ---- the rows' tile maxima, and the previous tile's P sums, over the waves ----
    if (W > 1) {
      const int par = t & 1;
      if (lane < 16) {
        sMax[par][w][lane] = mx;
        sSum[par][w][lane] = l_part;
      }
      __syncthreads();
      float tm = sMax[par][0][x], ls = sSum[par][0][x];
#pragma unroll
      for (int v = 1; v < W; ++v) {
        tm = fmaxf(tm, sMax[par][v][x]);
        ls += sSum[par][v][x];
      }
      mx = tm;
      l_run += ls;
    } else {
      l_run += l_part;
    }
    l_part = 0.f;
    // ---- per-row test against this split's partial normalizer; a head's rows
    // form one block, which retains the tile iff one of its rows passes -----------
    const bool legal = col_ok && t * BK <= pos;  // the row has a key in the tile
    const float margin = l_run > 0.f ? mx - m_run - test_log(l_run) - thr : INFINITY;
    const unsigned retmask = (unsigned)(__ballot(legal && margin >= 0.f) & 0xffffull);  // lanes 0..15
    const bool ret = col_ok && ((retmask >> (gl * nq)) & ((1u << nq) - 1u)) != 0u;
    const bool upd = ret && legal;  // rows of a retaining head with a key in the tile
    if (a.tile_mask && w == 0 && col_ok && tq == 0)
      a.tile_mask[((size_t)b * a.heads_q + g * G + gl) * a.num_tiles + t] = ret ? 1 : 0;
    if (w == 0) {
      n_ret += __builtin_popcount((unsigned)(__ballot(ret && tq == 0) & 0xffffull));
      n_vload += retmask != 0u ? 1 : 0;
    }
    if (retmask == 0u) return;  // no head retains the tile: V is not touched
    // ---- retained by some head: V_tile, softmax update, O^T += V^T P^T ------------
    const bool has_keys = k0 < n_k;  // wave-uniform: the wave's window holds keys
    if (has_keys) copy_v(t, pid_cur, &sV[w][0]);
    const float m_new = upd ? fmaxf(m_run, mx) : m_run;
    const float alpha = upd ? __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e) : 1.f;
#pragma unroll
    for (int db = 0; db < DD / 16; ++db) acc[db] *= alpha;
    l_run *= alpha;
    m_run = m_new;
    // P in the score registers; a row that does not update gets P = 0, so
    // its column of the accumulator and its l stay as they are
    const float msc = upd ? m_new * kLog2e : INFINITY;
    float ps = 0.f;
    u32x4_t pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float p[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f(fmaf(sc[2 * c][r], kLog2e, -msc));
        p[4 + r] = __builtin_amdgcn_exp2f(fmaf(sc[2 * c + 1][r], kLog2e, -msc));
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) ps += p[r];
      pb[c] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])};
    }
    l_part = wave_sum_halves(row_pair_sum(ps));
    if (has_keys) {
      wait_vmcnt<0>();  // the V rows landed (tile t - 1's K rows, requested earlier, too)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < DD / 16; ++db)
          acc[db] = mfma16(tile_col8_16(&sV[w][0], 32 * c, 16 * db, lane), pb[c], acc[db]);
    }
  };

  if (hi - 1 >= lo) {
    wait_vmcnt<0>();
    take_pages(id_req, pid_nxt);
    load_k(hi - 1, pid_nxt, kf);
    id_req = request_pages(hi - 2);
  }
  for (int t = hi - 1; t >= lo; --t) step(t);

  // ---- the waves' P sums of their last retained tile, and their outputs --------
  // (the partial outputs go through the V tiles: W x 16 columns x OSTRIDE
  // floats fit in W x 16 KB)
  float* sO = reinterpret_cast<float*>(&sV[0][0]);
  __syncthreads();  // every wave is done with its V tile and the exchange slots
  if (lane < 16) sSum[0][w][lane] = l_part;
  if (w == 0 && lane < 16) {
    sFin[0][lane] = m_run;
    sFin[1][lane] = l_run;
  }
#pragma unroll
  for (int db = 0; db < DD / 16; ++db)
    *reinterpret_cast<f32x4_t*>(&sO[(w * 16 + x) * OSTRIDE + 16 * db + 4 * g16]) = acc[db];
  __syncthreads();
  // one thread per (column, 8-dim slice)
  for (int e = tid; e < G * nq * (DD / 8); e += W * 64) {
    const int c = e / (DD / 8), d0 = 8 * (e % (DD / 8));
    float l = sFin[1][c];
#pragma unroll
    for (int v = 0; v < W; ++v) l += sSum[0][v][c];
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < W; ++v)
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] += sO[(v * 16 + c) * OSTRIDE + d0 + i];
    // a row without keys in this split leaves l = 0: o_s = 0, z_s = -inf
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t pi = (((size_t)b * a.heads_q + g * G + c / nq) * nq + c % nq) * a.num_splits + s;
    *reinterpret_cast<f32x4_t*>(a.part_o + pi * DD + d0) = f32x4_t{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    *reinterpret_cast<f32x4_t*>(a.part_o + pi * DD + d0 + 4) =
        f32x4_t{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
    if (d0 == 0) a.part_z[pi] = l > 0.f ? sFin[0][c] + __logf(l) : -INFINITY;
  }
  if (tid == 0 && a.stats) {
    // every tile of the range is legal for a head's block (its last row sees
    // all N_k keys); post-score slots count the block's rows with a position
    const unsigned long long rows = (unsigned long long)max(min(nq, n_k), 0);
    atomicAdd(&a.stats[0], (unsigned long long)(hi - lo) * G);
    atomicAdd(&a.stats[1], n_ret);
    atomicAdd(&a.stats[2], n_ret * BK * rows);
    atomicAdd(&a.stats[3], n_vload);
  }
}

// One wavefront per (batch, query head, token); lane covers DV / 64
// consecutive dims. Row r = (b H_q + h) N_q + t: the partials and z are
// [B, H_q, N_q, ...], o is [B, N_q, H_q, DV].
template <int DV>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeParams a) {
  constexpr int PER = DV / 64;
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= (long long)a.batch * a.heads_q * a.nq) return;
  const float* pz = a.part_z + r * a.num_splits;
  const long long bh = r / a.nq, t = r % a.nq;
  const long long orow_i = ((bh / a.heads_q) * a.nq + t) * a.heads_q + bh % a.heads_q;
  uint32_t* orow = reinterpret_cast<uint32_t*>(a.o) + orow_i * (DV / 2) + lane * (PER / 2);
  float zmax = -INFINITY;
  for (int s = 0; s < a.num_splits; ++s) zmax = fmaxf(zmax, pz[s]);
  if (zmax == -INFINITY) {  // no keys at all (an empty paged sequence, a row before the first key)
#pragma unroll
    for (int t = 0; t < PER / 2; ++t) orow[t] = 0u;
    if (lane == 0) a.z[r] = -INFINITY;
    return;
  }
  float wsum = 0.f, acc[PER];
#pragma unroll
  for (int x = 0; x < PER; ++x) acc[x] = 0.f;
  for (int s = 0; s < a.num_splits; ++s) {
    const float w = __builtin_amdgcn_exp2f((pz[s] - zmax) * kLog2e);
    const float* po = a.part_o + (r * a.num_splits + s) * DV + PER * lane;
    wsum += w;
#pragma unroll
    for (int x = 0; x < PER; ++x) acc[x] = fmaf(w, po[x], acc[x]);
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int t = 0; t < PER / 2; ++t) orow[t] = pack_bf16x2(acc[2 * t] * inv, acc[2 * t + 1] * inv);
  if (lane == 0) a.z[r] = zmax + __logf(wsum);
}

template <bool PAGED>
hipError_t run_decode(const mala_problem& p, const DecodeParams& a, hipStream_t s, bool* supported) {
  *supported = false;
  if (p.dtype != MALA_BF16 || p.head_dim != DD) return hipSuccess;
  const int G = (int)(p.heads_q / p.heads_kv);
  if (G < 1 || G * a.nq > 16) return hipSuccess;  // the (head, token) columns of one MFMA
  const dim3 grid((unsigned)((long long)a.batch * a.heads_kv * a.num_splits));
  if (p.block_k == 64)
    hipLaunchKernelGGL((decode_split_kernel<64, PAGED>), grid, dim3(64), 0, s, a, G);
  else if (p.block_k == 128)
    hipLaunchKernelGGL((decode_split_kernel<128, PAGED>), grid, dim3(128), 0, s, a, G);
  else if (p.block_k == 256)
    hipLaunchKernelGGL((decode_split_kernel<256, PAGED>), grid, dim3(256), 0, s, a, G);
  else
    return hipSuccess;
  *supported = true;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(a, DD, s);
}

}  // namespace

hipError_t launch_decode_combine(const DecodeParams& a, int d_v, hipStream_t s) {
  const long long rows = (long long)a.batch * a.heads_q * a.nq;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (d_v == DD)
    hipLaunchKernelGGL(decode_combine_kernel<DD>, grid, dim3(256), 0, s, a);
  else if (d_v == 512)
    hipLaunchKernelGGL(decode_combine_kernel<512>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode(const mala_problem& p, const DecodeParams& a, hipStream_t s,
                         bool* supported) {
  return a.block_table ? run_decode<true>(p, a, s, supported) : run_decode<false>(p, a, s, supported);
}

}  // namespace mala
