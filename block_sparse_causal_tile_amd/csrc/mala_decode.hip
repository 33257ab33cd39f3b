// MALA single-token decode with split-KV for gfx950 (MALA page, split-KV
// paragraph and "Fused decoding execution").
//
// decode_split: one wavefront per (batch, KV head, split). The wavefront
//   holds the G query heads of the KV group (GQA: K/V are read once for the
//   whole group) and walks its split's key tiles from the most recent one
//   down. For every tile it
//     1. streams K (16 lanes per key row, 8 dims per lane), forms the G
//        scores of every key with fp32 FMAs and a 16-lane DPP sum, keeps the
//        scores in LDS and each head's running tile maximum;
//     2. tests each head against its own partial normalizer of this split:
//        retain_h <=> rowmax_h - (m_h + log l_h) >= log tau - log L_0 with
//        L_0 = N_k (l_h = 0 counts as +inf);
//     3. only if some head retains: streams V once and applies the online
//        softmax update and P V to the retaining heads; the other heads keep
//        their state. A tile no head retains never touches V.
//   The split writes its normalized partial output and log-normalizer.
// decode_combine: normalizer-aware merge of the split partials,
//   z = log sum_s exp(z_s), o = sum_s exp(z_s - z) o_s.
//
// Paged caches (PAGED = true): K/V rows live in pages of page_size tokens,
// sequence b's key k in page block_table[b][k / page_size] at row
// k % page_size, and every sequence has its own length N_k(b) (so its own
// L_0 = N_k(b) and its own number of tiles T_b, cut into the same num_splits
// ranges). A split whose range is empty (T_b < num_splits) has no keys: it
// writes o_s = 0, z_s = -inf and drops out of the combine. Lengths are
// clamped to the table's capacity and page ids to the pool, so malformed
// tables cannot send a load out of bounds.
//
// The workload is bound by HBM bandwidth (K always, V when retained): the
// kernel is organised around keeping 16-byte loads in flight - K and V rows
// stream through two 32-key register buffers that alternate (one is
// consumed while the other loads) - and around staying small enough in
// registers for several wavefronts per SIMD, rather than around arithmetic.
#include <math.h>

#include "mala_common.hpp"

namespace mala {
namespace {

constexpr int DD = 128;        // head_dim
constexpr int WAVES = 4;       // independent splits per workgroup
constexpr int HALF = 32;       // keys per streamed half-chunk (8 rounds of 4 keys)
constexpr int HROUNDS = HALF / 4;

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same
// bits (each step adds a commutative pair).
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ void unpack8(const u32x4_t w, float f[8]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f[2 * t] = bf16_lo(w[t]);
    f[2 * t + 1] = bf16_hi(w[t]);
  }
}

template <int G, int BK, bool PAGED>
__global__ void __launch_bounds__(WAVES * 64) decode_split_kernel(DecodeParams a) {
  constexpr int NHALF = BK / HALF;  // 32-key half-chunks per tile
  __shared__ float sS[WAVES][G][BK];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int sub = lane & 15;   // 8-dim slice of a key row
  const int grp = lane >> 4;   // which of the 4 keys of a round
  const long long wid = (long long)blockIdx.x * WAVES + wv;
  const long long total = (long long)a.batch * a.heads_kv * a.num_splits;
  if (wid >= total) return;  // whole wavefront exits together
  const int s = (int)(wid % a.num_splits);
  const long long bg = wid / a.num_splits;
  const int g = (int)(bg % a.heads_kv);
  const int b = (int)(bg / a.heads_kv);
  int n_k = a.seqlen_k;
  if (PAGED) n_k = min(max(a.seq_lens[b], 0), a.max_pages * a.page_size);
  const int n_tiles = PAGED ? (n_k + BK - 1) / BK : a.num_tiles;
  const int lo = (int)(((long long)s * n_tiles) / a.num_splits);
  const int hi = (int)(((long long)(s + 1) * n_tiles) / a.num_splits);
  // log tau - log L_0, L_0 = N_k (of this sequence when paged); both layouts
  // take the logarithm here, so equal keys give equal decisions
  const float thr = a.log_tau - __logf((float)max(n_k, 1));

  const size_t kv_rs = (size_t)a.heads_kv * DD;
  const size_t seq_off = PAGED ? 0 : (size_t)b * a.seqlen_k * a.heads_kv * DD;
  const uint16_t* kbase = (const uint16_t*)a.k + seq_off + (size_t)g * DD + 8 * sub;
  const uint16_t* vbase = (const uint16_t*)a.v + seq_off + (size_t)g * DD + 8 * sub;
  const int* table = PAGED ? a.block_table + (size_t)b * a.max_pages : nullptr;
  // Page ids of a tile, fetched one tile ahead: lane i holds the id of the
  // tile's i-th page (a tile spans max(1, BK / page_size) <= 16 pages), so a
  // half-chunk reads its id from a register instead of waiting on memory.
  const int tile_pages = PAGED ? max(1, BK / a.page_size) : 0;
  const int seq_pages = PAGED ? (n_k + a.page_size - 1) / a.page_size : 0;
  auto fetch_pages = [&](int t) -> int {
    int id = 0;
    if (PAGED && t >= 0) {
      const int pi = (t * BK) / a.page_size + lane;
      if (lane < tile_pages && pi < seq_pages)
        id = (int)min(max((long long)table[pi], 0ll), a.num_pages - 1);  // clamped to the pool
    }
    return id;
  };
  int pids_next = fetch_pages(hi - 1), pids = 0;

  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4_t w = ld16((const uint16_t*)a.q + ((size_t)b * a.heads_q + g * G + h) * DD + 8 * sub);
    unpack8(w, qv[h]);
  }
  float acc[G][8];
  float m_run[G], l_run[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[h][x] = 0.f;
  }
  unsigned long long n_ret = 0, n_vload = 0;

  // two half-chunk register buffers: one is consumed while the other loads
  u32x4_t bufA[HROUNDS], bufB[HROUNDS];
  auto load_half = [&](u32x4_t* buf, const uint16_t* base, int key0) {
    if (!PAGED) {
#pragma unroll
      for (int r = 0; r < HROUNDS; ++r) {
        const int key = key0 + 4 * r + grp;
        buf[r] = key < n_k ? ld16(base + (size_t)key * kv_rs) : zero16();
      }
    } else {
      // A 32-key half-chunk (32-aligned) lies in one page, or in two pages of
      // 16 keys: one wave-uniform row pointer per page, then the same per-lane
      // offsets as a contiguous cache (row kk of the half-chunk at kk * kv_rs).
      const int ip = ((key0 % BK) / a.page_size);  // the half-chunk's page within the tile
      const long long p0 = __builtin_amdgcn_readlane(pids, ip);
      const uint16_t* b0 = base + ((size_t)p0 * a.page_size + (key0 & (a.page_size - 1))) * kv_rs;
      const uint16_t* b1 = b0;
      if (a.page_size == 16) {
        const long long p1 = __builtin_amdgcn_readlane(pids, ip + 1);
        b1 = base + ((size_t)p1 * 16 - 16) * kv_rs;  // + kk * kv_rs for kk in [16, 32)
      }
#pragma unroll
      for (int r = 0; r < HROUNDS; ++r) {
        const int kk = 4 * r + grp;  // r >= 4 <=> kk >= 16: the choice is uniform
        const uint16_t* row = (a.page_size == 16 && r >= 4 ? b1 : b0) + (size_t)kk * kv_rs;
        buf[r] = key0 + kk < n_k ? ld16(row) : zero16();
      }
    }
  };

  for (int t = hi - 1; t >= lo; --t) {
    const int tk0 = t * BK;
    if (PAGED) {
      pids = pids_next;
      pids_next = fetch_pages(t - 1 >= lo ? t - 1 : -1);
    }
    // ---- pass 1: scores of every key for the G heads, tile maxima -----------
    float tmax[G];
#pragma unroll
    for (int h = 0; h < G; ++h) tmax[h] = -INFINITY;
    auto score_half = [&](const u32x4_t* buf, int hc) {
#pragma unroll
      for (int r = 0; r < HROUNDS; ++r) {
        const int kl = hc * HALF + 4 * r + grp;  // key within the tile
        float kf[8];
        unpack8(buf[r], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float p = 0.f;
#pragma unroll
          for (int x = 0; x < 8; ++x) p = fmaf(qv[h][x], kf[x], p);
          p = row16_sum(p);
          if (tk0 + kl >= n_k) p = -INFINITY;
          tmax[h] = fmaxf(tmax[h], p);
          if (sub == h) sS[wv][h][kl] = p;
        }
      }
    };
    load_half(bufA, kbase, tk0);
#pragma unroll 1
    for (int hc = 0; hc < NHALF; hc += 2) {
      if (hc + 1 < NHALF) load_half(bufB, kbase, tk0 + (hc + 1) * HALF);
      score_half(bufA, hc);
      if (hc + 2 < NHALF) load_half(bufA, kbase, tk0 + (hc + 2) * HALF);
      if (hc + 1 < NHALF) score_half(bufB, hc + 1);
    }
    // scores written by one lane are read by others below: keep LDS order
    __builtin_amdgcn_wave_barrier();
    // ---- per-head test against this split's partial normalizer ------------
    unsigned retmask = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = fmaxf(tmax[h], __shfl_xor(tmax[h], 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      tmax[h] = mx;
      const float margin = (l_run[h] > 0.f) ? (mx - m_run[h] - __logf(l_run[h]) - thr) : INFINITY;
      if (margin >= 0.f) retmask |= 1u << h;
    }
    if (a.tile_mask && lane < G)
      a.tile_mask[((size_t)b * a.heads_q + g * G + lane) * a.num_tiles + t] = (retmask >> lane) & 1u;
    if (retmask == 0) continue;
    n_ret += __builtin_popcount(retmask);
    ++n_vload;
    // ---- pass 2: retained heads - online softmax update and P V -------------
    load_half(bufA, vbase, tk0);
    float m_new[G], msc[G], lsum[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bool rh = (retmask >> h) & 1u;
      m_new[h] = rh ? fmaxf(m_run[h], tmax[h]) : m_run[h];
      const float alpha = rh ? __builtin_amdgcn_exp2f((m_run[h] - m_new[h]) * kLog2e) : 1.f;
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[h][x] *= alpha;
      l_run[h] *= alpha;
      msc[h] = m_new[h] * kLog2e;
      lsum[h] = 0.f;
    }
    auto pv_half = [&](const u32x4_t* buf, int hc) {
#pragma unroll
      for (int r = 0; r < HROUNDS; ++r) {
        const int kl = hc * HALF + 4 * r + grp;
        float vf[8];
        unpack8(buf[r], vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (!((retmask >> h) & 1u)) continue;
          const float p = __builtin_amdgcn_exp2f(fmaf(sS[wv][h][kl], kLog2e, -msc[h]));
          lsum[h] += p;
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[h][x] = fmaf(p, vf[x], acc[h][x]);
        }
      }
    };
#pragma unroll 1
    for (int hc = 0; hc < NHALF; hc += 2) {
      if (hc + 1 < NHALF) load_half(bufB, vbase, tk0 + (hc + 1) * HALF);
      pv_half(bufA, hc);
      if (hc + 2 < NHALF) load_half(bufA, vbase, tk0 + (hc + 2) * HALF);
      if (hc + 1 < NHALF) pv_half(bufB, hc + 1);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((retmask >> h) & 1u)) continue;
      // lsum is per lane group (4 groups hold different keys)
      float ls = lsum[h] + __shfl_xor(lsum[h], 16);
      ls += __shfl_xor(ls, 32);
      l_run[h] += ls;
      m_run[h] = m_new[h];
    }
  }

  // ---- merge the 4 lane groups' partial outputs; write the split partial ----
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      float v = acc[h][x] + __shfl_xor(acc[h][x], 16);
      acc[h][x] = v + __shfl_xor(v, 32);
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const size_t pi = ((size_t)b * a.heads_q + g * G + h) * a.num_splits + s;
      // a split without keys (empty range) leaves l = 0: o_s = 0, z_s = -inf
      const float inv = l_run[h] > 0.f ? 1.f / l_run[h] : 0.f;
      f32x4_t o0 = {acc[h][0] * inv, acc[h][1] * inv, acc[h][2] * inv, acc[h][3] * inv};
      f32x4_t o1 = {acc[h][4] * inv, acc[h][5] * inv, acc[h][6] * inv, acc[h][7] * inv};
      *reinterpret_cast<f32x4_t*>(a.part_o + pi * DD + 8 * sub) = o0;
      *reinterpret_cast<f32x4_t*>(a.part_o + pi * DD + 8 * sub + 4) = o1;
      if (sub == 0) a.part_z[pi] = l_run[h] > 0.f ? m_run[h] + __logf(l_run[h]) : -INFINITY;
    }
  }
  if (lane == 0 && a.stats) {
    atomicAdd(&a.stats[0], (unsigned long long)(hi - lo) * G);
    atomicAdd(&a.stats[1], n_ret);
    atomicAdd(&a.stats[2], n_ret * BK);
    atomicAdd(&a.stats[3], n_vload);
  }
}

// One wavefront per (batch, query head); lane covers DV / 64 consecutive dims.
template <int DV>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeParams a) {
  constexpr int PER = DV / 64;
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= (long long)a.batch * a.heads_q) return;
  const float* pz = a.part_z + r * a.num_splits;
  uint32_t* orow = reinterpret_cast<uint32_t*>(a.o) + r * (DV / 2) + lane * (PER / 2);
  float zmax = -INFINITY;
  for (int s = 0; s < a.num_splits; ++s) zmax = fmaxf(zmax, pz[s]);
  if (zmax == -INFINITY) {  // no keys at all (an empty paged sequence)
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

template <int G, bool PAGED>
hipError_t run_g(int bk, const DecodeParams& a, hipStream_t st, bool* ok) {
  const long long waves = (long long)a.batch * a.heads_kv * a.num_splits;
  const dim3 grid((unsigned)((waves + WAVES - 1) / WAVES));
  *ok = true;
  if (bk == 64)
    hipLaunchKernelGGL((decode_split_kernel<G, 64, PAGED>), grid, dim3(WAVES * 64), 0, st, a);
  else if (bk == 128)
    hipLaunchKernelGGL((decode_split_kernel<G, 128, PAGED>), grid, dim3(WAVES * 64), 0, st, a);
  else if (bk == 256)
    hipLaunchKernelGGL((decode_split_kernel<G, 256, PAGED>), grid, dim3(WAVES * 64), 0, st, a);
  else
    *ok = false;
  return hipSuccess;
}

template <bool PAGED>
hipError_t run_decode(const mala_problem& p, const DecodeParams& a, hipStream_t s, bool* supported) {
  *supported = false;
  if (p.dtype != MALA_BF16 || p.head_dim != DD) return hipSuccess;
  const int G = (int)(p.heads_q / p.heads_kv);
  hipError_t e = hipSuccess;
  switch (G) {
    case 1: e = run_g<1, PAGED>(p.block_k, a, s, supported); break;
    case 2: e = run_g<2, PAGED>(p.block_k, a, s, supported); break;
    case 4: e = run_g<4, PAGED>(p.block_k, a, s, supported); break;
    case 8: e = run_g<8, PAGED>(p.block_k, a, s, supported); break;
    default: return hipSuccess;
  }
  if (!*supported || e != hipSuccess) return e;
  return launch_decode_combine(a, DD, s);
}

}  // namespace

hipError_t launch_decode_combine(const DecodeParams& a, int d_v, hipStream_t s) {
  const long long rows = (long long)a.batch * a.heads_q;
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
