// Operator-fidelity instrumentation (MALA page, experiments: the omitted-mass
// definition and the operator-fidelity protocol). These kernels sit beside
// the attention path: they compare a screened run with a screening-disabled
// (tau = 0, FullAttn) run of the same operator, histogram the realized
// post-score key slots per query, and draw the deterministic Rademacher
// direction used as the upstream gradient of the backward comparison.
//
//  omitted_mass : 1 - exp(z_screened - z_reference) per query row, written as
//                 -expm1(difference) (the same quantity without cancellation).
//  sq_err_heads : per (batch, head) sums of (x - ref)^2 and ref^2 in fp64;
//                 one workgroup per head, fixed reduction order, so the result
//                 is deterministic.
//  slot_hist    : per query block, the number c of retained tiles in its row
//                 of a tile mask; every valid row of the block adds 1 to bin c
//                 (post-score slots per query = c B_k).
//  rademacher   : x_i = SplitMix64 output i for a seed (the counter-based form
//                 of Steele, Lea and Flood's generator: the state after i + 1
//                 steps is seed + (i + 1) * golden gamma, then the published
//                 mixing function), value -1 if its top bit is set, else +1.
#include <math.h>

#include "mala_common.hpp"

namespace mala {
namespace {

__global__ void __launch_bounds__(256) omitted_mass_kernel(const float* zs, const float* zr, float* out,
                                                           long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = -expm1f(zs[i] - zr[i]);
}

template <typename T>
__device__ __forceinline__ double as_f64(T x);
template <>
__device__ __forceinline__ double as_f64<float>(float x) {
  return (double)x;
}
template <>
__device__ __forceinline__ double as_f64<uint16_t>(uint16_t x) {
  return (double)__uint_as_float((uint32_t)x << 16);
}

// One workgroup per (batch, head); threads stride over the seq x head_dim
// elements of the head, then a fixed-shape tree reduction.
template <typename T>
__global__ void __launch_bounds__(256) sq_err_heads_kernel(const T* x, const T* ref, long long seq,
                                                           int heads, int dim, double* sq_diff,
                                                           double* sq_ref) {
  const int bh = blockIdx.x;
  const int b = bh / heads, h = bh % heads;
  const long long per_head = seq * dim;
  double sd = 0.0, sr = 0.0;
  for (long long e = threadIdx.x; e < per_head; e += 256) {
    const long long row = e / dim;
    const int c = (int)(e % dim);
    const size_t off = (((size_t)b * seq + row) * heads + h) * dim + c;
    const double r = as_f64<T>(ref[off]);
    const double d = as_f64<T>(x[off]) - r;
    sd += d * d;
    sr += r * r;
  }
  __shared__ double s_d[256], s_r[256];
  s_d[threadIdx.x] = sd;
  s_r[threadIdx.x] = sr;
  __syncthreads();
  for (unsigned w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      s_d[threadIdx.x] += s_d[threadIdx.x + w];
      s_r[threadIdx.x] += s_r[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    sq_diff[bh] = s_d[0];
    sq_ref[bh] = s_r[0];
  }
}

__global__ void __launch_bounds__(256) slot_hist_kernel(const uint8_t* mask, long long blocks, int nqb,
                                                        int nkb, int block_q, long long seqlen_q,
                                                        unsigned long long* hist) {
  const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
  if (r >= blocks) return;
  const int i = (int)(r % nqb);
  const uint8_t* row = mask + (size_t)r * nkb;
  int c = 0;
  for (int j = 0; j < nkb; ++j) c += row[j] == 1;
  const long long rows = min((long long)block_q, seqlen_q - (long long)i * block_q);
  atomicAdd(&hist[c], (unsigned long long)rows);
}

__device__ __forceinline__ uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <typename T>
__global__ void __launch_bounds__(256) rademacher_kernel(T* out, long long n, uint64_t seed);
template <>
__global__ void __launch_bounds__(256) rademacher_kernel<float>(float* out, long long n, uint64_t seed) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint64_t x = splitmix64_mix(seed + (uint64_t)(i + 1) * 0x9E3779B97F4A7C15ull);
  out[i] = (x >> 63) ? -1.f : 1.f;
}
template <>
__global__ void __launch_bounds__(256) rademacher_kernel<uint16_t>(uint16_t* out, long long n, uint64_t seed) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint64_t x = splitmix64_mix(seed + (uint64_t)(i + 1) * 0x9E3779B97F4A7C15ull);
  out[i] = (x >> 63) ? (uint16_t)0xBF80u : (uint16_t)0x3F80u;  // bf16 -1 / +1
}

unsigned grid_of(long long n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_omitted_mass(const float* zs, const float* zr, float* out, long long n, hipStream_t s) {
  hipLaunchKernelGGL(omitted_mass_kernel, dim3(grid_of(n)), dim3(256), 0, s, zs, zr, out, n);
  return hipGetLastError();
}

hipError_t launch_sq_err_heads(const void* x, const void* ref, long long batch, long long seq, int heads,
                               int dim, int dtype, double* sq_diff, double* sq_ref, hipStream_t s) {
  const dim3 grid((unsigned)(batch * heads));
  if (dtype == MALA_BF16)
    hipLaunchKernelGGL(sq_err_heads_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)x,
                       (const uint16_t*)ref, seq, heads, dim, sq_diff, sq_ref);
  else
    hipLaunchKernelGGL(sq_err_heads_kernel<float>, grid, dim3(256), 0, s, (const float*)x,
                       (const float*)ref, seq, heads, dim, sq_diff, sq_ref);
  return hipGetLastError();
}

hipError_t launch_slot_hist(const uint8_t* mask, long long blocks, int nqb, int nkb, int block_q,
                            long long seqlen_q, unsigned long long* hist, hipStream_t s) {
  hipLaunchKernelGGL(slot_hist_kernel, dim3(grid_of(blocks)), dim3(256), 0, s, mask, blocks, nqb, nkb,
                     block_q, seqlen_q, hist);
  return hipGetLastError();
}

hipError_t launch_rademacher(void* out, long long n, int dtype, uint64_t seed, hipStream_t s) {
  if (dtype == MALA_BF16)
    hipLaunchKernelGGL(rademacher_kernel<uint16_t>, dim3(grid_of(n)), dim3(256), 0, s, (uint16_t*)out, n,
                       seed);
  else
    hipLaunchKernelGGL(rademacher_kernel<float>, dim3(grid_of(n)), dim3(256), 0, s, (float*)out, n, seed);
  return hipGetLastError();
}

}  // namespace mala
