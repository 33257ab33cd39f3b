// Internal launcher interface between the C ABI (mala_api.hip) and the
// kernel files. Arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mala.h"

namespace mala {

// Kernel arguments shared by the prefill forward kernels.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* z;
  unsigned long long* stats;  // may be null
  uint8_t* tile_mask;         // may be null
  int batch, heads_q, heads_kv;
  int seqlen_q, seqlen_k;
  int offset;    // causal offset
  float log_tau; // log(tau), -inf for tau == 0
  int nqb, nkb;  // number of query / key blocks (of the longest sequence when packed)
  // packed sequences (null for the BSHD layout): q/o rows [cu_q[b], cu_q[b+1])
  // and k/v rows [cu_k[b], cu_k[b+1]) belong to sequence b; seqlen_q/k are
  // then the longest lengths, z is [heads_q, total_q]
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
};

// Workgroups (and partial maxima) of the backward's |dO| maximum.
constexpr int kBwdMaxParts = 1024;

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* z;
  void* dq;
  void* dk;
  void* dv;
  float* delta;     // [B, Hq, Nq] workspace: D_q = sum_d dO * O
  float* rowst;     // [B, Hq, 3, rp] workspace: -z_q log2(e), the test offset and D_q per row
  int rp;           // rows of each rowst array: N_q rounded up to a multiple of 128
  uint16_t* do16;   // [B, Nq, Hq, d] workspace: dO 2^s_o as fp16 (the key-major role's dO)
  unsigned* absmax; // [kBwdMaxParts] workspace: partial maxima of |dO| (bf16 bits)
  int* do_scale;    // [1] workspace: s_o
  unsigned long long* stats;
  uint8_t* tile_mask;     // decisions of the key-major pass (may be null)
  uint8_t* tile_mask_dq;  // decisions of the query-major dQ pass (may be null)
  int batch, heads_q, heads_kv;
  int seqlen_q, seqlen_k;
  int offset;
  float log_tau;
  int nqb, nkb;
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* z;
  float* part_o;  // [B, Hq, N_q, S, d] split partial outputs (normalized)
  float* part_z;  // [B, Hq, N_q, S] split partial log-normalizers
  unsigned long long* stats;
  uint8_t* tile_mask;
  int batch, heads_q, heads_kv;
  int seqlen_k;
  int num_splits;
  int num_tiles;   // tiles of the longest sequence (tile_mask row length)
  int nq;          // query tokens per sequence (the newest N_q positions)
  float log_tau;
  // paged caches (k, v are [num_pages, page_size, heads_kv, head_dim])
  const int* block_table;  // [batch, max_pages] page ids
  const int* seq_lens;     // [batch] keys per sequence (L_0 of the sequence)
  int page_size;           // power of two >= 16
  int max_pages;
  long long num_pages;
};

hipError_t launch_fwd(const mala_problem& p, const FwdParams& a, hipStream_t s, bool* supported);
hipError_t launch_fwd_latent(const mala_problem& p, const FwdParams& a, int d_v, hipStream_t s,
                             bool* supported);
hipError_t launch_bwd(const mala_problem& p, const BwdParams& a, hipStream_t s, bool* supported);
// Latent backward: a.k is the cached rows, a.dk the output dKV; `part` holds
// (H_q / latent_bwd_heads_per_item(p)) fp32 partials of dKV.
int latent_bwd_heads_per_item(const mala_problem& p);
hipError_t launch_bwd_latent(const mala_problem& p, const BwdParams& a, int d_v, float* part, hipStream_t s,
                             bool* supported);
hipError_t launch_decode(const mala_problem& p, const DecodeParams& a, hipStream_t s,
                         bool* supported);
// LSE merge of the split partials (part_o rows of d_v floats) into o (bf16) and z.
hipError_t launch_decode_combine(const DecodeParams& a, int d_v, hipStream_t s);
hipError_t launch_decode_latent(const mala_problem& p, const DecodeParams& a, int d_v, hipStream_t s,
                                bool* supported);
hipError_t launch_omitted_mass(const float* zs, const float* zr, float* out, long long n, hipStream_t s);
hipError_t launch_sq_err_heads(const void* x, const void* ref, long long batch, long long seq, int heads,
                               int dim, int dtype, double* sq_diff, double* sq_ref, hipStream_t s);
hipError_t launch_slot_hist(const uint8_t* mask, long long blocks, int nqb, int nkb, int block_q,
                            long long seqlen_q, unsigned long long* hist, hipStream_t s);
hipError_t launch_rademacher(void* out, long long n, int dtype, uint64_t seed, hipStream_t s);

}  // namespace mala
