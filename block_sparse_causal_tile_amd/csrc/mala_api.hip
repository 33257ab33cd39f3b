// C ABI of the MALA library: synchronous argument validation, workspace
// carving, then asynchronous launches on the caller's stream. Nothing is
// allocated; the only global state is the per-device scratch address of
// mala_decode_noalloc.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "mala_internal.hpp"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxRow = int64_t(1) << 24;  // elements of one sequence position (heads x head_dim)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Checks shared by every entry point.
int check_common(const mala_problem* p) {
  if (!p) return MALA_EINVAL;
  if (p->batch <= 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->seqlen_q <= 0 ||
      p->seqlen_k <= 0 || p->head_dim <= 0 || p->block_q <= 0 || p->block_k <= 0)
    return MALA_EINVAL;
  if (p->batch > kMaxDim || p->heads_q > kMaxDim || p->seqlen_q > kMaxDim ||
      p->seqlen_k > kMaxDim)
    return MALA_EINVAL;
  // a tile's per-lane copy offsets (up to 128 rows) are 32-bit byte offsets
  if ((int64_t)p->heads_q * p->head_dim > kMaxRow) return MALA_EINVAL;
  if (p->heads_q % p->heads_kv != 0) return MALA_EINVAL;
  if (!(p->tau >= 0.f) || !isfinite(p->tau)) return MALA_EINVAL;  // rejects NaN too
  if (p->causal_offset < 0 || p->causal_offset > p->seqlen_k - p->seqlen_q) return MALA_EINVAL;
  if (p->dtype != MALA_BF16 && p->dtype != MALA_FP32) return MALA_EUNSUPPORTED;
  return MALA_OK;
}

float log_tau(float tau) { return tau == 0.f ? -INFINITY : logf(tau); }

bool ptrs_ok(std::initializer_list<const void*> ps) {
  for (const void* x : ps)
    if (!x || !aligned16(x)) return false;
  return true;
}

int grid_ok(int64_t blocks) { return blocks > 0 && blocks < (int64_t(1) << 31); }

// A decode problem's query rows: 1 <= N_q <= min(16, N_k), the newest N_q
// positions of the cache (causal offset N_k - N_q).
bool decode_rows_ok(const mala_problem* p) {
  return p->seqlen_q >= 1 && p->seqlen_q <= 16 && p->seqlen_q <= p->seqlen_k &&
         p->causal_offset == p->seqlen_k - p->seqlen_q;
}

// Validation and launch of the split-KV decode, shared by mala_decode (the
// caller's workspace) and mala_decode_noalloc (the library's scratch).
int decode_impl(const mala_problem* p, const void* q, const void* k_cache, const void* v_cache, void* o,
                float* z, int num_splits, void* workspace, size_t ws_bytes, int64_t* stats, uint8_t* tile_mask,
                void* stream);

// ---------------------------------------------------------------------------
// Scratch of mala_decode_noalloc: the split partials live in this file-scope
// device array instead of a caller workspace. Each GPU the library runs on
// holds its own copy until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MALA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first
// call on that device), or MALA_EHIP.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MALA_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MALA_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MALA_OK;
}

}  // namespace

extern "C" {

int mala_fwd(const mala_problem* p, const void* q, const void* k, const void* v, void* o,
             float* z, int64_t* stats, uint8_t* tile_mask, void* stream) {
  int st = check_common(p);
  if (st != MALA_OK) return st;
  if (!ptrs_ok({q, k, v, o, z})) return MALA_EINVAL;
  const int64_t nqb = ceil_div(p->seqlen_q, p->block_q);
  const int64_t nkb = ceil_div(p->seqlen_k, p->block_k);
  if (!grid_ok(p->batch * p->heads_q * nqb)) return MALA_EINVAL;
  mala::FwdParams a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.z = z;
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  a.tile_mask = tile_mask;
  a.batch = (int)p->batch;
  a.heads_q = (int)p->heads_q;
  a.heads_kv = (int)p->heads_kv;
  a.seqlen_q = (int)p->seqlen_q;
  a.seqlen_k = (int)p->seqlen_k;
  a.offset = (int)p->causal_offset;
  a.log_tau = log_tau(p->tau);
  a.nqb = (int)nqb;
  a.nkb = (int)nkb;
  bool supported = false;
  hipError_t e = mala::launch_fwd(*p, a, reinterpret_cast<hipStream_t>(stream), &supported);
  if (!supported) return MALA_EUNSUPPORTED;
  return e == hipSuccess ? MALA_OK : MALA_EHIP;
}

int mala_fwd_latent(const mala_problem* p, const void* q, const void* kv, int64_t d_v, void* o,
                    float* z, int64_t* stats, uint8_t* tile_mask, void* stream) {
  int st = check_common(p);
  if (st != MALA_OK) return st;
  if (p->heads_kv != 1) return MALA_EINVAL;  // one cached row per position
  if (d_v <= 0 || d_v > p->head_dim || d_v % 8 != 0) return MALA_EINVAL;
  if (!ptrs_ok({q, kv, o, z})) return MALA_EINVAL;
  const int64_t nqb = ceil_div(p->seqlen_q, p->block_q);
  const int64_t nkb = ceil_div(p->seqlen_k, p->block_k);
  if (!grid_ok(ceil_div(p->batch * nqb, 8) * 8 * p->heads_q)) return MALA_EINVAL;
  mala::FwdParams a{};
  a.q = q;
  a.k = kv;
  a.v = kv;
  a.o = o;
  a.z = z;
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  a.tile_mask = tile_mask;
  a.batch = (int)p->batch;
  a.heads_q = (int)p->heads_q;
  a.heads_kv = 1;
  a.seqlen_q = (int)p->seqlen_q;
  a.seqlen_k = (int)p->seqlen_k;
  a.offset = (int)p->causal_offset;
  a.log_tau = log_tau(p->tau);
  a.nqb = (int)nqb;
  a.nkb = (int)nkb;
  bool supported = false;
  hipError_t e = mala::launch_fwd_latent(*p, a, (int)d_v, reinterpret_cast<hipStream_t>(stream), &supported);
  if (!supported) return MALA_EUNSUPPORTED;
  return e == hipSuccess ? MALA_OK : MALA_EHIP;
}

int mala_fwd_varlen(const mala_problem* p, const void* q, const void* k, const void* v,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t total_q,
                    int64_t total_k, void* o, float* z, int64_t* stats, uint8_t* tile_mask, void* stream) {
  if (!p) return MALA_EINVAL;
  if (p->batch <= 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->seqlen_q <= 0 || p->seqlen_k <= 0 ||
      p->head_dim <= 0 || p->block_q <= 0 || p->block_k <= 0)
    return MALA_EINVAL;
  if (p->batch > kMaxDim || p->heads_q > kMaxDim || p->seqlen_q > kMaxDim || p->seqlen_k > kMaxDim)
    return MALA_EINVAL;
  if ((int64_t)p->heads_q * p->head_dim > kMaxRow) return MALA_EINVAL;
  if (p->heads_q % p->heads_kv != 0) return MALA_EINVAL;
  if (!(p->tau >= 0.f) || !isfinite(p->tau)) return MALA_EINVAL;
  if (p->causal_offset != 0) return MALA_EINVAL;  // the offset is per sequence: N_k(b) - N_q(b)
  if (total_q <= 0 || total_k <= 0 || total_q > kMaxDim || total_k > kMaxDim) return MALA_EINVAL;
  if (p->dtype != MALA_BF16) return MALA_EUNSUPPORTED;
  if (!ptrs_ok({q, k, v, o, z})) return MALA_EINVAL;
  if (!cu_seqlens_q || !cu_seqlens_k || (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return MALA_EINVAL;
  const int64_t nqb = ceil_div(p->seqlen_q, p->block_q);
  const int64_t nkb = ceil_div(p->seqlen_k, p->block_k);
  if (!grid_ok(p->batch * p->heads_q * nqb)) return MALA_EINVAL;
  mala::FwdParams a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.z = z;
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  a.tile_mask = tile_mask;
  a.batch = (int)p->batch;
  a.heads_q = (int)p->heads_q;
  a.heads_kv = (int)p->heads_kv;
  a.seqlen_q = (int)p->seqlen_q;
  a.seqlen_k = (int)p->seqlen_k;
  a.offset = 0;
  a.log_tau = log_tau(p->tau);
  a.nqb = (int)nqb;
  a.nkb = (int)nkb;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = (int)total_q;
  a.total_k = (int)total_k;
  bool supported = false;
  hipError_t e = mala::launch_fwd(*p, a, reinterpret_cast<hipStream_t>(stream), &supported);
  if (!supported) return MALA_EUNSUPPORTED;
  return e == hipSuccess ? MALA_OK : MALA_EHIP;
}

namespace {
// mala_bwd's workspace, in this order, each part 256-byte aligned: three
// fp32 values per query row (-z log2 e, the test offset, D_q; per (b, h)
// three arrays of rp rows, rp = N_q rounded up to a multiple of 128, the
// rows past N_q holding the values of a row that is never retained), the
// partial maxima of |dO|, the scale exponent s_o, and the fp16 copy dO 2^s_o
// (the layout of dO).
struct BwdWorkspace {
  size_t rowst, absmax, scale, do16, total;
  size_t rp;
  explicit BwdWorkspace(const mala_problem& p) {
    const size_t rows = (size_t)p.batch * p.heads_q * p.seqlen_q;
    rp = round_up((size_t)p.seqlen_q, 128);
    rowst = 0;
    absmax = round_up((size_t)p.batch * p.heads_q * 3 * rp * sizeof(float), 256);
    scale = absmax + round_up(mala::kBwdMaxParts * sizeof(unsigned), 256);
    do16 = scale + 256;
    total = do16 + round_up(rows * (size_t)p.head_dim * 2, 256);
  }
};
}  // namespace

size_t mala_bwd_workspace_size(const mala_problem* p) {
  if (check_common(p) != MALA_OK) return 0;
  return BwdWorkspace(*p).total;
}

int mala_bwd(const mala_problem* p, const void* q, const void* k, const void* v, const void* o,
             const void* dout, const float* z, void* dq, void* dk, void* dv, void* workspace,
             size_t ws_bytes, int64_t* stats, uint8_t* tile_mask, uint8_t* tile_mask_dq, void* stream) {
  int st = check_common(p);
  if (st != MALA_OK) return st;
  if (!ptrs_ok({q, k, v, o, dout, z, dq, dk, dv})) return MALA_EINVAL;
  const size_t need = mala_bwd_workspace_size(p);
  if (!workspace || !aligned16(workspace) || ws_bytes < need) return MALA_EWORKSPACE;
  const int64_t nqb = ceil_div(p->seqlen_q, p->block_q);
  const int64_t nkb = ceil_div(p->seqlen_k, p->block_k);
  if (!grid_ok(p->batch * p->heads_kv * nkb) || !grid_ok(p->batch * p->heads_q * nqb))
    return MALA_EINVAL;
  mala::BwdParams a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.z = z;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const BwdWorkspace wl(*p);
  char* const w = reinterpret_cast<char*>(workspace);
  a.rowst = reinterpret_cast<float*>(w + wl.rowst);
  a.rp = (int)wl.rp;
  a.absmax = reinterpret_cast<unsigned*>(w + wl.absmax);
  a.do_scale = reinterpret_cast<int*>(w + wl.scale);
  a.do16 = reinterpret_cast<uint16_t*>(w + wl.do16);
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  a.tile_mask = tile_mask;
  a.tile_mask_dq = tile_mask_dq;
  a.batch = (int)p->batch;
  a.heads_q = (int)p->heads_q;
  a.heads_kv = (int)p->heads_kv;
  a.seqlen_q = (int)p->seqlen_q;
  a.seqlen_k = (int)p->seqlen_k;
  a.offset = (int)p->causal_offset;
  a.log_tau = log_tau(p->tau);
  a.nqb = (int)nqb;
  a.nkb = (int)nkb;
  bool supported = false;
  hipError_t e = mala::launch_bwd(*p, a, reinterpret_cast<hipStream_t>(stream), &supported);
  if (!supported) return MALA_EUNSUPPORTED;
  return e == hipSuccess ? MALA_OK : MALA_EHIP;
}

size_t mala_bwd_latent_workspace_size(const mala_problem* p) {
  if (check_common(p) != MALA_OK || p->heads_kv != 1) return 0;
  const size_t rows = (size_t)p->batch * p->heads_q * p->seqlen_q;
  const size_t n_hg = (size_t)(p->heads_q / mala::latent_bwd_heads_per_item(*p));
  return round_up(rows * sizeof(float), 256) +
         round_up(n_hg * (size_t)p->batch * p->seqlen_k * p->head_dim * sizeof(float), 256);
}

int mala_bwd_latent(const mala_problem* p, const void* q, const void* kv, int64_t d_v, const void* o,
                    const void* dout, const float* z, void* dq, void* dkv, void* workspace, size_t ws_bytes,
                    int64_t* stats, uint8_t* tile_mask, uint8_t* tile_mask_dq, void* stream) {
  int st = check_common(p);
  if (st != MALA_OK) return st;
  if (p->heads_kv != 1) return MALA_EINVAL;  // one cached row per position
  if (d_v <= 0 || d_v > p->head_dim || d_v % 8 != 0) return MALA_EINVAL;
  if (!ptrs_ok({q, kv, o, dout, z, dq, dkv})) return MALA_EINVAL;
  const size_t need = mala_bwd_latent_workspace_size(p);
  if (!workspace || !aligned16(workspace) || ws_bytes < need) return MALA_EWORKSPACE;
  const int64_t nqb = ceil_div(p->seqlen_q, p->block_q);
  const int64_t nkb = ceil_div(p->seqlen_k, p->block_k);
  if (!grid_ok(ceil_div(p->batch * nqb, 8) * 8 * p->heads_q) || !grid_ok(nkb * p->batch * p->heads_q))
    return MALA_EINVAL;
  mala::BwdParams a{};
  a.q = q;
  a.k = kv;
  a.v = kv;
  a.o = o;
  a.dout = dout;
  a.z = z;
  a.dq = dq;
  a.dk = dkv;
  a.dv = dkv;
  a.delta = reinterpret_cast<float*>(workspace);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                         round_up((size_t)p->batch * p->heads_q * p->seqlen_q * sizeof(float), 256));
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  a.tile_mask = tile_mask;
  a.tile_mask_dq = tile_mask_dq;
  a.batch = (int)p->batch;
  a.heads_q = (int)p->heads_q;
  a.heads_kv = 1;
  a.seqlen_q = (int)p->seqlen_q;
  a.seqlen_k = (int)p->seqlen_k;
  a.offset = (int)p->causal_offset;
  a.log_tau = log_tau(p->tau);
  a.nqb = (int)nqb;
  a.nkb = (int)nkb;
  bool supported = false;
  hipError_t e = mala::launch_bwd_latent(*p, a, (int)d_v, part, reinterpret_cast<hipStream_t>(stream),
                                         &supported);
  if (!supported) return MALA_EUNSUPPORTED;
  return e == hipSuccess ? MALA_OK : MALA_EHIP;
}

size_t mala_decode_workspace_size(const mala_problem* p, int num_splits) {
  if (check_common(p) != MALA_OK || num_splits <= 0) return 0;
  const size_t parts = (size_t)p->batch * p->heads_q * p->seqlen_q * num_splits;
  return round_up(parts * p->head_dim * sizeof(float), 256) + round_up(parts * sizeof(float), 256);
}

}  // extern "C"

namespace {

int decode_impl(const mala_problem* p, const void* q, const void* k_cache, const void* v_cache, void* o,
                float* z, int num_splits, void* workspace, size_t ws_bytes, int64_t* stats, uint8_t* tile_mask,
                void* stream) {
  int st = check_common(p);
  if (st != MALA_OK) return st;
  if (!ptrs_ok({q, k_cache, v_cache, o, z})) return MALA_EINVAL;
  if (!decode_rows_ok(p)) return MALA_EINVAL;
  const int64_t T = ceil_div(p->seqlen_k, p->block_k);
  if (num_splits < 1 || num_splits > T) return MALA_EINVAL;
  const size_t need = mala_decode_workspace_size(p, num_splits);
  if (!workspace || !aligned16(workspace) || ws_bytes < need) return MALA_EWORKSPACE;
  if (!grid_ok(p->batch * p->heads_kv * num_splits)) return MALA_EINVAL;
  const size_t parts = (size_t)p->batch * p->heads_q * p->seqlen_q * num_splits;
  mala::DecodeParams a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = o;
  a.z = z;
  a.part_o = reinterpret_cast<float*>(workspace);
  a.part_z = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                      round_up(parts * p->head_dim * sizeof(float), 256));
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  a.tile_mask = tile_mask;
  a.batch = (int)p->batch;
  a.heads_q = (int)p->heads_q;
  a.heads_kv = (int)p->heads_kv;
  a.seqlen_k = (int)p->seqlen_k;
  a.num_splits = num_splits;
  a.num_tiles = (int)T;
  a.nq = (int)p->seqlen_q;
  a.log_tau = log_tau(p->tau);
  bool supported = false;
  hipError_t e = mala::launch_decode(*p, a, reinterpret_cast<hipStream_t>(stream), &supported);
  if (!supported) return MALA_EUNSUPPORTED;
  return e == hipSuccess ? MALA_OK : MALA_EHIP;
}

}  // namespace

extern "C" {

int mala_decode(const mala_problem* p, const void* q, const void* k_cache, const void* v_cache,
                void* o, float* z, int num_splits, void* workspace, size_t ws_bytes,
                int64_t* stats, uint8_t* tile_mask, void* stream) {
  return decode_impl(p, q, k_cache, v_cache, o, z, num_splits, workspace, ws_bytes, stats, tile_mask, stream);
}

int mala_decode_noalloc(const mala_problem* p, const void* q, const void* k_cache, const void* v_cache, void* o,
                        float* z, int num_splits, int64_t* stats, uint8_t* tile_mask, void* stream) {
  // the checks mala_decode makes before it looks at the workspace, so an
  // invalid problem reports MALA_EINVAL rather than a size error
  int st = check_common(p);
  if (st != MALA_OK) return st;
  if (!decode_rows_ok(p)) return MALA_EINVAL;
  const int64_t T = ceil_div(p->seqlen_k, p->block_k);
  if (num_splits < 1 || num_splits > T) return MALA_EINVAL;
  if (mala_decode_workspace_size(p, num_splits) > MALA_NOALLOC_SCRATCH_BYTES) return MALA_ETOOLARGE;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != MALA_OK) return st;
  return decode_impl(p, q, k_cache, v_cache, o, z, num_splits, ws, MALA_NOALLOC_SCRATCH_BYTES, stats, tile_mask,
                     stream);
}

int mala_decode_latent(const mala_problem* p, const void* q, const void* kv_cache, int64_t d_v,
                       void* o, float* z, int num_splits, void* workspace, size_t ws_bytes,
                       int64_t* stats, uint8_t* tile_mask, void* stream) {
  int st = check_common(p);
  if (st != MALA_OK) return st;
  if (p->heads_kv != 1) return MALA_EINVAL;  // one cached row per position
  if (d_v <= 0 || d_v > p->head_dim || d_v % 8 != 0) return MALA_EINVAL;
  if (!ptrs_ok({q, kv_cache, o, z})) return MALA_EINVAL;
  if (p->seqlen_q != 1 || p->causal_offset != p->seqlen_k - 1) return MALA_EINVAL;
  const int64_t T = ceil_div(p->seqlen_k, p->block_k);
  if (num_splits < 1 || num_splits > T) return MALA_EINVAL;
  const size_t need = mala_decode_workspace_size(p, num_splits);
  if (!workspace || !aligned16(workspace) || ws_bytes < need) return MALA_EWORKSPACE;
  if (!grid_ok(ceil_div(p->batch * num_splits, 8) * 8 * ceil_div(p->heads_q, 16))) return MALA_EINVAL;
  const size_t parts = (size_t)p->batch * p->heads_q * num_splits;
  mala::DecodeParams a{};
  a.q = q;
  a.k = kv_cache;
  a.v = kv_cache;
  a.o = o;
  a.z = z;
  a.part_o = reinterpret_cast<float*>(workspace);  // rows of d_v floats
  a.part_z = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                      round_up(parts * p->head_dim * sizeof(float), 256));
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  a.tile_mask = tile_mask;
  a.batch = (int)p->batch;
  a.heads_q = (int)p->heads_q;
  a.heads_kv = 1;
  a.seqlen_k = (int)p->seqlen_k;
  a.num_splits = num_splits;
  a.num_tiles = (int)T;
  a.nq = 1;
  a.log_tau = log_tau(p->tau);
  bool supported = false;
  hipError_t e =
      mala::launch_decode_latent(*p, a, (int)d_v, reinterpret_cast<hipStream_t>(stream), &supported);
  if (!supported) return MALA_EUNSUPPORTED;
  return e == hipSuccess ? MALA_OK : MALA_EHIP;
}

int mala_decode_paged(const mala_problem* p, const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* seq_lens, int64_t num_pages,
                      int32_t page_size, int32_t max_pages_per_seq, void* o, float* z, int num_splits,
                      void* workspace, size_t ws_bytes, int64_t* stats, uint8_t* tile_mask, void* stream) {
  int st = check_common(p);
  if (st != MALA_OK) return st;
  if (!ptrs_ok({q, k_pages, v_pages, o, z})) return MALA_EINVAL;
  if (!block_table || !seq_lens || (reinterpret_cast<uintptr_t>(block_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return MALA_EINVAL;
  if (page_size < 16 || page_size > 4096 || (page_size & (page_size - 1))) return MALA_EINVAL;
  if (max_pages_per_seq <= 0 || num_pages <= 0 || num_pages > kMaxDim) return MALA_EINVAL;
  if ((int64_t)max_pages_per_seq * page_size > kMaxDim) return MALA_EINVAL;
  if (p->seqlen_k != (int64_t)max_pages_per_seq * page_size || !decode_rows_ok(p)) return MALA_EINVAL;
  const int64_t T = ceil_div(p->seqlen_k, p->block_k);
  if (num_splits < 1 || num_splits > T) return MALA_EINVAL;
  const size_t need = mala_decode_workspace_size(p, num_splits);
  if (!workspace || !aligned16(workspace) || ws_bytes < need) return MALA_EWORKSPACE;
  if (!grid_ok(p->batch * p->heads_kv * num_splits)) return MALA_EINVAL;
  const size_t parts = (size_t)p->batch * p->heads_q * p->seqlen_q * num_splits;
  mala::DecodeParams a{};
  a.q = q;
  a.k = k_pages;
  a.v = v_pages;
  a.o = o;
  a.z = z;
  a.part_o = reinterpret_cast<float*>(workspace);
  a.part_z = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                      round_up(parts * p->head_dim * sizeof(float), 256));
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  a.tile_mask = tile_mask;
  a.batch = (int)p->batch;
  a.heads_q = (int)p->heads_q;
  a.heads_kv = (int)p->heads_kv;
  a.seqlen_k = (int)p->seqlen_k;
  a.num_splits = num_splits;
  a.num_tiles = (int)T;
  a.nq = (int)p->seqlen_q;
  a.log_tau = log_tau(p->tau);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.page_size = page_size;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  bool supported = false;
  hipError_t e = mala::launch_decode(*p, a, reinterpret_cast<hipStream_t>(stream), &supported);
  if (!supported) return MALA_EUNSUPPORTED;
  return e == hipSuccess ? MALA_OK : MALA_EHIP;
}

int mala_omitted_mass(const float* z_screened, const float* z_reference, float* omitted, int64_t n,
                      void* stream) {
  if (n <= 0 || n > (int64_t(1) << 40)) return MALA_EINVAL;
  if (!ptrs_ok({z_screened, z_reference, omitted})) return MALA_EINVAL;
  if (!grid_ok(ceil_div(n, 256))) return MALA_EINVAL;
  return mala::launch_omitted_mass(z_screened, z_reference, omitted, n,
                                   reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MALA_OK
             : MALA_EHIP;
}

int mala_sq_err_heads(const void* x, const void* ref, int64_t batch, int64_t seqlen, int64_t heads,
                      int64_t head_dim, int32_t dtype, double* sq_diff, double* sq_ref, void* stream) {
  if (batch <= 0 || seqlen <= 0 || heads <= 0 || head_dim <= 0) return MALA_EINVAL;
  if (batch > kMaxDim || seqlen > kMaxDim || heads > kMaxDim || head_dim > kMaxDim) return MALA_EINVAL;
  if (dtype != MALA_BF16 && dtype != MALA_FP32) return MALA_EUNSUPPORTED;
  if (!ptrs_ok({x, ref, sq_diff, sq_ref})) return MALA_EINVAL;
  if (!grid_ok(batch * heads)) return MALA_EINVAL;
  return mala::launch_sq_err_heads(x, ref, batch, seqlen, (int)heads, (int)head_dim, dtype, sq_diff,
                                   sq_ref, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MALA_OK
             : MALA_EHIP;
}

int mala_slot_histogram(const mala_problem* p, const uint8_t* tile_mask, int64_t* hist, void* stream) {
  int st = check_common(p);
  if (st != MALA_OK) return st;
  if (!ptrs_ok({tile_mask, hist})) return MALA_EINVAL;
  const int64_t nqb = ceil_div(p->seqlen_q, p->block_q), nkb = ceil_div(p->seqlen_k, p->block_k);
  const int64_t blocks = p->batch * p->heads_q * nqb;
  if (nkb > kMaxDim || !grid_ok(ceil_div(blocks, 256))) return MALA_EINVAL;
  return mala::launch_slot_hist(tile_mask, blocks, (int)nqb, (int)nkb, p->block_q, p->seqlen_q,
                                reinterpret_cast<unsigned long long*>(hist),
                                reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MALA_OK
             : MALA_EHIP;
}

int mala_rademacher(void* out, int64_t n, int32_t dtype, uint64_t seed, void* stream) {
  if (n <= 0 || n > (int64_t(1) << 40)) return MALA_EINVAL;
  if (dtype != MALA_BF16 && dtype != MALA_FP32) return MALA_EUNSUPPORTED;
  if (!ptrs_ok({out})) return MALA_EINVAL;
  if (!grid_ok(ceil_div(n, 256))) return MALA_EINVAL;
  return mala::launch_rademacher(out, n, dtype, seed, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MALA_OK
             : MALA_EHIP;
}

const char* mala_error_string(int status) {
  switch (status) {
    case MALA_OK: return "MALA_OK: success";
    case MALA_EINVAL: return "MALA_EINVAL: invalid argument";
    case MALA_EUNSUPPORTED: return "MALA_EUNSUPPORTED: head_dim/block/dtype combination not compiled";
    case MALA_EWORKSPACE: return "MALA_EWORKSPACE: workspace missing or too small";
    case MALA_EHIP: return "MALA_EHIP: HIP launch or runtime error";
    case MALA_ETOOLARGE:
      return "MALA_ETOOLARGE: the problem needs more scratch than the allocation-free entry point holds";
    default: return "MALA: unknown status";
  }
}

}  // extern "C"
