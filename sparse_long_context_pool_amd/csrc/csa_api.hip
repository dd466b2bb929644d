// csa_api.hip -- the extern "C" boundary of libcsa.so (declared in include/csa.h).
// Validates arguments on the host, picks a kernel and launch geometry, enqueues
// on the caller's stream and reports errors through a thread-local string.
// Never synchronizes, never allocates device memory, never throws.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/csa.h"
#include "csa_device.hpp"

namespace {

thread_local char g_err[512] = "";

csa_status_t fail(csa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

csa_status_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(CSA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return CSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(int32_t dt) { return dt == CSA_F32 || dt == CSA_BF16; }

// the argument checks of one cache update (CSA_OK: valid; nothing to do when
// B * n == 0)
csa_status_t check_cache_append(const char* fn, const void* x, const void* gate,
                                const float* slot_bias, void* ring_x, void* ring_g, void* pool,
                                void* win, const int32_t* count, int32_t B, int32_t n,
                                int32_t D, int32_t m, int32_t overlap, int32_t T_cap, int32_t W,
                                int32_t rope_dim, const float* cs, int32_t n_pos);

// the argument checks of one compressor pass (CSA_OK: valid; nothing to do
// when B * (S / m) == 0)
csa_status_t check_compress(const char* fn, const void* x, const void* gate,
                            const float* slot_bias, void* pool, int32_t B, int32_t S, int32_t D,
                            int32_t m, int32_t overlap, int32_t rope_dim, const float* cs,
                            int32_t n_pos, int32_t pos0);

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Shared checks of csa_sparse_attn / hca_attn.
csa_status_t check_attn(const char* fn, const void* q, const void* kv_win,
                        const int32_t* win_pos0, int32_t L_win, const void* pool, int32_t T,
                        void* out, const int32_t* q_pos, int32_t B, int32_t S, int32_t H,
                        int32_t D, int32_t dv, int32_t rope_dim, const float* cs,
                        int32_t n_pos, int32_t window, float scale, int32_t dtype) {
  if (!dtype_ok(dtype)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (B < 0 || S < 0 || H < 1 || D < 2 || T < 0 || L_win < 0 || window < 0)
    return fail(CSA_ERR_INVALID,
                "%s: bad sizes (B=%d S=%d H=%d D=%d T=%d L_win=%d window=%d)", fn, B, S, H,
                D, T, L_win, window);
  if (rope_dim < 0 || (rope_dim & 1) || rope_dim > D)
    return fail(CSA_ERR_INVALID, "%s: rope_dim=%d must be even and in [0, D=%d]", fn,
                rope_dim, D);
  if (dv != D && dv != D - rope_dim)
    return fail(CSA_ERR_INVALID, "%s: dv=%d must be D=%d or D-rope_dim=%d", fn, dv, D,
                D - rope_dim);
  if (dv < 1) return fail(CSA_ERR_INVALID, "%s: dv must be >= 1", fn);
  if (D % 8 != 0 || dv % 2 != 0)
    return fail(CSA_ERR_INVALID, "%s: D=%d must be a multiple of 8 and dv=%d even", fn, D,
                dv);
  if (D > 1024) return fail(CSA_ERR_UNSUPPORTED, "%s: D=%d > 1024", fn, D);
  if (!(scale > 0.f) || scale != scale)
    return fail(CSA_ERR_INVALID, "%s: scale must be positive", fn);
  if ((long)B * S == 0) return CSA_OK;
  if (!q || !out || !q_pos) return fail(CSA_ERR_INVALID, "%s: q, out, q_pos are required", fn);
  if (!aligned16(q) || !aligned16(out))
    return fail(CSA_ERR_INVALID, "%s: q and out must be 16-byte aligned", fn);
  if (window > 0 && L_win > 0) {
    if (!kv_win)
      return fail(CSA_ERR_INVALID, "%s: kv_win is required when window > 0", fn);
    if (!aligned16(kv_win)) return fail(CSA_ERR_INVALID, "%s: kv_win not 16-byte aligned", fn);
    // win_pos0 NULL: kv_win is a ring (position p at row p mod L_win) that
    // must still hold every window position of every query row
    if (!win_pos0 && L_win < window + S - 1)
      return fail(CSA_ERR_INVALID, "%s: a ring window needs L_win >= window + S - 1 (%d < %d)",
                  fn, L_win, window + S - 1);
  }
  if (T > 0) {
    if (!pool) return fail(CSA_ERR_INVALID, "%s: pool is required when T > 0", fn);
    if (!aligned16(pool)) return fail(CSA_ERR_INVALID, "%s: pool not 16-byte aligned", fn);
  }
  if (rope_dim > 0 && (!cs || n_pos < 1))
    return fail(CSA_ERR_INVALID, "%s: the RoPE table (cs, n_pos) is required", fn);
  return CSA_OK;
}

csa::AttnParams make_params(const void* q, const void* kv_win, const int32_t* win_pos0,
                            int32_t L_win, const void* pool, int32_t T, const int32_t* idx,
                            int32_t k, int32_t m, const float* sink, void* out,
                            const int32_t* q_pos, int32_t B, int32_t S, int32_t H, int32_t D,
                            int32_t dv, int32_t rope_dim, const float* cs, int32_t n_pos,
                            int32_t window, float scale, int32_t dtype) {
  csa::AttnParams p;
  const bool has_win = window > 0 && L_win > 0;
  p.q = q;
  p.kv_win = has_win ? kv_win : nullptr;
  p.win_pos0 = has_win ? win_pos0 : nullptr;
  p.win_ring = has_win && win_pos0 == nullptr;
  p.L_win = has_win ? L_win : 0;
  p.pool = T > 0 ? pool : nullptr;
  p.T = T;
  p.idx = idx;
  p.k = idx ? k : 0;
  p.dense = idx ? 0 : 1;
  p.m = m;
  p.sink = sink;
  p.out = out;
  p.q_pos = q_pos;
  p.B = B; p.S = S; p.H = H; p.D = D; p.dv = dv; p.rope_dim = rope_dim;
  p.cs = rope_dim > 0 ? cs : nullptr;
  p.n_pos = n_pos;
  p.window = has_win ? window : 0;
  p.scale = scale;
  p.bf16 = dtype == CSA_BF16;
  return p;
}

csa_status_t run_attn(const char* fn, const csa::AttnParams& p, int npool_max,
                      void* workspace, size_t ws_bytes, hipStream_t s) {
  csa::AttnPlan plan = csa::plan_attention(p.B, p.S, p.H, p.D, p.dv, p.rope_dim, p.window,
                                           npool_max, p.bf16, std::max<long>(p.L_win, p.T),
                                           p.dense ? 0 : p.k);
  void* ws = nullptr;
  if (plan.nsplit > 1) {
    if (workspace && ws_bytes >= plan.ws_bytes && aligned16(workspace)) ws = workspace;
    else plan.nsplit = 1;
  }
  return launched(csa::launch_attention(p, plan, ws, s), fn);
}

// ---- the workspace of csa_sparse_attn_noalloc: a device array of the library
// (each GPU the library runs on holds its own copy until the process ends).
// Host code never uses the array's name as an address: the device address of
// each GPU's copy comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is passed to kernels.
constexpr size_t kScratchBytes = size_t(24) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

csa_status_t scratch_on_current_device(const char* fn, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(CSA_ERR_LAUNCH, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CSA_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library serves", fn, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(CSA_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s",
                  fn, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CSA_OK;
}

#ifdef CSA_DEBUG
// ---- debug build: the index rows are checked on the device before attention
// runs (the stream is synchronized, so a debug build is not for graph
// capture).  The two result words live in a device array of the library,
// addressed like the scratch array above.
static __device__ __align__(16) int dbg_res[4];
std::mutex g_dbg_mu;
void* g_dbg_ptr[kMaxDevices] = {};

csa_status_t debug_check_idx(const char* fn, const int32_t* idx, long n, int32_t T,
                             hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(CSA_ERR_LAUNCH, "%s: debug check: no usable device", fn);
  std::lock_guard<std::mutex> lock(g_dbg_mu);
  if (!g_dbg_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_res));
    if (e != hipSuccess || p == nullptr)
      return fail(CSA_ERR_LAUNCH, "%s: debug check: hipGetSymbolAddress failed: %s", fn,
                  hipGetErrorString(e));
    g_dbg_ptr[dev] = p;
  }
  int* res = static_cast<int*>(g_dbg_ptr[dev]);
  const int init[2] = {0, 0x7fffffff};
  int got[2] = {0, 0};
  e = hipMemcpyAsync(res, init, sizeof(init), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = csa::launch_check_idx(idx, n, T, res, s);
  if (e == hipSuccess) e = hipMemcpyAsync(got, res, sizeof(got), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess)
    return fail(CSA_ERR_LAUNCH, "%s: debug check of idx failed: %s", fn, hipGetErrorString(e));
  if (got[0] != 0)
    return fail(CSA_ERR_INVALID,
                "%s: idx holds %d entries outside [-1, T=%d); the first at element %d", fn,
                got[0], T, got[1]);
  return CSA_OK;
}
#endif

}  // namespace

extern "C" {

const char* csa_last_error(void) { return g_err; }

#ifdef CSA_DEBUG
const char* csa_version(void) { return "csa-mi355x 0.1 (gfx950, debug checks)"; }
#else
const char* csa_version(void) { return "csa-mi355x 0.1 (gfx950)"; }
#endif

csa_status_t csa_rope_table(float* cs, int32_t n_pos, int32_t rope_dim, double theta,
                            void* stream) {
  if (!cs) return fail(CSA_ERR_INVALID, "csa_rope_table: cs is NULL");
  if (n_pos < 1 || rope_dim < 2 || (rope_dim & 1) || !(theta > 0.0))
    return fail(CSA_ERR_INVALID,
                "csa_rope_table: need n_pos >= 1, even rope_dim >= 2, theta > 0 "
                "(n_pos=%d rope_dim=%d theta=%g)",
                n_pos, rope_dim, theta);
  return launched(
      csa::launch_rope_table(cs, n_pos, rope_dim, theta, 1.0, 1, 32.0, 1.0, as_stream(stream)),
      "csa_rope_table");
}

csa_status_t csa_rope_table_yarn(float* cs, int32_t n_pos, int32_t rope_dim, double theta,
                                 double factor, int32_t original_max_pos, double beta_fast,
                                 double beta_slow, void* stream) {
  if (!cs) return fail(CSA_ERR_INVALID, "csa_rope_table_yarn: cs is NULL");
  if (n_pos < 1 || rope_dim < 2 || (rope_dim & 1) || !(theta > 1.0))
    return fail(CSA_ERR_INVALID,
                "csa_rope_table_yarn: need n_pos >= 1, even rope_dim >= 2, theta > 1 "
                "(n_pos=%d rope_dim=%d theta=%g)",
                n_pos, rope_dim, theta);
  if (!(factor >= 1.0) || original_max_pos < 1 || !(beta_slow > 0.0) ||
      !(beta_fast > beta_slow))
    return fail(CSA_ERR_INVALID,
                "csa_rope_table_yarn: need factor >= 1, original_max_pos >= 1 and "
                "beta_fast > beta_slow > 0 (factor=%g original_max_pos=%d beta_fast=%g "
                "beta_slow=%g)",
                factor, original_max_pos, beta_fast, beta_slow);
  return launched(csa::launch_rope_table(cs, n_pos, rope_dim, theta, factor, original_max_pos,
                                         beta_fast, beta_slow, as_stream(stream)),
                  "csa_rope_table_yarn");
}

csa_status_t csa_compress(const void* x, const void* gate, const float* slot_bias,
                          void* pool, int32_t B, int32_t S, int32_t D, int32_t m,
                          int32_t overlap, int32_t rope_dim, const float* cs,
                          int32_t n_pos, int32_t pos0, int32_t dtype, void* stream) {
  const char* fn = "csa_compress";
  if (!dtype_ok(dtype)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  csa_status_t st = check_compress(fn, x, gate, slot_bias, pool, B, S, D, m, overlap, rope_dim,
                                   cs, n_pos, pos0);
  if (st != CSA_OK || (long)B * (S / m) == 0) return st;
  return launched(csa::launch_compress(x, gate, slot_bias, pool, B, S, D, m, overlap,
                                       rope_dim, cs, pos0, dtype == CSA_BF16,
                                       as_stream(stream)),
                  fn);
}

csa_status_t csa_compress_many(const csa_compress_pass_t* passes, int32_t n_passes,
                               int32_t dtype, void* stream) {
  const char* fn = "csa_compress_many";
  if (!dtype_ok(dtype)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (n_passes < 0 || n_passes > 16 || (n_passes > 0 && !passes))
    return fail(CSA_ERR_INVALID, "%s: need 0 <= n_passes <= 16 and a pass array", fn);
  csa::CompressPass cp[16];
  int n = 0;
  for (int q = 0; q < n_passes; ++q) {
    const csa_compress_pass_t& c = passes[q];
    char name[48];
    snprintf(name, sizeof(name), "%s: pass %d", fn, q);
    csa_status_t st = check_compress(name, c.x, c.gate, c.slot_bias, c.pool, c.B, c.S, c.D, c.m,
                                     c.overlap, c.rope_dim, c.cs, c.n_pos, c.pos0);
    if (st != CSA_OK) return st;
    if ((long)c.B * (c.S / c.m) == 0) continue;
    cp[n++] = csa::CompressPass{c.x, c.gate, c.slot_bias, c.pool, c.B, c.S, c.D, c.m, c.overlap,
                                c.rope_dim, c.rope_dim > 0 ? c.cs : nullptr, c.pos0};
  }
  return launched(csa::launch_compress_many(cp, n, dtype == CSA_BF16, as_stream(stream)), fn);
}

}  // extern "C"

namespace {
csa_status_t check_compress(const char* fn, const void* x, const void* gate,
                            const float* slot_bias, void* pool, int32_t B, int32_t S, int32_t D,
                            int32_t m, int32_t overlap, int32_t rope_dim, const float* cs,
                            int32_t n_pos, int32_t pos0) {
  if (B < 0 || S < 0 || D < 8 || m < 1 || (overlap != 0 && overlap != 1))
    return fail(CSA_ERR_INVALID, "%s: bad sizes (B=%d S=%d D=%d m=%d overlap=%d)", fn, B, S,
                D, m, overlap);
  if (D % 8 != 0) return fail(CSA_ERR_INVALID, "%s: D=%d must be a multiple of 8", fn, D);
  if (D > 1024) return fail(CSA_ERR_UNSUPPORTED, "%s: D=%d > 1024", fn, D);
  if (rope_dim < 0 || (rope_dim & 1) || rope_dim > D)
    return fail(CSA_ERR_INVALID, "%s: rope_dim=%d must be even and in [0, D]", fn, rope_dim);
  const int32_t T = S / m;
  if ((long)B * T == 0) return CSA_OK;
  if (!x || !pool) return fail(CSA_ERR_INVALID, "%s: x and pool are required", fn);
  if (!aligned16(x) || !aligned16(pool) || (gate && !aligned16(gate)) ||
      (slot_bias && !aligned16(slot_bias)))
    return fail(CSA_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
  if (rope_dim > 0) {
    if (!cs) return fail(CSA_ERR_INVALID, "%s: the RoPE table is required", fn);
    if (pos0 < 0 || (long)pos0 + (long)(T - 1) * m >= n_pos)
      return fail(CSA_ERR_INVALID,
                  "%s: entry positions pos0=%d .. %ld exceed the RoPE table (n_pos=%d)", fn,
                  pos0, (long)pos0 + (long)(T - 1) * m, n_pos);
  }
  return CSA_OK;
}
}  // namespace

extern "C" {

csa_status_t csa_cache_append(const void* x, const void* gate, const float* slot_bias,
                              void* ring_x, void* ring_g, void* pool, void* win,
                              const int32_t* count, int32_t B, int32_t n, int32_t D, int32_t m,
                              int32_t overlap, int32_t T_cap, int32_t W, int32_t rope_dim,
                              const float* cs, int32_t n_pos, int32_t dtype, void* stream) {
  const char* fn = "csa_cache_append";
  if (!dtype_ok(dtype)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  csa_status_t st = check_cache_append(fn, x, gate, slot_bias, ring_x, ring_g, pool, win, count,
                                       B, n, D, m, overlap, T_cap, W, rope_dim, cs, n_pos);
  if (st != CSA_OK || (long)B * n == 0) return st;
  return launched(csa::launch_cache_append(x, gate, slot_bias, ring_x, ring_g, pool, win,
                                           count, B, n, D, m, overlap, T_cap, W, rope_dim, cs,
                                           n_pos, dtype == CSA_BF16, as_stream(stream)),
                  fn);
}

csa_status_t csa_cache_append_many(const csa_cache_pass_t* passes, int32_t n_passes,
                                   int32_t dtype, void* stream) {
  const char* fn = "csa_cache_append_many";
  if (!dtype_ok(dtype)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (n_passes < 0 || n_passes > 16 || (n_passes > 0 && !passes))
    return fail(CSA_ERR_INVALID, "%s: need 0 <= n_passes <= 16 and a pass array", fn);
  csa::CachePass cp[16];
  int n = 0;
  for (int q = 0; q < n_passes; ++q) {
    const csa_cache_pass_t& c = passes[q];
    char name[48];
    snprintf(name, sizeof(name), "%s: pass %d", fn, q);
    csa_status_t st = check_cache_append(name, c.x, c.gate, c.slot_bias, c.ring_x, c.ring_g,
                                         c.pool, c.win, c.count, c.B, c.n, c.D, c.m, c.overlap,
                                         c.T_cap, c.W, c.rope_dim, c.cs, c.n_pos);
    if (st != CSA_OK) return st;
    if ((long)c.B * c.n == 0) continue;
    cp[n++] = csa::CachePass{c.x, c.gate, c.slot_bias, c.ring_x, c.ring_g, c.pool, c.win,
                             c.count, c.B, c.n, c.D, c.m, c.overlap, c.T_cap, c.W, c.rope_dim,
                             c.cs, c.n_pos};
  }
  return launched(csa::launch_cache_append_many(cp, n, dtype == CSA_BF16, as_stream(stream)),
                  fn);
}

}  // extern "C"

namespace {
csa_status_t check_cache_append(const char* fn, const void* x, const void* gate,
                                const float* slot_bias, void* ring_x, void* ring_g, void* pool,
                                void* win, const int32_t* count, int32_t B, int32_t n,
                                int32_t D, int32_t m, int32_t overlap, int32_t T_cap, int32_t W,
                                int32_t rope_dim, const float* cs, int32_t n_pos) {
  if (B < 0 || n < 0 || D < 8 || m < 1 || (overlap != 0 && overlap != 1) || T_cap < 0 ||
      W < 0)
    return fail(CSA_ERR_INVALID, "%s: bad sizes (B=%d n=%d D=%d m=%d overlap=%d T_cap=%d W=%d)",
                fn, B, n, D, m, overlap, T_cap, W);
  if (D % 8 != 0) return fail(CSA_ERR_INVALID, "%s: D=%d must be a multiple of 8", fn, D);
  if (D > 1024) return fail(CSA_ERR_UNSUPPORTED, "%s: D=%d > 1024", fn, D);
  if ((1 + overlap) * m > 256)
    return fail(CSA_ERR_UNSUPPORTED, "%s: window of %d rows > 256", fn, (1 + overlap) * m);
  if (rope_dim < 0 || (rope_dim & 1) || rope_dim > D)
    return fail(CSA_ERR_INVALID, "%s: rope_dim=%d must be even and in [0, D]", fn, rope_dim);
  if ((long)B * n == 0) return CSA_OK;
  if ((long)n * (D / 8) >= (1L << 30))
    return fail(CSA_ERR_UNSUPPORTED, "%s: n=%d too large", fn, n);
  if (!x || !ring_x || !pool || !count)
    return fail(CSA_ERR_INVALID, "%s: x, ring_x, pool and count are required", fn);
  if ((gate == nullptr) != (ring_g == nullptr))
    return fail(CSA_ERR_INVALID, "%s: gate and ring_g go together", fn);
  if ((W > 0) != (win != nullptr))
    return fail(CSA_ERR_INVALID, "%s: win is required exactly when W > 0", fn);
  if (!aligned16(x) || !aligned16(ring_x) || !aligned16(pool) || (gate && !aligned16(gate)) ||
      (ring_g && !aligned16(ring_g)) || (win && !aligned16(win)) ||
      (slot_bias && !aligned16(slot_bias)))
    return fail(CSA_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
  if (rope_dim > 0 && (!cs || n_pos < 1))
    return fail(CSA_ERR_INVALID, "%s: the RoPE table is required", fn);
  return CSA_OK;
}
}  // namespace

extern "C" {

csa_status_t csa_index_scores(const void* q_idx, const float* w_idx, const void* k_pool,
                              float* scores, const int32_t* q_pos, int32_t B, int32_t S,
                              int32_t T, int32_t n_heads, int32_t head_dim, int32_t m,
                              int32_t dtype, void* stream) {
  const char* fn = "csa_index_scores";
  if (!dtype_ok(dtype)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (B < 0 || S < 0 || T < 0 || n_heads < 1 || head_dim < 1 || m < 1)
    return fail(CSA_ERR_INVALID, "%s: bad sizes (B=%d S=%d T=%d heads=%d dim=%d m=%d)", fn,
                B, S, T, n_heads, head_dim, m);
  if (head_dim % 8 != 0)
    return fail(CSA_ERR_INVALID, "%s: head_dim=%d must be a multiple of 8", fn, head_dim);
  if ((long)n_heads * head_dim + n_heads > 16384)
    return fail(CSA_ERR_UNSUPPORTED, "%s: n_heads*head_dim=%d too large", fn,
                n_heads * head_dim);
  if ((long)B * S * T == 0) return CSA_OK;
  if (!q_idx || !w_idx || !k_pool || !scores || !q_pos)
    return fail(CSA_ERR_INVALID, "%s: NULL tensor", fn);
  if (!aligned16(q_idx) || !aligned16(k_pool))
    return fail(CSA_ERR_INVALID, "%s: q_idx and k_pool must be 16-byte aligned", fn);
  return launched(csa::launch_index_scores(q_idx, w_idx, k_pool, scores, q_pos, B, S, T,
                                           n_heads, head_dim, m, dtype == CSA_BF16,
                                           as_stream(stream)),
                  fn);
}

csa_status_t csa_topk(const float* scores, int32_t* idx, const int32_t* q_pos, int32_t B,
                      int32_t S, int32_t T, int32_t k, int32_t m, void* stream) {
  const char* fn = "csa_topk";
  if (B < 0 || S < 0 || T < 0 || k < 1 || m < 1)
    return fail(CSA_ERR_INVALID, "%s: bad sizes (B=%d S=%d T=%d k=%d m=%d)", fn, B, S, T, k,
                m);
  if ((long)B * S == 0) return CSA_OK;
  if (!idx || !q_pos || (T > 0 && !scores)) return fail(CSA_ERR_INVALID, "%s: NULL tensor", fn);
  return launched(csa::launch_topk(scores, idx, q_pos, B, S, T, k, m, as_stream(stream)), fn);
}

size_t csa_index_topk_workspace_size(int32_t B, int32_t S, int32_t T, int32_t n_heads,
                                     int32_t head_dim, int32_t k, int32_t m, int32_t dtype) {
  if (B < 0 || S < 0 || T < 0 || n_heads < 1 || head_dim < 1 || k < 1 || m < 1) return 0;
  if (csa::index_topk_fused_shape(S, T, n_heads, head_dim, k, m, dtype == CSA_BF16)) return 0;
  return (size_t)B * S * T * sizeof(float);
}

csa_status_t csa_index_topk(const void* q_idx, const float* w_idx, const void* k_pool,
                            int32_t* idx, const int32_t* q_pos, int32_t B, int32_t S, int32_t T,
                            int32_t n_heads, int32_t head_dim, int32_t k, int32_t m,
                            void* workspace, size_t ws_bytes, int32_t dtype, void* stream) {
  const char* fn = "csa_index_topk";
  if (!dtype_ok(dtype)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (B < 0 || S < 0 || T < 0 || n_heads < 1 || head_dim < 1 || m < 1 || k < 1)
    return fail(CSA_ERR_INVALID,
                "%s: bad sizes (B=%d S=%d T=%d heads=%d dim=%d k=%d m=%d)", fn, B, S, T,
                n_heads, head_dim, k, m);
  if (head_dim % 8 != 0)
    return fail(CSA_ERR_INVALID, "%s: head_dim=%d must be a multiple of 8", fn, head_dim);
  if ((long)n_heads * head_dim + n_heads > 16384)
    return fail(CSA_ERR_UNSUPPORTED, "%s: n_heads*head_dim=%d too large", fn,
                n_heads * head_dim);
  if ((long)B * S == 0) return CSA_OK;
  if (!idx || !q_pos || (T > 0 && (!q_idx || !w_idx || !k_pool)))
    return fail(CSA_ERR_INVALID, "%s: NULL tensor", fn);
  if (T > 0 && (!aligned16(q_idx) || !aligned16(k_pool)))
    return fail(CSA_ERR_INVALID, "%s: q_idx and k_pool must be 16-byte aligned", fn);
  const hipStream_t s = as_stream(stream);
  if (csa::index_topk_fused_shape(S, T, n_heads, head_dim, k, m, dtype == CSA_BF16))
    return launched(csa::launch_index_topk_fused(q_idx, w_idx, k_pool, idx, q_pos, B, S, T, m,
                                                 k, s),
                    fn);
  // other shapes: the scores go through the caller's workspace
  const size_t need = (size_t)B * S * T * sizeof(float);
  if (!workspace || ws_bytes < need || !aligned16(workspace))
    return fail(CSA_ERR_INVALID,
                "%s: this shape needs a 16-byte aligned workspace of %zu bytes (got %zu)", fn,
                need, ws_bytes);
  float* sc = reinterpret_cast<float*>(workspace);
  hipError_t e = csa::launch_index_scores(q_idx, w_idx, k_pool, sc, q_pos, B, S, T, n_heads,
                                          head_dim, m, dtype == CSA_BF16, s);
  if (e != hipSuccess) return launched(e, fn);
  return launched(csa::launch_topk(sc, idx, q_pos, B, S, T, k, m, s), fn);
}

size_t csa_sparse_attn_workspace_size(int32_t B, int32_t S, int32_t H, int32_t D, int32_t dv,
                                      int32_t rope_dim, int32_t k, int32_t window,
                                      int32_t dtype) {
  if (B < 0 || S < 0 || H < 1 || D < 1 || dv < 1 || k < 0 || window < 0) return 0;
  return csa::plan_attention(B, S, H, D, dv, rope_dim, window, k, dtype == CSA_BF16, 0, k)
      .ws_bytes;
}

size_t hca_attn_workspace_size(int32_t B, int32_t S, int32_t H, int32_t D, int32_t dv,
                               int32_t rope_dim, int32_t T, int32_t window, int32_t dtype) {
  if (B < 0 || S < 0 || H < 1 || D < 1 || dv < 1 || T < 0 || window < 0) return 0;
  return csa::plan_attention(B, S, H, D, dv, rope_dim, window, T, dtype == CSA_BF16, T, 0)
      .ws_bytes;
}

csa_status_t csa_sparse_attn(const void* q, const void* kv_win, const int32_t* win_pos0,
                             int32_t L_win, const void* pool, int32_t T, const int32_t* idx,
                             int32_t k, const float* sink, void* out, const int32_t* q_pos,
                             int32_t B, int32_t S, int32_t H, int32_t D, int32_t dv,
                             int32_t rope_dim, const float* cs, int32_t n_pos,
                             int32_t window, float scale, void* workspace, size_t ws_bytes,
                             int32_t dtype, void* stream) {
  const char* fn = "csa_sparse_attn";
  csa_status_t st = check_attn(fn, q, kv_win, win_pos0, L_win, pool, T, out, q_pos, B, S, H,
                               D, dv, rope_dim, cs, n_pos, window, scale, dtype);
  if (st != CSA_OK) return st;
  if (k < 0) return fail(CSA_ERR_INVALID, "%s: k=%d must be >= 0", fn, k);
  if ((long)B * S == 0) return CSA_OK;
  if (k > 0 && !idx) return fail(CSA_ERR_INVALID, "%s: idx is required when k > 0", fn);
  csa::AttnParams p = make_params(q, kv_win, win_pos0, L_win, pool, T, idx, k, 1, sink, out,
                                  q_pos, B, S, H, D, dv, rope_dim, cs, n_pos, window, scale,
                                  dtype);
  if (k == 0) {  // no pool slot at all: window-only attention
    p.idx = nullptr;
    p.k = 0;
    p.dense = 0;
  }
#ifdef CSA_DEBUG
  if (p.k > 0) {
    st = debug_check_idx(fn, idx, (long)B * S * k, T, as_stream(stream));
    if (st != CSA_OK) return st;
  }
#endif
  return run_attn(fn, p, p.k, workspace, ws_bytes, as_stream(stream));
}

csa_status_t csa_sparse_attn_noalloc(const void* q, const void* kv_win,
                                     const int32_t* win_pos0, int32_t L_win, const void* pool,
                                     int32_t T, const int32_t* idx, int32_t k,
                                     const float* sink, void* out, const int32_t* q_pos,
                                     int32_t B, int32_t S, int32_t H, int32_t D, int32_t dv,
                                     int32_t rope_dim, const float* cs, int32_t n_pos,
                                     int32_t window, float scale, int32_t dtype,
                                     void* stream) {
  const char* fn = "csa_sparse_attn_noalloc";
  csa_status_t st = check_attn(fn, q, kv_win, win_pos0, L_win, pool, T, out, q_pos, B, S, H,
                               D, dv, rope_dim, cs, n_pos, window, scale, dtype);
  if (st != CSA_OK) return st;
  if (k < 0) return fail(CSA_ERR_INVALID, "%s: k=%d must be >= 0", fn, k);
  if ((long)B * S == 0) return CSA_OK;
  if (k > 0 && !idx) return fail(CSA_ERR_INVALID, "%s: idx is required when k > 0", fn);
  csa::AttnParams p = make_params(q, kv_win, win_pos0, L_win, pool, T, idx, k, 1, sink, out,
                                  q_pos, B, S, H, D, dv, rope_dim, cs, n_pos, window, scale,
                                  dtype);
  if (k == 0) {
    p.idx = nullptr;
    p.k = 0;
    p.dense = 0;
  }
#ifdef CSA_DEBUG
  if (p.k > 0) {
    st = debug_check_idx(fn, idx, (long)B * S * k, T, as_stream(stream));
    if (st != CSA_OK) return st;
  }
#endif
  // the same plan as csa_sparse_attn with a large enough workspace
  const csa::AttnPlan plan =
      csa::plan_attention(p.B, p.S, p.H, p.D, p.dv, p.rope_dim, p.window, p.k, p.bf16,
                          std::max<long>(p.L_win, p.T), p.k);
  void* ws = nullptr;
  if (plan.nsplit > 1) {
    if (plan.ws_bytes > kScratchBytes)
      return fail(CSA_ERR_UNSUPPORTED,
                  "%s: this shape needs %zu bytes of scratch, more than the library's "
                  "%zu (use csa_sparse_attn with a workspace)",
                  fn, plan.ws_bytes, kScratchBytes);
    st = scratch_on_current_device(fn, &ws);
    if (st != CSA_OK) return st;
  }
  return launched(csa::launch_attention(p, plan, ws, as_stream(stream)), fn);
}

csa_status_t csa_grouped_out_proj(const void* o, const void* w_a, const void* w_b, void* mid,
                                  void* out, int32_t M, int32_t groups, int32_t group_in,
                                  int32_t rank, int32_t hidden, int32_t dtype, void* stream) {
  const char* fn = "csa_grouped_out_proj";
  if (!dtype_ok(dtype)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (M < 0 || groups < 1 || group_in < 1 || rank < 1 || hidden < 1)
    return fail(CSA_ERR_INVALID,
                "%s: bad sizes (M=%d groups=%d group_in=%d rank=%d hidden=%d)", fn, M, groups,
                group_in, rank, hidden);
  if (group_in % 8 != 0 || rank % 8 != 0 || hidden % 8 != 0)
    return fail(CSA_ERR_INVALID, "%s: group_in, rank and hidden must be multiples of 8", fn);
  const long elems_o = (long)groups * group_in, elems_mid = (long)groups * rank;
  if ((long)M * elems_o >= (1L << 31) || (long)M * elems_mid >= (1L << 31) ||
      (long)M * hidden >= (1L << 31) || (long)hidden * elems_mid >= (1L << 31) ||
      (long)groups * rank * group_in >= (1L << 31))
    return fail(CSA_ERR_UNSUPPORTED, "%s: tensors of 2^31 elements or more", fn);
  if (M == 0) return CSA_OK;
  if (!o || !w_a || !w_b || !mid || !out)
    return fail(CSA_ERR_INVALID, "%s: o, w_a, w_b, mid and out are required", fn);
  if (!aligned16(o) || !aligned16(w_a) || !aligned16(w_b) || !aligned16(mid) || !aligned16(out))
    return fail(CSA_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
  return launched(csa::launch_out_proj(o, w_a, w_b, mid, out, M, groups, group_in, rank, hidden,
                                       dtype == CSA_BF16, as_stream(stream)),
                  fn);
}

csa_status_t hca_attn(const void* q, const void* kv_win, const int32_t* win_pos0,
                      int32_t L_win, const void* pool, int32_t T, int32_t m,
                      const float* sink, void* out, const int32_t* q_pos, int32_t B,
                      int32_t S, int32_t H, int32_t D, int32_t dv, int32_t rope_dim,
                      const float* cs, int32_t n_pos, int32_t window, float scale,
                      void* workspace, size_t ws_bytes, int32_t dtype, void* stream) {
  const char* fn = "hca_attn";
  csa_status_t st = check_attn(fn, q, kv_win, win_pos0, L_win, pool, T, out, q_pos, B, S, H,
                               D, dv, rope_dim, cs, n_pos, window, scale, dtype);
  if (st != CSA_OK) return st;
  if (m < 1) return fail(CSA_ERR_INVALID, "%s: m=%d must be >= 1", fn, m);
  if ((long)B * S == 0) return CSA_OK;
  csa::AttnParams p = make_params(q, kv_win, win_pos0, L_win, pool, T, nullptr, 0, m, sink,
                                  out, q_pos, B, S, H, D, dv, rope_dim, cs, n_pos, window,
                                  scale, dtype);
  return run_attn(fn, p, T, workspace, ws_bytes, as_stream(stream));
}

}  // extern "C"
