// csa_device.hpp -- device helpers and kernel launch declarations shared by the
// gfx950 kernels of libcsa.so.  CDNA4 only: 64-wide wavefronts, bf16 matrix
// cores (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_32x32x16_bf16), 160 KiB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf2f(u16 h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN): the gfx950
// conversion instruction (v_cvt_pk_bf16_f32) does exactly this.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 8 consecutive elements (one 16-byte bf16 chunk, or two 16-byte fp32 chunks)
// loaded as fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, long elem, float v[8]) {
  if (BF16) {
    uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(base) + elem);
    v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
    v[4] = bf_lo(u.z); v[5] = bf_hi(u.z); v[6] = bf_lo(u.w); v[7] = bf_hi(u.w);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, long elem, const float v[8]) {
  if (BF16) {
    uint4 u;
    u.x = pack2(v[0], v[1]); u.y = pack2(v[2], v[3]);
    u.z = pack2(v[4], v[5]); u.w = pack2(v[6], v[7]);
    *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(base) + elem) = u;
  } else {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + elem);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, long elem) {
  if (BF16) return bf2f(reinterpret_cast<const u16*>(base)[elem]);
  return reinterpret_cast<const float*>(base)[elem];
}

template <bool BF16>
__device__ __forceinline__ void store1(void* base, long elem, float v) {
  if (BF16) reinterpret_cast<u16*>(base)[elem] = f2bf(v);
  else reinterpret_cast<float*>(base)[elem] = v;
}

// ---------------------------------------------------------------- readiness
// Query at absolute position t sees pool entries w < min(T, floor((t+1)/m)).
__device__ __forceinline__ int ready_count(long t, int m, int T) {
  if (t + 1 <= 0) return 0;
  long r = (t + 1) / m;
  return r > T ? T : (int)r;
}

// ---------------------------------------------------------------- matrix cores
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// ---------------------------------------------------------------- misc
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// LDS barrier that waits only for this wave's LDS traffic, not for global
// loads still in flight (the gathers of later tiles must stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Wait until at most N of this wave's vector memory operations (loads, stores
// and direct-to-LDS loads, retired in issue order) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// LDS pointer type of the direct-to-LDS buffer loads
typedef __attribute__((address_space(3))) void lds_void;

// Reductions over the four lanes l, l^16, l^32, l^48 of a wave with the gfx950
// lane-swap instructions (VALU, no LDS round trip).  v_permlane16_swap(x, x)
// returns, in its two results, x of lanes l and l^16 (in an order that depends
// on the lane, which a commutative operation does not see); v_permlane32_swap
// does the same for lanes l and l^32.  Every lane ends with the same value.
__device__ __forceinline__ float xgroup_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xgroup_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace csa

// ------------------------------------------------------------------------
// Host-side launchers (defined in the kernel sources, called by csa_api.hip).
// Each returns hipSuccess or the launch error.
namespace csa {

// factor <= 1: plain RoPE; factor > 1: YaRN-scaled frequencies
hipError_t launch_rope_table(float* cs, int n_pos, int rope_dim, double theta, double factor,
                             int orig_len, double beta_fast, double beta_slow, hipStream_t s);

hipError_t launch_compress(const void* x, const void* gate, const float* slot_bias,
                           void* pool, int B, int S, int D, int m, int overlap,
                           int rope_dim, const float* cs, int pos0, bool bf16,
                           hipStream_t s);

// one pass of launch_compress_many (the arguments of launch_compress)
struct CompressPass {
  const void* x;
  const void* gate;
  const float* slot_bias;
  void* pool;
  int B, S, D, m, overlap, rope_dim;
  const float* cs;
  int pos0;
};
hipError_t launch_compress_many(const CompressPass* p, int n, bool bf16, hipStream_t s);

hipError_t launch_cache_append(const void* x, const void* gate, const float* slot_bias,
                               void* ring_x, void* ring_g, void* pool, void* win,
                               const int* count, int B, int n, int D, int m, int overlap,
                               int T_cap, int W, int rope_dim, const float* cs, int n_pos,
                               bool bf16, hipStream_t s);

// one csa_cache_append pass; launch_cache_append_many runs the single-token
// passes of a list in shared launches and the others on their own
struct CachePass {
  const void* x;
  const void* gate;
  const float* slot_bias;
  void* ring_x;
  void* ring_g;
  void* pool;
  void* win;
  const int* count;
  int B, n, D, m, overlap, T_cap, W, rope_dim;
  const float* cs;
  int n_pos;
};
hipError_t launch_cache_append_many(const CachePass* p, int n, bool bf16, hipStream_t s);

hipError_t launch_index_scores(const void* q_idx, const float* w_idx, const void* k_pool,
                               float* scores, const int* q_pos, int B, int S, int T,
                               int n_heads, int head_dim, int m, bool bf16,
                               hipStream_t s);

bool index_topk_fused_shape(int S, int T, int n_heads, int head_dim, int k, int m, bool bf16);
hipError_t launch_index_topk_fused(const void* q_idx, const float* w_idx, const void* k_pool,
                                   int* idx, const int* q_pos, int B, int S, int T, int m,
                                   int k, hipStream_t s);

hipError_t launch_topk(const float* scores, int* idx, const int* q_pos, int B, int S,
                       int T, int k, int m, hipStream_t s);

// Grouped low-rank output projection: mid = grouped(o, w_a), out = mid w_b^T
// (two GEMMs with both operands contiguous along the reduction).
bool gemm_nt_mfma_shape(int N, int K, int G, int ldx, int ldc, int M);
hipError_t launch_out_proj(const void* o, const void* w_a, const void* w_b, void* mid,
                           void* out, int M, int G, int Kg, int r, int hidden, bool bf16,
                           hipStream_t s);

struct AttnParams {
  const void* q;          // [B][S][H][D]
  const void* kv_win;     // [B][L_win][D]
  const int* win_pos0;    // [B]; nullptr with kv_win: a ring, position p at row p % L_win
  int win_ring;
  int L_win;
  const void* pool;       // [B][T][D]
  int T;
  const int* idx;         // [B][S][k] selected entries (CSA / DSA); unused when dense
  int k;
  int dense;              // 1: pool slots are all ready entries w < R(t) (HCA)
  int m;                  // readiness rate of the dense mode
  const float* sink;      // [H] or nullptr
  void* out;              // [B][S][H][dv]
  const int* q_pos;       // [B]
  int B, S, H, D, dv, rope_dim;
  const float* cs;        // [n_pos][rope_dim/2][2]
  int n_pos;
  int window;
  float scale;
  bool bf16;
};

// Plan for splitting a row's key slots over several workgroups.
struct AttnPlan {
  int kernel;             // 0 = generic, 1 = bf16 matrix-core kernel
  int nsplit;             // workgroups per query row (1 = no split)
  int tiles_per_split;
  size_t ws_bytes;        // workspace the split needs
};

// window: window slots per query; npool_max: pool slots per query (k, or T in
// dense mode); max_rows: the larger of L_win and T (rows of one sequence a
// gather addresses); k: index slots per query (0 in dense mode)
AttnPlan plan_attention(int B, int S, int H, int D, int dv, int rope_dim, int window,
                        int npool_max, bool bf16, long max_rows, int k);
hipError_t launch_attention(const AttnParams& p, const AttnPlan& plan, void* ws,
                            hipStream_t s);

// debug builds: counts the entries of idx[0 .. n) outside [-1, T) into res[0]
// and the first such element index into res[1] (res preset to {0, INT_MAX})
hipError_t launch_check_idx(const int* idx, long n, int T, int* res, hipStream_t s);

}  // namespace csa
