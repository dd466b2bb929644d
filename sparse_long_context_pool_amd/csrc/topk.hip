// topk.hip -- per-query top-k over the ready pool entries.
//
// Page "DeepSeek-V4", DeepseekV4Config: index_topk entries are kept per query
// (eq. 17); section "Attention mask layout": slots that cannot be filled yet
// carry the -1 sentinel.  Result: the min(k, R(t)) ready entries with the
// largest scores, equal scores resolved toward the lower index, emitted in
// ascending index order and padded with -1.  That result is unique, so the
// kernel is deterministic and matches any correct implementation bit for bit.
//
// One workgroup (8 wavefronts) per query row.  Scores become order-preserving
// 32-bit keys (-0 folded onto +0); the row is kept in LDS when it fits (up to
// 32768 entries = 128 KiB of the 160 KiB LDS), otherwise re-read from global
// memory on every pass.  A most-significant-digit-first radix select (four
// 8-bit digits, per-wave LDS histograms to cut atomic contention, a one-wave
// suffix scan to pick the digit) finds the k-th largest key K and how many
// copies of K to keep.  A final pass in index order keeps every key > K and the
// first copies of K; positions come from wave ballots and popcounts, so the
// output is written in ascending index order without any sort.
#include "csa_device.hpp"

namespace csa {
namespace {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkLdsCap = 32768;
constexpr int kHistWords = kTopkWaves * 256;
constexpr int kMetaWords = 64;

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;  // -0 equals +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

template <bool IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float* __restrict__ scores, int* __restrict__ idx, const int* __restrict__ q_pos,
    int S, int T, int k, int m) {
  extern __shared__ uint32_t sm[];
  uint32_t* hist = sm;                            // [waves][256]
  int* meta = reinterpret_cast<int*>(sm + kHistWords);  // selection + per-wave counts
  uint32_t* keys = sm + kHistWords + kMetaWords;  // [R] when IN_LDS

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const long row = blockIdx.x;
  const int b = (int)(row / S), i = (int)(row - (long)b * S);
  const int R = ready_count((long)q_pos[b] + i, m, T);
  int* out = idx + row * k;
  const float* src = scores + row * T;

  if (R <= k) {  // every ready entry is kept
    for (int j = tid; j < k; j += kTopkThreads) out[j] = j < R ? j : -1;
    return;
  }
  if (IN_LDS)
    for (int j = tid; j < R; j += kTopkThreads) keys[j] = score_key(src[j]);

  uint32_t prefix = 0u, pmask = 0u;
  int kk = k;  // rank still to find among keys matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int j = tid; j < kHistWords; j += kTopkThreads) hist[j] = 0u;
    __syncthreads();
    for (int j = tid; j < R; j += kTopkThreads) {
      const uint32_t key = IN_LDS ? keys[j] : score_key(src[j]);
      if ((key & pmask) == prefix) atomicAdd(&hist[wave * 256 + ((key >> shift) & 255u)], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns digits 4*lane .. 4*lane+3
      int tot[4], local = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int s = 0;
#pragma unroll
        for (int q = 0; q < kTopkWaves; ++q) s += (int)hist[q * 256 + 4 * lane + u];
        tot[u] = s;
        local += s;
      }
      // inclusive suffix sum over lanes >= lane
      int suf = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += v;
      }
      int above = suf - local;  // keys with a digit in a higher lane
#pragma unroll
      for (int u = 3; u >= 0; --u) {
        if (above < kk && above + tot[u] >= kk) {
          meta[0] = 4 * lane + u;
          meta[1] = above;
        }
        above += tot[u];
      }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)meta[0];
    kk -= meta[1];
    prefix |= digit << shift;
    pmask |= 255u << shift;
    __syncthreads();  // meta is rewritten by the next pass
  }

  // prefix is the k-th largest key K; keep all keys > K and the first kk
  // copies of K, in index order.
  const uint32_t K = prefix;
  int* cnt = meta + 2;  // [2 buffers][waves][gt, eq]
  int sel_base = 0, eq_base = 0;
  int it = 0;
  for (int base = 0; base < R && sel_base < k; base += kTopkThreads, ++it) {
    const int j = base + tid;
    uint32_t key = 0u;
    if (j < R) key = IN_LDS ? keys[j] : score_key(src[j]);
    const bool gt = j < R && key > K;
    const bool eq = j < R && key == K;
    const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
    int* c = cnt + (it & 1) * kTopkWaves * 2;
    if (lane == 0) {
      c[wave * 2] = __popcll(mgt);
      c[wave * 2 + 1] = __popcll(meq);
    }
    __syncthreads();
    int eq_before = eq_base, sel_before = sel_base;
    int eq_tot = 0, sel_tot = 0;
    for (int q = 0; q < kTopkWaves; ++q) {
      const int g = c[q * 2], e = c[q * 2 + 1];
      const int take_e = min(max(kk - (eq_base + eq_tot), 0), e);
      if (q < wave) { eq_before += e; sel_before += g + take_e; }
      eq_tot += e;
      sel_tot += g + take_e;
    }
    const int take_here = min(max(kk - eq_before, 0), __popcll(meq));
    const uint64_t lt = lanemask_lt(lane);
    const bool take = gt || (eq && __popcll(meq & lt) < take_here);
    const uint64_t mtake = __ballot(take);
    const int pos = sel_before + __popcll(mtake & lt);
    if (take && pos < k) out[pos] = j;
    sel_base += sel_tot;
    eq_base += eq_tot;
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int* idx, const int* q_pos, int B, int S,
                       int T, int k, int m, hipStream_t s) {
  const long rows = (long)B * S;
  if (rows == 0) return hipSuccess;
  const bool in_lds = T <= kTopkLdsCap;
  const size_t lds = (size_t)(kHistWords + kMetaWords + (in_lds ? T : 0)) * sizeof(uint32_t);
  if (in_lds)
    hipLaunchKernelGGL(topk_kernel<true>, dim3((unsigned)rows), dim3(kTopkThreads), lds, s,
                       scores, idx, q_pos, S, T, k, m);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3((unsigned)rows), dim3(kTopkThreads), lds, s,
                       scores, idx, q_pos, S, T, k, m);
  return hipGetLastError();
}

}  // namespace csa
