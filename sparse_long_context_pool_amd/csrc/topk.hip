// topk.hip -- per-query top-k over the ready pool entries.
//
// Page "DeepSeek-V4", DeepseekV4Config: index_topk entries are kept per query
// (eq. 17); section "Attention mask layout": slots that cannot be filled yet
// carry the -1 sentinel.  Result: the min(k, R(t)) ready entries with the
// largest scores, equal scores resolved toward the lower index, emitted in
// ascending index order and padded with -1.  That result is unique, so the
// kernel is deterministic and matches any correct implementation bit for bit.
//
// One workgroup per query row (4, 8 or 16 wavefronts by row length).  Scores
// become order-preserving 32-bit keys (-0 folded onto +0).  A most-significant-digit-first radix
// select finds the k-th largest key K and how many copies of K to keep; a
// final pass in index order keeps every key > K and the first copies of K,
// with output positions from wave ballots and popcounts, so the result is
// written in ascending index order without any sort.  Rows of up to 32768
// entries keep their keys in registers for the whole selection (three passes
// over 11 + 11 + 10 bits); longer rows re-read the scores from global memory
// on each of four 8-bit passes.
#include "csa_device.hpp"

namespace csa {
namespace {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / 64;
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

__global__ __launch_bounds__(kTopkThreads) void topk_global(
    const float* __restrict__ scores, int* __restrict__ idx, const int* __restrict__ q_pos,
    int S, int T, int k, int m) {
  __shared__ uint32_t sm[kHistWords + kMetaWords];
  uint32_t* hist = sm;                            // [waves][256]
  int* meta = reinterpret_cast<int*>(sm + kHistWords);  // selection + per-wave counts

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
  uint32_t prefix = 0u, pmask = 0u;
  int kk = k;  // rank still to find among keys matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int j = tid; j < kHistWords; j += kTopkThreads) hist[j] = 0u;
    __syncthreads();
    for (int j = tid; j < R; j += kTopkThreads) {
      const uint32_t key = score_key(src[j]);
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
    if (j < R) key = score_key(src[j]);
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

// Register path (rows of up to 512 * KPT entries): thread t keeps the keys
// of entries 512 j + t (j < KPT) in registers for the whole selection.  Radix
// select over 11 + 11 + 10 bits with one shared LDS histogram (2048 bins, two
// copies so that clearing the next one needs no extra barrier), each pass a
// block-wide suffix scan of the bins.  Final pass: for each 512-entry slice,
// wave ballots of (key > K) and (key == K) give every entry its rank among the
// earlier ones; the per-(slice, wave) totals are prefix-summed once, so the
// ordered compaction needs a single barrier.
// NT threads per row (NT / 64 waves), KPT keys per thread; the 2048 histogram
// bins are scanned BPT = 2048 / NT per thread.
template <int KPT, int NT>
__global__ __launch_bounds__(NT) void topk_reg(
    const float* __restrict__ scores, int* __restrict__ idx, const int* __restrict__ q_pos,
    int S, int T, int k, int m) {
  constexpr int NW = NT / 64;
  constexpr int BPT = 2048 / NT;
  static_assert(BPT == 2 || BPT == 4 || BPT == 8, "bins per thread");
  // the first pass spreads its counts over HC copies of the histogram (lane
  // l counts into copy l % HC; copies one word apart in bank order), so that
  // lanes of one atomic instruction whose keys share a bin mostly hit
  // different words; the rows of up to 2048 entries (eight workgroups per
  // compute unit) keep one copy for their LDS budget
  constexpr int HC = NT >= 512 ? 4 : 1;
  constexpr int HS = HC > 1 ? 2049 : 2048;  // words between copies
  __shared__ __attribute__((aligned(16))) uint32_t hist0[HC * HS];
  __shared__ __attribute__((aligned(16))) uint32_t hist1[2048];
  __shared__ int wtot[NW];
  __shared__ int meta[3];  // digit, keys above its bin, bin taken whole
  __shared__ int gtot[KPT * NW], etot[KPT * NW];  // per (slice, wave) counts, then prefixes
  __shared__ int wsg[NW], wse[NW];                // wave totals of the prefix scan
  static_assert(KPT <= 64, "one (slice, wave) entry per thread");

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const long row = blockIdx.x;
  const int b = (int)(row / S), i = (int)(row - (long)b * S);
  const int R = ready_count((long)q_pos[b] + i, m, T);
  int* out = idx + row * k;
  const float* src = scores + row * T;

  if (R <= k) {  // every ready entry is kept
    for (int j = tid; j < k; j += NT) out[j] = j < R ? j : -1;
    return;
  }
  // keys of entries 512 j + tid.  Entries past R get key 0, below the key of
  // any score that is not NaN (-inf maps to 0x007fffff), so they fall in the
  // lowest bin of the first pass, never match a later prefix and are never
  // kept: no separate validity test is needed.
  // The first histogram is cleared before the loads are issued, so that the
  // first pass's atomics run as the keys arrive (each key is counted as soon
  // as its load has landed) instead of after all of them.
  // (the loads are unconditional, clamped into the row, so that all of them
  // are in flight together)
  for (int j = tid; j < HC * HS; j += NT) hist0[j] = 0u;
  __syncthreads();  // the first histogram is clear
  // (rows of more than 8192 entries -- decode, token-level rows -- load
  // their scores non-temporally: each is read once, and this measured ~1 us
  // faster on the decode rows; the short prefill rows, still in the caches
  // from the index kernel, measured ~1 us slower with it)
  float sv[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const float* a = src + min(j * NT + tid, R - 1);
    sv[j] = NT >= 1024 ? __builtin_nontemporal_load(a) : *a;
  }
  uint32_t key[KPT];
  {
    // first pass's atomics (digit = the top 11 bits; entries past R, key 0,
    // are skipped: they would all hit one bin and serialise the atomics)
    uint32_t* hc0 = hist0 + (lane % HC) * HS;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      key[j] = j * NT + tid < R ? score_key(sv[j]) : 0u;
      if (key[j] != 0u) atomicAdd(&hc0[key[j] >> 21], 1u);
    }
  }

  uint32_t prefix = 0u, pmask = 0u;
  int kk = k;
  int buf = 0;
  // Pass p: atomics into h (pass 0's were issued with the loads), barrier, bin
  // counts and wave suffix sums, barrier, the digit, barrier.  A pass needs no barrier before its atomics: its
  // histogram was cleared during the previous pass, and the previous pass's
  // reads of wtot, meta and the other histogram all precede its last barrier.
  // The passes stop early once the bin holding the kk-th largest key is taken
  // whole (its count is exactly kk): every key matching the prefix so far is
  // kept, and K = the prefix with zero low bits keeps exactly them (keys above
  // it, and the copies of K itself, all of which kk admits).
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    // pass 0: hist0 (HC copies); pass 1: hist1; pass 2: hist0's first copy
    uint32_t* h = buf == 0 ? hist0 : hist1;
    // (the first pass counted its keys as they were loaded)
    if (pass > 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (key[j] != 0u && (key[j] & pmask) == prefix) atomicAdd(&h[(key[j] >> shift) & dmask], 1u);
    }
    // clear the other histogram for the next pass meanwhile (its first 2048
    // words: a later pass uses one copy)
    for (int j = tid; j < 2048; j += NT) (buf == 0 ? hist1 : hist0)[j] = 0u;
    __syncthreads();
    // thread t owns bins BPT t .. BPT t + BPT-1; suffix sums over the bins above
    int cnt[BPT];
    if (HC > 1 && pass == 0) {
#pragma unroll
      for (int u = 0; u < BPT; ++u) {
        int c = 0;
#pragma unroll
        for (int q = 0; q < HC; ++q) c += (int)hist0[q * HS + BPT * tid + u];
        cnt[u] = c;
      }
    } else if constexpr (BPT == 2) {
      const uint2 hb = *reinterpret_cast<const uint2*>(&h[2 * tid]);
      cnt[0] = (int)hb.x; cnt[1] = (int)hb.y;
    } else {
#pragma unroll
      for (int q = 0; q < BPT / 4; ++q) {
        const uint4 hb = *reinterpret_cast<const uint4*>(&h[BPT * tid + 4 * q]);
        cnt[4 * q] = (int)hb.x; cnt[4 * q + 1] = (int)hb.y;
        cnt[4 * q + 2] = (int)hb.z; cnt[4 * q + 3] = (int)hb.w;
      }
    }
    int loc = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) loc += cnt[u];
    int suf = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += v;
    }
    if (lane == 0) wtot[wave] = suf;
    __syncthreads();
    int above = suf - loc;
#pragma unroll
    for (int w = 0; w < NW; ++w) above += w > wave ? wtot[w] : 0;
#pragma unroll
    for (int u = BPT - 1; u >= 0; --u) {
      if (above < kk && above + cnt[u] >= kk) {
        meta[0] = BPT * tid + u;
        meta[1] = above;
        meta[2] = above + cnt[u] == kk ? 1 : 0;
      }
      above += cnt[u];
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)meta[0];
    kk -= meta[1];
    prefix |= digit << shift;
    pmask |= dmask << shift;
    buf ^= 1;
    if (meta[2] != 0) break;  // uniform: the bin is taken whole
  }

  // prefix is the k-th largest key K: keep every key > K and the first kk
  // copies of K, in index order
  const uint32_t K = prefix;
  const uint64_t lt = lanemask_lt(lane);
  // slices in groups of GS: the ballots of a group are in flight together
  // (all 2 KPT of them would not fit the scalar registers)
  constexpr int GS = KPT < 8 ? KPT : 8;
#pragma unroll
  for (int j0 = 0; j0 < KPT; j0 += GS) {
    uint64_t mg[GS], me[GS];
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      mg[u] = __ballot(key[j0 + u] > K);
      me[u] = __ballot(key[j0 + u] == K);
    }
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < GS; ++u) {
        gtot[(j0 + u) * NW + wave] = __popcll(mg[u]);
        etot[(j0 + u) * NW + wave] = __popcll(me[u]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  // exclusive prefix over the KPT x NW (slice, wave) counts in index order:
  // thread s takes entry s (KPT NW <= NT), inclusive scans within each wave,
  // then each wave adds the totals of the waves before it
  {
    constexpr int E = KPT * NW;
    const int g = tid < E ? gtot[tid] : 0, e = tid < E ? etot[tid] : 0;
    int ig = g, ie = e;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int vg = __shfl_up(ig, off, 64), ve = __shfl_up(ie, off, 64);
      if (lane >= off) { ig += vg; ie += ve; }
    }
    if (lane == 63) { wsg[wave] = ig; wse[wave] = ie; }
    __syncthreads();
    int bg = 0, be = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) { bg += wsg[w]; be += wse[w]; }
    if (tid < E) { gtot[tid] = bg + ig - g; etot[tid] = be + ie - e; }
  }
  __syncthreads();
  // the ballots are recomputed rather than kept: opaque keys stop the
  // compiler from reusing the first ones
#pragma unroll
  for (int j = 0; j < KPT; ++j) asm volatile("" : "+v"(key[j]));
  // (the row's k slots through a bounded descriptor: 32-bit offsets)
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(out, 0, k * 4, 0x00020000);
#pragma unroll
  for (int j0 = 0; j0 < KPT; j0 += GS) {
    int gb0[GS], eb0[GS];
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      gb0[u] = gtot[(j0 + u) * NW + wave];
      eb0[u] = etot[(j0 + u) * NW + wave];
    }
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int j = j0 + u;
      const bool gt = key[j] > K, eq = key[j] == K;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      int pos;
      bool take;
      if (me == 0ull) {
        // no copy of K among this wave's keys of the slice (nearly every
        // slice): the copies before it are all counted in eb0
        pos = gb0[u] + __popcll(mg & lt) + min(eb0[u], kk);
        take = gt;
      } else {
        const int eb = eb0[u] + __popcll(me & lt);
        pos = gb0[u] + __popcll(mg & lt) + min(eb, kk);
        take = gt || (eq && eb < kk);
      }
      if (take) __builtin_amdgcn_raw_buffer_store_b32(j * NT + tid, ors, 4 * pos, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int* idx, const int* q_pos, int B, int S,
                       int T, int k, int m, hipStream_t s) {
  const long rows = (long)B * S;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)rows);
  // short rows: 256 threads, so that eight rows share a compute unit; rows of
  // more than 8192 entries: 1024 threads with 32 keys each (measured 13%
  // faster on the DSA rows than 512 threads with 64 keys, whose 168 registers
  // also leave room for one row per compute unit)
  if (T <= 2048)
    hipLaunchKernelGGL((topk_reg<8, 256>), grid, dim3(256), 0, s, scores, idx, q_pos, S, T, k, m);
  else if (T <= 16 * 512)
    hipLaunchKernelGGL((topk_reg<16, 512>), grid, dim3(512), 0, s, scores, idx, q_pos, S, T, k, m);
  else if (T <= 32 * 1024)
    hipLaunchKernelGGL((topk_reg<32, 1024>), grid, dim3(1024), 0, s, scores, idx, q_pos, S, T, k,
                       m);
  else
    hipLaunchKernelGGL(topk_global, grid, dim3(kTopkThreads), 0, s, scores, idx, q_pos, S, T, k,
                       m);
  return hipGetLastError();
}

}  // namespace csa
