// index_scores.hip -- Lightning-Indexer index scores.
//
// Page "DeepSeek-V4", section "Hybrid attention (§2.3)": the indexer scores
// each query against the compressed pool (eqs. 13-17) with n_h^I heads of
// width c^I (DeepseekV4Config index_n_heads, index_head_dim).  Page
// "DeepSeek-V3.2", section "DeepSeek Sparse Attention (DSA)": the score is a
// low-head-count dot product between the query heads and one shared key head,
// combined with per-head weights.  Score of entry w for the query at t:
//     I(t, w) = sum_j w_idx[t, j] * max(0, <q_idx[t, j], k_pool[w]>),  w < R(t)
//
// bf16 path (the hot one): a GEMM with the indexer HEADS on the matrix-core M
// dimension and pool entries on N (K = c^I).  v_mfma_f32_32x32x16_bf16 leaves
// each lane 16 heads of one entry, so the ReLU-and-weight epilogue reduces over
// heads inside the lane and one cross-half swap finishes the head sum: no LDS
// round trip for the reduction.  Query fragments (the A operand) stay in
// registers; pool rows come in through direct-to-LDS loads of whole cache
// lines, their 16-byte chunks swizzled by row so that B-fragment reads fall in
// distinct banks.  Two kernels:
//   many query rows (prefill, token-level indexer): 4 rows per workgroup share
//     each 64-entry tile of the pool, two workgroups per compute unit
//     (MFMA-bound);
//   few query rows (decode): a pool entry meets one query row only, so each
//     wave streams its own blocks and the pool is split over workgroups so
//     that the whole chip streams it (HBM-bound).
// fp32 (and unusual shapes): a plain kernel, one thread per (row, entry).
#include "csa_device.hpp"

#include <type_traits>

namespace csa {
namespace {

constexpr int kIdxTile = 128;  // pool entries per LDS tile
// cache-policy operand of a buffer load: the non-temporal hint ("nt")
constexpr int kCacheNT = 2;

// max(x, 0) as one integer max on the bit pattern: a negative float (sign bit
// set) is a negative integer, so it becomes +0; everything else is unchanged.
// (fmaxf would cost a second instruction per value: the compiler first quiets
// a possible signalling NaN coming out of the matrix core.)
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Many query rows (prefill, token-level indexer): workgroup = QR consecutive
// query rows (one per wave) x one chunk of the pool.  The pool is walked in
// NT-entry tiles (NT = 16 QR, so QR x 4 KiB), triple-buffered in LDS and
// shared by the QR rows: each wave fills four 1 KiB slices of every tile, two
// tiles ahead of the products, with one barrier per tile.  Each wave keeps its row's
// query fragments (the A operand, 64 heads x 128) in registers and, per
// 32-entry block, runs 16 matrix instructions, the ReLU-and-weight epilogue
// and one 128-byte store.  Row blocks are launched heaviest first.
template <int NI, int CI, int QR, int NT>
__global__ __launch_bounds__(64 * QR) void index_scores_mfma(
    const u16* __restrict__ q_idx, const float* __restrict__ w_idx,
    const u16* __restrict__ k_pool, float* __restrict__ scores,
    const int* __restrict__ q_pos, int S, int T, int m, int chunk) {
  // QR query rows = waves per workgroup, NT entries per tile
  constexpr int MB = NI / 32;      // 32-head blocks
  constexpr int KS = CI / 16;      // k-steps of 16
  constexpr int TB = NT * CI * 2;  // bytes per tile
  constexpr int SPT = NT / 32;     // 32-entry blocks (and stores) per tile
  static_assert(TB == QR * 4096, "each wave fills four 1 KiB slices of a tile");
  static_assert(CI == 128, "a key row is 16 chunks of 16 bytes");
  static_assert(NI <= 64, "one head weight per lane");
  // one static array per buffer (a load in flight into one buffer then does
  // not look like it aliases reads of another)
  __shared__ __attribute__((aligned(16))) unsigned char kb0[TB];
  __shared__ __attribute__((aligned(16))) unsigned char kb1[TB];
  __shared__ __attribute__((aligned(16))) unsigned char kb2[TB];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int b = blockIdx.z;
  const int rb = gridDim.x - 1 - blockIdx.x;  // heaviest (latest) rows first
  const int i0 = rb * QR;
  const long qp = q_pos[b];
  int r_wg = 0;
#pragma unroll
  for (int r = 0; r < QR; ++r)
    if (i0 + r < S) r_wg = max(r_wg, ready_count(qp + i0 + r, m, T));
  const int lo = blockIdx.y * chunk;
  const int hi = min(r_wg, lo + chunk);
  if (lo >= hi) return;  // uniform over the workgroup
  const int my_i = i0 + wave;
  const bool valid = my_i < S;
  const int hi_my = valid ? min(ready_count(qp + my_i, m, T), lo + chunk) : lo;
  const long row = (long)b * S + (valid ? my_i : 0);

  // A fragments: a[mb][ks] = q_idx[row][32mb + lane%32][16ks + 8(lane/32) .. +7]
  bf16x8 a[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a[mb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(
          q_idx + (row * NI + 32 * mb + (lane & 31)) * CI + 16 * ks + 8 * (lane >> 5)));
  // head weights in accumulator order: wreg[mb][q] = w_idx[row][32mb + 8q +
  // 4(lane/32) .. +3]
  float4 wreg[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      wreg[mb][q] = *reinterpret_cast<const float4*>(w_idx + row * NI + 32 * mb + 8 * q +
                                                     4 * (lane >> 5));

  // pool rows lo .. hi-1 of this sequence
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(k_pool + ((long)b * T + lo) * CI), 0, (hi - lo) * CI * 2, 0x00020000);
  const int klim = (hi - lo) * CI * 2 - 16;   // the range's last 16-byte chunk
  // this wave's slices of a tile: 1 KiB slice g = 4 wave + q (rows 4g .. 4g+3);
  // lane l fills LDS slot l of the slice with chunk (l % 16) ^ (row % 16) of
  // row 4g + l / 16 (row % 16 depends on q only)
  int loff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    loff[q] = (lane >> 4) * 256 + 16 * ((lane & 15) ^ ((4 * q + (lane >> 4)) & 15));
  auto issue = [&](auto JC, int tile) __attribute__((always_inline)) {
    constexpr int J = decltype(JC)::value;
    unsigned char* buf = J == 0 ? kb0 : J == 1 ? kb1 : kb2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int g = 4 * wave + q;
      // (every lane's address is clamped into the key rows of the range: a
      // slot past the range re-reads its last chunk, which no score uses, so
      // no load ever touches memory past the tensor)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(buf + g * 1024), 16,
                                               min(loff[q] + tile * TB + g * 1024, klim), 0, 0,
                                               0);
    }
  };
  // B-fragment read address: row 32nb + lane%32, chunk 2ks + lane/32
  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    roff[ks] = (lane & 31) * 256 + 16 * ((2 * ks + (lane >> 5)) ^ (lane & 15));

  // scores of this row within the chunk: a bounded buffer store drops lanes
  // past the row's ready entries (and the upper half, which holds copies).
  // A row of the block can end before the chunk starts (rows of one block
  // differ in readiness by up to three entries at m = 1): its range is then
  // empty, never negative, which would wrap the descriptor's byte count and
  // let every store through.
  const __amdgpu_buffer_rsrc_t out_rs = __builtin_amdgcn_make_buffer_rsrc(
      scores + row * T + lo, 0, max(hi_my - lo, 0) * 4, 0x00020000);

  // tile j: the products of the 8 rows on buffer J, four 32-entry blocks per
  // wave; blocks past the row's entries are skipped, but every block issues
  // exactly one store (dropped past the row's entries), which keeps the wait
  // counts below exact.  The epilogue sums in four independent chains.
  auto compute = [&](auto JC, int tile) __attribute__((always_inline)) {
    constexpr int J = decltype(JC)::value;
    const unsigned char* buf = J == 0 ? kb0 : J == 1 ? kb1 : kb2;
#pragma unroll
    for (int nb = 0; nb < NT / 32; ++nb) {
      const int e0 = tile * NT + 32 * nb;  // first entry of the block, from lo
      float part = 0.f;
      if (lo + e0 < hi_my) {
        f32x16 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
        // the B fragment of k-step ks + 1 is read before the products of
        // k-step ks, so its LDS latency hides under them
        uint4 bv[2];
        bv[0] = *reinterpret_cast<const uint4*>(buf + nb * 8192 + roff[0]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS)
            bv[(ks + 1) & 1] = *reinterpret_cast<const uint4*>(buf + nb * 8192 + roff[ks + 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb] = mfma32x32x16(a[mb][ks], as_bf16x8(bv[ks & 1]), acc[mb]);
          __builtin_amdgcn_sched_barrier(0);
        }
        // accumulator register r holds head 32mb + 8(r/4) + 4(lane/32) + r%4
        float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 w4 = wreg[mb][q];
            p4[0] += w4.x * relu_bits(acc[mb][4 * q]);
            p4[1] += w4.y * relu_bits(acc[mb][4 * q + 1]);
            p4[2] += w4.z * relu_bits(acc[mb][4 * q + 2]);
            p4[3] += w4.w * relu_bits(acc[mb][4 * q + 3]);
          }
        part = (p4[0] + p4[1]) + (p4[2] + p4[3]);
        // the other half of the heads sits in lane l ^ 32
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                         __float_as_uint(part), false, false);
        part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      const int off = (lane < 32) ? (e0 + lane) * 4 : 0x40000000;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((part == 0.f) ? 0.f : part), out_rs,
                                            off, 0, 0);
    }
  };

  // Tile j: wait for this wave's slices of tile j, barrier (then every slice
  // of tile j has landed and every wave is done with tile j-1, whose buffer
  // takes tile j+2), refill, products.  After the loads of tile j a wave has
  // issued at most: 4 stores (tile j-2), 4 loads (tile j+1), 4 stores (tile
  // j-1).
  const int ntiles = (hi - lo + NT - 1) / NT;
  issue(std::integral_constant<int, 0>{}, 0);
  issue(std::integral_constant<int, 1>{}, 1);
  wait_vmcnt<4>();
  lds_barrier();
  issue(std::integral_constant<int, 2>{}, 2);
  compute(std::integral_constant<int, 0>{}, 0);
  wait_vmcnt<4 + SPT>();
  lds_barrier();
  issue(std::integral_constant<int, 0>{}, 3);
  compute(std::integral_constant<int, 1>{}, 1);
  for (int j = 2; j < ntiles; j += 3) {  // whole rounds: every wave, every path
    wait_vmcnt<4 + 2 * SPT>();
    lds_barrier();
    issue(std::integral_constant<int, 1>{}, j + 2);
    compute(std::integral_constant<int, 2>{}, j);
    wait_vmcnt<4 + 2 * SPT>();
    lds_barrier();
    issue(std::integral_constant<int, 2>{}, j + 3);
    compute(std::integral_constant<int, 0>{}, j + 1);
    wait_vmcnt<4 + 2 * SPT>();
    lds_barrier();
    issue(std::integral_constant<int, 0>{}, j + 4);
    compute(std::integral_constant<int, 1>{}, j + 2);
  }
  wait_vmcnt<0>();  // no load into LDS outlives the workgroup
}

// ---------------------------------------------------------------- fused top-k
// Order-preserving 32-bit key of a score (-0 folded onto +0): larger score,
// larger key; every non-NaN score maps above 0.
__device__ __forceinline__ uint32_t topk_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k of one row by one wave: the row's R scores (R <= 64 KPL) sit in LDS
// (`sc`); lane l takes entries 64 u + l.  Radix select (most significant digit
// first, up to three digits of up to 11 bits over the key's offset above the
// row's smallest key) with the wave's own 2048-bin histogram `h` in LDS, then
// an ordered compaction by ballots: every key above the k-th largest K, and
// the first copies of K in index order, written in ascending index order,
// then -1 in the remaining slots.  (LDS operations of one wave complete in
// order, so the wave needs no barrier between its own writes and reads.)
template <int KPL>
__device__ __forceinline__ void wave_topk(const float* sc, uint32_t* h, int R, int k, int* out,
                                          int lane) {
  if (R <= k) {
    for (int j = lane; j < k; j += 64) out[j] = j < R ? j : -1;
    return;
  }
  uint32_t key[KPL];
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int j = 64 * u + lane;
    key[u] = j < R ? topk_key(sc[j]) : 0u;
    if (key[u] != 0u) { lo = min(lo, key[u]); hi = max(hi, key[u]); }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
  }
#pragma unroll
  for (int u = 0; u < KPL; ++u) key[u] = key[u] != 0u ? key[u] - lo + 1u : 0u;
  const int nbits = 32 - (int)__builtin_clz(hi - lo + 1u);
  uint32_t prefix = 0u, pmask = 0u;
  int kk = k;
  for (int pass = 0; pass < 3; ++pass) {
    const int top = nbits - 11 * pass;
    if (top <= 0) break;
    const int shift = max(top - 11, 0);
    const uint32_t dmask = (1u << (top - shift)) - 1u;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      *reinterpret_cast<uint4*>(h + 256 * q + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < KPL; ++u)
      if (key[u] != 0u && (key[u] & pmask) == prefix) atomicAdd(&h[(key[u] >> shift) & dmask], 1u);
    // lane l owns bins 32 l .. 32 l + 31: suffix sums over the bins above
    int cnt[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 v = *reinterpret_cast<const uint4*>(h + 32 * lane + 4 * q);
      cnt[4 * q] = (int)v.x; cnt[4 * q + 1] = (int)v.y;
      cnt[4 * q + 2] = (int)v.z; cnt[4 * q + 3] = (int)v.w;
    }
    int loc = 0;
#pragma unroll
    for (int u = 0; u < 32; ++u) loc += cnt[u];
    int suf = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += v;
    }
    int above = suf - loc, dig = -1, abv = 0;
#pragma unroll
    for (int u = 31; u >= 0; --u) {
      if (above < kk && above + cnt[u] >= kk) { dig = 32 * lane + u; abv = above; }
      above += cnt[u];
    }
    const uint64_t own = __ballot(dig >= 0);
    const int src = (int)__builtin_ctzll(own);
    const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane(dig, src);
    kk -= __builtin_amdgcn_readlane(abv, src);
    prefix |= digit << shift;
    pmask |= dmask << shift;
  }
  const uint32_t K = prefix;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int sel = 0, eqs = 0;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const bool gt = key[u] > K, eq = key[u] == K;
    const uint64_t me = __ballot(eq);
    const bool take = gt || (eq && eqs + __popcll(me & lt) < kk);
    const uint64_t mt = __ballot(take);
    if (take) out[sel + __popcll(mt & lt)] = 64 * u + lane;
    sel += __popcll(mt);
    eqs += __popcll(me);
  }
  for (int j = sel + lane; j < k; j += 64) out[j] = -1;
}

// Index scores and top-k in one kernel (rows of at most TMAX ready entries):
// the scores of index_scores_mfma (the same products, epilogue and order, so
// the same bits) go to LDS instead of HBM, one TMAX-entry array per row, and
// when every tile is done each wave selects its own row's top-k from its
// array (wave_topk), its histogram in the freed tile buffers.  Nothing but the
// index rows is written.
template <int NI, int CI, int QR, int NT, int TMAX>
__global__ __launch_bounds__(64 * QR) void index_topk_fused(
    const u16* __restrict__ q_idx, const float* __restrict__ w_idx,
    const u16* __restrict__ k_pool, int* __restrict__ idx, const int* __restrict__ q_pos,
    int S, int T, int m, int k) {
  constexpr int MB = NI / 32;
  constexpr int KS = CI / 16;
  constexpr int TB = NT * CI * 2;
  static_assert(TB == QR * 4096, "each wave fills four 1 KiB slices of a tile");
  static_assert(CI == 128 && NI <= 64, "shape");
  static_assert(QR * 8192 <= 3 * TB, "the histograms fit the tile buffers");
  __shared__ __attribute__((aligned(16))) unsigned char kb0[TB];
  __shared__ __attribute__((aligned(16))) unsigned char kb1[TB];
  __shared__ __attribute__((aligned(16))) unsigned char kb2[TB];
  __shared__ __attribute__((aligned(16))) float sc[QR][TMAX];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int b = blockIdx.z;
  const int rb = gridDim.x - 1 - blockIdx.x;  // heaviest (latest) rows first
  const int i0 = rb * QR;
  const long qp = q_pos[b];
  int r_wg = 0;
#pragma unroll
  for (int r = 0; r < QR; ++r)
    if (i0 + r < S) r_wg = max(r_wg, ready_count(qp + i0 + r, m, T));
  const int my_i = i0 + wave;
  const bool valid = my_i < S;
  const int R_my = valid ? ready_count(qp + my_i, m, T) : 0;
  const long row = (long)b * S + (valid ? my_i : 0);

  bf16x8 a[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a[mb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(
          q_idx + (row * NI + 32 * mb + (lane & 31)) * CI + 16 * ks + 8 * (lane >> 5)));
  float4 wreg[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      wreg[mb][q] = *reinterpret_cast<const float4*>(w_idx + row * NI + 32 * mb + 8 * q +
                                                     4 * (lane >> 5));
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(k_pool + (long)b * T * CI), 0, r_wg * CI * 2, 0x00020000);
  const int klim = r_wg * CI * 2 - 16;        // the range's last 16-byte chunk
  int loff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    loff[q] = (lane >> 4) * 256 + 16 * ((lane & 15) ^ ((4 * q + (lane >> 4)) & 15));
  auto issue = [&](auto JC, int tile) __attribute__((always_inline)) {
    constexpr int J = decltype(JC)::value;
    unsigned char* buf = J == 0 ? kb0 : J == 1 ? kb1 : kb2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int g = 4 * wave + q;
      // (every lane's address is clamped into the key rows of the range: a
      // slot past the range re-reads its last chunk, which no score uses, so
      // no load ever touches memory past the tensor)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(buf + g * 1024), 16,
                                               min(loff[q] + tile * TB + g * 1024, klim), 0, 0,
                                               0);
    }
  };
  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    roff[ks] = (lane & 31) * 256 + 16 * ((2 * ks + (lane >> 5)) ^ (lane & 15));
  float* my_sc = sc[wave];
  auto compute = [&](auto JC, int tile) __attribute__((always_inline)) {
    constexpr int J = decltype(JC)::value;
    const unsigned char* buf = J == 0 ? kb0 : J == 1 ? kb1 : kb2;
#pragma unroll
    for (int nb = 0; nb < NT / 32; ++nb) {
      const int e0 = tile * NT + 32 * nb;
      if (e0 < R_my) {
        f32x16 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
        // the B fragment of k-step ks + 1 is read before the products of
        // k-step ks, so its LDS latency hides under them
        uint4 bv[2];
        bv[0] = *reinterpret_cast<const uint4*>(buf + nb * 8192 + roff[0]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS)
            bv[(ks + 1) & 1] = *reinterpret_cast<const uint4*>(buf + nb * 8192 + roff[ks + 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb] = mfma32x32x16(a[mb][ks], as_bf16x8(bv[ks & 1]), acc[mb]);
          __builtin_amdgcn_sched_barrier(0);
        }
        float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 w4 = wreg[mb][q];
            p4[0] += w4.x * relu_bits(acc[mb][4 * q]);
            p4[1] += w4.y * relu_bits(acc[mb][4 * q + 1]);
            p4[2] += w4.z * relu_bits(acc[mb][4 * q + 2]);
            p4[3] += w4.w * relu_bits(acc[mb][4 * q + 3]);
          }
        float part = (p4[0] + p4[1]) + (p4[2] + p4[3]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                         __float_as_uint(part), false, false);
        part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if (lane < 32 && e0 + lane < R_my) my_sc[e0 + lane] = (part == 0.f) ? 0.f : part;
      }
    }
  };

  // tile j: wait for this wave's slices of tile j (the loads of tile j + 1
  // may stay in flight), barrier, refill the buffer of tile j - 1 with tile
  // j + 2, products
  const int ntiles = (r_wg + NT - 1) / NT;
  if (ntiles > 0) {
    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
    wait_vmcnt<4>();
    lds_barrier();
    issue(std::integral_constant<int, 2>{}, 2);
    compute(std::integral_constant<int, 0>{}, 0);
    wait_vmcnt<4>();
    lds_barrier();
    issue(std::integral_constant<int, 0>{}, 3);
    compute(std::integral_constant<int, 1>{}, 1);
    for (int j = 2; j < ntiles; j += 3) {
      wait_vmcnt<4>();
      lds_barrier();
      issue(std::integral_constant<int, 1>{}, j + 2);
      compute(std::integral_constant<int, 2>{}, j);
      wait_vmcnt<4>();
      lds_barrier();
      issue(std::integral_constant<int, 2>{}, j + 3);
      compute(std::integral_constant<int, 0>{}, j + 1);
      wait_vmcnt<4>();
      lds_barrier();
      issue(std::integral_constant<int, 0>{}, j + 4);
      compute(std::integral_constant<int, 1>{}, j + 2);
    }
  }
  wait_vmcnt<0>();
  lds_barrier();  // every wave is done with the tile buffers
  if (!valid) return;
  unsigned char* hb = (wave >> 1) == 0 ? kb0 : (wave >> 1) == 1 ? kb1 : kb2;
  wave_topk<TMAX / 64>(my_sc, reinterpret_cast<uint32_t*>(hb + (wave & 1) * 8192), R_my, k,
                       idx + row * k, lane);
}

// Streaming kernel for few query rows.  Workgroup (x = query row, y = pool
// chunk); wave w scores 32-entry blocks w, w + 4, w + 8, ... of the chunk.
// A block (32 rows x 256 bytes, contiguous in HBM) comes in with eight
// direct-to-LDS 16-byte buffer loads, each reading 1 KiB contiguous (whole
// cache lines, once); lane l of load i fills LDS slot l of rows 4i .. 4i+3
// with the 16-byte chunk (l % 16) ^ (row % 16) of its row, so that the
// B-fragment reads (32 rows, one chunk each) fall in distinct banks.  Two
// buffers per wave: a block's fragments are read into registers as soon as it
// lands, and its buffer is refilled at once, so two blocks stay in flight per
// wave.  Query fragments (the A operand) stay in registers.  A wave with no
// block leaves at once; the chunk is covered in whole rounds of two blocks
// (blocks past the end re-read the chunk's last bytes; their scores are
// dropped).
template <int NI, int CI>
__global__ __launch_bounds__(256, 2) void index_scores_stream(
    const u16* __restrict__ q_idx, const float* __restrict__ w_idx,
    const u16* __restrict__ k_pool, float* __restrict__ scores,
    const int* __restrict__ q_pos, int S, int T, int m, int chunk) {
  constexpr int MB = NI / 32;      // 32-head blocks
  constexpr int KS = CI / 16;      // k-steps of 16
  constexpr int BLK = 32 * CI * 2;  // bytes per block
  static_assert(CI == 128, "a key row is 16 chunks of 16 bytes");
  static_assert(NI <= 64, "one head weight per lane");
  // one static array per buffer: the compiler then sees that a load in flight
  // into one buffer does not alias reads of the other
  __shared__ __attribute__((aligned(16))) unsigned char kb0[4][BLK];
  __shared__ __attribute__((aligned(16))) unsigned char kb1[4][BLK];
  __shared__ __attribute__((aligned(16))) float wsh[4][64];
  // the wave index is uniform: keep it (and the block loop) scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const long row = blockIdx.x;
  const int b = (int)(row / S), i = (int)(row - (long)b * S);
  const int R = ready_count((long)q_pos[b] + i, m, T);
  const int lo = blockIdx.y * chunk;
  const int hi = min(R, lo + chunk);
  const int nblk = (hi - lo + 31) >> 5;
  int blk = wave;
  if (blk >= nblk) return;  // wave-uniform

  // key rows lo .. hi-1 of this sequence
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(k_pool + ((long)b * T + lo) * CI), 0, (hi - lo) * CI * 2, 0x00020000);
  const int klim = (hi - lo) * CI * 2 - 16;   // the chunk's last 16-byte chunk
  // per-lane source offset of load i within its 1 KiB (rows 4i .. 4i+3); it
  // depends on i % 4 only
  int loff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * q + (lane >> 4);  // row within the block, mod 16
    loff[q] = (lane >> 4) * 256 + 16 * ((lane & 15) ^ (r & 15));
  }
  auto issue = [&](auto JC, int bk) __attribute__((always_inline)) {
    unsigned char* buf = decltype(JC)::value ? kb1[wave] : kb0[wave];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      // (addresses clamped into the chunk's rows: a block past the chunk
      // re-reads its last 16 bytes, whose scores are dropped, so no load
      // touches memory past the tensor)
      // (non-temporal: the pool is streamed once, and the loads marked so
      // measured 11% faster than plain ones on the 537 MB decode pool)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(buf + q * 1024), 16,
                                               min(loff[q & 3] + bk * BLK + q * 1024, klim), 0,
                                               0, kCacheNT);
    }
  };
  // head weights to LDS (lane l: 4 bytes at +4l), A fragments to registers:
  // a[mb][ks] = q_idx[row][32mb + lane%32][16ks + 8(lane/32) .. +7]
  {
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(w_idx + row * NI), 0, NI * 4, 0x00020000);
    const int woff = lane * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void*)&wsh[wave][0], 4, woff, 0, 0, 0);
  }
  bf16x8 a[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a[mb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(
          q_idx + (row * NI + 32 * mb + (lane & 31)) * CI + 16 * ks + 8 * (lane >> 5)));

  // query loads first, then the key blocks: waits count loads in issue order
  __builtin_amdgcn_sched_barrier(0);
  issue(std::integral_constant<int, 0>{}, blk);
  issue(std::integral_constant<int, 1>{}, blk + 4);
  __builtin_amdgcn_sched_barrier(0);

  // B-fragment read addresses: row lane%32, chunk 2ks + lane/32 (swizzled)
  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int r = lane & 31, c = 2 * ks + (lane >> 5);
    roff[ks] = r * 256 + 16 * (c ^ (r & 15));
  }

  // scores of this row and chunk go out through a bounded buffer store: lanes
  // past the chunk (and the upper half, which holds copies) are dropped by the
  // hardware, so the store needs no branch
  const __amdgpu_buffer_rsrc_t out_rs = __builtin_amdgcn_make_buffer_rsrc(
      scores + row * T + lo, 0, (hi - lo) * 4, 0x00020000);

  auto step = [&](auto JC, int bk) __attribute__((always_inline)) {
    const unsigned char* buf = decltype(JC)::value ? kb1[wave] : kb0[wave];
    uint4 bv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bv[ks] = *reinterpret_cast<const uint4*>(buf + roff[ks]);
    // the fragments are in registers once these reads are done: refill (the
    // scheduling barriers keep one block's reads, refill and products
    // together, in this order)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    issue(JC, bk + 8);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32x32x16(a[mb][ks], as_bf16x8(bv[ks]), acc[mb]);
    // accumulator register r holds head 32mb + 8(r/4) + 4(lane/32) + r%4
    float part = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 w4 = *reinterpret_cast<const float4*>(
            &wsh[wave][32 * mb + 8 * q + 4 * (lane >> 5)]);
        part += w4.x * relu_bits(acc[mb][4 * q]);
        part += w4.y * relu_bits(acc[mb][4 * q + 1]);
        part += w4.z * relu_bits(acc[mb][4 * q + 2]);
        part += w4.w * relu_bits(acc[mb][4 * q + 3]);
      }
    // the other half of the heads sits in lane l ^ 32
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                     __float_as_uint(part), false, false);
    part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int off = (lane < 32) ? (32 * bk + lane) * 4 : 0x40000000;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((part == 0.f) ? 0.f : part), out_rs,
                                          off, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  const int rounds = ((nblk - wave + 3) / 4 + 1) / 2;  // >= 1
  int it = 0;
  do {
    step(std::integral_constant<int, 0>{}, blk);
    step(std::integral_constant<int, 1>{}, blk + 4);
    blk += 8;
  } while (++it < rounds);
}

template <bool BF16>
__global__ __launch_bounds__(256) void index_scores_generic(
    const void* __restrict__ q_idx, const float* __restrict__ w_idx,
    const void* __restrict__ k_pool, float* __restrict__ scores,
    const int* __restrict__ q_pos, int S, int T, int n_heads, int head_dim, int m) {
  extern __shared__ float sq[];  // [n_heads * head_dim] queries, then [n_heads] weights
  const long row = blockIdx.x;
  const int b = (int)(row / S), i = (int)(row - (long)b * S);
  const int R = ready_count((long)q_pos[b] + i, m, T);
  if ((int)blockIdx.y * 256 >= R) return;  // uniform
  const int nq = n_heads * head_dim;
  for (int e = threadIdx.x; e < nq; e += 256) sq[e] = load1<BF16>(q_idx, row * nq + e);
  for (int e = threadIdx.x; e < n_heads; e += 256) sq[nq + e] = w_idx[row * n_heads + e];
  __syncthreads();
  const int w = blockIdx.y * 256 + threadIdx.x;
  if (w >= R) return;
  const long kr = ((long)b * T + w) * head_dim;
  float s = 0.f;
  {
    // sequential sums, every product and sum rounded on its own (no fused
    // multiply-add): with fp32 inputs the scores equal a plain scalar loop's
#pragma clang fp contract(off)
    for (int j = 0; j < n_heads; ++j) {
      float dot = 0.f;
      for (int c = 0; c < head_dim; ++c)
        dot += sq[j * head_dim + c] * load1<BF16>(k_pool, kr + c);
      s += sq[nq + j] * fmaxf(dot, 0.f);
    }
  }
  scores[row * T + w] = (s == 0.f) ? 0.f : s;
}

}  // namespace

// Shapes the fused kernel takes: bf16, 64 x 128 indexer heads, at least 16
// query rows per sequence, rows of at most 2048 entries, compressed pools
// (m >= 2: the CSA prefill shape; token-level rows take the workspace path).
bool index_topk_fused_shape(int S, int T, int n_heads, int head_dim, int k, int m, bool bf16) {
  return bf16 && n_heads == 64 && head_dim == 128 && S >= 16 && T <= 2048 && k >= 1 && m >= 2;
}

hipError_t launch_index_topk_fused(const void* q_idx, const float* w_idx, const void* k_pool,
                                   int* idx, const int* q_pos, int B, int S, int T, int m,
                                   int k, hipStream_t s) {
  if (B == 0 || S == 0) return hipSuccess;
  // 4 rows per workgroup, 64-entry tiles: 48 KiB of tiles + 32 KiB of scores,
  // two workgroups per compute unit
  constexpr int QR = 4, NT = 16 * QR;
  dim3 grid((S + QR - 1) / QR, 1, B);
  hipLaunchKernelGGL((index_topk_fused<64, 128, QR, NT, 2048>), grid, dim3(64 * QR), 0, s,
                     reinterpret_cast<const u16*>(q_idx), w_idx,
                     reinterpret_cast<const u16*>(k_pool), idx, q_pos, S, T, m, k);
  return hipGetLastError();
}

hipError_t launch_index_scores(const void* q_idx, const float* w_idx, const void* k_pool,
                               float* scores, const int* q_pos, int B, int S, int T,
                               int n_heads, int head_dim, int m, bool bf16,
                               hipStream_t s) {
  if (B == 0 || S == 0 || T == 0) return hipSuccess;
  if (bf16 && n_heads == 64 && head_dim == 128) {
    const int tiles = (T + kIdxTile - 1) / kIdxTile;
    if (S < 16) {
      // about two workgroups per compute unit over all rows, each a whole
      // number of 128-entry tiles
      const long rows = (long)B * S;
      const int nchunk = (int)std::min<long>(tiles, std::max<long>(1, (512 + rows - 1) / rows));
      const int chunk_tiles = (tiles + nchunk - 1) / nchunk;
      const int chunk = chunk_tiles * kIdxTile;
      dim3 grid((unsigned)rows, (tiles + chunk_tiles - 1) / chunk_tiles);
      hipLaunchKernelGGL((index_scores_stream<64, 128>), grid, dim3(256), 0, s,
                         reinterpret_cast<const u16*>(q_idx), w_idx,
                         reinterpret_cast<const u16*>(k_pool), scores, q_pos, S, T, m, chunk);
      return hipGetLastError();
    }
    // 4 rows per workgroup and 64-entry tiles (48 KiB of LDS): two workgroups
    // share a compute unit, so one's query loads overlap the other's products
    constexpr int QR = 4, NT = 16 * QR;
    const int ntile = (T + NT - 1) / NT;
    const int nrb = (S + QR - 1) / QR;
    // split the pool over workgroups until the chip has enough of them
    const long wgs = (long)nrb * B;
    int nchunk = 1;
    if (wgs < 1024) nchunk = (int)std::min<long>(ntile, (1024 + wgs - 1) / wgs);
    int chunk_tiles = (ntile + nchunk - 1) / nchunk;
    nchunk = (ntile + chunk_tiles - 1) / chunk_tiles;
    const int chunk = chunk_tiles * NT;
    dim3 grid(nrb, nchunk, B);
    hipLaunchKernelGGL((index_scores_mfma<64, 128, QR, NT>), grid, dim3(64 * QR), 0, s,
                       reinterpret_cast<const u16*>(q_idx), w_idx,
                       reinterpret_cast<const u16*>(k_pool), scores, q_pos, S, T, m, chunk);
    return hipGetLastError();
  }
  const size_t lds = (size_t)(n_heads * head_dim + n_heads) * sizeof(float);
  dim3 grid((unsigned)((long)B * S), (T + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(index_scores_generic<true>, grid, dim3(256), lds, s, q_idx, w_idx,
                       k_pool, scores, q_pos, S, T, n_heads, head_dim, m);
  else
    hipLaunchKernelGGL(index_scores_generic<false>, grid, dim3(256), lds, s, q_idx, w_idx,
                       k_pool, scores, q_pos, S, T, n_heads, head_dim, m);
  return hipGetLastError();
}

}  // namespace csa
