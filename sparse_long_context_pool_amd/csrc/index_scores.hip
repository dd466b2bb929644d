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
// round trip for the reduction.  Query fragments stay in registers for the
// whole row; 128-entry key tiles are staged in LDS (16-byte padded rows, so the
// 32 rows a B-fragment read touches fall in distinct banks) and shared by the
// four wavefronts of a workgroup:
//   prefill (QR = 4): four consecutive query rows per workgroup, one per wave,
//     all sharing each key tile; causal row blocks are launched heaviest first.
//   decode  (QR = 1): one query row per workgroup; the four waves take the four
//     32-entry blocks of each tile, and the pool is split over workgroups so the
//     whole chip streams the key pool (HBM-bound).
// fp32 (and unusual shapes): a plain kernel, one thread per (row, entry).
#include "csa_device.hpp"

namespace csa {
namespace {

constexpr int kIdxTile = 128;  // pool entries per LDS tile

template <int NI, int CI, int QR>
__global__ __launch_bounds__(256) void index_scores_mfma(
    const u16* __restrict__ q_idx, const float* __restrict__ w_idx,
    const u16* __restrict__ k_pool, float* __restrict__ scores,
    const int* __restrict__ q_pos, int S, int T, int m, int chunk) {
  constexpr int MB = NI / 32;      // 32-head blocks
  constexpr int KS = CI / 16;      // k-steps of 16
  constexpr int ROWB = CI * 2 + 16;
  constexpr int CPR = CI / 8;      // 16-byte chunks per key row
  __shared__ __attribute__((aligned(16))) unsigned char tile[kIdxTile * ROWB];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.z;
  const int rb = gridDim.x - 1 - blockIdx.x;  // heaviest (latest) rows first
  const int i0 = rb * QR;
  const int my_i = (QR == 4) ? i0 + wave : i0;
  const bool valid = my_i < S;
  const long qp = q_pos[b];

  int r_wg = 0;
#pragma unroll
  for (int r = 0; r < QR; ++r)
    if (i0 + r < S) r_wg = max(r_wg, ready_count(qp + i0 + r, m, T));
  const int lo = blockIdx.y * chunk;
  const int hi = min(r_wg, lo + chunk);
  if (lo >= hi) return;  // uniform over the workgroup
  const int r_my = valid ? ready_count(qp + my_i, m, T) : 0;
  const long row = (long)b * S + my_i;

  // A fragments: a[mb][ks] = q_idx[row][32mb + lane%32][16ks + 8(lane/32) .. +7]
  bf16x8 a[MB][KS];
  float wv[MB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int head = 32 * mb + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (valid)
        u = *reinterpret_cast<const uint4*>(q_idx + (row * NI + head) * CI + 16 * ks +
                                            8 * (lane >> 5));
      a[mb][ks] = as_bf16x8(u);
    }
    // accumulator register r holds head 32mb + 8(r/4) + 4(lane/32) + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wv[mb][r] = valid ? w_idx[row * NI + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)]
                        : 0.f;
  }

  const long kbase = (long)b * T;
  for (int t0 = lo; t0 < hi; t0 += kIdxTile) {
    __syncthreads();
    for (int c = threadIdx.x; c < kIdxTile * CPR; c += 256) {
      const int r = c / CPR, col = c - (c / CPR) * CPR;
      const int w = t0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (w < hi) v = *reinterpret_cast<const uint4*>(k_pool + (kbase + w) * CI + col * 8);
      *reinterpret_cast<uint4*>(tile + r * ROWB + col * 16) = v;
    }
    __syncthreads();
    const int nb0 = (QR == 4) ? 0 : wave;
    const int nb1 = (QR == 4) ? kIdxTile / 32 : wave + 1;
    for (int nb = nb0; nb < nb1; ++nb) {
      const int wb = t0 + nb * 32;
      if (wb >= min(hi, r_my)) continue;  // uniform over the wave
      f32x16 acc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 bv = *reinterpret_cast<const uint4*>(
            tile + (nb * 32 + (lane & 31)) * ROWB + (16 * ks + 8 * (lane >> 5)) * 2);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32x32x16(a[mb][ks], as_bf16x8(bv), acc[mb]);
      }
      float part = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) part += wv[mb][r] * fmaxf(acc[mb][r], 0.f);
      part += shfl_xor(part, 32);
      const int w = wb + lane;
      if (lane < 32 && w < hi && w < r_my) scores[row * T + w] = (part == 0.f) ? 0.f : part;
    }
  }
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

hipError_t launch_index_scores(const void* q_idx, const float* w_idx, const void* k_pool,
                               float* scores, const int* q_pos, int B, int S, int T,
                               int n_heads, int head_dim, int m, bool bf16,
                               hipStream_t s) {
  if (B == 0 || S == 0 || T == 0) return hipSuccess;
  if (bf16 && n_heads == 64 && head_dim == 128) {
    const int QR = (S >= 16) ? 4 : 1;
    const int nrb = (S + QR - 1) / QR;
    // split the pool over workgroups until the chip has enough of them
    int tiles = (T + kIdxTile - 1) / kIdxTile;
    long wgs = (long)nrb * B;
    int nchunk = 1;
    if (QR == 1) nchunk = tiles < 8 ? 1 : tiles / 8;             // ~1024 entries each
    else if (wgs < 1024) nchunk = (int)std::min<long>(tiles, (1024 + wgs - 1) / wgs);
    int chunk_tiles = (tiles + nchunk - 1) / nchunk;
    nchunk = (tiles + chunk_tiles - 1) / chunk_tiles;
    const int chunk = chunk_tiles * kIdxTile;
    dim3 grid(nrb, nchunk, B);
    if (QR == 4)
      hipLaunchKernelGGL((index_scores_mfma<64, 128, 4>), grid, dim3(256), 0, s,
                         reinterpret_cast<const u16*>(q_idx), w_idx,
                         reinterpret_cast<const u16*>(k_pool), scores, q_pos, S, T, m, chunk);
    else
      hipLaunchKernelGGL((index_scores_mfma<64, 128, 1>), grid, dim3(256), 0, s,
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
