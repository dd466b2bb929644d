// out_proj.hip -- grouped low-rank output projection of the attention output.
//
// Page "DeepSeek-V4", section "Hybrid attention (§2.3)", bullet on the grouped
// low-rank output projection: the H attention heads are split into o_groups
// groups; each group's concatenated head outputs go through their own
// projection to o_lora_rank values (o_a_proj, a grouped linear map), the
// o_groups results are concatenated and one more linear map (o_b_proj) takes
// them to hidden_size.  DeepseekV4Config: o_groups = 8, o_lora_rank = 1024,
// hidden_size = 4096, no bias.  With the attention output o[M][H][dv]:
//     mid[m][g r + j] = sum_c o[m][g Kg + c] * Wa[g][j][c]     (Kg = H dv / G)
//     out[m][n]      = sum_i mid[m][i] * Wb[n][i]
// Both are GEMMs with both operands contiguous along the reduction ("NT"):
// activations [rows][K] and nn.Linear-style weights [out][K].
//
// Matrix-core kernel (bf16, fp32 accumulation): a 256 x 256 output tile per
// workgroup of 8 waves, K in steps of 32 through a 5-deep ring of LDS tiles
// (160 KiB: four tiles in flight, one static array per stage) filled by
// direct-to-LDS 16-byte buffer loads (each wave loads 4 KiB of each tile,
// spread between its products).  The MFMA (v_mfma_f32_32x32x16_bf16) takes weight rows as its A
// operand and token rows as its B operand, so the accumulator of a lane holds
// four consecutive output features of one token: 8-byte bf16 stores.  Each
// wave owns 128 features x 64 tokens (4 x 2 blocks of 32 x 32).  Tile rows are
// 64 bytes (four 16-byte chunks); chunk c of row r sits at c ^ ((r / 4) % 4),
// so the 16 lanes of one LDS read phase (16 consecutive rows, one chunk) hit
// distinct banks.  Token rows past M re-read row M - 1 and their stores are
// dropped (bounded descriptor).
// Generic kernel (fp32, other shapes): one thread per output element, the
// sum taken in k order.
#include <type_traits>

#include "csa_device.hpp"

namespace csa {
namespace {

constexpr int kGM = 256;     // tokens per workgroup tile
constexpr int kGN = 256;     // output features per workgroup tile
constexpr int kGK = 32;      // reduction step
constexpr int kGStages = 5;  // LDS ring depth (160 KiB)
constexpr int kGTileBytes = kGM * kGK * 2;  // one operand tile (16 KiB)

struct GemmArgs {
  const u16* x;   // [M][ldx], group g's K columns start at g K
  const u16* w;   // [G][N][K]
  u16* c;         // [M][ldc], group g's N columns start at g N
  int M, N, K, G, ldx, ldc;
};

__device__ __forceinline__ int gswz(int r) { return (r >> 2) & 3; }

__global__ __launch_bounds__(512) void gemm_nt_mfma(GemmArgs a) {
  // One static array per ring stage (weight tile, then token tile): with
  // distinct objects the compiler sees that the loads in flight into the
  // later stages do not alias the reads of the current one, and waits only
  // for the loads of the stage it reads (one array for the whole ring made it
  // wait for every load in flight before each LDS read).
  __shared__ __attribute__((aligned(16))) unsigned char st0[2 * kGTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char st1[2 * kGTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char st2[2 * kGTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char st3[2 * kGTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char st4[2 * kGTileBytes];
  static_assert(kGStages == 5, "one array per stage");
  auto stage = [&](auto JC) __attribute__((always_inline)) -> unsigned char* {
    constexpr int J = decltype(JC)::value % kGStages;
    if constexpr (J == 0) return st0;
    else if constexpr (J == 1) return st1;
    else if constexpr (J == 2) return st2;
    else if constexpr (J == 3) return st3;
    else return st4;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.z;
  const int m0 = blockIdx.x * kGM, n0 = blockIdx.y * kGN;
  const int wn = wave & 1, wm = wave >> 1;      // 2 x 4 waves: 128 features x 64 tokens each

  // bounded descriptors (the store of a token row past M is dropped)
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(a.x), 0, a.M * a.ldx * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(a.w), 0, a.G * a.N * a.K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      a.c, 0, a.M * a.ldc * 2, 0x00020000);

  // Loads: a 1 KiB load covers 16 tile rows (lane l: row 16 i + l / 4,
  // physical chunk l % 4 holding logical chunk (l % 4) ^ swizzle(row)).  Wave
  // w loads blocks 2w and 2w + 1 of both operand tiles.
  int woff[2], xoff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 16 * (2 * wave + u) + (lane >> 2);
    const int lc = (lane & 3) ^ gswz(r);
    woff[u] = (((g * a.N + n0 + r) * a.K) + 8 * lc) * 2;
    // (token rows past M re-read row M - 1, whose products are never stored:
    // no load touches memory past the tensor)
    xoff[u] = ((min(m0 + r, a.M - 1) * a.ldx) + g * a.K + 8 * lc) * 2;
  }
  // load u (0, 1: weight blocks; 2, 3: token blocks) of tile kt into stage J
  auto issue_one = [&](auto JC, int kt, int u) __attribute__((always_inline)) {
    unsigned char* sb = stage(JC);
    const int kb = kt * kGK * 2;
    if (u < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wrs, (lds_void*)(sb + 1024 * (2 * wave + u)), 16, woff[u], kb, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (lds_void*)(sb + kGTileBytes + 1024 * (2 * wave + u - 2)), 16, xoff[u - 2], kb,
          0, 0);
  };

  // Fragment reads: block of 32 rows from row rb, k-step s: lane l reads row
  // rb + l % 32, logical chunk 2 s + l / 32.
  int wrd[4][2], xrd[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int r = 128 * wn + 32 * bn + (lane & 31);
      wrd[bn][s] = r * 64 + 16 * ((2 * s + (lane >> 5)) ^ gswz(r));
    }
#pragma unroll
    for (int bm = 0; bm < 2; ++bm) {
      const int r = 64 * wm + 32 * bm + (lane & 31);
      xrd[bm][s] = kGTileBytes + r * 64 + 16 * ((2 * s + (lane >> 5)) ^ gswz(r));
    }
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int bn = 0; bn < 4; ++bn)
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bn][bm][e] = 0.f;

  // The products of the tile in stage J with the four loads of tile kn (into
  // stage J + 4) spread between them (one after every four products), so that
  // the loads do not stall the wave in one burst.
  auto compute_loading = [&](auto JC, int kn) __attribute__((always_inline)) {
    constexpr int J = decltype(JC)::value;
    const unsigned char* t = stage(JC);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 wf[4], xf[2];
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) wf[bn] = as_bf16x8(*reinterpret_cast<const uint4*>(t + wrd[bn][s]));
#pragma unroll
      for (int bm = 0; bm < 2; ++bm) xf[bm] = as_bf16x8(*reinterpret_cast<const uint4*>(t + xrd[bm][s]));
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) acc[bn][bm] = mfma32x32x16(wf[bn], xf[bm], acc[bn][bm]);
        if ((bn & 1) == 1) {
          __builtin_amdgcn_sched_barrier(0);
          issue_one(std::integral_constant<int, J + kGStages - 1>{}, kn, 2 * s + (bn >> 1));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // Iteration kt (stage J = kt % 5): wait for this wave's loads of tile kt,
  // barrier (every wave's loads of tile kt have landed, and every wave is done
  // with tile kt - 1, whose stage takes tile kt + 4), products of tile kt with
  // the loads of tile kt + 4.  Every iteration issues its four loads (a tile
  // past the last re-reads the last one into a stage that is not read again),
  // so a wave always has 16 loads in flight at the wait and 12 of them may
  // stay; with no path that skips loads, the compiler too waits only for the
  // loads of the stage it reads.  Rounds of five iterations keep every stage
  // index a constant; only the last, partial round checks kt against nk.
  const int nk = a.K / kGK;
  auto tile = [&](int kt) __attribute__((always_inline)) { return min(kt, nk - 1); };
#pragma unroll
  for (int u = 0; u < 4; ++u) issue_one(std::integral_constant<int, 0>{}, 0, u);
#pragma unroll
  for (int u = 0; u < 4; ++u) issue_one(std::integral_constant<int, 1>{}, tile(1), u);
#pragma unroll
  for (int u = 0; u < 4; ++u) issue_one(std::integral_constant<int, 2>{}, tile(2), u);
#pragma unroll
  for (int u = 0; u < 4; ++u) issue_one(std::integral_constant<int, 3>{}, tile(3), u);
  auto iter = [&](auto JC, int kt) __attribute__((always_inline)) {
    wait_vmcnt<12>();
    lds_barrier();
    compute_loading(JC, tile(kt + kGStages - 1));
  };
  const int nfull = nk / kGStages;
  for (int r = 0; r < nfull; ++r) {
    const int k0 = r * kGStages;
    iter(std::integral_constant<int, 0>{}, k0);
    iter(std::integral_constant<int, 1>{}, k0 + 1);
    iter(std::integral_constant<int, 2>{}, k0 + 2);
    iter(std::integral_constant<int, 3>{}, k0 + 3);
    iter(std::integral_constant<int, 4>{}, k0 + 4);
  }
  {
    const int k0 = nfull * kGStages, rest = nk - k0;  // 0 to 4 iterations
    if (rest > 0) iter(std::integral_constant<int, 0>{}, k0);
    if (rest > 1) iter(std::integral_constant<int, 1>{}, k0 + 1);
    if (rest > 2) iter(std::integral_constant<int, 2>{}, k0 + 2);
    if (rest > 3) iter(std::integral_constant<int, 3>{}, k0 + 3);
  }
  // no load may still be writing this workgroup's LDS when it exits
  wait_vmcnt<0>();

  // Output: accumulator register e of block (bn, bm) holds feature
  // 32 bn + 8 (e / 4) + 4 (lane / 32) + e % 4 of token 32 bm + lane % 32.
#pragma unroll
  for (int bn = 0; bn < 4; ++bn)
#pragma unroll
    for (int bm = 0; bm < 2; ++bm) {
      const int m = m0 + 64 * wm + 32 * bm + (lane & 31);
      const int nb = g * a.N + n0 + 128 * wn + 32 * bn + 4 * (lane >> 5);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = {pack2(acc[bn][bm][4 * j], acc[bn][bm][4 * j + 1]),
                         pack2(acc[bn][bm][4 * j + 2], acc[bn][bm][4 * j + 3])};
        __builtin_amdgcn_raw_buffer_store_b64(v, crs, (m * a.ldc + nb + 8 * j) * 2, 0, 0);
      }
    }
}

// fp32 / any shape: one thread per output element, k in order
template <bool BF16>
__global__ __launch_bounds__(256) void gemm_nt_generic(const void* x, const void* w, void* c,
                                                       int M, int N, int K, int G, int ldx,
                                                       int ldc) {
  const long e = blockIdx.x * (long)blockDim.x + threadIdx.x;
  const long total = (long)M * N * G;
  if (e >= total) return;
  const int m = (int)(e / ((long)N * G));
  const int gn = (int)(e - (long)m * N * G);
  const int g = gn / N, n = gn - g * N;
  float s = 0.f;
  for (int k = 0; k < K; ++k)
    s += load1<BF16>(x, (long)m * ldx + (long)g * K + k) * load1<BF16>(w, ((long)g * N + n) * K + k);
  store1<BF16>(c, (long)m * ldc + (long)g * N + n, s);
}

hipError_t launch_gemm_nt(const void* x, const void* w, void* c, int M, int N, int K, int G,
                          int ldx, int ldc, bool bf16, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (bf16 && gemm_nt_mfma_shape(N, K, G, ldx, ldc, M)) {
    GemmArgs a{reinterpret_cast<const u16*>(x), reinterpret_cast<const u16*>(w),
               reinterpret_cast<u16*>(c), M, N, K, G, ldx, ldc};
    hipLaunchKernelGGL(gemm_nt_mfma, dim3((unsigned)((M + kGM - 1) / kGM), (unsigned)(N / kGN),
                                          (unsigned)G),
                       dim3(512), 0, s, a);
    return hipGetLastError();
  }
  const long total = (long)M * N * G;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (bf16) hipLaunchKernelGGL(gemm_nt_generic<true>, dim3(blocks), dim3(256), 0, s, x, w, c, M, N, K, G, ldx, ldc);
  else hipLaunchKernelGGL(gemm_nt_generic<false>, dim3(blocks), dim3(256), 0, s, x, w, c, M, N, K, G, ldx, ldc);
  return hipGetLastError();
}

}  // namespace

// The matrix-core kernel's shapes: whole 256-feature tiles and whole 32-wide
// K steps (at least one), 16-byte aligned rows, and byte offsets that fit its 32-bit buffer
// addressing (rows past M included).
bool gemm_nt_mfma_shape(int N, int K, int G, int ldx, int ldc, int M) {
  if (N % kGN != 0 || K < kGK || K % kGK != 0 || ldx % 8 != 0 || ldc % 8 != 0) return false;
  const long mr = ((long)M + kGM - 1) / kGM * kGM;
  return mr * ldx * 2 < 0x7fffffffL && mr * ldc * 2 < 0x7fffffffL &&
         (long)G * N * K * 2 < 0x7fffffffL;
}

hipError_t launch_out_proj(const void* o, const void* w_a, const void* w_b, void* mid,
                           void* out, int M, int G, int Kg, int r, int hidden, bool bf16,
                           hipStream_t s) {
  hipError_t e = launch_gemm_nt(o, w_a, mid, M, r, Kg, G, G * Kg, G * r, bf16, s);
  if (e != hipSuccess) return e;
  return launch_gemm_nt(mid, w_b, out, M, hidden, G * r, 1, G * r, hidden, bf16, s);
}

}  // namespace csa
