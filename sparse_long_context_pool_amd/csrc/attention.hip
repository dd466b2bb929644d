// attention.hip -- core attention of CSA / HCA / DSA layers.
//
// Page "DeepSeek-V4", section "Hybrid attention (§2.3)": one shared K=V head
// read as both key and value (multi-query attention), partial RoPE on the
// trailing qk_rope_head_dim channels of q, the output rope slice rotated back
// at position -t (eq. 26), a learnable per-head sink (eq. 27) and the sliding
// window K=V branch concatenated with the compressed entries.  Section
// "Attention mask layout": the query at t sees window positions (t-W, t], its
// k selected entries (CSA; -1 = empty) or every entry w < (t+1)//m (HCA).
// Page "DeepSeek-V3.2", section "DeepSeek Sparse Attention": attention over
// the selected tokens only (the m = 1 case, value = the latent part).
//
// Matrix-core kernel (bf16).  One workgroup = one query row, all H heads
// (H/16 wavefronts).  The key list (window slots, then pool slots) is walked in
// tiles of 32 rows.  Each tile's rows are gathered from HBM with 16-byte loads
// into ONE LDS tile that serves as both K and V, so a selected row is read from
// HBM once per query row for all heads:
//   S-phase: each wave computes S^T = K * Q^T for its 16 heads with
//     v_mfma_f32_16x16x32_bf16 (keys on M, heads on N; Q stays in registers as
//     the B operand).  That layout leaves each lane one head and 8 keys, i.e.
//     exactly the A-operand layout of the P*V product, so the online softmax
//     (seeded with the sink logit) runs in registers and P goes to LDS once.
//   PV-phase: the waves split the value columns: each computes O[all heads]
//     [its dv/NW columns] += P * V, reusing every V fragment for all heads.
// Rows whose keys exceed one workgroup's share (decode: few query rows, 2176
// keys each) are split over workgroups; partial (max, sum, O) go to the
// caller's workspace and a combine kernel merges them with the sink.
// Generic kernel: one wave per (row, head), any dtype and shape.
#include "csa_device.hpp"

#include <algorithm>

namespace csa {
namespace {

constexpr int kNK = 32;     // keys per tile

struct RowInfo {
  int b;
  long t;
  int nslots;
  int window;
};

__device__ __forceinline__ RowInfo row_info(const AttnParams& p, long row) {
  RowInfo ri;
  ri.b = (int)(row / p.S);
  const int i = (int)(row - (long)ri.b * p.S);
  ri.t = (long)p.q_pos[ri.b] + i;
  ri.window = p.window;
  const int npool = p.dense ? ready_count(ri.t, p.m, p.T) : p.k;
  ri.nslots = p.window + npool;
  return ri;
}

// Element offset of the K=V row behind slot s, or -1 for an empty slot.  The
// second output tells whether it lives in kv_win (true) or in pool (false).
__device__ __forceinline__ long slot_row(const AttnParams& p, const RowInfo& ri, long row,
                                         int s, bool* from_win) {
  if (s < ri.window) {
    *from_win = true;
    const long pos = ri.t - ri.window + 1 + s;
    if (pos < 0 || p.kv_win == nullptr) return -1;
    const long r = pos - (long)p.win_pos0[ri.b];
    if (r < 0 || r >= p.L_win) return -1;
    return ((long)ri.b * p.L_win + r) * p.D;
  }
  *from_win = false;
  const int j = s - ri.window;
  const int w = p.dense ? j : p.idx[row * p.k + j];
  if (w < 0 || w >= p.T || p.pool == nullptr) return -1;
  return ((long)ri.b * p.T + w) * p.D;
}

// ------------------------------------------------------------------ generic
template <bool BF16, int VPL>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnParams p) {
  const long row = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave;
  if (h >= p.H) return;
  const RowInfo ri = row_info(p, row);
  const int D = p.D, dv = p.dv, half = p.rope_dim >> 1, rbase = D - p.rope_dim;
  const long oo = (row * p.H + h) * dv;
  if (p.rope_dim > 0 && (ri.t < 0 || ri.t >= p.n_pos)) {
    for (int c = lane; c < dv; c += 64) store1<BF16>(p.out, oo + c, __int_as_float(0x7fc00000));
    return;
  }
  const float2* cs = reinterpret_cast<const float2*>(p.cs);
  const int c0 = lane * VPL;
  float q[VPL], o[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    q[v] = (c0 + v < D) ? load1<BF16>(p.q, (row * p.H + h) * D + c0 + v) : 0.f;
    o[v] = 0.f;
  }
#pragma unroll
  for (int v = 0; v < VPL; v += 2) {
    if (c0 + v >= rbase && c0 + v < D) {
      const float2 r = cs[ri.t * half + ((c0 + v - rbase) >> 1)];
      const float a = q[v], bb = q[v + 1];
      q[v] = a * r.x - bb * r.y;
      q[v + 1] = a * r.y + bb * r.x;
    }
  }
  const float sl2 = p.scale * kLog2e;
  float mrun = p.sink ? p.sink[h] * kLog2e : -INFINITY;
  float lrun = p.sink ? 1.f : 0.f;
  for (int s = 0; s < ri.nslots; ++s) {
    bool from_win;
    const long off = slot_row(p, ri, row, s, &from_win);
    if (off < 0) continue;
    const void* base = from_win ? p.kv_win : p.pool;
    float kv[VPL];
    float d = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      kv[v] = (c0 + v < D) ? load1<BF16>(base, off + c0 + v) : 0.f;
      d += q[v] * kv[v];
    }
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) d += shfl_xor(d, sh);
    const float x = d * sl2;
    const float mn = fmaxf(mrun, x);
    const float alpha = exp2f(mrun - mn);
    const float pe = exp2f(x - mn);
    lrun = lrun * alpha + pe;
#pragma unroll
    for (int v = 0; v < VPL; ++v) o[v] = o[v] * alpha + pe * kv[v];
    mrun = mn;
  }
  const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
#pragma unroll
  for (int v = 0; v < VPL; ++v) o[v] *= inv;
  if (dv == D) {
#pragma unroll
    for (int v = 0; v < VPL; v += 2) {
      if (c0 + v >= rbase && c0 + v < D) {
        const float2 r = cs[ri.t * half + ((c0 + v - rbase) >> 1)];
        const float a = o[v], bb = o[v + 1];
        o[v] = a * r.x + bb * r.y;
        o[v + 1] = -a * r.y + bb * r.x;
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v)
    if (c0 + v < dv) store1<BF16>(p.out, oo + c0 + v, o[v]);
}

// ------------------------------------------------------------------ matrix-core
struct MfmaArgs {
  AttnParams p;
  float* ws;              // split partials, or nullptr
  int nsplit;
  int tiles_per_split;
  int rows_per_xcd;       // query-row remap: consecutive rows on one XCD
};

// Split workspace (fp32): [rows][nsplit][H][2] running (max, sum) in the log2
// domain, then [rows][nsplit][H][dv] unnormalised partial outputs.
//
// Template: NW waves (16 heads each in the S phase, dv/NW output columns each
// in the PV phase), NB = 16-column blocks per wave, D = K=V row width, R =
// rope_dim (trailing rotated channels).  Lane c16 of a wave owns the NB
// consecutive output columns wave*16*NB + NB*c16 ..; its V operand for one key
// is then a single NB*2-byte LDS read.
//
// Key list of a query row: the visible window rows (one contiguous run of
// kv_win), then the pool slots; each part is padded to whole 32-key tiles so
// that every tile reads one tensor.  Rows are fetched with buffer loads whose
// bound is the sequence's slice of that tensor: an empty slot gets an offset
// past the bound and reads zeros, with no branch.
template <int NW, int NB, int D, int R>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(MfmaArgs args) {
  constexpr int NT = NW * 64;
  constexpr int HG = 16 * NW;           // heads per workgroup (one head group)
  constexpr int DVW = 16 * NB;          // output columns per wave
  constexpr int KS = D / 32;            // k-steps of the S phase
  constexpr int ROWB = D * 2 + 16;      // padded LDS row (bytes)
  constexpr int CPR = D / 8;            // 16-byte chunks per K=V row
  constexpr int GATHER_IT = (kNK * CPR + NT - 1) / NT;
  constexpr int half = R / 2, rbase = D - R;
  static_assert(NB == 2 || NB == 4 || NB == 8, "V read width");
  const AttnParams& p = args.p;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* ktile = smem;                                   // [32][ROWB]
  u16* Ps = reinterpret_cast<u16*>(smem + kNK * ROWB);           // [HG][32] bf16
  float* alpha_s = reinterpret_cast<float*>(Ps + HG * kNK);      // [HG]
  float* fin_s = alpha_s + HG;                                   // [HG] 1/l
  int* rid_s = reinterpret_cast<int*>(fin_s + HG);               // [2][32] row ids
  int* flags = rid_s + 2 * kNK;                                  // [2] rescale, [NW] scan

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;

  // query row: consecutive rows stay on one XCD (workgroups go round-robin
  // over the 8 XCDs), so neighbouring rows share window rows in one L2
  const long bid = blockIdx.x;
  const long row = (bid & 7) * (long)args.rows_per_xcd + (bid >> 3);
  if (row >= (long)p.B * p.S) return;
  const int split = blockIdx.y;
  const int h0 = blockIdx.z * HG;
  const int H = p.H, dv = p.dv;
  const int b = (int)(row / p.S);
  const long t = (long)p.q_pos[b] + (row - (long)b * p.S);
  const float2* cs = reinterpret_cast<const float2*>(p.cs);
  const bool split_mode = args.nsplit > 1;

  if (R > 0 && (t < 0 || t >= p.n_pos)) {
    // position outside the RoPE table: the row is written as NaN
    if (split_mode) {
      float* ml = args.ws + ((size_t)row * args.nsplit + split) * H * 2;
      for (int e = tid; e < HG; e += NT) {
        ml[2 * (h0 + e)] = __int_as_float(0x7fc00000);
        ml[2 * (h0 + e) + 1] = 0.f;
      }
      return;
    }
    for (int e = tid; e < HG * dv; e += NT)
      store1<true>(p.out, (row * H + h0) * dv + e, __int_as_float(0x7fc00000));
    return;
  }

  // ---- effective key list
  int n_win = 0, r_lo = 0;
  if (p.window > 0 && p.kv_win != nullptr) {
    const long wp0 = p.win_pos0[b];
    const long lo = max(t - p.window + 1, max(0L, wp0));
    const long hi = min(t, wp0 + (long)p.L_win - 1);
    if (hi >= lo) { n_win = (int)(hi - lo + 1); r_lo = (int)(lo - wp0); }
  }
  int npool = 0;
  const int* idx_row = p.dense ? nullptr : p.idx + row * p.k;
  if (p.dense) {
    npool = p.pool ? ready_count(t, p.m, p.T) : 0;
  } else if (p.k > 0 && p.pool) {
    // the last non-empty slot bounds the list (top-k pads with -1 at the tail)
    int last = -1;
    for (int j = tid; j < p.k; j += NT) {
      const int w = idx_row[j];
      if (w >= 0 && w < p.T) last = j;
    }
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) last = max(last, __shfl_xor(last, sh, 64));
    if (lane == 0) flags[2 + wave] = last;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NW; ++q) npool = max(npool, flags[2 + q] + 1);
  }
  const int WT = (n_win + kNK - 1) / kNK;
  const int ntiles = WT + (npool + kNK - 1) / kNK;
  const int tile0 = split * args.tiles_per_split;
  const int tile1 = min(ntiles, tile0 + args.tiles_per_split);

  const u16* win_base = p.kv_win ? reinterpret_cast<const u16*>(p.kv_win) + (size_t)b * p.L_win * D
                                 : nullptr;
  const u16* pool_base = p.pool ? reinterpret_cast<const u16*>(p.pool) + (size_t)b * p.T * D
                                : nullptr;
  const __amdgpu_buffer_rsrc_t rs_win = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(win_base), 0, win_base ? p.L_win * D * 2 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_pool = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(pool_base), 0, pool_base ? p.T * D * 2 : 0, 0x00020000);

  // row id of key j of a tile: kv_win / pool row of this sequence, -1 = empty
  auto resolve = [&](int tile, int buf) {
    if (wave == 0 && lane < kNK) {
      int rid = -1;
      if (tile < WT) {
        const int jj = tile * kNK + lane;
        if (jj < n_win) rid = r_lo + jj;
      } else {
        const int jj = (tile - WT) * kNK + lane;
        if (jj < npool) {
          const int w = p.dense ? jj : idx_row[jj];
          if (w >= 0 && w < p.T) rid = w;
        }
      }
      rid_s[buf * kNK + lane] = rid;
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T): head hl, dims 32ks + 8g .. +7,
  // rotated at +t on the rope slice, rounded to bf16
  const int hl = 16 * wave + c16;
  bf16x8 qf[KS];
  {
    const u16* qrow = reinterpret_cast<const u16*>(p.q) + (row * H + h0 + hl) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      uint4 u = *reinterpret_cast<const uint4*>(qrow + d0);
      if (32 * ks + 32 > rbase && d0 >= rbase) {
        float v[8] = {bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y),
                      bf_lo(u.z), bf_hi(u.z), bf_lo(u.w), bf_hi(u.w)};
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float2 r = cs[t * half + ((d0 + e - rbase) >> 1)];
          const float a = v[e], bb = v[e + 1];
          v[e] = a * r.x - bb * r.y;
          v[e + 1] = a * r.y + bb * r.x;
        }
        u.x = pack2(v[0], v[1]); u.y = pack2(v[2], v[3]);
        u.z = pack2(v[4], v[5]); u.w = pack2(v[6], v[7]);
      }
      qf[ks] = as_bf16x8(u);
    }
  }

  // ---- softmax state of head hl (replicated over the 4 lane groups), log2 domain
  const float sl2 = p.scale * kLog2e;
  float mrun = -INFINITY, lrun = 0.f;
  if (p.sink && !split_mode) { mrun = p.sink[h0 + hl] * kLog2e; lrun = 1.f; }

  f32x4 acc[NW][NB];
#pragma unroll
  for (int mb = 0; mb < NW; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int col0 = wave * DVW + NB * c16;  // this lane's first output column

  if (tid == 0) { flags[0] = 1; flags[1] = 1; }
  if (tile0 < tile1) resolve(tile0, 0);
  __syncthreads();

  for (int tile = tile0; tile < tile1; ++tile) {
    const int buf = (tile - tile0) & 1;
    // ---- gather: 32 rows x D bf16 into the LDS tile (16-byte buffer loads)
    {
      const __amdgpu_buffer_rsrc_t rs = tile < WT ? rs_win : rs_pool;
#pragma unroll
      for (int it = 0; it < GATHER_IT; ++it) {
        const int c = tid + it * NT;
        if (GATHER_IT * NT == kNK * CPR || c < kNK * CPR) {
          const int r = c / CPR, col = c - r * CPR;
          const int rid = rid_s[buf * kNK + r];
          const int off = rid >= 0 ? rid * (D * 2) + col * 16 : 0x7ffffff0;
          const uint4 v =
              __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
          *reinterpret_cast<uint4*>(ktile + r * ROWB + col * 16) = v;
        }
      }
    }
    if (tid == 0) flags[buf ^ 1] = 0;  // next tile's rescale flag starts clear
    __syncthreads();
    if (tile + 1 < tile1) resolve(tile + 1, buf ^ 1);

    // ---- S phase: S^T[key][head] for this wave's 16 heads, 4 k-steps per
    // group (the scheduling barrier bounds the K fragments in flight)
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int k4 = 0; k4 < KS; k4 += 4) {
      uint4 kv[4][2];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          if (k4 + kk < KS)
            kv[kk][h2] = *reinterpret_cast<const uint4*>(
                ktile + (16 * h2 + c16) * ROWB + 64 * (k4 + kk) + 16 * g);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          if (k4 + kk < KS) st[h2] = mfma16x16x32(as_bf16x8(kv[kk][h2]), qf[k4 + kk], st[h2]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane holds keys 16*h2 + 4g + j of head hl
    const int4 ra = *reinterpret_cast<const int4*>(rid_s + buf * kNK + 4 * g);
    const int4 rb = *reinterpret_cast<const int4*>(rid_s + buf * kNK + 16 + 4 * g);
    const int rv[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = rv[4 * h2 + j] >= 0 ? st[h2][j] * sl2 : -INFINITY;
        sv[4 * h2 + j] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float mnew = fmaxf(mrun, tmax);
    const float mbase = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = exp2f(mrun - mbase);
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = exp2f(sv[e] - mbase), p1 = exp2f(sv[e + 1] - mbase);
      psum += p0 + p1;
      pk[e >> 1] = pack2(p0, p1);
    }
    psum += shfl_xor(psum, 16);
    psum += shfl_xor(psum, 32);
    lrun = lrun * alpha + psum;
    mrun = mnew;
    // P row of head hl; key 16*h2 + 4g + j sits at position 8g + 4*h2 + j
    *reinterpret_cast<uint4*>(Ps + hl * kNK + 8 * g) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    if (g == 0) alpha_s[hl] = alpha;
    if (__ballot(alpha != 1.f) != 0ull && lane == 0) flags[buf] = 1;
    __syncthreads();

    // ---- PV phase: O[all HG heads][this wave's DVW columns] += P V
    if (flags[buf]) {
#pragma unroll
      for (int mb = 0; mb < NW; ++mb) {
        const float4 al = *reinterpret_cast<const float4*>(alpha_s + 16 * mb + 4 * g);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[mb][nb][0] *= al.x; acc[mb][nb][1] *= al.y;
          acc[mb][nb][2] *= al.z; acc[mb][nb][3] *= al.w;
        }
      }
    }
    bf16x8 pa[NW];
#pragma unroll
    for (int mb = 0; mb < NW; ++mb)
      pa[mb] = as_bf16x8(*reinterpret_cast<const uint4*>(Ps + (16 * mb + c16) * kNK + 8 * g));
    // V: for key position q (key 16*(q/4) + 4g + q%4), this lane's NB columns
    uint32_t vr[8][NB / 2];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const unsigned char* src =
          ktile + (16 * (q >> 2) + 4 * g + (q & 3)) * ROWB + col0 * 2;
      if constexpr (NB == 8) {
        const uint4 u = *reinterpret_cast<const uint4*>(src);
        vr[q][0] = u.x; vr[q][1] = u.y; vr[q][2] = u.z; vr[q][3] = u.w;
      } else if constexpr (NB == 4) {
        const uint2 u = *reinterpret_cast<const uint2*>(src);
        vr[q][0] = u.x; vr[q][1] = u.y;
      } else {
        vr[q][0] = *reinterpret_cast<const uint32_t*>(src);
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int dw = nb >> 1;
      uint32_t f[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t a = vr[2 * d][dw], bq = vr[2 * d + 1][dw];
        f[d] = (nb & 1) ? ((a >> 16) | (bq & 0xffff0000u)) : ((a & 0xffffu) | (bq << 16));
      }
      const bf16x8 vb = as_bf16x8(make_uint4(f[0], f[1], f[2], f[3]));
#pragma unroll
      for (int mb = 0; mb < NW; ++mb) acc[mb][nb] = mfma16x16x32(pa[mb], vb, acc[mb][nb]);
    }
    __syncthreads();
  }

  // ---- epilogue
  if (split_mode) {
    float* ml = args.ws + ((size_t)row * args.nsplit + split) * H * 2;
    if (g == 0) { ml[2 * (h0 + hl)] = mrun; ml[2 * (h0 + hl) + 1] = lrun; }
    float* po = args.ws + (size_t)((long)p.B * p.S) * args.nsplit * H * 2 +
                ((size_t)row * args.nsplit + split) * H * dv;
#pragma unroll
    for (int mb = 0; mb < NW; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* dst = po + (size_t)(h0 + 16 * mb + 4 * g + j) * dv + col0;
#pragma unroll
        for (int nb = 0; nb < NB; nb += 2)
          *reinterpret_cast<float2*>(dst + nb) = make_float2(acc[mb][nb][j], acc[mb][nb + 1][j]);
      }
    return;
  }
  if (g == 0) fin_s[hl] = lrun > 0.f ? 1.f / lrun : 0.f;
  __syncthreads();
  u16* out = reinterpret_cast<u16*>(p.out) + (row * H + h0) * dv;
  const bool derot = (dv == D) && R > 0 && col0 + NB > rbase;
#pragma unroll
  for (int mb = 0; mb < NW; ++mb) {
    const float4 li = *reinterpret_cast<const float4*>(fin_s + 16 * mb + 4 * g);
    const float lv[4] = {li.x, li.y, li.z, li.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) v[nb] = acc[mb][nb][j] * lv[j];
      if (derot) {
#pragma unroll
        for (int nb = 0; nb < NB; nb += 2) {
          const int col = col0 + nb;
          if (col >= rbase) {
            const float2 r = cs[t * half + ((col - rbase) >> 1)];
            const float a = v[nb], bb = v[nb + 1];
            v[nb] = a * r.x + bb * r.y;
            v[nb + 1] = -a * r.y + bb * r.x;
          }
        }
      }
      uint32_t w[NB / 2];
#pragma unroll
      for (int nb = 0; nb < NB; nb += 2) w[nb >> 1] = pack2(v[nb], v[nb + 1]);
      u16* dst = out + (16 * mb + 4 * g + j) * dv + col0;
      if constexpr (NB == 8)
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      else if constexpr (NB == 4)
        *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
      else
        *reinterpret_cast<uint32_t*>(dst) = w[0];
    }
  }
}

// Merge split partials: M = max(z, m_s), L = e^(z-M) + sum e^(m_s-M) l_s,
// O = sum e^(m_s-M) O_s / L, then the output rope slice is rotated at -t.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p, const float* ws,
                                                           int nsplit) {
  const long row = blockIdx.x;
  const int H = p.H, dv = p.dv;
  const RowInfo ri = row_info(p, row);
  const int half = p.rope_dim >> 1, rbase = p.D - p.rope_dim;
  const float2* cs = reinterpret_cast<const float2*>(p.cs);
  const float* ml = ws + (size_t)row * nsplit * H * 2;
  const float* po = ws + (size_t)(p.B * (long)p.S) * nsplit * H * 2 + (size_t)row * nsplit * H * dv;
  u16* out = reinterpret_cast<u16*>(p.out) + row * H * dv;
  for (int e = threadIdx.x; e < H * (dv >> 1); e += blockDim.x) {
    const int h = e / (dv >> 1);
    const int c = 2 * (e - h * (dv >> 1));
    float M = p.sink ? p.sink[h] * kLog2e : -INFINITY;
    bool nan = false;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = ml[(s * H + h) * 2];
      if (ms != ms) nan = true;
      M = fmaxf(M, ms);
    }
    const float Mb = (M == -INFINITY) ? 0.f : M;
    float L = p.sink ? exp2f(p.sink[h] * kLog2e - Mb) : 0.f;
    float o0 = 0.f, o1 = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float f = exp2f(ml[(s * H + h) * 2] - Mb);
      L += f * ml[(s * H + h) * 2 + 1];
      const float* os = po + ((size_t)s * H + h) * dv;
      o0 += f * os[c];
      o1 += f * os[c + 1];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    o0 *= inv;
    o1 *= inv;
    if (p.dv == p.D && p.rope_dim > 0 && c >= rbase && ri.t >= 0 && ri.t < p.n_pos) {
      const float2 r = cs[ri.t * half + ((c - rbase) >> 1)];
      const float a = o0, bb = o1;
      o0 = a * r.x + bb * r.y;
      o1 = -a * r.y + bb * r.x;
    }
    if (nan) o0 = o1 = __int_as_float(0x7fc00000);
    out[h * dv + c] = f2bf(o0);
    out[h * dv + c + 1] = f2bf(o1);
  }
}

// Matrix-core shapes compiled in.  Heads run in groups of 16*NW; every
// group is its own workgroup (so H = 128 runs as two 64-head groups).
struct MfmaShape {
  int nw, nb, d, r;
};

bool mfma_shape(int H, int D, int dv, int rope_dim, MfmaShape* sh) {
  if (H % 64 == 0 && dv == 512 && rope_dim == 64 && (D == 512 || D == 576)) {
    *sh = {4, 8, D, 64};
    return true;
  }
  if (H % 16 == 0 && dv == 64 && ((D == 64 && rope_dim == 16) || (D == 96 && rope_dim == 32))) {
    *sh = {1, 4, D, rope_dim};
    return true;
  }
  return false;
}

size_t mfma_lds_bytes(int nw, int D) {
  const int hg = 16 * nw;
  return (size_t)kNK * (D * 2 + 16) + (size_t)hg * kNK * 2 + (size_t)hg * 4 * 2 +
         2 * kNK * sizeof(int) + (2 + nw) * sizeof(int);
}

int device_cus() {
  static thread_local int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached_dev = dev;
    cached_cus = cus;
  }
  return cached_cus;
}

}  // namespace

AttnPlan plan_attention(int B, int S, int H, int D, int dv, int rope_dim, int max_slots,
                        bool bf16, long max_rows) {
  AttnPlan pl{0, 1, 1 << 30, 0};
  MfmaShape sh;
  if (!bf16 || !mfma_shape(H, D, dv, rope_dim, &sh)) return pl;
  // the gather addresses one sequence's rows with 32-bit buffer offsets
  if (max_rows * D * 2 >= 0x7ffffff0L) return pl;
  pl.kernel = 1;
  const long wgs = (long)B * S * (H / (16 * sh.nw));
  const int tiles = (max_slots + kNK - 1) / kNK;
  const int cus = device_cus();
  if (wgs < cus && tiles > 1) {
    int ns = (int)std::min<long>(tiles, (cus + wgs - 1) / wgs);
    const int tps = (tiles + ns - 1) / ns;
    ns = (tiles + tps - 1) / tps;
    if (ns > 1) {
      pl.nsplit = ns;
      pl.tiles_per_split = tps;
      pl.ws_bytes = (size_t)B * S * ns * H * (dv + 2) * sizeof(float);
    }
  }
  return pl;
}

hipError_t launch_attention(const AttnParams& p, const AttnPlan& plan, void* ws,
                            hipStream_t s) {
  const long rows = (long)p.B * p.S;
  if (rows == 0) return hipSuccess;
  if (plan.kernel == 0) {
    dim3 grid((unsigned)rows, (p.H + 3) / 4);
    const int vpl = 2 * ((p.D + 127) / 128);
#define CSA_GENERIC(V)                                                                   \
  if (p.bf16) hipLaunchKernelGGL((attn_generic_kernel<true, V>), grid, dim3(256), 0, s, p); \
  else hipLaunchKernelGGL((attn_generic_kernel<false, V>), grid, dim3(256), 0, s, p);
    if (vpl <= 2) { CSA_GENERIC(2) }
    else if (vpl <= 4) { CSA_GENERIC(4) }
    else if (vpl <= 8) { CSA_GENERIC(8) }
    else if (vpl <= 10) { CSA_GENERIC(10) }
    else { CSA_GENERIC(16) }
#undef CSA_GENERIC
    return hipGetLastError();
  }
  MfmaShape sh;
  mfma_shape(p.H, p.D, p.dv, p.rope_dim, &sh);
  MfmaArgs a;
  a.p = p;
  const bool split = plan.nsplit > 1 && ws != nullptr;
  a.ws = split ? reinterpret_cast<float*>(ws) : nullptr;
  a.nsplit = split ? plan.nsplit : 1;
  a.tiles_per_split = split ? plan.tiles_per_split : (1 << 30);
  a.rows_per_xcd = (int)((rows + 7) / 8);
  dim3 grid((unsigned)(8 * (long)a.rows_per_xcd), a.nsplit, p.H / (16 * sh.nw));
  const size_t lds = mfma_lds_bytes(sh.nw, p.D);
  if (sh.nw == 4 && sh.d == 512)
    hipLaunchKernelGGL((attn_mfma_kernel<4, 8, 512, 64>), grid, dim3(256), lds, s, a);
  else if (sh.nw == 4 && sh.d == 576)
    hipLaunchKernelGGL((attn_mfma_kernel<4, 8, 576, 64>), grid, dim3(256), lds, s, a);
  else if (sh.nw == 1 && sh.d == 64)
    hipLaunchKernelGGL((attn_mfma_kernel<1, 4, 64, 16>), grid, dim3(64), lds, s, a);
  else if (sh.nw == 1 && sh.d == 96)
    hipLaunchKernelGGL((attn_mfma_kernel<1, 4, 96, 32>), grid, dim3(64), lds, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !split) return err;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)rows), dim3(256), 0, s, p,
                     reinterpret_cast<const float*>(ws), a.nsplit);
  return hipGetLastError();
}

}  // namespace csa
