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
#include <type_traits>

namespace csa {
namespace {

constexpr int kNK = 32;     // keys per tile
constexpr int kPS = kNK + 8;  // P row stride (u16): 80 bytes keeps P reads conflict-free

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
typedef __attribute__((address_space(3))) void lds_void;

struct MfmaArgs {
  AttnParams p;
  float* ws;              // split partials, or nullptr
  int nsplit;
  int tiles_per_split;
  int rows_per_xcd;       // query-row remap: consecutive rows on one XCD
};

// LDS barrier that waits only for this wave's LDS traffic, not for global
// loads still in flight (the gathers of later tiles must stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// K=V tile of 32 rows in LDS, each row padded by 16 bytes (row stride
// 2D+16 bytes = 4 or 36 dwords mod 64 banks), so that the S-phase reads (16
// rows, one 16-byte chunk) and the PV-phase reads (4 rows x 8 consecutive
// chunks) fall in distinct banks, while every address is a per-lane base plus
// an immediate offset.  Rows are filled by direct global->LDS 16-byte buffer
// loads: one wave instruction writes up to 1 KiB contiguous (lane l at +16*l),
// one instruction per row (plus an 8-lane one for the last 128 bytes when
// D = 576); lanes whose row slot is empty read past the buffer bound, which
// writes zeros.
template <int D>
struct KTile {
  static constexpr int ROWB = D * 2 + 16;
  static constexpr int BYTES = kNK * ROWB;
  static constexpr int G = (D > 512) ? 8 : 4;   // loads per wave per tile (8 waves)
};

// Split workspace (fp32): [rows][nsplit][H][2] running (max, sum) in the log2
// domain, then [rows][nsplit][H][dv] unnormalised partial outputs.
//
// One workgroup = one query row x one group of 64 heads, 8 waves (2 per SIMD).
// S phase: wave w computes S^T for heads 16(w%4) .. +15 over keys 16(w/4) ..
// +15 of the 32-key tile; the two key halves of a head exchange their tile
// maxima through LDS.  PV phase: wave w owns output columns 64w .. 64w+63,
// lane c16 the 4 consecutive columns 64w + 4*c16 .. (one 8-byte LDS read per
// key, 8-byte output stores, lane-local de-rotation).  The gathers run
// NBUF-1 tiles ahead of the compute.
//
// Softmax: a per-head reference max m (the sink logit to start with) is raised
// only when a tile's max exceeds it by more than 8 (log2 units); otherwise the
// probabilities exp2(s - m) may reach 2^8, which bf16 and fp32 carry exactly
// in relative terms, and O / l is unchanged.  So the accumulators are rescaled
// only in the rare tile that raises m.
template <int D, int NBUF>
__global__ __launch_bounds__(512) void attn_mfma_kernel(MfmaArgs args) {
  constexpr int NW = 8, NT = 512, HG = 64, NB = 4;
  constexpr int KS = D / 32;
  constexpr int KH = KS / 2;  // k-steps per wave: the two waves of a head block split D
  constexpr int R = 64, half = R / 2, rbase = D - R;
  constexpr float kLazy = 8.f;
  using KT = KTile<D>;
  static_assert(NBUF == 3 || NBUF == 4, "buffer count");
  // One static array per K buffer: with distinct objects the compiler can
  // tell that an in-flight gather into one buffer does not alias reads of
  // another, so it does not wait for the gather before those reads.
  __shared__ __attribute__((aligned(16))) unsigned char kb0[KT::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char kb1[KT::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char kb2[KT::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char kb3[NBUF == 4 ? KT::BYTES : 16];
  // every other LDS array is static as well, for the same reason
  __shared__ __attribute__((aligned(16))) u16 Ps[HG * kPS];        // P, bf16
  __shared__ __attribute__((aligned(16))) float spart[NW * 2 * 64 * 4];  // S^T partials
  __shared__ __attribute__((aligned(16))) float alpha_s[HG];       // rescale factors
  __shared__ __attribute__((aligned(16))) float fin_s[HG];         // 1/l
  __shared__ __attribute__((aligned(16))) float l_s[HG];           // second half's sum
  __shared__ __attribute__((aligned(16))) float bias_s[NBUF * kNK];  // 0 / -inf per key slot
  __shared__ int flags[20];                                        // rescale, scan
  const AttnParams& p = args.p;
  auto kbuf_of = [&](auto JC) __attribute__((always_inline)) -> unsigned char* {
    constexpr int J = decltype(JC)::value;
    if constexpr (J == 0) return kb0;
    else if constexpr (J == 1) return kb1;
    else if constexpr (J == 2) return kb2;
    else return kb3;
  };

  // the wave index is uniform: keep it (and everything derived from it) scalar
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int hgrp = wave & 3, kh = wave >> 2;   // head block; D half in S, key half in P

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

  if (t < 0 || t >= p.n_pos) {
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

  // ---- effective key list: visible window rows, then the pool slots, each
  // part padded to whole tiles so that a tile reads one tensor
  int n_win = 0, r_lo = 0;
  if (p.window > 0 && p.kv_win != nullptr) {
    const long wp0 = p.win_pos0[b];
    const long lo = max(t - p.window + 1, max(0L, wp0));
    const long hi = min(t, wp0 + (long)p.L_win - 1);
    if (hi >= lo) { n_win = (int)(hi - lo + 1); r_lo = (int)(lo - wp0); }
  }
  int npool = 0, pool_stand_in = 0;
  if (p.dense) {
    npool = p.pool ? ready_count(t, p.m, p.T) : 0;
  } else if (p.k > 0 && p.pool) {
    // the last non-empty slot of the index row bounds the list; the row of the
    // first non-empty one stands in for the empty slots
    const int* idx_row = p.idx + row * p.k;
    int last = -1, first = p.k;
    for (int j = tid; j < p.k; j += NT) {
      const int w = idx_row[j];
      if (w >= 0 && w < p.T) { last = j; first = min(first, j); }
    }
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) {
      last = max(last, __shfl_xor(last, sh, 64));
      first = min(first, __shfl_xor(first, sh, 64));
    }
    if (lane == 0) { flags[2 + wave] = last; flags[10 + wave] = first; }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      npool = max(npool, flags[2 + q] + 1);
      first = min(first, flags[10 + q]);
    }
    // (values read back from LDS or memory: made wave-uniform explicitly so
    // that they stay in scalar registers)
    npool = __builtin_amdgcn_readfirstlane(npool);
    if (npool > 0) pool_stand_in = __builtin_amdgcn_readfirstlane(idx_row[first]);
  }
  const int WT = (n_win + kNK - 1) / kNK;
  const int ntiles = WT + (npool + kNK - 1) / kNK;
  const int tile0 = split * args.tiles_per_split;
  const int tile1 = min(ntiles, tile0 + args.tiles_per_split);

  const u16* win_base = p.kv_win ? reinterpret_cast<const u16*>(p.kv_win) + (size_t)b * p.L_win * D
                                 : nullptr;
  const u16* pool_base = p.pool ? reinterpret_cast<const u16*>(p.pool) + (size_t)b * p.T * D
                                : nullptr;
  // gather descriptors are built per tile from these (a zero size past the
  // tile range: the loads then fill zeros)
  const int win_bytes = win_base ? p.L_win * D * 2 : 0;
  const int pool_bytes = pool_base ? p.T * D * 2 : 0;
  const int lane_off = lane << 4;

  // row ids of this wave's 4 rows (4w .. 4w+3) of a tile: kv_win / pool row of
  // this sequence, -1 = empty (or past the tile range).  Wave-uniform: the
  // index entries come in with scalar loads (read through the constant
  // address space: the index is never written while the kernel runs).
  typedef __attribute__((address_space(4))) const int cint;
  cint* idx_row = p.idx ? (cint*)(p.idx + row * p.k) : nullptr;
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(4))) const i32x4 ci32x4;
  auto rid4 = [=](int tile) __attribute__((always_inline)) -> int4 {
    int4 r = make_int4(-1, -1, -1, -1);
    if (tile >= tile1) return r;
    if (tile < WT) {
      const int jj = tile * kNK + wave * 4;
      r.x = jj + 0 < n_win ? r_lo + jj + 0 : -1;
      r.y = jj + 1 < n_win ? r_lo + jj + 1 : -1;
      r.z = jj + 2 < n_win ? r_lo + jj + 2 : -1;
      r.w = jj + 3 < n_win ? r_lo + jj + 3 : -1;
      return r;
    }
    const int jj = (tile - WT) * kNK + wave * 4;
    int4 w;
    if (p.dense) {
      w = make_int4(jj, jj + 1, jj + 2, jj + 3);
    } else if (jj + 4 <= p.k) {
      const i32x4 v = *(ci32x4*)(idx_row + jj);  // one scalar load of the 4 entries
      w = make_int4(v[0], v[1], v[2], v[3]);
    } else {
      w.x = jj + 0 < p.k ? idx_row[jj + 0] : -1;
      w.y = jj + 1 < p.k ? idx_row[jj + 1] : -1;
      w.z = jj + 2 < p.k ? idx_row[jj + 2] : -1;
      w.w = jj + 3 < p.k ? idx_row[jj + 3] : -1;
    }
    r.x = (jj + 0 < npool && w.x >= 0 && w.x < p.T) ? w.x : -1;
    r.y = (jj + 1 < npool && w.y >= 0 && w.y < p.T) ? w.y : -1;
    r.z = (jj + 2 < npool && w.z >= 0 && w.z < p.T) ? w.z : -1;
    r.w = (jj + 3 < npool && w.w >= 0 && w.w < p.T) ? w.w : -1;
    return r;
  };

  // this wave's share of a tile's gather into buffer J: rows 4*wave ..
  // 4*wave+3, one 1 KiB load per row (and one 8-lane load of the last 128
  // bytes when D = 576)
  // An empty slot gathers a stand-in row of the same tensor (finite data that
  // the -inf bias of the slot cancels: its probability is exactly 0); a tile
  // past the range gathers through a zero-size descriptor (zero fill).  The
  // row is wave-uniform: its offset goes in the scalar operand, so the
  // per-lane operand is the loop-invariant lane_off (the compiler's wait-count
  // model treats a register that fed a gather as pending until the gather
  // lands, so a per-gather temporary reused later for other data would cost a
  // wait).
  auto issue = [=](auto JC, int tile, const int4 rids) __attribute__((always_inline)) {
    constexpr int J = decltype(JC)::value;
    unsigned char* kbuf = kbuf_of(JC);
    const int rl = lane == 0 ? rids.x : lane == 1 ? rids.y : lane == 2 ? rids.z : rids.w;
    if (lane < 4) bias_s[J * kNK + wave * 4 + lane] = rl >= 0 ? 0.f : -INFINITY;
    const bool win = tile < WT;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(win ? win_base : pool_base), 0,
        tile >= tile1 ? 0 : win ? win_bytes : pool_bytes, 0x00020000);
    const int stand_in = win ? r_lo : pool_stand_in;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = wave * 4 + q;
      const int rid = q == 0 ? rids.x : q == 1 ? rids.y : q == 2 ? rids.z : rids.w;
      const int soff = (rid >= 0 ? rid : stand_in) * (D * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(kbuf + r * KT::ROWB), 16,
                                               lane_off, soff, 0, 0);
      if constexpr (D > 512) {
        // (the immediate offset would move the LDS address too: the extra
        // 1024 bytes go in the scalar offset, which addresses memory only)
        if (lane < (D - 512) / 8)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(kbuf + r * KT::ROWB + 1024),
                                                   16, lane_off, soff + 1024, 0, 0);
      }
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T): head hq, this wave's half of
  // the k-steps, dims 32ks + 8g .. +7
  const int hq = 16 * hgrp + c16;
  const int ks0 = KH * kh;                       // first k-step of this wave
  uint4 qraw[KH];
  {
    const u16* qrow = reinterpret_cast<const u16*>(p.q) + (row * H + h0 + hq) * D;
#pragma unroll
    for (int ks = 0; ks < KH; ++ks)
      qraw[ks] = *reinterpret_cast<const uint4*>(qrow + 32 * (ks0 + ks) + 8 * g);
  }
  // the sink logit, loaded before the gathers so that waiting for it does not
  // wait for them
  const bool use_sink = p.sink && !split_mode;
  const float sink_l2 = use_sink ? p.sink[h0 + hq] * kLog2e : -INFINITY;
  if (tid == 0) { flags[0] = 1; flags[1] = 1; }
  // the first NBUF-1 gathers (issued whether or not the tiles exist, as in the
  // loop, so that the wait counts are the same on every path)
  issue(std::integral_constant<int, 0>{}, tile0, rid4(tile0));
  issue(std::integral_constant<int, 1>{}, tile0 + 1, rid4(tile0 + 1));
  if constexpr (NBUF == 4) issue(std::integral_constant<int, 2>{}, tile0 + 2, rid4(tile0 + 2));

  // rotate the rope slice of q at +t, round to bf16
  bf16x8 qf[KH];
#pragma unroll
  for (int ks = 0; ks < KH; ++ks) {
    // the rope slice is the last R dims: the last R/32 k-steps of the upper half
    const int d0 = 32 * (ks0 + ks) + 8 * g;
    uint4 u = qraw[ks];
    if (ks >= KH - R / 32 && kh == 1) {
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

  // ---- softmax state of head hq (replicated over the 4 lane groups, and the
  // same in both waves of the head block), log2 domain; lrun sums the keys of
  // this wave's key half only
  const float sl2 = p.scale * kLog2e;
  float mref = sink_l2, lrun = (use_sink && kh == 0) ? 1.f : 0.f;

  f32x4 acc[4][NB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int col0 = 64 * wave + 4 * c16;          // this lane's first output column

  // this wave's partial S^T of the pending tile (its half of the k-steps),
  // key blocks 0 and 1; empty key slots hold -inf
  f32x4 sp[2];

  // ---- S phase pieces.  Lane supplies K row 16kb + c16, 16-byte chunk
  // 4(ks0 + ks) + g for key block kb and k-step ks of this wave's half.
  auto k_row = [&](auto JC) __attribute__((always_inline)) -> const unsigned char* {
    return kbuf_of(JC) + c16 * KT::ROWB + 16 * g + 64 * ks0;
  };
  // bias the partials (0 / -inf per key slot; the lower D-half wave adds it,
  // so the sum of the two partials carries it once) and publish them for the
  // other wave of the head block
  auto s_finish = [&](auto JC, const f32x4 st0, const f32x4 st1) __attribute__((always_inline)) {
    constexpr int J = decltype(JC)::value;
    sp[0] = st0;
    sp[1] = st1;
    if (kh == 0) {
      sp[0] += *reinterpret_cast<const f32x4*>(bias_s + J * kNK + 4 * g);
      sp[1] += *reinterpret_cast<const f32x4*>(bias_s + J * kNK + 16 + 4 * g);
    }
    *reinterpret_cast<f32x4*>(spart + (wave * 2 + 0) * 64 * 4 + 4 * lane) = sp[0];
    *reinterpret_cast<f32x4*>(spart + (wave * 2 + 1) * 64 * 4 + 4 * lane) = sp[1];
  };
  // the S phase on its own (first tile): groups of 2 k-steps x 2 key blocks,
  // the fence bounds the K fragments held in registers at once
  auto s_phase = [&](auto JC) __attribute__((always_inline)) {
    const unsigned char* krow = k_row(JC);
    f32x4 st0 = f32x4{0.f, 0.f, 0.f, 0.f}, st1 = st0;  // key blocks 0 / 1
#pragma unroll
    for (int k2 = 0; k2 < KH; k2 += 2) {
      uint4 kv[2][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        if (k2 + kk < KH) {
          kv[kk][0] = *reinterpret_cast<const uint4*>(krow + 64 * (k2 + kk));
          kv[kk][1] = *reinterpret_cast<const uint4*>(krow + 16 * KT::ROWB + 64 * (k2 + kk));
        }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        if (k2 + kk < KH) {
          st0 = mfma16x16x32(as_bf16x8(kv[kk][0]), qf[k2 + kk], st0);
          st1 = mfma16x16x32(as_bf16x8(kv[kk][1]), qf[k2 + kk], st1);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    s_finish(JC, st0, st1);
  };

  // ---- softmax of the pending tile, once both waves' partials are in LDS:
  // the full logits of the 32 keys of head hq (identical in both waves: the
  // two partials are added in either order), the new reference max, P of this
  // wave's key half to LDS (key 16kh + 4g + j at position 8g + 4kh + j), the
  // rescale factor of head hq, and the rescale flag of parity par
  auto softmax = [&](auto JC, int par) __attribute__((always_inline)) {
    const int pw = wave ^ 4;
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(spart + (pw * 2 + 0) * 64 * 4 + 4 * lane);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(spart + (pw * 2 + 1) * 64 * 4 + 4 * lane);
    // raw logits; the scale (> 0) commutes with the max and goes into the
    // exponent's fused multiply-add
    const f32x4 f0 = sp[0] + o0, f1 = sp[1] + o1;
    const float m0 = fmaxf(fmaxf(f0[0], f0[1]), fmaxf(f0[2], f0[3]));
    const float m1 = fmaxf(fmaxf(f1[0], f1[1]), fmaxf(f1[2], f1[3]));
    const float tmax = xgroup_max(fmaxf(m0, m1)) * sl2;
    const f32x4 sv = kh ? f1 : f0;
    const float mnew = (tmax > mref + kLazy) ? tmax : mref;
    const float alpha = (mnew == mref) ? 1.f : __builtin_amdgcn_exp2f(mref - mnew);
    const float mbase = (mnew == -INFINITY) ? 0.f : mnew;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[0], sl2, -mbase));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[1], sl2, -mbase));
    const float p2 = __builtin_amdgcn_exp2f(fmaf(sv[2], sl2, -mbase));
    const float p3 = __builtin_amdgcn_exp2f(fmaf(sv[3], sl2, -mbase));
    lrun = lrun * alpha + xgroup_sum((p0 + p1) + (p2 + p3));
    mref = mnew;
    *reinterpret_cast<uint2*>(Ps + hq * kPS + 8 * g + 4 * kh) =
        make_uint2(pack2(p0, p1), pack2(p2, p3));
    if (kh == 0 && g == 0) alpha_s[hq] = alpha;
    if (kh == 0 && __ballot(alpha != 1.f) != 0ull && lane == 0) flags[par] = 1;
  };

  // ---- PV phase of the tile in buffer J: O[all 64 heads][this wave's 64
  // columns] += P V (after the rescale when some head raised its maximum),
  // then, when WITH_S, the S phase of the tile in the next buffer.  The
  // operand reads run ahead of the matrix instructions: the PV operands and
  // the first K fragments are read before the PV products, and every group of
  // S products is followed by the reads of the group after next.
  auto pv_s = [&](auto JC, auto WITH_S, int par) __attribute__((always_inline)) {
    constexpr bool kS = decltype(WITH_S)::value;
    using JN = std::integral_constant<int, (decltype(JC)::value + 1) % NBUF>;
    const unsigned char* kbuf = kbuf_of(JC);
    if (flags[par]) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const float4 al = *reinterpret_cast<const float4*>(alpha_s + 16 * mb + 4 * g);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[mb][nb][0] *= al.x; acc[mb][nb][1] *= al.y;
          acc[mb][nb][2] *= al.z; acc[mb][nb][3] *= al.w;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pa[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      pa[mb] = as_bf16x8(*reinterpret_cast<const uint4*>(Ps + (16 * mb + c16) * kPS + 8 * g));
    // V: for key position q (key 16*(q/4) + 4g + q%4), this lane's 4 columns
    uint32_t vr[8][2];
    const unsigned char* vcol = kbuf + 4 * g * KT::ROWB + 2 * col0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint2 u = *reinterpret_cast<const uint2*>(
          vcol + (16 * (q >> 2) + (q & 3)) * KT::ROWB);
      vr[q][0] = u.x; vr[q][1] = u.y;
    }
    uint4 kv[KH][2];
    const unsigned char* krow = k_row(JN{});
    // the first half of the K fragments now, the second half once the PV
    // operands are consumed (bounds the registers held at once)
    constexpr int KA = KH / 2;
    auto k_reads = [&](int k_lo, int k_hi) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < KH; ++ks)
        if (ks >= k_lo && ks < k_hi) {
          kv[ks][0] = *reinterpret_cast<const uint4*>(krow + 64 * ks);
          kv[ks][1] = *reinterpret_cast<const uint4*>(krow + 16 * KT::ROWB + 64 * ks);
        }
    };
    if constexpr (kS) k_reads(0, KA);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int dw = nb >> 1;
      uint32_t f[4];
#pragma unroll
      for (int d = 0; d < 4; ++d)  // low halves (even nb) or high halves (odd nb) of two keys
        f[d] = __builtin_amdgcn_perm(vr[2 * d + 1][dw], vr[2 * d][dw],
                                     (nb & 1) ? 0x07060302u : 0x05040100u);
      const bf16x8 vb = as_bf16x8(make_uint4(f[0], f[1], f[2], f[3]));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = mfma16x16x32(pa[mb], vb, acc[mb][nb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kS) {
      k_reads(KA, KH);
      f32x4 st0 = f32x4{0.f, 0.f, 0.f, 0.f}, st1 = st0;  // key blocks 0 / 1
#pragma unroll
      for (int ks = 0; ks < KH; ++ks) {
        st0 = mfma16x16x32(as_bf16x8(kv[ks][0]), qf[ks], st0);
        st1 = mfma16x16x32(as_bf16x8(kv[ks][1]), qf[ks], st1);
      }
      s_finish(JN{}, st0, st1);
    }
  };

  // ---- software pipeline over the tiles, two barriers per tile:
  //   X(j): partials of tile j published; buffer (j-1) and P free
  //         -> softmax of tile j, gather tile j+NBUF-1 into buffer (j-1)
  //   Y(j): P(j) and the rescale factors visible; tile j+1 landed
  //         -> PV of tile j, then S of tile j+1 (matrix cores back to back)
  // Gathers are issued past the last tile as well (every row empty: the
  // buffer is zero-filled), so that every iteration issues the same loads and
  // the wait counts are exact; the row ids of the next gather are looked up
  // an iteration ahead.
  constexpr int kAhead = (NBUF - 2) * KT::G;   // loads still in flight at a wait
  wait_vmcnt<kAhead>();
  lds_barrier();  // tile0 landed
  s_phase(std::integral_constant<int, 0>{});
  int4 rid_next = rid4(tile0 + NBUF - 1);
  auto iter = [&](auto JC, int j) __attribute__((always_inline)) {
    constexpr int J = decltype(JC)::value;
    const int par = (j - tile0) & 1;
    const bool live = j < tile1;
    lds_barrier();  // X(j)
    if (live) softmax(JC, par);
    issue(std::integral_constant<int, (J + NBUF - 1) % NBUF>{}, j + NBUF - 1, rid_next);
    wait_vmcnt<kAhead>();  // this wave's loads of tile j+1 have landed
    lds_barrier();  // Y(j)
    if (tid == 0) flags[par ^ 1] = 0;  // the next tile's rescale flag starts clear
    // the S phase runs after the last tile too, on a zero-filled buffer: one
    // code path keeps the register allocation tight
    if (live) pv_s(JC, std::true_type{}, par);
    rid_next = rid4(j + NBUF);
  };
  // whole rounds of NBUF iterations: the ones past the last tile only keep the
  // barriers and the (empty) gathers, so that the loads issued are the same
  // on every path through the loop
  for (int tile = tile0; tile < tile1; tile += NBUF) {
    iter(std::integral_constant<int, 0>{}, tile);
    iter(std::integral_constant<int, 1>{}, tile + 1);
    iter(std::integral_constant<int, 2>{}, tile + 2);
    if constexpr (NBUF == 4) iter(std::integral_constant<int, 3>{}, tile + 3);
  }
  // no gather may still be writing this workgroup's LDS when it exits
  wait_vmcnt<0>();

  // ---- epilogue: l = sum over both key halves
  if (kh == 1 && g == 0) l_s[hq] = lrun;
  lds_barrier();
  if (kh == 0 && g == 0) {
    const float l = lrun + l_s[hq];
    if (split_mode) {
      float* ml = args.ws + ((size_t)row * args.nsplit + split) * H * 2;
      ml[2 * (h0 + hq)] = mref;
      ml[2 * (h0 + hq) + 1] = l;
    } else {
      fin_s[hq] = l > 0.f ? 1.f / l : 0.f;
    }
  }
  if (split_mode) {
    float* po = args.ws + (size_t)((long)p.B * p.S) * args.nsplit * H * 2 +
                ((size_t)row * args.nsplit + split) * H * dv;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(po + (size_t)(h0 + 16 * mb + 4 * g + j) * dv + col0) =
            make_float4(acc[mb][0][j], acc[mb][1][j], acc[mb][2][j], acc[mb][3][j]);
    return;
  }
  lds_barrier();
  u16* out = reinterpret_cast<u16*>(p.out) + (row * H + h0) * dv;
  const bool derot = (dv == D) && col0 + NB > rbase;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
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
            const float2 rr = cs[t * half + ((col - rbase) >> 1)];
            const float a = v[nb], bb = v[nb + 1];
            v[nb] = a * rr.x + bb * rr.y;
            v[nb + 1] = -a * rr.y + bb * rr.x;
          }
        }
      }
      *reinterpret_cast<uint2*>(out + (16 * mb + 4 * g + j) * dv + col0) =
          make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
    }
  }
}

// Merge split partials: M = max(z, m_s), L = e^(z-M) + sum e^(m_s-M) l_s,
// O = sum e^(m_s-M) O_s / L, then the output rope slice is rotated at -t.
// Thread = 8 consecutive columns of one head; 4 heads per workgroup.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p, const float* ws,
                                                           int nsplit) {
  const long row = blockIdx.x;
  const int H = p.H, dv = p.dv;
  const int per_head = dv >> 3;
  const int h = blockIdx.y * (256 / per_head) + threadIdx.x / per_head;
  if (h >= H) return;
  const int c = (threadIdx.x % per_head) * 8;
  const int b = (int)(row / p.S);
  const long t = (long)p.q_pos[b] + (row - (long)b * p.S);
  const int half = p.rope_dim >> 1, rbase = p.D - p.rope_dim;
  const float2* cs = reinterpret_cast<const float2*>(p.cs);
  const float* ml = ws + (size_t)row * nsplit * H * 2;
  const float* po =
      ws + (size_t)((long)p.B * p.S) * nsplit * H * 2 + (size_t)row * nsplit * H * dv;
  float M = p.sink ? p.sink[h] * kLog2e : -INFINITY;
  bool nan = false;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = ml[(s * H + h) * 2];
    if (ms != ms) nan = true;
    M = fmaxf(M, ms);
  }
  const float Mb = (M == -INFINITY) ? 0.f : M;
  float L = p.sink ? exp2f(p.sink[h] * kLog2e - Mb) : 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float f = exp2f(ml[(s * H + h) * 2] - Mb);
    L += f * ml[(s * H + h) * 2 + 1];
    const float4* os = reinterpret_cast<const float4*>(po + ((size_t)s * H + h) * dv + c);
    const float4 a = os[0], bq = os[1];
    o[0] += f * a.x; o[1] += f * a.y; o[2] += f * a.z; o[3] += f * a.w;
    o[4] += f * bq.x; o[5] += f * bq.y; o[6] += f * bq.z; o[7] += f * bq.w;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] *= inv;
  const bool tin = t >= 0 && t < p.n_pos;
  if (p.dv == p.D && p.rope_dim > 0 && tin) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      if (c + e >= rbase) {
        const float2 r = cs[t * half + ((c + e - rbase) >> 1)];
        const float a = o[e], bb = o[e + 1];
        o[e] = a * r.x + bb * r.y;
        o[e + 1] = -a * r.y + bb * r.x;
      }
    }
  }
  if (nan || !tin)
    for (int e = 0; e < 8; ++e) o[e] = __int_as_float(0x7fc00000);
  *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.out) + (row * H + h) * dv + c) =
      make_uint4(pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7]));
}

// Matrix-core shapes: heads in groups of 64 (H = 128 runs as two groups),
// D = 512 (CSA / HCA) or 576 (DSA: 512 latent + 64 rope), dv = 512, rope 64.

bool mfma_shape(int H, int D, int dv, int rope_dim, int k) {
  (void)k;
  return H % 64 == 0 && dv == 512 && rope_dim == 64 && (D == 512 || D == 576);
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
                        bool bf16, long max_rows, int k) {
  AttnPlan pl{0, 1, 1 << 30, 0};
  if (!bf16 || !mfma_shape(H, D, dv, rope_dim, k)) return pl;
  // the gather addresses one sequence's rows with 32-bit buffer offsets
  if (max_rows * D * 2 >= 0x7ffffff0L) return pl;
  pl.kernel = 1;
  const long wgs = (long)B * S * (H / 64);
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
  MfmaArgs a;
  a.p = p;
  const bool split = plan.nsplit > 1 && ws != nullptr;
  a.ws = split ? reinterpret_cast<float*>(ws) : nullptr;
  a.nsplit = split ? plan.nsplit : 1;
  a.tiles_per_split = split ? plan.tiles_per_split : (1 << 30);
  a.rows_per_xcd = (int)((rows + 7) / 8);
  dim3 grid((unsigned)(8 * (long)a.rows_per_xcd), a.nsplit, p.H / 64);
  if (p.D == 512)
    hipLaunchKernelGGL((attn_mfma_kernel<512, 4>), grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<576, 3>), grid, dim3(512), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !split) return err;
  const int per_wg = 256 / (p.dv / 8);
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)rows, (p.H + per_wg - 1) / per_wg),
                     dim3(256), 0, s, p, reinterpret_cast<const float*>(ws), a.nsplit);
  return hipGetLastError();
}

}  // namespace csa
