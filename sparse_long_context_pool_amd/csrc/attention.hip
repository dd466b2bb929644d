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
// Matrix-core kernel (bf16).  One workgroup = one query row x 64 heads.  The
// key list (window slots, then pool slots) is walked in tiles of 32 rows; each
// tile's rows are gathered from HBM straight into LDS (16-byte direct-to-LDS
// buffer loads, several tiles in flight) into ONE tile that serves as both K
// and V, so a selected row is read once per query row for all heads.  Half of
// the waves compute S^T = K Q^T (v_mfma_f32_16x16x32_bf16, Q in registers) and
// the softmax (seeded with the sink logit), the other half P V with the value
// columns split between them; the two halves work one tile apart.  Rows whose
// keys exceed one workgroup's share (decode: few query rows, 2176 keys each)
// are split over workgroups; partial (max, sum, O) go to the caller's
// workspace and a combine kernel merges them with the sink.
// Generic kernel: one wave per (row, head), any dtype and shape.
#include "csa_device.hpp"

#include <algorithm>
#include <type_traits>

namespace csa {
namespace {

constexpr int kNK = 32;     // keys per tile
constexpr int kPS = kNK + 8;  // P row stride (u16): 80 bytes keeps P reads conflict-free
constexpr int kMaxK = 2048;   // index slots per query the matrix-core kernel keeps in LDS
// Cache-policy operand of buffer loads and stores: the non-temporal hint.  On
// the 512-wide rows (CSA, HCA) the queries (each read once) and the outputs
// (each written once, and together far larger than the 256 MB last-level
// cache: 512 MB for an 8192-token prefill) carry it, so that streaming them
// does not evict what the caches hold for the stages around the attention
// (measured: the next step's compression 21.5 -> 19.5 us and index scores
// 130 -> 126 us on CSA prefill, HCA compression 80 -> 62 us; the attention
// itself unchanged).  The 576-wide DSA rows keep plain queries and outputs:
// with the hint their attention fetched 53 GB instead of 40 GB and ran 1%
// slower.
constexpr int kNT = 2;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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
    const long r = p.win_ring ? pos % p.L_win : pos - (long)p.win_pos0[ri.b];
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

// Division of n < 2^31 by an invariant d < 2^31 with one multiply-high: m =
// floor(2^32 / d) + 1 makes floor(n m / 2^32) either n / d or one more (the
// excess n (m - 2^32 / d) / 2^32 is below 1/2), which one compare settles.
// m = 0 stands for d = 1.
struct FastDiv {
  unsigned d, m;
};
inline FastDiv make_fastdiv(unsigned d) {
  FastDiv f;
  f.d = d;
  f.m = d <= 1 ? 0u : (unsigned)((1ull << 32) / d + 1);
  return f;
}
__device__ __forceinline__ unsigned fdiv(unsigned n, FastDiv f) {
  if (f.m == 0) return n;
  const unsigned q = __umulhi(n, f.m);
  return q * f.d > n ? q - 1 : q;
}

struct MfmaArgs {
  AttnParams p;
  float* ws;              // split partials, or nullptr
  int nsplit;             // splits of a row's key list (1: none)
  int tiles_per_split;    // tiles of a split (huge: no split)
  int nhg;                // groups of 64 heads
  int rows;               // query rows B * S
  long n_items;           // work items: rows rounded up to 8, x splits x head groups
  FastDiv by_nhg, by_nsplit, by_S, by_m;
};

// K=V tile of 32 rows in LDS, 1 KiB per row, the 16-byte chunks of row r
// stored XOR-swizzled: logical chunk c sits at chunk c ^ f(r), with
// f(r) = 2 ((r + 4 h) % 8) + h, h = (r / 8) % 2 (rows r and r + 16 alike).
// The PV-phase transposing reads (8-byte, served 32 lanes at a time: eight
// consecutive rows x two adjacent chunks {2i, 2i + 1}) need f / 2 distinct
// over eight consecutive rows, which any such f gives; among those, this one
// was measured (with the LDS bank-conflict counter, over candidate swizzles)
// to leave the S-phase reads (16-byte, sixteen rows x one chunk, four chunks
// per wave instruction) free of bank conflicts as well.  Rows are filled by
// direct global->LDS 16-byte buffer loads: one wave instruction per row writes
// 1 KiB contiguous (lane l at +16 l), lane l reading logical chunk l ^ f(r)
// from memory; lanes whose row slot is past the tile range read past the
// buffer bound, which writes zeros.
//
// When D > 512 (a 512-wide latent part followed by the rope dims) the first 512
// dims of each row are laid out as above and the rest goes to a tail area: one
// block per wave of 8 rows, chunk-major ([16-byte chunk][row]), blocks 1152
// bytes apart.  One 64-lane load then gathers the tails of a wave's 8 rows,
// and the S-phase reads of the tail (16 rows, one chunk) still fall in
// distinct banks.
// chunk swizzle of tile row r (see above); rows r and r + 16 share it
__device__ __forceinline__ int swz(int r) {
  const int h = (r >> 3) & 1;
  return ((((r & 7) + 4 * h) & 7) << 1) | h;
}

template <int D>
struct KTile {
  static constexpr int MAIN = D > 512 ? 512 : D;    // dims in the row area
  static constexpr int ROWB = MAIN * 2;
  static_assert(MAIN == 512, "the chunk swizzle assumes 64 chunks per row");
  static constexpr int TAIL = D - MAIN;             // dims in the tail area
  static constexpr int TBLK = 1152;                 // tail block stride (8 rows)
  static_assert(TAIL == 0 || TAIL == 64, "tail of 64 dims");
  static constexpr int BYTES = kNK * ROWB;
  static constexpr int TBYTES = TAIL ? 4 * TBLK : 16;
};

// Split workspace: [rows][nsplit][H][2] fp32 running (max, sum) in the log2
// domain, then [rows][nsplit][H][dv] unnormalised partial outputs in bf16.
//
// Work items: (query row, split of its key list, group of 64 heads).  The
// grid is persistent (one workgroup per compute unit) and workgroup w takes
// items w, w + grid, w + 2 grid, ...; item i stands for row 8 (i / 8 / (splits
// x groups)) + i % 8 with its group and split from the middle digits, so the
// workgroups of one XCD (which gets every 8th workgroup) run the head groups
// and splits of the same rows side by side and share their gathers in the
// XCD's L2.  The tiles of a workgroup's items form ONE stream: each item's
// tile count is padded to whole rounds of NBUF tiles (the padding tiles are
// skipped), and the gathers, index entries, query fragments and list length
// of the next item are fetched while the current one is still running, so
// a row costs no pipeline fill or drain.
//
// 8 waves in two roles, one wave of each role per SIMD (so the hardware
// interleaves them):
//   S waves (0..3): wave w owns heads 16w .. 16w+15 for the S products and
//     the softmax (all keys of a tile, so a head's softmax state lives in one
//     wave), and reads each item's metadata, index-row length and queries;
//   PV waves (4..7): wave 4+w owns output columns 128w .. 128w+127 and their
//     accumulators, and loads the index entries and gathers rows 8w .. 8w+7
//     of each tile.
// S phase: S^T[keys][heads] = K Q^T with 16x16x32 matrix instructions, the
// query fragments held in registers; a lane ends with the logits of keys
// 4g + r and 16 + 4g + r (g = lane / 16, r = 0..3) of its head, which are
// exactly a P operand of the PV product (O^T = V^T P^T, P the B operand) in
// the key order position 8g + e <-> key 16(e/4) + 4g + (e%4).  P goes through LDS in that order, and
// V is read with the gfx950 transposing LDS load (ds_read_b64_tr_b16: 4 keys
// x 1 column per lane) in the same key order.
//
// Pipeline, one barrier per tile: between barriers B(j) and B(j+1) (stream
// positions) the S waves run S + softmax of tile j+1 while the PV waves run
// PV of tile j, load the index entries of tile j+NBUF and gather tile
// j+NBUF-1 into the buffer of tile j-1; before B(j+1) the PV waves wait for
// their loads of tile j+2.
//
// Softmax: per head a reference max m (log2 domain) that only ever rises:
// the first tile of an item sets it (from the sink logit and the tile), and a
// later tile whose max exceeds it by more than 64 raises it to that max, the
// running sum and the accumulators being scaled by 2^(m_old - m_new) (the S
// waves publish the factors with the tile's P, the PV waves apply them before
// adding the tile's P V).  So P <= 2^64 and the rescale is rare.
// NTG: the gathers carry the non-temporal hint.  Split launches (few query rows,
// each gathering thousands of distinct pool rows once: decode) take it;
// prefill-like launches do not, since neighbouring rows re-read their window
// and pool rows from L2 (measured: decode attention 2.5 us faster with it,
// CSA prefill attention 6-8% slower).
template <int D, int NBUF, bool NTG>
__global__ __launch_bounds__(512) void attn_mfma_kernel(MfmaArgs args) {
  constexpr int HG = 64, NB = 8;                     // NB: 16-column blocks per PV wave
  constexpr int KS = D / 32;
  constexpr int R = 64, half = R / 2, rbase = D - R;
  constexpr float kRescale = 64.f;
  constexpr int QO = D == 512 ? kNT : 0;             // cache policy of queries and outputs
  constexpr int NS = 4;                              // S waves (and PV waves)
  constexpr int RPW = kNK / NS;                      // gathered rows per PV wave per tile
  constexpr int NSCAN = kMaxK / (NS * 64);           // index-row loads per S lane
  using KT = KTile<D>;
  constexpr int G = RPW + (KT::TAIL ? 1 : 0);         // gather loads per wave per tile
  static_assert(NBUF == 3 || NBUF == 4, "buffer count");
  // One static array per K buffer: with distinct objects the compiler can
  // tell that an in-flight gather into one buffer does not alias reads of
  // another, so it does not wait for the gather before those reads.
  __shared__ __attribute__((aligned(16))) unsigned char kb0[KT::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char kb1[KT::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char kb2[KT::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char kb3[NBUF == 4 ? KT::BYTES : 16];
  // tail areas (D > 512), one object per buffer as well
  __shared__ __attribute__((aligned(16))) unsigned char tb0[KT::TBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char tb1[KT::TBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char tb2[KT::TBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char tb3[NBUF == 4 ? KT::TBYTES : 16];
  // every other LDS array is static as well, for the same reason
  __shared__ __attribute__((aligned(16))) u16 Ps[2 * HG * kPS];     // P, bf16, 2 tiles
  __shared__ __attribute__((aligned(16))) float bias_s[NBUF * kNK]; // 0 / -inf per slot
  __shared__ __attribute__((aligned(16))) float alpha_s[2][HG];     // rescale factors
  __shared__ __attribute__((aligned(16))) int rfl_s[2][NS];         // rescale flags
  __shared__ __attribute__((aligned(16))) float fin_s[2][HG];       // 1/l per item parity
  __shared__ __attribute__((aligned(16))) int scan_s[2][NS];        // last live slot, per wave
  __shared__ __attribute__((aligned(16))) int meta_s[2][4];         // t, n_win, r_lo, bad
  __shared__ __attribute__((aligned(16))) float2 cs_s[2][R / 2];    // RoPE factors at t
  __shared__ __attribute__((aligned(16))) int idx_s[2][kMaxK];      // index rows of 2 items
  const AttnParams& p = args.p;
  auto kbuf_of = [&](auto JC) __attribute__((always_inline)) -> unsigned char* {
    constexpr int J = decltype(JC)::value;
    if constexpr (J == 0) return kb0;
    else if constexpr (J == 1) return kb1;
    else if constexpr (J == 2) return kb2;
    else return kb3;
  };
  auto tbuf_of = [&](auto JC) __attribute__((always_inline)) -> unsigned char* {
    constexpr int J = decltype(JC)::value;
    if constexpr (J == 0) return tb0;
    else if constexpr (J == 1) return tb1;
    else if constexpr (J == 2) return tb2;
    else return tb3;
  };

  // the wave index is uniform: keep it (and everything derived from it) scalar
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const bool s_role = wave < NS;                  // S wave, else PV wave
  const int w4 = wave & (NS - 1);
  const int hq = 16 * w4 + c16;                   // S phase / softmax head
  const int cbase = 128 * w4;                     // PV phase columns
  const int H = p.H, dv = p.dv;
  const float2* cs = reinterpret_cast<const float2*>(p.cs);
  const bool split_mode = args.nsplit > 1;
  const bool use_sink = p.sink && !split_mode;
  const bool scan = !p.dense && p.k > 0 && p.pool;

  // ---- work items (wave-uniform)
  struct Item {
    int row;              // query row, -1: past the end of this workgroup's list
    int split, h0, b;
  };
  auto item_at = [&](int i) __attribute__((always_inline)) -> Item {
    Item it;
    it.row = -1; it.split = 0; it.h0 = 0; it.b = 0;
    const long n = (long)blockIdx.x + (long)i * gridDim.x;
    if (n >= args.n_items) return it;
    const int x = (int)(n & 7);
    const unsigned rest = (unsigned)(n >> 3);
    const unsigned rest2 = fdiv(rest, args.by_nhg);
    const int hg = (int)(rest - rest2 * args.nhg);
    const unsigned rest3 = fdiv(rest2, args.by_nsplit);
    it.split = (int)(rest2 - rest3 * args.nsplit);
    const int row = (int)rest3 * 8 + x;
    if (row >= args.rows) return it;
    it.row = row;
    it.h0 = hg * HG;
    it.b = (int)fdiv((unsigned)row, args.by_S);
    return it;
  };
  // ready pool entries of a valid position t (0 <= t < n_pos)
  auto ready_of = [&](int t) __attribute__((always_inline)) -> int {
    return min((int)fdiv((unsigned)t + 1u, args.by_m), p.T);
  };
  // what the gathers of an item need (t, the window range and the validity
  // come from the S waves through LDS)
  struct Meta {
    int row, split, h0, b, t, bad, n_win, r_lo, WT, tile0, tlim, bound;
  };
  auto meta_of = [&](const Item& it, int t, int n_win, int r_lo, int bad)
      __attribute__((always_inline)) -> Meta {
    Meta m;
    m.row = it.row; m.split = it.split; m.h0 = it.h0; m.b = it.b;
    m.t = t; m.bad = it.row < 0 ? 1 : bad; m.n_win = n_win; m.r_lo = r_lo;
    m.WT = (n_win + kNK - 1) / kNK;
    m.tile0 = it.split * args.tiles_per_split;
    m.tlim = m.tile0 + args.tiles_per_split;
    // pool slots a gather may read: every ready entry (dense) or the k slots
    m.bound = m.bad ? 0 : p.dense ? (p.pool ? ready_of(t) : 0) : p.k;
    return m;
  };
  // tiles of an item's slice of the key list (at least one, so that every
  // item has a first tile; the list length npool comes from the scan) and
  // that count padded to whole rounds
  auto tiles_of = [&](const Meta& m, int npool) __attribute__((always_inline)) -> int {
    if (m.bad) return 1;
    const int nt = min(m.WT + (npool + kNK - 1) / kNK, m.tlim) - m.tile0;
    return max(nt, 1);
  };
  auto padded = [&](int nt) __attribute__((always_inline)) -> int {
    return (nt + NBUF - 1) / NBUF * NBUF;
  };

  // ======================================================================
  // S waves
  // ======================================================================
  if (s_role) {
    // per-sequence values through bounded descriptors (no branch, zero when
    // absent)
    const __amdgpu_buffer_rsrc_t qpos_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int*>(p.q_pos), 0, p.B * 4, 0x00020000);
    const bool has_win = p.window > 0 && p.kv_win != nullptr;
    const bool lin_win = has_win && !p.win_ring;
    const __amdgpu_buffer_rsrc_t wpos_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int*>(lin_win ? p.win_pos0 : p.q_pos), 0, lin_win ? p.B * 4 : 0,
        0x00020000);
    const __amdgpu_buffer_rsrc_t sink_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(use_sink ? p.sink : p.cs), 0, use_sink ? H * 4 : 0, 0x00020000);
    auto load_pos = [&](const Item& it, int& qp, int& wp) __attribute__((always_inline)) {
      qp = (int)__builtin_amdgcn_raw_buffer_load_b32(qpos_rs, 4 * it.b, 0, 0);
      wp = (int)__builtin_amdgcn_raw_buffer_load_b32(wpos_rs, 4 * it.b, 0, 0);
    };
    // t, window range and validity of an item from its sequence's values
    auto pos_meta = [&](const Item& it, int qp, int wp, int (&mt)[4])
        __attribute__((always_inline)) {
      qp = __builtin_amdgcn_readfirstlane(qp);
      wp = __builtin_amdgcn_readfirstlane(wp);
      const long t = (long)qp + (it.row - (long)it.b * p.S);
      const int bad = (it.row < 0 || t < 0 || t >= p.n_pos) ? 1 : 0;
      int n_win = 0, r_lo = 0;
      if (!bad && has_win) {
        if (p.win_ring) {
          // the ring holds positions (t - L_win, t]: row of position lo
          const long lo = max(t - p.window + 1, 0L);
          n_win = (int)(t - lo + 1);
          r_lo = (int)(lo % p.L_win);
        } else {
          const long lo = max(t - p.window + 1, max(0L, (long)wp));
          const long hi = min(t, (long)wp + (long)p.L_win - 1);
          if (hi >= lo) { n_win = (int)(hi - lo + 1); r_lo = (int)(lo - wp); }
        }
      }
      mt[0] = bad ? 0 : (int)t; mt[1] = n_win; mt[2] = r_lo; mt[3] = bad;
    };
    // index-row scan of an item: NSCAN loads per lane (through a descriptor
    // bounded by the row, so nothing is read without one), reduced later
    auto scan_load = [&](const Item& it, int (&w)[NSCAN]) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<int*>(scan && it.row >= 0 ? p.idx + (long)it.row * p.k : p.q_pos), 0,
          scan && it.row >= 0 ? p.k * 4 : 0, 0x00020000);
#pragma unroll
      for (int u = 0; u < NSCAN; ++u)
        w[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (NS * 64 * u + tid), 0, 0);
    };
    // an item's index row into LDS (slot = item parity) for the gathers, and
    // this wave's last live slot of it (-1: none) for the list length
    auto scan_publish = [&](const int (&w)[NSCAN], int slot) __attribute__((always_inline)) {
      // (the wave's last live slot from ballots: scalar work, no lane
      // exchange)
      int last = -1;
#pragma unroll
      for (int u = 0; u < NSCAN; ++u) {
        const int jj = NS * 64 * u + tid;
        idx_s[slot][jj] = w[u];
        const uint64_t live = __ballot(jj < p.k && w[u] >= 0 && w[u] < p.T);
        if (live != 0ull) last = NS * 64 * u + 64 * w4 + 63 - (int)__builtin_clzll(live);
      }
      if (lane == 0) scan_s[slot][w4] = last;
    };
    auto npool_of = [&](const int (&mt)[4], int slot) __attribute__((always_inline)) -> int {
      if (p.dense) return p.pool ? ready_of(mt[0]) : 0;
      if (!scan) return 0;
      const int4 s4 = *reinterpret_cast<const int4*>(scan_s[slot]);
      return __builtin_amdgcn_readfirstlane(max(max(s4.x, s4.y), max(s4.z, s4.w)) + 1);
    };

    // query fragments of an item (B operand of S^T = K Q^T): head h0 + hq,
    // dims 32ks + 8g .. +7, loaded raw with the RoPE factors of the rope
    // slice, rotated at +t and rounded to bf16 once they are in
    bf16x8 qf[KS];
    constexpr int KR = R / 32;                      // rope k-steps
    float2 csr[KR][4];
    float sink_raw = 0.f;
    auto q_load = [&](const Item& it, int t) __attribute__((always_inline)) {
      const long row = it.row < 0 ? 0 : it.row;
      const u16* qrow = reinterpret_cast<const u16*>(p.q) + (row * H + it.h0 + hq) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[ks] = QO != 0 ? __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                                                   reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * g)))
                         : as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g));
#pragma unroll
      for (int kr = 0; kr < KR; ++kr) {
        const float4* c4 = reinterpret_cast<const float4*>(cs + (long)t * half + 16 * kr + 4 * g);
        const float4 a = c4[0], bq = c4[1];
        csr[kr][0] = make_float2(a.x, a.y); csr[kr][1] = make_float2(a.z, a.w);
        csr[kr][2] = make_float2(bq.x, bq.y); csr[kr][3] = make_float2(bq.z, bq.w);
      }
      sink_raw = __builtin_bit_cast(
          float, (int)__builtin_amdgcn_raw_buffer_load_b32(sink_rs, 4 * (it.h0 + hq), 0, 0));
    };
    // D = 512: the next item's queries go into a second register set, their
    // loads spread over the first three iterations of the current item's last
    // round (a few per iteration, where the S waves have slack) instead of one
    // burst at its end; the RoPE factors and the rope k-steps go first (the
    // rotation needs them first).  The RoPE factors and the sink value of the
    // current item are dead once its first tile has started, so those go
    // straight into their registers.
    constexpr bool kSpread = D == 512;
    bf16x8 qn[KS];
    auto q_load_part = [&](const Item& it, int t, auto PART) __attribute__((always_inline)) {
      constexpr int part = decltype(PART)::value;
      const long row = it.row < 0 ? 0 : it.row;
      // (through a descriptor over the item's 64 query rows: one lane offset,
      // the k-step in the scalar offset)
      const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<u16*>(reinterpret_cast<const u16*>(p.q) + (row * H + it.h0) * D), 0,
          HG * D * 2, 0x00020000);
      const int qoff = (hq * D + 8 * g) * 2;
      auto qld = [&](int ks) __attribute__((always_inline)) -> bf16x8 {
        return __builtin_bit_cast(bf16x8,
                                  __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff, 64 * ks, QO));
      };
      if constexpr (part == 0) {
#pragma unroll
        for (int kr = 0; kr < KR; ++kr) {
          const float4* c4 =
              reinterpret_cast<const float4*>(cs + (long)t * half + 16 * kr + 4 * g);
          const float4 a = c4[0], bq = c4[1];
          csr[kr][0] = make_float2(a.x, a.y); csr[kr][1] = make_float2(a.z, a.w);
          csr[kr][2] = make_float2(bq.x, bq.y); csr[kr][3] = make_float2(bq.z, bq.w);
        }
      }
      // part 0: the rope k-steps and the first 8 - KR; part 1: the next 6;
      // part 2: the rest and the sink
      constexpr int lo = part == 0 ? 0 : part == 1 ? 8 - KR : 14 - KR;
      constexpr int hi = part == 0 ? 8 - KR : part == 1 ? 14 - KR : KS - KR;
      if constexpr (part == 0) {
#pragma unroll
        for (int kr = 0; kr < KR; ++kr) qn[KS - KR + kr] = qld(KS - KR + kr);
      }
#pragma unroll
      for (int ks = lo; ks < hi; ++ks) qn[ks] = qld(ks);
      if constexpr (part == 2)
        sink_raw = __builtin_bit_cast(
            float, (int)__builtin_amdgcn_raw_buffer_load_b32(sink_rs, 4 * (it.h0 + hq), 0, 0));
    };
    auto q_take = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = qn[ks];
    };
    // the RoPE factors of the item's position, for the PV waves' output
    auto cs_publish = [&](int slot) __attribute__((always_inline)) {
      if (w4 == 0 && c16 == 0) {
#pragma unroll
        for (int kr = 0; kr < KR; ++kr)
#pragma unroll
          for (int e = 0; e < 4; ++e) cs_s[slot][16 * kr + 4 * g + e] = csr[kr][e];
      }
    };
    auto q_rotate = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kr = 0; kr < KR; ++kr) {
        uint4 u = __builtin_bit_cast(uint4, qf[rbase / 32 + kr]);
        float v[8] = {bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y),
                      bf_lo(u.z), bf_hi(u.z), bf_lo(u.w), bf_hi(u.w)};
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float2 r = csr[kr][e >> 1];
          const float a = v[e], bb = v[e + 1];
          v[e] = a * r.x - bb * r.y;
          v[e + 1] = a * r.y + bb * r.x;
        }
        u.x = pack2(v[0], v[1]); u.y = pack2(v[2], v[3]);
        u.z = pack2(v[4], v[5]); u.w = pack2(v[6], v[7]);
        qf[rbase / 32 + kr] = as_bf16x8(u);
      }
    };

    // ---- softmax state of head hq (replicated over the 4 lane groups), log2
    // domain
    const float sl2 = p.scale * kLog2e;
    float mref = -INFINITY, lrun = 0.f;
    auto state_reset = [&]() __attribute__((always_inline)) {
      mref = use_sink ? sink_raw * kLog2e : -INFINITY;
      lrun = use_sink ? 1.f : 0.f;
    };

    // ---- S phase pieces.  S^T for keys 16kb + c16 (kb = 0, 1) and the 16
    // heads of this wave, in groups of 4 k-steps; lane supplies K row
    // 16kb + c16, 16-byte chunk 4ks + g.  Four accumulation chains (key block x
    // even/odd k-step).
    constexpr int GK = 4;                             // k-steps per group
    constexpr int NG = (KS + GK - 1) / GK;
    // K row c16 (and 16 + c16, same swizzle), logical chunk 4ks + g: physical
    // chunk ((4 (ks % 4) + g) ^ f(c16)) + 16 (ks / 4)
    const int fk = swz(c16);
    int koff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) koff[u] = c16 * KT::ROWB + 16 * ((4 * u + g) ^ fk);
    auto k_group = [&](auto JC, int grp, uint4 (&kv)[GK][2]) __attribute__((always_inline)) {
      const unsigned char* kbase = kbuf_of(JC);
      // tail area: rows c16 and 16 + c16 sit in wave blocks c16/8 and 2 + c16/8
      const unsigned char* ktail = tbuf_of(JC) + (c16 >> 3) * KT::TBLK + (c16 & 7) * 16 + 128 * g;
#pragma unroll
      for (int kk = 0; kk < GK; ++kk) {
        const int ks = GK * grp + kk;
        if (ks < KT::MAIN / 32) {
          const unsigned char* kp = kbase + koff[ks & 3] + 256 * (ks >> 2);
          kv[kk][0] = *reinterpret_cast<const uint4*>(kp);
          kv[kk][1] = *reinterpret_cast<const uint4*>(kp + 16 * KT::ROWB);
        } else if (ks < KS) {
          const int u = ks - KT::MAIN / 32;   // tail chunk 4u + g
          kv[kk][0] = *reinterpret_cast<const uint4*>(ktail + 512 * u);
          kv[kk][1] = *reinterpret_cast<const uint4*>(ktail + 2 * KT::TBLK + 512 * u);
        }
      }
    };
    auto s_group = [&](int grp, const uint4 (&kv)[GK][2], f32x4 (&sa)[4])
        __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < GK; ++kk) {
        const int ks = GK * grp + kk;
        if (ks < KS) {
          sa[(kk & 1) * 2 + 0] = mfma16x16x32(as_bf16x8(kv[kk][0]), qf[ks], sa[(kk & 1) * 2 + 0]);
          sa[(kk & 1) * 2 + 1] = mfma16x16x32(as_bf16x8(kv[kk][1]), qf[ks], sa[(kk & 1) * 2 + 1]);
        }
      }
    };
    // ---- softmax of a tile (buffer J) from its logits: P to P buffer par (key
    // position 8g + e <-> key 16(e/4) + 4g + (e%4)), with the rescale request
    auto bias_of = [&](auto JC, int kb) __attribute__((always_inline)) -> f32x4 {
      return *reinterpret_cast<const f32x4*>(bias_s + decltype(JC)::value * kNK + 16 * kb + 4 * g);
    };
    auto softmax = [&](int par, const f32x4 x0, const f32x4 x1, bool first)
        __attribute__((always_inline)) {
      // raw logits; the scale (> 0) commutes with the max and goes into the
      // exponent's fused multiply-add
      const float m0 = fmaxf(fmaxf(x0[0], x0[1]), fmaxf(x0[2], x0[3]));
      const float m1 = fmaxf(fmaxf(x1[0], x1[1]), fmaxf(x1[2], x1[3]));
      const float tmax = xgroup_max(fmaxf(m0, m1)) * sl2;
      float alpha = 1.f;
      if (first) {
        const float mnew = fmaxf(mref, tmax);
        if (mnew != mref) alpha = __builtin_amdgcn_exp2f(mref - mnew);
        mref = mnew;
        rfl_s[par][w4] = 0;
      } else {
        const bool up = tmax > mref + kRescale;
        if (up) {
          alpha = __builtin_amdgcn_exp2f(mref - tmax);
          mref = tmax;
        }
        // every lane writes the wave's verdict (no branch: this chain is
        // interleaved with matrix instructions)
        rfl_s[par][w4] = __ballot(up) != 0ull ? 1 : 0;
        if (g == 0) alpha_s[par][hq] = alpha;
      }
      const float mbase = (mref == -INFINITY) ? 0.f : mref;
      float pv[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(fmaf(x0[r], sl2, -mbase));
        pv[4 + r] = __builtin_amdgcn_exp2f(fmaf(x1[r], sl2, -mbase));
      }
      const float ps = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
      lrun = lrun * alpha + xgroup_sum(ps);
      *reinterpret_cast<uint4*>(Ps + (par * HG + hq) * kPS + 8 * g) =
          make_uint4(pack2(pv[0], pv[1]), pack2(pv[2], pv[3]), pack2(pv[4], pv[5]),
                     pack2(pv[6], pv[7]));
    };
    // ---- S-wave step: S + softmax of the tile in buffer JN (P buffer par),
    // the K groups read one group ahead of their products
    auto s_step = [&](auto JN, int par, bool first) __attribute__((always_inline)) {
      uint4 kv[2][GK][2];
      k_group(JN, 0, kv[0]);
      const f32x4 bias0 = bias_of(JN, 0), bias1 = bias_of(JN, 1);
      f32x4 sa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int grp = 0; grp < NG; ++grp) {
        __builtin_amdgcn_sched_barrier(0);
        if (grp + 1 < NG) k_group(JN, grp + 1, kv[(grp + 1) & 1]);
        s_group(grp, kv[grp & 1], sa);
      }
      __builtin_amdgcn_sched_barrier(0);
      softmax(par, sa[0] + sa[2] + bias0, sa[1] + sa[3] + bias1, first);
    };
    // ---- an item's end: running max and sum of each head, for the PV waves
    // (1/l) or the merge of the splits
    auto finish = [&](const Item& it, const int (&mt)[4], int slot) __attribute__((always_inline)) {
      if (g == 0) {
        const float nanv = __int_as_float(0x7fc00000);
        if (split_mode) {
          float* ml = args.ws + ((size_t)it.row * args.nsplit + it.split) * H * 2;
          ml[2 * (it.h0 + hq)] = mt[3] ? nanv : mref;
          ml[2 * (it.h0 + hq) + 1] = mt[3] ? 0.f : lrun;
        } else {
          fin_s[slot][hq] = mt[3] ? nanv : lrun > 0.f ? 1.f / lrun : 0.f;
        }
      }
    };

    // ---- prologue: items 0 and 1 (metadata, scan of item 0, queries of
    // item 0), the loads that item 0's last round will need (scan of item 1,
    // positions of item 2), then the first tile
    Item cur = item_at(0);
    if (cur.row < 0) return;                // no item (the PV waves leave as well)
    Item nx = item_at(1), nx2 = item_at(2);
    int qp0, wp0, qp1, wp1, qp2, wp2;
    load_pos(cur, qp0, wp0);
    load_pos(nx, qp1, wp1);
    load_pos(nx2, qp2, wp2);
    int wsc[NSCAN], wsc1[NSCAN];
    scan_load(cur, wsc);
    scan_load(nx, wsc1);
    int mt_cur[4], mt_nx[4], mt_nx2[4];
    pos_meta(cur, qp0, wp0, mt_cur);
    q_load(cur, mt_cur[0]);
    scan_publish(wsc, 0);
    scan_publish(wsc1, 1);
    scan_load(nx2, wsc);
    pos_meta(nx, qp1, wp1, mt_nx);
    if (w4 == 0 && lane == 0) {
      *reinterpret_cast<int4*>(meta_s[0]) = make_int4(mt_cur[0], mt_cur[1], mt_cur[2], mt_cur[3]);
      *reinterpret_cast<int4*>(meta_s[1]) = make_int4(mt_nx[0], mt_nx[1], mt_nx[2], mt_nx[3]);
    }
    lds_barrier();  // L0: metadata and index rows of items 0 and 1 published
    int n = 0;
    int ntl = tiles_of(meta_of(cur, mt_cur[0], mt_cur[1], mt_cur[2], mt_cur[3]),
                       npool_of(mt_cur, 0));
    int start = 0, end = padded(ntl);
    // (the queries land while the first gathers are in flight)
    q_rotate();
    cs_publish(0);
    state_reset();
    lds_barrier();  // tile 0 landed
    s_step(std::integral_constant<int, 0>{}, 0, true);
    lds_barrier();  // B(0)

    // ---- an item's last round, after its last S step (the query registers
    // are free): publish the index row, list length and metadata of the item
    // after next (loaded one item ago), load the next item's queries, then the
    // index row and positions of the item after that (issued after the
    // queries, so that waiting for the queries never waits for them)
    auto publish = [&]() __attribute__((always_inline)) {
      scan_publish(wsc, n & 1);
      pos_meta(nx2, qp2, wp2, mt_nx2);
      if (w4 == 0 && lane == 0)
        *reinterpret_cast<int4*>(meta_s[n & 1]) =
            make_int4(mt_nx2[0], mt_nx2[1], mt_nx2[2], mt_nx2[3]);
    };
    auto prefetch = [&]() __attribute__((always_inline)) {
      if constexpr (!kSpread) {
        publish();
        q_load(nx, mt_nx[0]);
      } else {
        q_load_part(nx, mt_nx[0], std::integral_constant<int, 2>{});
      }
      const Item n3 = item_at(n + 3);
      scan_load(n3, wsc);
      load_pos(n3, qp2, wp2);
    };
    // ---- the move to the next item, at the last iteration of an item's
    // last round (before S of the next item's first tile)
    bool moved = false;
    auto advance = [&]() __attribute__((always_inline)) {
      finish(cur, mt_cur, n & 1);
      ++n;
      cur = nx;
      nx = nx2;
      nx2 = item_at(n + 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) { mt_cur[e] = mt_nx[e]; mt_nx[e] = mt_nx2[e]; }
      if (cur.row >= 0) {
        if constexpr (kSpread) q_take();
        q_rotate();
        cs_publish(n & 1);
        state_reset();
      }
      // the new item starts here; its tile count is known after the round
      // (its first tile is always computed)
      start = end;
      ntl = 1;
      moved = true;
    };

    for (int r = 0;; ++r) {
      const bool last_round = (r + 1) * NBUF == end;
      auto iter = [&](auto JC, int j) __attribute__((always_inline)) {
        constexpr int J = decltype(JC)::value;
        const int q = j + 1;                // the tile this step computes
        if constexpr (J == NBUF - 1) {
          if (last_round) advance();
        }
        const int u = q - start;
        if (cur.row >= 0 && u < ntl)
          s_step(std::integral_constant<int, (J + 1) % NBUF>{}, q & 1, u == 0);
        if constexpr (kSpread && J == 0) {
          if (last_round && nx.row >= 0) q_load_part(nx, mt_nx[0], std::integral_constant<int, 0>{});
        }
        if constexpr (kSpread && J == 1) {
          // (not at J = 0: the PV waves read this item's list length and the
          // next item's metadata at the round start, before the first barrier)
          if (last_round && nx.row >= 0) {
            publish();
            q_load_part(nx, mt_nx[0], std::integral_constant<int, 1>{});
          }
        }
        if constexpr (J == NBUF - 2) {
          if (last_round && nx.row >= 0) prefetch();
        }
        lds_barrier();  // B(j+1)
      };
      iter(std::integral_constant<int, 0>{}, r * NBUF);
      iter(std::integral_constant<int, 1>{}, r * NBUF + 1);
      iter(std::integral_constant<int, 2>{}, r * NBUF + 2);
      if constexpr (NBUF == 4) iter(std::integral_constant<int, 3>{}, r * NBUF + 3);
      if (moved) {
        moved = false;
        if (cur.row < 0) break;
        ntl = tiles_of(meta_of(cur, mt_cur[0], mt_cur[1], mt_cur[2], mt_cur[3]),
                       npool_of(mt_cur, n & 1));
        end = start + padded(ntl);
      }
    }
    return;
  }

  // ======================================================================
  // PV waves
  // ======================================================================
  // The PV waves' chain (gathers, LDS reads, products) sets the tile time;
  // the S wave on the same SIMD finishes its share early and waits at the
  // barrier.  A higher issue priority lets a PV wave's instructions go first
  // when both are ready (measured against the default priority, A/B in one
  // process on three boxes: CSA prefill attention 2-4% faster, HCA 3-4%,
  // decode and DSA unchanged; the level, 1 to 3, made no difference).
  __builtin_amdgcn_s_setprio(2);
  // gather source offset of lane l for tile row 8w + q: logical chunk
  // l ^ f(8w + q) (loop-invariant registers)
  int lane_off[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) lane_off[q] = (lane ^ swz(RPW * w4 + q)) << 4;
  const int win_bytes = p.kv_win ? p.L_win * D * 2 : 0;
  const int pool_bytes = p.pool ? p.T * D * 2 : 0;

  // Row id of row 8w + lane % 8 of a tile (w = the wave's index in its role):
  // kv_win / pool row of the item's sequence, -1 = empty (or past the item's
  // range); pool entries come from the item's index row, which the S waves
  // put in LDS (slot = item parity) one item ahead.
  auto rid_of = [&](const Meta& m, int tile, int slot) __attribute__((always_inline)) -> int {
    if (m.bad || tile >= m.tlim) return -1;
    if (tile < m.WT) {
      const int jj = tile * kNK + w4 * RPW + (lane & 7);
      if (jj >= m.n_win) return -1;
      const int r = m.r_lo + jj;       // (a ring wraps once at most: n_win <= L_win)
      return r >= p.L_win ? r - p.L_win : r;
    }
    const int jj = (tile - m.WT) * kNK + w4 * RPW + (lane & 7);
    const int w = p.dense ? jj : idx_s[slot][min(jj, kMaxK - 1)];
    return (jj < m.bound && w >= 0 && w < p.T) ? w : -1;
  };

  // This wave's share of a tile's gather into buffer J: rows 8w .. 8w+7, one
  // 1 KiB load per row (and one 8-lane load of the last 128 bytes when D =
  // 576).  An empty slot gathers a stand-in row, the first non-empty one of
  // the 8 (finite data that the -inf bias of the slot cancels: its
  // probability is exactly 0); when all 8 are empty the loads go through a
  // zero-size descriptor (zero fill).  The row is wave-uniform: its offset
  // goes in the scalar operand, so the per-lane operands are the
  // loop-invariant lane_off[q] (the compiler's wait-count model treats a
  // register that fed a gather as pending until the gather lands, so a
  // per-gather temporary reused later for other data would cost a wait).
  auto issue = [&](auto JC, const Meta& m, int tile, int rid) __attribute__((always_inline)) {
    constexpr int J = decltype(JC)::value;
    unsigned char* kbuf = kbuf_of(JC);
    if (lane < RPW) bias_s[J * kNK + w4 * RPW + lane] = rid >= 0 ? 0.f : -INFINITY;
    const uint64_t live = __ballot(lane < RPW && rid >= 0);
    const bool win = tile < m.WT;
    const u16* base = win ? reinterpret_cast<const u16*>(p.kv_win) + (size_t)m.b * p.L_win * D
                          : reinterpret_cast<const u16*>(p.pool) + (size_t)m.b * p.T * D;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(base), 0, live == 0ull ? 0 : win ? win_bytes : pool_bytes,
        0x00020000);
    const int stand_in =
        live == 0ull ? 0 : __builtin_amdgcn_readlane(rid, (int)__builtin_ctzll(live));
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int r = w4 * RPW + q;
      const int rq = __builtin_amdgcn_readlane(rid, q);
      const int soff = (rq >= 0 ? rq : stand_in) * (D * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(kbuf + r * KT::ROWB), 16,
                                               lane_off[q], soff, 0, NTG ? kNT : 0);
    }
    if constexpr (KT::TAIL > 0) {
      // the tails of this wave's 8 rows: lane l takes row l%8, chunk l/8
      const int rid_l = rid >= 0 ? rid : stand_in;
      unsigned char* tbuf = tbuf_of(JC) + w4 * KT::TBLK;
      // (the offset goes through a named value: written inline in the call,
      // the host pass of this template drops the kernel's launch stub)
      const int tvoff = rid_l * (D * 2) + 2 * KT::MAIN + 16 * (lane >> 3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)tbuf, 16, tvoff, 0, 0,
                                               NTG ? kNT : 0);
    }
  };

  // V: column block nb, keys 4g + e (first read) and 16 + 4g + e (second):
  // lane (g, s) of a 16-lane block reads row 4g + s/4, columns 4(s%4) ..
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  // (row r = 4g + s/4 and 16 + r share the swizzle f(r); logical chunk
  // cbase/8 + 2nb + (s/2) % 2, byte 8 (s % 2) within it)
  const int rv = 4 * g + (c16 >> 2);
  const int fv = swz(rv);
  const int voff0 = rv * KT::ROWB + 2 * cbase + 8 * (c16 & 1);
  auto v_read = [&](auto JC, int nb) __attribute__((always_inline)) -> bf16x8 {
    const unsigned char* vrow =
        kbuf_of(JC) + voff0 + 16 * ((2 * nb + ((c16 >> 1) & 1)) ^ fv);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vrow);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vrow + 16 * KT::ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // O^T = V^T P^T: V is the A operand and P the B operand, so lane (g, c16)
  // holds, for head block mb and column block nb, the four adjacent columns
  // cbase + 16nb + 4g .. +3 of head 16mb + c16.
  f32x4 acc[4][NB];
  // ---- PV-wave step: PV of the tile in buffer J (P buffer par), after the
  // rescale the S waves may have asked for with this P.  An item's first tile
  // starts the sums from zero (no reset of the accumulators between items).
  auto pv_step = [&](auto JC, int par, auto FIRST) __attribute__((always_inline)) {
    constexpr bool first = decltype(FIRST)::value;
    if constexpr (!first) {
      const int4 rf = *reinterpret_cast<const int4*>(rfl_s[par]);
      if (__builtin_amdgcn_readfirstlane(rf.x | rf.y | rf.z | rf.w) != 0) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const float a = alpha_s[par][16 * mb + c16];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[mb][nb] *= a;
        }
      }
    }
    bf16x8 pa[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      pa[mb] = as_bf16x8(
          *reinterpret_cast<const uint4*>(Ps + (par * HG + 16 * mb + c16) * kPS + 8 * g));
    bf16x8 vb[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) vb[nb] = v_read(JC, nb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb][nb] = mfma16x16x32(vb[nb], pa[mb],
                                   first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mb][nb]);
  };

  // ---- output of an item (lane: head 16mb + c16, columns cbase + 16nb + 4g
  // .. +3 of each block)
  auto output = [&](const Meta& m, int slot) __attribute__((always_inline)) {
    if (split_mode) {
      // unnormalised partial outputs in bf16 (their scale is the split's
      // running max; the merge weighs them in fp32)
      u16* po = reinterpret_cast<u16*>(args.ws + (size_t)args.rows * args.nsplit * H * 2) +
                ((size_t)m.row * args.nsplit + m.split) * H * dv + (size_t)m.h0 * dv;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          *reinterpret_cast<uint2*>(po + (size_t)(16 * mb + c16) * dv + cbase + 16 * nb + 4 * g) =
              make_uint2(pack2(acc[mb][nb][0], acc[mb][nb][1]),
                         pack2(acc[mb][nb][2], acc[mb][nb][3]));
      return;
    }
    // The bf16 results go out through LDS as 16-byte stores: the buffer the
    // next gather (issued after this) fills is free here, and this wave
    // stages in the rows it gathers itself, so no other wave touches them.
    // Two passes of 32 heads x 128 columns (8 KiB).  Staged head row h holds
    // 16 chunks of 8 columns, chunk c at position c ^ 2 (h % 8): an 8-byte
    // write instruction (16 heads x 2 chunks) spreads evenly over the banks.
    // (stores through a descriptor: one lane offset register, the head and
    // pass in the scalar offset)
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<u16*>(p.out) + ((long)m.row * H + m.h0) * dv + cbase, 0, HG * dv * 2,
        0x00020000);
    const int olane = (g * dv + 8 * c16) * 2;
    unsigned char* stg = kbuf_of(std::integral_constant<int, NBUF - 1>{}) + w4 * RPW * KT::ROWB;
    auto stg_pos = [](int h, int c) __attribute__((always_inline)) -> int {
      return h * 256 + ((c ^ ((h & 7) << 1)) << 4);
    };
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
        const int mb = 2 * pass + mh;
        const float li = fin_s[slot][16 * mb + c16];
        const int hl = 16 * mh + c16;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          f32x4 v = acc[mb][nb] * li;
          if (dv == D && cbase + 16 * nb + 16 > rbase) {
            // de-rotate the rope slice at -t: the pairs (4g, 4g+1) and
            // (4g+2, 4g+3) of the block
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              const float2 rr = cs_s[slot][(cbase + 16 * nb + 4 * g + e - rbase) >> 1];
              const float a = v[e], bq = v[e + 1];
              v[e] = a * rr.x + bq * rr.y;
              v[e + 1] = bq * rr.x - a * rr.y;
            }
          }
          const int cl = 16 * nb + 4 * g;
          *reinterpret_cast<uint2*>(stg + stg_pos(hl, cl >> 3) + 2 * (cl & 7)) =
              make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
        }
      }
      // (LDS accesses of one wave complete in order: no barrier)
      // (four reads in flight, then their four stores)
#pragma unroll
      for (int i0 = 0; i0 < 8; i0 += 4) {
        u32x4 d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          d[i] = *reinterpret_cast<const u32x4*>(stg + stg_pos(4 * (i0 + i) + g, c16));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(d[i], ors, olane,
                                                 (32 * pass + 4 * (i0 + i)) * dv * 2, QO);
      }
    }
  };

  auto meta_read = [&](const Item& it, int slot) __attribute__((always_inline)) -> Meta {
    const int4 mt = *reinterpret_cast<const int4*>(meta_s[slot]);
    return meta_of(it, __builtin_amdgcn_readfirstlane(mt.x), __builtin_amdgcn_readfirstlane(mt.y),
                   __builtin_amdgcn_readfirstlane(mt.z), __builtin_amdgcn_readfirstlane(mt.w));
  };
  auto npool_read = [&](const Meta& m, int slot) __attribute__((always_inline)) -> int {
    if (p.dense) return m.bound;
    if (!scan) return 0;
    const int4 s4 = *reinterpret_cast<const int4*>(scan_s[slot]);
    return __builtin_amdgcn_readfirstlane(max(max(s4.x, s4.y), max(s4.z, s4.w)) + 1);
  };

  // ---- prologue: the first NBUF-1 gathers (an item has at least NBUF
  // tiles)
  Item it_cur = item_at(0);
  if (it_cur.row < 0) return;
  lds_barrier();  // L0
  Meta mc = meta_read(it_cur, 0);
  Meta mn = meta_read(item_at(1), 1);
  int n = 0;
  int ntl = tiles_of(mc, npool_read(mc, 0));
  int start = 0, end = padded(ntl);
  issue(std::integral_constant<int, 0>{}, mc, mc.tile0, rid_of(mc, mc.tile0, 0));
  issue(std::integral_constant<int, 1>{}, mc, mc.tile0 + 1, rid_of(mc, mc.tile0 + 1, 0));
  if constexpr (NBUF == 4)
    issue(std::integral_constant<int, 2>{}, mc, mc.tile0 + 2, rid_of(mc, mc.tile0 + 2, 0));
  // row ids of the next gather, looked up one iteration ahead of its issue so
  // that the index-row read is off the issue's path
  int rid_pend = rid_of(mc, mc.tile0 + NBUF - 1, 0);
  wait_vmcnt<(NBUF - 2) * G>();
  lds_barrier();  // tile 0 landed
  wait_vmcnt<(NBUF - 3) * G>();
  lds_barrier();  // B(0)

  for (int r = 0;; ++r) {
    if (r * NBUF == end) {
      // item n ended with the previous round: its output (the S waves wrote
      // its 1/l before the last barrier), then the next item's list length
      // and the metadata of the one after (published with that barrier)
      output(mc, n & 1);
      ++n;
      mc = mn;
      if (mc.row < 0) break;
      mn = meta_read(item_at(n + 1), (n + 1) & 1);
      start = end;
      ntl = tiles_of(mc, npool_read(mc, n & 1));
      end = start + padded(ntl);
    }
    // the item of the next round (the gathers run up to a round ahead)
    const bool ahead_next = (r + 1) * NBUF >= end;
    const Meta& ma = ahead_next ? mn : mc;
    const int sa = ahead_next ? end : start;
    const int slot_a = ahead_next ? (n + 1) & 1 : n & 1;
    auto iter = [&](auto JC, int j) __attribute__((always_inline)) {
      constexpr int J = decltype(JC)::value;
      // gather of position j+NBUF-1 (in this round for J = 0, in the next one
      // after), then the row ids of position j+NBUF (always the next round's)
      if constexpr (J == 0) {
        issue(std::integral_constant<int, NBUF - 1>{}, mc, mc.tile0 + (j + NBUF - 1 - start),
              rid_pend);
      } else {
        issue(std::integral_constant<int, (J + NBUF - 1) % NBUF>{}, ma,
              ma.tile0 + (j + NBUF - 1 - sa), rid_pend);
      }
      rid_pend = rid_of(ma, ma.tile0 + (j + NBUF - sa), slot_a);
      if constexpr (J == 0) {
        // (a round start can be an item's first tile)
        if (j == start) pv_step(JC, j & 1, std::true_type{});
        else if (j - start < ntl) pv_step(JC, j & 1, std::false_type{});
      } else {
        if (j - start < ntl) pv_step(JC, j & 1, std::false_type{});
      }
      // this wave's gathers of position j+2 have landed (NBUF = 4: those of
      // j+3 may be in flight)
      wait_vmcnt<(NBUF - 3) * G>();
      lds_barrier();  // B(j+1)
    };
    iter(std::integral_constant<int, 0>{}, r * NBUF);
    iter(std::integral_constant<int, 1>{}, r * NBUF + 1);
    iter(std::integral_constant<int, 2>{}, r * NBUF + 2);
    if constexpr (NBUF == 4) iter(std::integral_constant<int, 3>{}, r * NBUF + 3);
  }
  // no gather may still be writing this workgroup's LDS when it exits
  wait_vmcnt<0>();
}

// Merge split partials: M = max(z, m_s), L = e^(z-M) + sum e^(m_s-M) l_s,
// O = sum e^(m_s-M) O_s / L, then the output rope slice is rotated at -t.
// Thread = 8 consecutive columns of one head; 4 heads per workgroup.  With at
// most NSM splits (NSM > 0: the decode shapes) every load of a thread --
// sink, (m, l) pairs, partial outputs, RoPE factors -- is issued before any
// arithmetic, one memory round trip instead of a chain of them; NSM = 0
// loops over any number of splits.
template <int NSM>
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
  const u16* po = reinterpret_cast<const u16*>(ws + (size_t)((long)p.B * p.S) * nsplit * H * 2) +
                  (size_t)row * nsplit * H * dv;
  const bool tin = t >= 0 && t < p.n_pos;
  const bool rot = p.dv == p.D && p.rope_dim > 0 && tin;
  float zs = p.sink ? p.sink[h] * kLog2e : -INFINITY;
  float M = zs;
  bool nan = false;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L;
  // the output's rope pairs: RoPE factors at t (loaded with the rest)
  float2 r4[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2)
    r4[e >> 1] = (rot && c + e >= rbase) ? cs[t * half + ((c + e - rbase) >> 1)]
                                         : make_float2(1.f, 0.f);
  auto acc8 = [&](float f, const uint4 u) __attribute__((always_inline)) {
    o[0] += f * bf_lo(u.x); o[1] += f * bf_hi(u.x); o[2] += f * bf_lo(u.y); o[3] += f * bf_hi(u.y);
    o[4] += f * bf_lo(u.z); o[5] += f * bf_hi(u.z); o[6] += f * bf_lo(u.w); o[7] += f * bf_hi(u.w);
  };
  if constexpr (NSM > 0) {
    float2 msl[NSM];
    uint4 u[NSM];
#pragma unroll
    for (int s = 0; s < NSM; ++s) {
      if (s < nsplit) {
        msl[s] = *reinterpret_cast<const float2*>(ml + (s * H + h) * 2);
        u[s] = *reinterpret_cast<const uint4*>(po + ((size_t)s * H + h) * dv + c);
      }
    }
#pragma unroll
    for (int s = 0; s < NSM; ++s)
      if (s < nsplit) {
        if (msl[s].x != msl[s].x) nan = true;
        M = fmaxf(M, msl[s].x);
      }
    const float Mb = (M == -INFINITY) ? 0.f : M;
    L = p.sink ? exp2f(zs - Mb) : 0.f;
#pragma unroll
    for (int s = 0; s < NSM; ++s)
      if (s < nsplit) {
        const float f = exp2f(msl[s].x - Mb);
        L += f * msl[s].y;
        acc8(f, u[s]);
      }
  } else {
    for (int s = 0; s < nsplit; ++s) {
      const float ms = ml[(s * H + h) * 2];
      if (ms != ms) nan = true;
      M = fmaxf(M, ms);
    }
    const float Mb = (M == -INFINITY) ? 0.f : M;
    L = p.sink ? exp2f(zs - Mb) : 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float f = exp2f(ml[(s * H + h) * 2] - Mb);
      L += f * ml[(s * H + h) * 2 + 1];
      acc8(f, *reinterpret_cast<const uint4*>(po + ((size_t)s * H + h) * dv + c));
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] *= inv;
  if (rot) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      if (c + e >= rbase) {
        const float2 r = r4[e >> 1];
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
  return H % 64 == 0 && dv == 512 && rope_dim == 64 && (D == 512 || D == 576) && k <= kMaxK;
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

AttnPlan plan_attention(int B, int S, int H, int D, int dv, int rope_dim, int window,
                        int npool_max, bool bf16, long max_rows, int k) {
  AttnPlan pl{0, 1, 1 << 30, 0};
  if (!bf16 || !mfma_shape(H, D, dv, rope_dim, k)) return pl;
  // the gather addresses one sequence's rows with 32-bit buffer offsets
  if (max_rows * D * 2 >= 0x7ffffff0L) return pl;
  const long rows = (long)B * S;
  const int tiles = (window + kNK - 1) / kNK + (npool_max + kNK - 1) / kNK;
  // work items are counted in 32-bit arithmetic
  if ((rows + 7) / 8 * 8 * (H / 64) * (long)std::max(tiles, 1) >= 0x7fffffffL) return pl;
  pl.kernel = 1;
  const long wgs = rows * (H / 64);
  const int cus = device_cus();
  if (wgs < cus && tiles > 1) {
    int ns = (int)std::min<long>(tiles, (cus + wgs - 1) / wgs);
    const int tps = (tiles + ns - 1) / ns;
    ns = (tiles + tps - 1) / tps;
    if (ns > 1) {
      pl.nsplit = ns;
      pl.tiles_per_split = tps;
      // fp32 (max, sum) per head, then bf16 partial outputs
      pl.ws_bytes = (size_t)B * S * ns * H * (2 * sizeof(float) + dv * 2);
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
  a.nhg = p.H / 64;
  a.rows = (int)rows;
  a.n_items = (rows + 7) / 8 * 8 * a.nsplit * a.nhg;
  a.by_nhg = make_fastdiv((unsigned)a.nhg);
  a.by_nsplit = make_fastdiv((unsigned)a.nsplit);
  a.by_S = make_fastdiv((unsigned)p.S);
  a.by_m = make_fastdiv((unsigned)std::max(p.m, 1));
  // persistent: one workgroup per compute unit (the LDS use allows no more),
  // a multiple of 8 so that a workgroup's items keep one residue mod 8
  const long grid = (std::min<long>(device_cus(), a.n_items) + 7) / 8 * 8;
  if (p.D == 512 && split)
    hipLaunchKernelGGL((attn_mfma_kernel<512, 4, true>), dim3((unsigned)grid), dim3(512), 0, s, a);
  else if (p.D == 512)
    hipLaunchKernelGGL((attn_mfma_kernel<512, 4, false>), dim3((unsigned)grid), dim3(512), 0, s, a);
  else if (split)
    hipLaunchKernelGGL((attn_mfma_kernel<576, 3, true>), dim3((unsigned)grid), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<576, 3, false>), dim3((unsigned)grid), dim3(512), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !split) return err;
  const int per_wg = 256 / (p.dv / 8);
  const dim3 cgrid((unsigned)rows, (p.H + per_wg - 1) / per_wg);
  if (a.nsplit <= 8)
    hipLaunchKernelGGL((attn_combine_kernel<8>), cgrid, dim3(256), 0, s, p,
                       reinterpret_cast<const float*>(ws), a.nsplit);
  else
    hipLaunchKernelGGL((attn_combine_kernel<0>), cgrid, dim3(256), 0, s, p,
                       reinterpret_cast<const float*>(ws), a.nsplit);
  return hipGetLastError();
}

}  // namespace csa
