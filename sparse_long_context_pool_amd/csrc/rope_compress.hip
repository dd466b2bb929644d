// rope_compress.hip -- RoPE cos/sin table and the window compressor.
//
// Page "DeepSeek-V4", section "Hybrid attention (§2.3)": partial RoPE with
// interleaved pairs on the trailing qk_rope_head_dim channels; the CSA pool
// compresses K=V at rate m with overlapping windows, the HCA pool at rate m'
// with non-overlapping windows.  Section "Cache layers": the compressor keeps
// overlap state for CSA and runs a parallel compressor at index_head_dim for
// the indexer keys.
//
// The compressor is HBM-bound (it reads each token row of x and gate once and
// writes one row per m tokens).  A thread (or lane) owns 8 consecutive
// channels (one 16-byte bf16 load per row); the RoPE pair rotation is applied
// to the finished entry before the store.  By window shape:
//   m = 1, no gate: the entry is its token, rotated (a streaming copy);
//   windows of exactly 4 or 8 rows (CSA at m = 4 or 2 with overlap): one
//     thread per (entry, chunk), the window's rows loaded together, then
//     max, weights and weighted sum per channel;
//   other windows of up to 32 rows: one wave per entry, an online softmax
//     per channel over the rows;
//   longer windows (HCA, m' = 128): one workgroup per entry, its four waves
//     split the rows and merge their online-softmax states through LDS.
#include "csa_device.hpp"

namespace csa {
namespace {

// Frequency scaling of the table.  factor <= 1: plain RoPE, pair i turns at
// theta^(-2i/d).  factor > 1: YaRN (DeepseekV4Config: compress_rope_theta is
// used together with rope scaling for YaRN; the method's published
// "NTK-by-parts" rule): over the original context L pair i turns
// L f_i / (2 pi) times, which is r turns at the fractional pair index
// i(r) = d ln(L / (2 pi r)) / (2 ln theta); pairs up to low = floor(i(beta_fast))
// keep f_i, pairs from high = ceil(i(beta_slow)) run at f_i / factor, and the
// pairs between blend the two with a weight linear in i.  Only the angle
// changes: the table stays a pure rotation.
struct RopeScaling {
  double factor;               // <= 1: plain RoPE
  double orig_len, beta_fast, beta_slow;
};

__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ cs, int n_pos,
                                                         int rope_dim, double theta,
                                                         RopeScaling sc) {
  const int half = rope_dim / 2;
  const long n = (long)n_pos * half;
  const double d = (double)rope_dim;
  const bool yarn = sc.factor > 1.0;
  double low = 0.0, high = 1.0;
  if (yarn) {
    // (every thread forms the two ramp ends itself: fp64 logs, once)
    const double two_pi = 6.283185307179586;
    low = fmax(floor(d * log(sc.orig_len / (two_pi * sc.beta_fast)) / (2.0 * log(theta))), 0.0);
    high = fmin(ceil(d * log(sc.orig_len / (two_pi * sc.beta_slow)) / (2.0 * log(theta))),
                d - 1.0);
    if (high == low) high += 0.001;
  }
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n;
       e += (long)gridDim.x * blockDim.x) {
    const long p = e / half;
    const int i = (int)(e - p * half);
    double f = pow(theta, -2.0 * (double)i / d);
    if (yarn) {
      const double ramp = fmin(fmax(((double)i - low) / (high - low), 0.0), 1.0);
      f = (f / sc.factor) * ramp + f * (1.0 - ramp);
    }
    const double ang = (double)p * f;
    cs[e] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

constexpr int kCompressWaves = 4;
constexpr int kMaxChunksPerLane = 2;  // D <= 64 lanes * 2 chunks * 8 channels

template <bool BF16>
__global__ __launch_bounds__(256) void compress_kernel(
    const void* __restrict__ x, const void* __restrict__ gate,
    const float* __restrict__ slot_bias, void* __restrict__ pool, int S, int D, int m,
    int overlap, int rope_dim, const float2* __restrict__ cs, int pos0) {
  extern __shared__ float smem[];  // [waves][3][D]: running max, sum, weighted sum
  const int T = S / m;
  const int w = blockIdx.x;
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nchunk = D >> 3;

  const long first = (long)(w - overlap) * m;  // token held by slot 0
  const long j0 = first < 0 ? 0 : first;
  const long j1 = (long)(w + 1) * m;
  const long row0 = (long)b * S;

  float mx[kMaxChunksPerLane][8], sm[kMaxChunksPerLane][8], ac[kMaxChunksPerLane][8];
#pragma unroll
  for (int cc = 0; cc < kMaxChunksPerLane; ++cc)
#pragma unroll
    for (int v = 0; v < 8; ++v) { mx[cc][v] = -INFINITY; sm[cc][v] = 0.f; ac[cc][v] = 0.f; }

  for (long j = j0 + wave; j < j1; j += kCompressWaves) {
#pragma unroll
    for (int cc = 0; cc < kMaxChunksPerLane; ++cc) {
      const int ch = lane + 64 * cc;
      if (ch >= nchunk) break;
      float xv[8], a[8];
      load8<BF16>(x, (row0 + j) * D + ch * 8, xv);
      if (gate) {
        load8<BF16>(gate, (row0 + j) * D + ch * 8, a);
      } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) a[v] = 0.f;
      }
      if (slot_bias) {
        const float4* sb = reinterpret_cast<const float4*>(slot_bias + (j - first) * D + ch * 8);
        float4 s0 = sb[0], s1 = sb[1];
        a[0] += s0.x; a[1] += s0.y; a[2] += s0.z; a[3] += s0.w;
        a[4] += s1.x; a[5] += s1.y; a[6] += s1.z; a[7] += s1.w;
      }
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        // online softmax: keep (max, sum e^(a-max), sum e^(a-max) x)
        if (a[v] > mx[cc][v]) {
          const float r = __expf(mx[cc][v] - a[v]);
          sm[cc][v] = sm[cc][v] * r + 1.f;
          ac[cc][v] = ac[cc][v] * r + xv[v];
          mx[cc][v] = a[v];
        } else {
          const float e = __expf(a[v] - mx[cc][v]);
          sm[cc][v] += e;
          ac[cc][v] += e * xv[v];
        }
      }
    }
  }

  float* st = smem + wave * 3 * D;
#pragma unroll
  for (int cc = 0; cc < kMaxChunksPerLane; ++cc) {
    const int ch = lane + 64 * cc;
    if (ch >= nchunk) break;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      st[ch * 8 + v] = mx[cc][v];
      st[D + ch * 8 + v] = sm[cc][v];
      st[2 * D + ch * 8 + v] = ac[cc][v];
    }
  }
  __syncthreads();

  // merge the wave states; thread owns a channel pair (2p, 2p+1)
  const int rope_base = D - rope_dim;
  const long out_row = ((long)b * T + w) * D;
  for (int p = threadIdx.x; p < (D >> 1); p += blockDim.x) {
    float val[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = 2 * p + u;
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < kCompressWaves; ++q) M = fmaxf(M, smem[q * 3 * D + c]);
      float den = 0.f, num = 0.f;
#pragma unroll
      for (int q = 0; q < kCompressWaves; ++q) {
        const float mq = smem[q * 3 * D + c];
        if (mq == -INFINITY) continue;  // wave saw no row of this window
        const float f = __expf(mq - M);
        den += f * smem[q * 3 * D + D + c];
        num += f * smem[q * 3 * D + 2 * D + c];
      }
      val[u] = num / den;
    }
    if (2 * p >= rope_base) {
      const int i = (2 * p - rope_base) >> 1;
      const float2 r = cs[((long)pos0 + (long)w * m) * (rope_dim >> 1) + i];
      const float a0 = val[0], a1 = val[1];
      val[0] = a0 * r.x - a1 * r.y;
      val[1] = a0 * r.y + a1 * r.x;
    }
    store1<BF16>(pool, out_row + 2 * p, val[0]);
    store1<BF16>(pool, out_row + 2 * p + 1, val[1]);
  }
}

// Short windows (at most 32 rows): one wave per entry, 4 entries per
// workgroup; lane l owns channel chunks l and l + 64 and runs the per-channel
// online softmax over the whole window, so no merge is needed.
template <bool BF16>
__global__ __launch_bounds__(256) void compress_wave_kernel(
    const void* __restrict__ x, const void* __restrict__ gate,
    const float* __restrict__ slot_bias, void* __restrict__ pool, int B, int S, int D, int m,
    int overlap, int rope_dim, const float2* __restrict__ cs, int pos0) {
  const int T = S / m;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long e = (long)blockIdx.x * 4 + wave;   // entry over all sequences
  if (e >= (long)B * T) return;
  const int b = (int)(e / T), w = (int)(e - (long)b * T);
  const int nchunk = D >> 3;
  const long first = (long)(w - overlap) * m;  // token held by slot 0
  const long j0 = first < 0 ? 0 : first;
  const long j1 = (long)(w + 1) * m;
  const long row0 = (long)b * S;
  const int rope_base = D - rope_dim;
#pragma unroll
  for (int cc = 0; cc < kMaxChunksPerLane; ++cc) {
    const int ch = lane + 64 * cc;
    if (ch >= nchunk) break;
    float mx[8], sm[8], ac[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) { mx[v] = -INFINITY; sm[v] = 0.f; ac[v] = 0.f; }
    for (long j = j0; j < j1; ++j) {
      float xv[8], a[8];
      load8<BF16>(x, (row0 + j) * D + ch * 8, xv);
      if (gate) {
        load8<BF16>(gate, (row0 + j) * D + ch * 8, a);
      } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) a[v] = 0.f;
      }
      if (slot_bias) {
        const float4* sb = reinterpret_cast<const float4*>(slot_bias + (j - first) * D + ch * 8);
        float4 s0 = sb[0], s1 = sb[1];
        a[0] += s0.x; a[1] += s0.y; a[2] += s0.z; a[3] += s0.w;
        a[4] += s1.x; a[5] += s1.y; a[6] += s1.z; a[7] += s1.w;
      }
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        if (a[v] > mx[v]) {
          const float r = __expf(mx[v] - a[v]);
          sm[v] = sm[v] * r + 1.f;
          ac[v] = ac[v] * r + xv[v];
          mx[v] = a[v];
        } else {
          const float ev = __expf(a[v] - mx[v]);
          sm[v] += ev;
          ac[v] += ev * xv[v];
        }
      }
    }
    float val[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) val[v] = ac[v] / sm[v];
#pragma unroll
    for (int v = 0; v < 8; v += 2) {
      const int c = ch * 8 + v;
      if (c >= rope_base) {
        const float2 r = cs[((long)pos0 + (long)w * m) * (rope_dim >> 1) + ((c - rope_base) >> 1)];
        const float a0 = val[v], a1 = val[v + 1];
        val[v] = a0 * r.x - a1 * r.y;
        val[v + 1] = a0 * r.y + a1 * r.x;
      }
    }
    store8<BF16>(pool, ((long)b * T + w) * D + ch * 8, val);
  }
}

// Rotation of a channel slice [8ch, 8ch + 8) at position pos: the pairs at or
// above rope_base turn by the table's angle.
__device__ __forceinline__ void rope8(float v[8], int ch, int rope_base, int rope_dim,
                                      const float2* __restrict__ cs, long pos) {
  if (ch * 8 + 8 <= rope_base) return;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const int c = ch * 8 + e;
    if (c >= rope_base) {
      const float2 rr = cs[pos * (rope_dim >> 1) + ((c - rope_base) >> 1)];
      const float a0 = v[e], a1 = v[e + 1];
      v[e] = a0 * rr.x - a1 * rr.y;
      v[e + 1] = a0 * rr.y + a1 * rr.x;
    }
  }
}

// The same rotation in two halves: the factors of the slice's rope pairs
// first (so their loads can go out with the data's), then the rotation.
__device__ __forceinline__ void rope8_load(float2 rr[4], int ch, int rope_base, int rope_dim,
                                          const float2* __restrict__ cs, long pos) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = ch * 8 + 2 * e;
    rr[e] = c >= rope_base ? cs[pos * (rope_dim >> 1) + ((c - rope_base) >> 1)]
                           : make_float2(1.f, 0.f);
  }
}
__device__ __forceinline__ void rope8_apply(float v[8], const float2 rr[4], int ch,
                                            int rope_base) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (ch * 8 + 2 * e >= rope_base) {
      const float a0 = v[2 * e], a1 = v[2 * e + 1];
      v[2 * e] = a0 * rr[e].x - a1 * rr[e].y;
      v[2 * e + 1] = a0 * rr[e].y + a1 * rr[e].x;
    }
  }
}

// m = 1 without overlap, gate or slot bias: the window of an entry is its own
// token, whose softmax weight is exactly 1, so the entry is the token with
// its rope slice rotated at pos0 + w.  A streaming pass: thread i takes the
// 8-channel chunks i, i + n/4, i + 2n/4, i + 3n/4 of the n = rows x D/8
// chunks, their four loads in flight together (a wave still reads 1 KiB
// contiguous per load).
constexpr int kCopyUnroll = 4;
template <bool BF16>
__device__ __forceinline__ void rope_copy_body(
    const void* __restrict__ x, void* __restrict__ pool, long rows, int S, int D,
    int rope_dim, const float2* __restrict__ cs, int pos0, unsigned i0) {
  // (index arithmetic in 32 bits: the launcher keeps rows x D/8 < 2^31)
  const unsigned nchunk = (unsigned)D >> 3;
  const unsigned n = (unsigned)rows * nchunk;
  const unsigned q = (n + kCopyUnroll - 1) / kCopyUnroll;
  if (i0 >= q) return;
  const int rope_base = D - rope_dim;
  float v[kCopyUnroll][8];
  float2 rr[kCopyUnroll][4];
  bool rot[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const unsigned i = i0 + u * q;
    rot[u] = false;
    if (i < n) {
      load8<BF16>(x, (long)i * 8, v[u]);   // row r, chunk c: element 8 (r D/8 + c)
      const unsigned r = i / nchunk;
      const int ch = (int)(i - r * nchunk);
      rot[u] = ch * 8 + 8 > rope_base;
      if (rot[u])
        rope8_load(rr[u], ch, rope_base, rope_dim, cs, (long)pos0 + (long)(r % (unsigned)S));
    }
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const unsigned i = i0 + u * q;
    if (i < n) {
      if (rot[u]) rope8_apply(v[u], rr[u], (int)((i0 + u * q) % nchunk), rope_base);
      store8<BF16>(pool, (long)i * 8, v[u]);
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void rope_copy_kernel(
    const void* __restrict__ x, void* __restrict__ pool, long rows, int S, int D,
    int rope_dim, const float2* __restrict__ cs, int pos0) {
  rope_copy_body<BF16>(x, pool, rows, S, D, rope_dim, cs, pos0,
                       blockIdx.x * blockDim.x + threadIdx.x);
}

// Windows of exactly NR = m (1 + overlap) rows (the token-window sizes in
// use): one thread per (entry, 8-channel chunk), so small widths (an index key
// of 128 channels is 16 chunks) still fill whole waves.  The window's rows are
// loaded together (all loads in flight at once), then per channel the max of
// the gate logits, the softmax weights and the weighted sum.  Rows before
// token 0 (the first entry's overlap half) take no part.
template <bool BF16, int NR>
__device__ __forceinline__ void compress_rows_body(
    const void* __restrict__ x, const void* __restrict__ gate,
    const float* __restrict__ slot_bias, void* __restrict__ pool, int B, int S, int D, int m,
    int overlap, int rope_dim, const float2* __restrict__ cs, int pos0, unsigned i) {
  // (index arithmetic in 32 bits: the launcher keeps B x T x D/8 < 2^31)
  const unsigned nchunk = (unsigned)D >> 3;
  const unsigned T = (unsigned)(S / m);
  if (i >= (unsigned)B * T * nchunk) return;
  const unsigned e = i / nchunk;
  const int ch = (int)(i - e * nchunk);
  const int b = (int)(e / T);
  const long w = (long)(e - (unsigned)b * T);
  const long first = (w - overlap) * m;            // token held by slot 0
  const long row0 = (long)b * S;
  const int rope_base = D - rope_dim;
  const bool rot = ch * 8 + 8 > rope_base;
  float2 rr[4];
  if (rot) rope8_load(rr, ch, rope_base, rope_dim, cs, (long)pos0 + w * m);
  float xv[NR][8], a[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const long j = first + r;
    if (j >= 0) {
      load8<BF16>(x, (row0 + j) * D + ch * 8, xv[r]);
      if (gate) {
        load8<BF16>(gate, (row0 + j) * D + ch * 8, a[r]);
      } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) a[r][v] = 0.f;
      }
      if (slot_bias) {
        const float4* sb = reinterpret_cast<const float4*>(slot_bias + r * D + ch * 8);
        const float4 s0 = sb[0], s1 = sb[1];
        a[r][0] += s0.x; a[r][1] += s0.y; a[r][2] += s0.z; a[r][3] += s0.w;
        a[r][4] += s1.x; a[r][5] += s1.y; a[r][6] += s1.z; a[r][7] += s1.w;
      }
    }
  }
  float val[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (first + r >= 0) mx = fmaxf(mx, a[r][v]);
    float sm = 0.f, ac = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (first + r >= 0) {
        const float ev = __expf(a[r][v] - mx);
        sm += ev;
        ac += ev * xv[r][v];
      }
    val[v] = ac / sm;
  }
  if (rot) rope8_apply(val, rr, ch, rope_base);
  store8<BF16>(pool, ((long)b * T + w) * D + ch * 8, val);
}

template <bool BF16, int NR>
__global__ __launch_bounds__(256) void compress_rows_kernel(
    const void* __restrict__ x, const void* __restrict__ gate,
    const float* __restrict__ slot_bias, void* __restrict__ pool, int B, int S, int D, int m,
    int overlap, int rope_dim, const float2* __restrict__ cs, int pos0) {
  compress_rows_body<BF16, NR>(x, gate, slot_bias, pool, B, S, D, m, overlap, rope_dim, cs, pos0,
                               blockIdx.x * blockDim.x + threadIdx.x);
}

// Several compressor passes in one launch (a prefill step's window rows, K=V
// pool and index keys): each pass takes a contiguous range of the grid's
// workgroups and runs the per-thread body of its single-pass kernel (the
// streaming copy, or the 8- or 4-row window), so the passes share one launch
// and fill the chip together instead of one after another.
constexpr int kMaxJobs = 4;
struct CompressJob {
  const void* x;
  const void* gate;
  const float* slot_bias;
  void* pool;
  const float2* cs;
  int B, S, D, m, overlap, rope_dim, pos0;
  int kind;        // 0: streaming copy (m = 1), 1: 8-row windows, 2: 4-row windows
  int block0;      // first workgroup of the pass
};
struct CompressBatch {
  CompressJob job[kMaxJobs];
  int n;
};

template <bool BF16>
__global__ __launch_bounds__(256) void compress_batch_kernel(CompressBatch bt) {
  int j = 0;
#pragma unroll
  for (int q = 1; q < kMaxJobs; ++q)
    if (q < bt.n && (int)blockIdx.x >= bt.job[q].block0) j = q;
  const CompressJob& jb = bt.job[j];
  const unsigned i = ((unsigned)blockIdx.x - (unsigned)jb.block0) * blockDim.x + threadIdx.x;
  if (jb.kind == 0)
    rope_copy_body<BF16>(jb.x, jb.pool, (long)jb.B * jb.S, jb.S, jb.D, jb.rope_dim, jb.cs,
                         jb.pos0, i);
  else if (jb.kind == 1)
    compress_rows_body<BF16, 8>(jb.x, jb.gate, jb.slot_bias, jb.pool, jb.B, jb.S, jb.D, jb.m,
                                jb.overlap, jb.rope_dim, jb.cs, jb.pos0, i);
  else
    compress_rows_body<BF16, 4>(jb.x, jb.gate, jb.slot_bias, jb.pool, jb.B, jb.S, jb.D, jb.m,
                                jb.overlap, jb.rope_dim, jb.cs, jb.pos0, i);
}

// Cache update (page "DeepSeek-V4", section "Cache layers": the compressor's
// buffer / pool / count with the CSA overlap state, and the sliding window of
// K=V rows).  Per sequence b: ring_x / ring_g hold the raw rows of the last
// L = (1+overlap) m tokens at row p mod L (the compressor's buffer and overlap
// state), win the last W rotated rows at row p mod W, pool the entries; count[b]
// tokens came before this call, which appends tokens count[b] .. count[b]+n-1
// (x and gate [B][n][D]).  Positions past the RoPE table give NaN rows.
//
// Pass 1: the entries whose window closes within the call, w from
// count/m to (count+n)/m - 1; window row j comes from x when the call brings
// it (j >= count), else from the ring.  Pooled as the compressor pools them:
// per channel the max of the logits, the weights, the weighted sum.
// entry w of sequence b, channels [8ch, 8ch + 8)
constexpr int kEntryRows = 8;
template <bool BF16>
__device__ __forceinline__ void cache_entry(
    const void* __restrict__ x, const void* __restrict__ gate,
    const float* __restrict__ slot_bias, const void* __restrict__ ring_x,
    const void* __restrict__ ring_g, void* __restrict__ pool, int b, long c0, long w, int ch,
    int n, int D, int m, int overlap, int T_cap, int rope_dim, const float2* __restrict__ cs,
    int n_pos) {
  const int L = (1 + overlap) * m;
  const long first = (w - overlap) * m;             // token held by slot 0
  const long j0 = first < 0 ? 0 : first, j1 = (w + 1) * m;
  // (j >= 0 and counts below 2^31: the ring slot is a 32-bit remainder)
  auto row_x = [&](long j, float v[8]) {
    if (j >= c0) load8<BF16>(x, ((long)b * n + (j - c0)) * D + ch * 8, v);
    else load8<BF16>(ring_x, ((long)b * L + (unsigned)j % (unsigned)L) * D + ch * 8, v);
  };
  auto row_a = [&](long j, float a[8]) {
    if (gate) {
      if (j >= c0) load8<BF16>(gate, ((long)b * n + (j - c0)) * D + ch * 8, a);
      else load8<BF16>(ring_g, ((long)b * L + (unsigned)j % (unsigned)L) * D + ch * 8, a);
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v) a[v] = 0.f;
    }
    if (slot_bias) {
      const float4* sb = reinterpret_cast<const float4*>(slot_bias + (j - first) * D + ch * 8);
      const float4 s0 = sb[0], s1 = sb[1];
      a[0] += s0.x; a[1] += s0.y; a[2] += s0.z; a[3] += s0.w;
      a[4] += s1.x; a[5] += s1.y; a[6] += s1.z; a[7] += s1.w;
    }
  };
  float val[8];
  if (L <= kEntryRows) {
    // windows of up to 8 rows: every row's loads in flight together, then the
    // max, the weights and the weighted sum in row order (the compressor
    // kernels' arithmetic, so an entry pooled here equals theirs bit for bit)
    float xv[kEntryRows][8], a[kEntryRows][8];
#pragma unroll
    for (int r = 0; r < kEntryRows; ++r) {
      const long j = first + r;
      if (r < L && j >= 0) {
        row_a(j, a[r]);
        row_x(j, xv[r]);
      }
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < kEntryRows; ++r)
        if (r < L && first + r >= 0) mx = fmaxf(mx, a[r][v]);
      float sm = 0.f, ac = 0.f;
#pragma unroll
      for (int r = 0; r < kEntryRows; ++r)
        if (r < L && first + r >= 0) {
          const float ev = __expf(a[r][v] - mx);
          sm += ev;
          ac += ev * xv[r][v];
        }
      val[v] = ac / sm;
    }
  } else {
    float mx[8], sm[8], ac[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) { mx[v] = -INFINITY; sm[v] = 0.f; ac[v] = 0.f; }
    for (long j = j0; j < j1; ++j) {
      float a[8];
      row_a(j, a);
#pragma unroll
      for (int v = 0; v < 8; ++v) mx[v] = fmaxf(mx[v], a[v]);
    }
    for (long j = j0; j < j1; ++j) {
      float a[8], xv[8];
      row_a(j, a);
      row_x(j, xv);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float ev = __expf(a[v] - mx[v]);
        sm[v] += ev;
        ac[v] += ev * xv[v];
      }
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) val[v] = ac[v] / sm[v];
  }
  const long pos = w * m;
  if (rope_dim > 0) {
    if (pos < n_pos) {
      rope8(val, ch, D - rope_dim, rope_dim, cs, pos);
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v) val[v] = __int_as_float(0x7fc00000);
    }
  }
  store8<BF16>(pool, ((long)b * T_cap + w) * D + ch * 8, val);
}

// token k of this call (position p) of sequence b into the ring (if it is
// among the call's last L) and the window (if among the last W)
template <bool BF16>
__device__ __forceinline__ void cache_token(
    const void* __restrict__ x, const void* __restrict__ gate, void* __restrict__ ring_x,
    void* __restrict__ ring_g, void* __restrict__ win, int b, long p, int k, int ch, int n,
    int D, int L, int W, int rope_dim, const float2* __restrict__ cs, int n_pos) {
  const long src = ((long)b * n + k) * D + ch * 8;
  float v[8];
  load8<BF16>(x, src, v);
  if (k >= n - L) {
    // (bf16 -> fp32 -> bf16 is exact: the ring keeps the rows bit for bit)
    store8<BF16>(ring_x, ((long)b * L + p % L) * D + ch * 8, v);
    if (gate) {
      float g[8];
      load8<BF16>(gate, src, g);
      store8<BF16>(ring_g, ((long)b * L + p % L) * D + ch * 8, g);
    }
  }
  if (win != nullptr && k >= n - W) {
    if (rope_dim > 0) {
      if (p < n_pos) {
        rope8(v, ch, D - rope_dim, rope_dim, cs, p);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __int_as_float(0x7fc00000);
      }
    }
    store8<BF16>(win, ((long)b * W + p % W) * D + ch * 8, v);
  }
}

// Pass 1: the entries whose window closes within the call, w from count/m
// to (count+n)/m - 1; window row j comes from x when the call brings it
// (j >= count), else from the ring.  Pooled as the compressor pools them: per
// channel the max of the logits, the weights, the weighted sum.
template <bool BF16>
__global__ __launch_bounds__(256) void cache_entries_kernel(
    const void* __restrict__ x, const void* __restrict__ gate,
    const float* __restrict__ slot_bias, const void* __restrict__ ring_x,
    const void* __restrict__ ring_g, void* __restrict__ pool, const int* __restrict__ count,
    int n, int D, int m, int overlap, int T_cap, int E, int rope_dim,
    const float2* __restrict__ cs, int n_pos) {
  const int nchunk = D >> 3;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  if (i >= E * nchunk) return;
  const int e = i / nchunk, ch = i - e * nchunk;
  const long c0 = count[b];
  const long w = c0 / m + e;
  if (c0 < 0 || w >= (c0 + n) / m || w >= T_cap) return;
  cache_entry<BF16>(x, gate, slot_bias, ring_x, ring_g, pool, b, c0, w, ch, n, D, m, overlap,
                    T_cap, rope_dim, cs, n_pos);
}

// Pass 2 (after pass 1, which reads the ring): the call's last L tokens into
// the ring, its last W tokens, rotated at their positions, into the window.
template <bool BF16>
__global__ __launch_bounds__(256) void cache_tokens_kernel(
    const void* __restrict__ x, const void* __restrict__ gate, void* __restrict__ ring_x,
    void* __restrict__ ring_g, void* __restrict__ win, const int* __restrict__ count, int n,
    int D, int L, int W, int rope_dim, const float2* __restrict__ cs, int n_pos) {
  const int nchunk = D >> 3;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  if (i >= n * nchunk) return;
  const int k = i / nchunk, ch = i - k * nchunk;
  const long c0 = count[b];
  if (c0 < 0) return;
  cache_token<BF16>(x, gate, ring_x, ring_g, win, b, c0 + k, k, ch, n, D, L, W, rope_dim, cs,
                    n_pos);
}

// One token per sequence (decode): both passes in one kernel.  The thread of
// a chunk pools its entry (if the token closes one) before it overwrites the
// ring row of the token L positions back, which that entry does not read.
template <bool BF16>
__device__ __forceinline__ void cache_one_body(
    const void* __restrict__ x, const void* __restrict__ gate,
    const float* __restrict__ slot_bias, void* __restrict__ ring_x, void* __restrict__ ring_g,
    void* __restrict__ pool, void* __restrict__ win, const int* __restrict__ count, int D,
    int m, int overlap, int T_cap, int W, int rope_dim, const float2* __restrict__ cs,
    int n_pos, int b, int ch) {
  if (ch >= (D >> 3)) return;
  const long c0 = count[b];
  if (c0 < 0) return;
  if ((c0 + 1) % m == 0 && (c0 + 1) / m - 1 < T_cap)
    cache_entry<BF16>(x, gate, slot_bias, ring_x, ring_g, pool, b, c0, (c0 + 1) / m - 1, ch, 1,
                      D, m, overlap, T_cap, rope_dim, cs, n_pos);
  cache_token<BF16>(x, gate, ring_x, ring_g, win, b, c0, 0, ch, 1, D, (1 + overlap) * m, W,
                    rope_dim, cs, n_pos);
}

template <bool BF16>
__global__ __launch_bounds__(256) void cache_one_kernel(
    const void* __restrict__ x, const void* __restrict__ gate,
    const float* __restrict__ slot_bias, void* __restrict__ ring_x, void* __restrict__ ring_g,
    void* __restrict__ pool, void* __restrict__ win, const int* __restrict__ count, int D,
    int m, int overlap, int T_cap, int W, int rope_dim, const float2* __restrict__ cs,
    int n_pos) {
  cache_one_body<BF16>(x, gate, slot_bias, ring_x, ring_g, pool, win, count, D, m, overlap,
                       T_cap, W, rope_dim, cs, n_pos, blockIdx.y,
                       blockIdx.x * blockDim.x + threadIdx.x);
}

// One token per sequence for several caches in one launch (a decode step's
// K=V cache and index-key cache): each cache owns a contiguous range of the
// grid's workgroups, one workgroup of 128 threads per sequence (a thread per
// 8-channel chunk, D <= 1024), and runs the single-cache kernel's body, so the
// caches come out exactly as separate updates leave them.
constexpr int kMaxCacheJobs = 4;
struct CacheJob {
  const void* x;
  const void* gate;
  const float* slot_bias;
  void* ring_x;
  void* ring_g;
  void* pool;
  void* win;
  const int* count;
  const float2* cs;
  int D, m, overlap, T_cap, W, rope_dim, n_pos;
  int block0;  // first workgroup of the cache
};
struct CacheBatch {
  CacheJob job[kMaxCacheJobs];
  int n;
};

template <bool BF16>
__global__ __launch_bounds__(128) void cache_one_batch_kernel(CacheBatch bt) {
  int j = 0;
#pragma unroll
  for (int q = 1; q < kMaxCacheJobs; ++q)
    if (q < bt.n && (int)blockIdx.x >= bt.job[q].block0) j = q;
  const CacheJob& c = bt.job[j];
  cache_one_body<BF16>(c.x, c.gate, c.slot_bias, c.ring_x, c.ring_g, c.pool, c.win, c.count,
                       c.D, c.m, c.overlap, c.T_cap, c.W, c.rope_dim, c.cs, c.n_pos,
                       (int)blockIdx.x - c.block0, threadIdx.x);
}

}  // namespace

hipError_t launch_rope_table(float* cs, int n_pos, int rope_dim, double theta, double factor,
                             int orig_len, double beta_fast, double beta_slow, hipStream_t s) {
  const long n = (long)n_pos * (rope_dim / 2);
  long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  RopeScaling sc{factor, (double)orig_len, beta_fast, beta_slow};
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<float2*>(cs), n_pos, rope_dim, theta, sc);
  return hipGetLastError();
}

namespace {
// The batched kernel's kind for a pass (-1: it needs its own kernel), and its
// workgroup count.
int batch_kind(const void* gate, const float* slot_bias, int B, int S, int D, int m,
               int overlap, long* blocks) {
  const int T = S / m;
  if (m == 1 && overlap == 0 && gate == nullptr && slot_bias == nullptr && D % 8 == 0 &&
      (long)B * S * (D / 8) < (1L << 31)) {
    *blocks = (((long)B * S * (D / 8) + kCopyUnroll - 1) / kCopyUnroll + 255) / 256;
    return 0;
  }
  if ((m * (1 + overlap) == 8 || m * (1 + overlap) == 4) && D % 8 == 0 &&
      (long)B * T * (D / 8) < (1L << 31)) {
    *blocks = ((long)B * T * (D / 8) + 255) / 256;
    return m * (1 + overlap) == 8 ? 1 : 2;
  }
  return -1;
}
}  // namespace

hipError_t launch_compress_many(const CompressPass* p, int n, bool bf16, hipStream_t s) {
  // passes the batched kernel takes go into launches of up to kMaxJobs passes;
  // the others run on their own
  CompressBatch bt;
  bt.n = 0;
  long blocks = 0;
  int lone = 0;      // the pass of bt.job[0]
  auto flush = [&]() -> hipError_t {
    if (bt.n == 0) return hipSuccess;
    if (bt.n == 1) {
      // a lone pass runs on its own kernel, whose occupancy is set by its body
      // alone (the batched kernel's register count is that of its largest body)
      const CompressPass& c = p[lone];
      bt.n = 0;
      blocks = 0;
      return launch_compress(c.x, c.gate, c.slot_bias, c.pool, c.B, c.S, c.D, c.m, c.overlap,
                             c.rope_dim, c.cs, c.pos0, bf16, s);
    }
    if (bf16)
      hipLaunchKernelGGL(compress_batch_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, bt);
    else
      hipLaunchKernelGGL(compress_batch_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, bt);
    bt.n = 0;
    blocks = 0;
    return hipGetLastError();
  };
  for (int q = 0; q < n; ++q) {
    const CompressPass& c = p[q];
    if (c.S / c.m == 0 || c.B == 0) continue;
    long nb = 0;
    const int kind = batch_kind(c.gate, c.slot_bias, c.B, c.S, c.D, c.m, c.overlap, &nb);
    if (kind < 0) {
      hipError_t e = launch_compress(c.x, c.gate, c.slot_bias, c.pool, c.B, c.S, c.D, c.m,
                                     c.overlap, c.rope_dim, c.cs, c.pos0, bf16, s);
      if (e != hipSuccess) return e;
      continue;
    }
    // one pass takes at most 2^23 workgroups; a launch keeps its grid under
    // 2^31 work-items (the 32-bit thread index of the bodies)
    if (blocks + nb > (1L << 23)) {
      hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
    if (bt.n == 0) lone = q;
    CompressJob& jb = bt.job[bt.n++];
    jb.x = c.x; jb.gate = c.gate; jb.slot_bias = c.slot_bias; jb.pool = c.pool;
    jb.cs = reinterpret_cast<const float2*>(c.cs);
    jb.B = c.B; jb.S = c.S; jb.D = c.D; jb.m = c.m; jb.overlap = c.overlap;
    jb.rope_dim = c.rope_dim; jb.pos0 = c.pos0; jb.kind = kind; jb.block0 = (int)blocks;
    blocks += nb;
    if (bt.n == kMaxJobs) {
      hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
  }
  return flush();
}

hipError_t launch_compress(const void* x, const void* gate, const float* slot_bias,
                           void* pool, int B, int S, int D, int m, int overlap,
                           int rope_dim, const float* cs, int pos0, bool bf16,
                           hipStream_t s) {
  const int T = S / m;
  if (T == 0 || B == 0) return hipSuccess;
  if (m == 1 && overlap == 0 && gate == nullptr && slot_bias == nullptr && D % 8 == 0 &&
      (long)B * S * (D / 8) < (1L << 31)) {
    const long rows = (long)B * S;
    const long blocks = ((rows * (D / 8) + kCopyUnroll - 1) / kCopyUnroll + 255) / 256;
    if (bf16)
      hipLaunchKernelGGL(rope_copy_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, x,
                         pool, rows, S, D, rope_dim, reinterpret_cast<const float2*>(cs), pos0);
    else
      hipLaunchKernelGGL(rope_copy_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, x,
                         pool, rows, S, D, rope_dim, reinterpret_cast<const float2*>(cs), pos0);
    return hipGetLastError();
  }
  if ((m * (1 + overlap) == 8 || m * (1 + overlap) == 4) && D % 8 == 0 &&
      (long)B * T * (D / 8) < (1L << 31)) {
    const long blocks = ((long)B * T * (D / 8) + 255) / 256;
#define CSA_ROWS(NR)                                                                         \
  if (bf16)                                                                                  \
    hipLaunchKernelGGL((compress_rows_kernel<true, NR>), dim3((unsigned)blocks), dim3(256), 0, \
                       s, x, gate, slot_bias, pool, B, S, D, m, overlap, rope_dim,            \
                       reinterpret_cast<const float2*>(cs), pos0);                           \
  else                                                                                       \
    hipLaunchKernelGGL((compress_rows_kernel<false, NR>), dim3((unsigned)blocks), dim3(256), 0, \
                       s, x, gate, slot_bias, pool, B, S, D, m, overlap, rope_dim,            \
                       reinterpret_cast<const float2*>(cs), pos0);
    if (m * (1 + overlap) == 8) { CSA_ROWS(8) } else { CSA_ROWS(4) }
#undef CSA_ROWS
    return hipGetLastError();
  }
  if (m * (1 + overlap) <= 32 && D % 8 == 0) {
    const long blocks = ((long)B * T + 3) / 4;
    if (bf16)
      hipLaunchKernelGGL(compress_wave_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, x,
                         gate, slot_bias, pool, B, S, D, m, overlap, rope_dim,
                         reinterpret_cast<const float2*>(cs), pos0);
    else
      hipLaunchKernelGGL(compress_wave_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, x,
                         gate, slot_bias, pool, B, S, D, m, overlap, rope_dim,
                         reinterpret_cast<const float2*>(cs), pos0);
    return hipGetLastError();
  }
  const size_t lds = (size_t)kCompressWaves * 3 * D * sizeof(float);
  dim3 grid(T, B);
  if (bf16)
    hipLaunchKernelGGL(compress_kernel<true>, grid, dim3(256), lds, s, x, gate, slot_bias,
                       pool, S, D, m, overlap, rope_dim,
                       reinterpret_cast<const float2*>(cs), pos0);
  else
    hipLaunchKernelGGL(compress_kernel<false>, grid, dim3(256), lds, s, x, gate, slot_bias,
                       pool, S, D, m, overlap, rope_dim,
                       reinterpret_cast<const float2*>(cs), pos0);
  return hipGetLastError();
}

hipError_t launch_cache_append(const void* x, const void* gate, const float* slot_bias,
                               void* ring_x, void* ring_g, void* pool, void* win,
                               const int* count, int B, int n, int D, int m, int overlap,
                               int T_cap, int W, int rope_dim, const float* cs, int n_pos,
                               bool bf16, hipStream_t s) {
  if (B == 0 || n == 0) return hipSuccess;
  const int nchunk = D / 8;
  if (n == 1) {
    const dim3 g((unsigned)((nchunk + 255) / 256), (unsigned)B);
    if (bf16)
      hipLaunchKernelGGL(cache_one_kernel<true>, g, dim3(256), 0, s, x, gate, slot_bias, ring_x,
                         ring_g, pool, win, count, D, m, overlap, T_cap, W, rope_dim,
                         reinterpret_cast<const float2*>(cs), n_pos);
    else
      hipLaunchKernelGGL(cache_one_kernel<false>, g, dim3(256), 0, s, x, gate, slot_bias,
                         ring_x, ring_g, pool, win, count, D, m, overlap, T_cap, W, rope_dim,
                         reinterpret_cast<const float2*>(cs), n_pos);
    return hipGetLastError();
  }
  const int E = n / m + 2;  // entries that can close within n tokens, and spare
  const float2* cs2 = reinterpret_cast<const float2*>(cs);
  const dim3 g1((unsigned)((E * nchunk + 255) / 256), (unsigned)B);
  if (bf16)
    hipLaunchKernelGGL(cache_entries_kernel<true>, g1, dim3(256), 0, s, x, gate, slot_bias,
                       ring_x, ring_g, pool, count, n, D, m, overlap, T_cap, E, rope_dim, cs2,
                       n_pos);
  else
    hipLaunchKernelGGL(cache_entries_kernel<false>, g1, dim3(256), 0, s, x, gate, slot_bias,
                       ring_x, ring_g, pool, count, n, D, m, overlap, T_cap, E, rope_dim, cs2,
                       n_pos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int L = (1 + overlap) * m;
  const dim3 g2((unsigned)((n * nchunk + 255) / 256), (unsigned)B);
  if (bf16)
    hipLaunchKernelGGL(cache_tokens_kernel<true>, g2, dim3(256), 0, s, x, gate, ring_x, ring_g,
                       win, count, n, D, L, W, rope_dim, cs2, n_pos);
  else
    hipLaunchKernelGGL(cache_tokens_kernel<false>, g2, dim3(256), 0, s, x, gate, ring_x, ring_g,
                       win, count, n, D, L, W, rope_dim, cs2, n_pos);
  return hipGetLastError();
}

hipError_t launch_cache_append_many(const CachePass* p, int n, bool bf16, hipStream_t s) {
  // single-token updates share launches of up to kMaxCacheJobs caches; the
  // others run as launch_cache_append runs them
  CacheBatch bt;
  bt.n = 0;
  long blocks = 0;
  auto flush = [&]() -> hipError_t {
    if (bt.n == 0) return hipSuccess;
    if (bf16)
      hipLaunchKernelGGL(cache_one_batch_kernel<true>, dim3((unsigned)blocks), dim3(128), 0, s,
                         bt);
    else
      hipLaunchKernelGGL(cache_one_batch_kernel<false>, dim3((unsigned)blocks), dim3(128), 0, s,
                         bt);
    bt.n = 0;
    blocks = 0;
    return hipGetLastError();
  };
  for (int q = 0; q < n; ++q) {
    const CachePass& c = p[q];
    if (c.B == 0 || c.n == 0) continue;
    if (c.n != 1 || c.D > 1024) {
      hipError_t e = launch_cache_append(c.x, c.gate, c.slot_bias, c.ring_x, c.ring_g, c.pool,
                                         c.win, c.count, c.B, c.n, c.D, c.m, c.overlap, c.T_cap,
                                         c.W, c.rope_dim, c.cs, c.n_pos, bf16, s);
      if (e != hipSuccess) return e;
      continue;
    }
    if (blocks + c.B >= (1L << 31)) {
      hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
    CacheJob& jb = bt.job[bt.n++];
    jb.x = c.x; jb.gate = c.gate; jb.slot_bias = c.slot_bias; jb.ring_x = c.ring_x;
    jb.ring_g = c.ring_g; jb.pool = c.pool; jb.win = c.win; jb.count = c.count;
    jb.cs = reinterpret_cast<const float2*>(c.cs);
    jb.D = c.D; jb.m = c.m; jb.overlap = c.overlap; jb.T_cap = c.T_cap; jb.W = c.W;
    jb.rope_dim = c.rope_dim; jb.n_pos = c.n_pos; jb.block0 = (int)blocks;
    blocks += c.B;
    if (bt.n == kMaxCacheJobs) {
      hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
  }
  return flush();
}

}  // namespace csa
