// peaks.hip -- achievable-peak probes (libcsa_probe.so, include/csa_probe.h).
//
// The published MI355X peaks (2.5 PFLOP/s dense bf16, 8 TB/s HBM3E) assume the
// 2.4 GHz peak engine clock and every HBM channel busy; a kernel on a real box
// runs at the clock the power limit allows under its load.  These two kernels
// measure what the device sustains for the two resources the hot path is
// bound by, so that each kernel's fraction can be read against both.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// a value in (-1, 1) from a 32-bit integer (one round of a multiplicative hash)
__device__ __forceinline__ float hash_unit(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (float)(int32_t)x * (1.0f / 2147483648.0f);
}

// Eight independent chains per wave keep the matrix pipe fed without any
// dependence on instruction latency; the operands never change, so the loop
// has no memory traffic at all.
__global__ __launch_bounds__(256, 2) void mfma_loop(float* __restrict__ sink, int iters) {
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[u][e] = (__bf16)hash_unit(gid * 64u + 8u * u + e);
      b[u][e] = (__bf16)hash_unit(0x9e3779b9u + gid * 64u + 8u * u + e);
    }
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c & 3], b[c >> 1], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  sink[gid] = s;
}

// Grid-stride 16-byte loads, eight in flight per thread per iteration, marked
// non-temporal (streamed once).  Swept on one box (4 GiB, best of five): plain
// loads 5.4-6.0 TB/s over 4-64 workgroups per compute unit and 4-16 loads in
// flight; non-temporal loads 5.7-6.5 TB/s, the most with 8 in flight and 32
// workgroups per compute unit -- the shape the bench runs.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_loop(const uint4* __restrict__ buf, size_t n16,
                                                 uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const size_t stride = (size_t)gridDim.x * 256u;
  size_t i = (size_t)blockIdx.x * 256u + threadIdx.x;
  const u32x4* b = reinterpret_cast<const u32x4*>(buf);
  uint32_t x = 0u;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(b + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(b + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * 256u + threadIdx.x] = x;
}

// LDS reads, 512 threads per workgroup over a 64 KiB array: every wave issues
// 8 independent reads per round, each to a 1 KiB row picked by (round, read,
// wave) so that no two rounds read the same rows in the same order.  Mode 0:
// 16-byte reads (ds_read_b128), lane l at +16 l of the row.  Mode 1: the
// transposing 8-byte reads (ds_read_b64_tr_b16) of the matrix-core operand
// path, lane l at +8 l of the row's first 512 bytes.  Thread i adds up what it
// read (sink[2 i]) and wave 0 of each workgroup writes the shader-clock cycles
// of its loop (sink[2 i + 1] of thread 0).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int MODE>
__global__ __launch_bounds__(512) void lds_loop(uint32_t* __restrict__ sink, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char buf[65536];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 65536 / 16; i += 512)
    reinterpret_cast<uint4*>(buf)[i] = make_uint4(i, 3 * i + 1, 5 * i + 2, 7 * i + 3);
  __syncthreads();
  const long long t0 = clock64();
  uint32_t acc = 0u;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = (it * 9 + u * 8 + wave) & 63;  // < 64 rows of 1 KiB
      if (MODE == 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(buf + row * 1024 + 16 * lane);
        acc += v.x + v.y + v.z + v.w;
      } else {
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(buf + row * 1024 + 8 * lane));
        acc += (uint32_t)(v[0] + v[1] + v[2] + v[3]);
      }
    }
  }
  const long long t1 = clock64();
  const size_t g = (size_t)blockIdx.x * 512u + tid;
  sink[2 * g] = acc;
  sink[2 * g + 1] = tid == 0 ? (uint32_t)(t1 - t0) : 0u;
}

}  // namespace

extern "C" int csa_probe_lds(uint32_t* sink, int32_t n_wg, int32_t iters, int32_t mode,
                             hipStream_t stream) {
  if (sink == nullptr || n_wg < 1 || iters < 1 || (mode != 0 && mode != 1))
    return (int)hipErrorInvalidValue;
  if (mode == 0)
    hipLaunchKernelGGL(lds_loop<0>, dim3((unsigned)n_wg), dim3(512), 0, stream, sink, iters);
  else
    hipLaunchKernelGGL(lds_loop<1>, dim3((unsigned)n_wg), dim3(512), 0, stream, sink, iters);
  return (int)hipGetLastError();
}

extern "C" double csa_probe_lds_bytes(int32_t n_wg, int32_t iters, int32_t mode) {
  // 8 waves x 8 reads per round, 1 KiB (mode 0) or 512 bytes (mode 1) each
  return (double)n_wg * 8.0 * 8.0 * (mode == 0 ? 1024.0 : 512.0) * (double)iters;
}

extern "C" int csa_probe_mfma_bf16(float* sink, int32_t n_wg, int32_t iters, hipStream_t stream) {
  if (sink == nullptr || n_wg < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop, dim3((unsigned)n_wg), dim3(256), 0, stream, sink, iters);
  return (int)hipGetLastError();
}

extern "C" double csa_probe_mfma_flops(int32_t n_wg, int32_t iters) {
  // 4 waves x 8 chains x (32 x 32 x 16 multiply-adds = 32768 flop) per round
  return (double)n_wg * 4.0 * 8.0 * 32768.0 * (double)iters;
}

extern "C" int csa_probe_read(const void* buf, size_t bytes, uint32_t* sink, int32_t n_wg,
                              hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || n_wg < 1 || bytes % 16 != 0 ||
      ((uintptr_t)buf & 15u) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_loop, dim3((unsigned)n_wg), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(buf), bytes / 16, sink);
  return (int)hipGetLastError();
}
