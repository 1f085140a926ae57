// probe.hip -- measured ceilings of the chip that the Indexer's kernels are
// compared with (measurement support, not page operations):
//
//   idx_probe_stream_read  a plain streaming read: each workgroup reads one
//                          contiguous span in 16-byte loads, eight loads in
//                          flight per thread, and folds what it read into
//                          one word (so no load is dropped).  The decode
//                          score kernel's key stream is this pattern plus
//                          the contraction.
//   idx_probe_mfma_fp4     back-to-back v_mfma_scale_f32_32x32x64_f8f6f4 on
//                          fp4 operands held in registers, four independent
//                          accumulators per wave: the matrix-core rate the
//                          prefill score kernel is bounded by.
//
// Each call launches its kernel with a HIP event pair attached
// (hipExtLaunchKernel), waits for it and returns the kernel's duration.
#include "idx_common.hpp"

#include <hip/hip_ext.h>

namespace idx {

typedef int v8i_p __attribute__((ext_vector_type(8)));
typedef float v16f_p __attribute__((ext_vector_type(16)));

constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ buf,
                                                          int64_t n16, int64_t per_wg,
                                                          uint32_t* __restrict__ sink) {
  const int64_t beg = (int64_t)blockIdx.x * per_wg;
  const int64_t end = beg + per_wg < n16 ? beg + per_wg : n16;
  uint32_t acc = 0;
  for (int64_t i = beg + threadIdx.x; i < end; i += 256 * kProbeUnroll) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + 256 * u;
      v[u] = j < end ? buf[j] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one word per workgroup: the xor of everything it read
  acc ^= (uint32_t)__shfl_xor((int)acc, 32, 64);
  acc ^= (uint32_t)__shfl_xor((int)acc, 16, 64);
  acc ^= (uint32_t)__shfl_xor((int)acc, 8, 64);
  acc ^= (uint32_t)__shfl_xor((int)acc, 4, 64);
  acc ^= (uint32_t)__shfl_xor((int)acc, 2, 64);
  acc ^= (uint32_t)__shfl_xor((int)acc, 1, 64);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ __launch_bounds__(256) void mfma_fp4_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  // operands from the lane id: any fp4 bit patterns do; the scale bytes 127
  // (2^0) keep every product finite
  v8i_p a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = i < 4 ? (int)(0x11111111u * (uint32_t)((lane + i) & 7)) : 0;
    b[i] = i < 4 ? (int)(0x22222222u * (uint32_t)((lane + 3 * i) & 3)) : 0;
  }
  v16f_p c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 4, 4, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 4, 4, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 4, 4, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 4, 4, 0, 127, 0, 127);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (s == 12345.0f) sink[blockIdx.x * 256 + threadIdx.x] = s;  // keeps the chain live
}

}  // namespace idx

namespace {
hipEvent_t g_probe_ev[2] = {nullptr, nullptr};

idx_status probe_events() {
  for (auto& e : g_probe_ev)
    if (!e && hipEventCreate(&e) != hipSuccess) return IDX_EHIP;
  return IDX_OK;
}

idx_status probe_wait(float* ms) {
  if (hipGetLastError() != hipSuccess) return IDX_EHIP;
  if (hipEventSynchronize(g_probe_ev[1]) != hipSuccess) return IDX_EHIP;
  return hipEventElapsedTime(ms, g_probe_ev[0], g_probe_ev[1]) == hipSuccess ? IDX_OK : IDX_EHIP;
}
}  // namespace

extern "C" idx_status idx_probe_stream_read(const void* buf, int64_t bytes, int grid,
                                            uint32_t* sink, float* ms, void* stream) {
  if (!buf || !sink || !ms || bytes < 16 || (bytes & 15) || grid <= 0) return IDX_EINVAL;
  if (!idx_host::aligned(buf, 16)) return IDX_EINVAL;
  const idx_status e = probe_events();
  if (e != IDX_OK) return e;
  const int64_t n16 = bytes / 16;
  const int64_t per_wg = (n16 + grid - 1) / grid;
  hipExtLaunchKernelGGL(idx::stream_read_kernel, dim3((unsigned)grid), dim3(256), 0,
                        (hipStream_t)stream, g_probe_ev[0], g_probe_ev[1], 0u,
                        (const uint4*)buf, n16, per_wg, sink);
  return probe_wait(ms);
}

extern "C" idx_status idx_probe_mfma_fp4(int grid, int iters, float* sink, double* flops,
                                         float* ms, void* stream) {
  if (grid <= 0 || iters <= 0 || !sink || !flops || !ms) return IDX_EINVAL;
  const idx_status e = probe_events();
  if (e != IDX_OK) return e;
  // 4 waves a workgroup, 4 MFMAs an iteration, 2 * 32 * 32 * 64 flop each
  *flops = (double)grid * 4.0 * iters * 4.0 * 131072.0;
  hipExtLaunchKernelGGL(idx::mfma_fp4_kernel, dim3((unsigned)grid), dim3(256), 0,
                        (hipStream_t)stream, g_probe_ev[0], g_probe_ev[1], 0u, iters, sink);
  return probe_wait(ms);
}

// The bf16 conversion instruction against the software round-to-nearest-even
// over every finite fp32 bit pattern (pairs 2i, 2i + 1 per conversion).
__global__ __launch_bounds__(256) void bf16_convert_probe_kernel(unsigned long long* bad) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  unsigned long long mine = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 31); i += stride) {
    const uint32_t u0 = (uint32_t)(2 * i), u1 = u0 + 1u;
    const float a = __uint_as_float(u0), b = __uint_as_float(u1);
    const uint32_t hw = idx::f32x2_to_bf16x2(a, b);
    const bool fa = (u0 & 0x7f800000u) != 0x7f800000u, fb = (u1 & 0x7f800000u) != 0x7f800000u;
    mine += (fa && (hw & 0xffffu) != idx::f32_to_bf16(a)) ? 1u : 0u;
    mine += (fb && (hw >> 16) != idx::f32_to_bf16(b)) ? 1u : 0u;
  }
  if (mine) atomicAdd(bad, mine);
}

extern "C" idx_status idx_probe_bf16_convert(unsigned long long* count,
                                              unsigned long long* mismatches, void* stream) {
  if (!count || !mismatches || !idx_host::aligned(count, 8)) return IDX_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (hipMemsetAsync(count, 0, sizeof(unsigned long long), st) != hipSuccess) return IDX_EHIP;
  hipLaunchKernelGGL(bf16_convert_probe_kernel, dim3(16384), dim3(256), 0, st, count);
  const idx_status s = idx_host::launch_status();
  if (s != IDX_OK) return s;
  if (hipMemcpyAsync(mismatches, count, sizeof(unsigned long long), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return IDX_EHIP;
  return IDX_OK;
}
