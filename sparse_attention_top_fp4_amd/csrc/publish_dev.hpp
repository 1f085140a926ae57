// publish_dev.hpp -- device steps of the index-key publish ([IDX, forward:
// k = k_norm(wk(latent)), RoPE on the last rope_head_dim dims, fp4 round
// trip, store]; [VLLM, DeepseekV4Indexer._produce_k]), shared by the
// publish kernels and the score launch that publishes a decode step's key
// itself.  Every floating-point step has a fixed order and explicit
// rounding (the library is built with -ffp-contract=off).
#pragma once

#include "idx_common.hpp"

#include <math.h>

namespace idx {

// y_o = sum_i fma(wk[o][i], latent[i]), i ascending from +0 (fp32; the
// caller rounds it to bf16): the wk row in chunks of CH values, each
// chunk's wk loads and latent reads issued together before its
// fixed-order fma chain (CH only batches the loads: the chain, and so
// the result, is the same for every CH; it costs CH / 2 registers).
// lat_s: the latent in LDS (Din bf16).
template <int CH = 256>
__device__ __forceinline__ float publish_linear(int o, const uint16_t* lat_s,
                                                const uint16_t* __restrict__ wk, int Din) {
  static_assert(CH % 8 == 0, "chunks of whole 16-byte words");
  constexpr int NW = CH / 8;
  const uint16_t* wrow = wk + (int64_t)o * Din;
  float acc = 0.0f;
  int i = 0;
  if ((Din & 7) == 0 && (reinterpret_cast<uintptr_t>(wk) & 15) == 0) {
    const uint4* w4 = reinterpret_cast<const uint4*>(wrow);
    const uint4* l4 = reinterpret_cast<const uint4*>(lat_s);
    for (; i + CH <= Din; i += CH) {
      uint4 wv[NW], lv[NW];
#pragma unroll
      for (int j = 0; j < NW; ++j) wv[j] = w4[i / 8 + j];
#pragma unroll
      for (int j = 0; j < NW; ++j) lv[j] = l4[i / 8 + j];
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const uint32_t u[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
        const uint32_t l[4] = {lv[j].x, lv[j].y, lv[j].z, lv[j].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc = __builtin_fmaf(bf16f(u[m] & 0xffffu), bf16f(l[m] & 0xffffu), acc);
          acc = __builtin_fmaf(bf16f(u[m] >> 16), bf16f(l[m] >> 16), acc);
        }
      }
    }
  }
  for (; i < Din; ++i) acc = __builtin_fmaf(bf16f(wrow[i]), bf16f(lat_s[i]), acc);
  return acc;
}

// Steps after the linear layer, for the 128 threads o = 0..127 of a group
// (every thread of the workgroup takes the barriers; threads with o >= 128
// only take them): k_norm, RoPE with the table row cs_row (the rd / 2
// (cos, sin) pairs of the group's position), quantise, store the row at
// dst (null: not stored).  y_s: the group's bf16 outputs as floats.
__device__ __forceinline__ void publish_finish(int o, const float* y_s, uint32_t* z_s,
                                               float* inv_s, const float* __restrict__ gamma,
                                               const float* __restrict__ cs_row, int rd,
                                               float eps, uint8_t* __restrict__ dst, bool f8,
                                               uint32_t* row_copy = nullptr) {

  if (o == 0) {
    float yv[kHeadDim];
#pragma unroll
    for (int j = 0; j < kHeadDim; ++j) yv[j] = y_s[j];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kHeadDim; ++j) ss = __builtin_fmaf(yv[j], yv[j], ss);
    const float mean = ss / (float)kHeadDim;
    *inv_s = 1.0f / sqrtf(mean + eps);
  }
  __syncthreads();
  if (o < kHeadDim) {
    float v = y_s[o] * *inv_s;
    v = v * gamma[o];
    z_s[o] = f32_to_bf16(v);
  }
  __syncthreads();

  const int base = kHeadDim - rd;
  uint32_t r0 = 0, r1 = 0;
  const bool lead = o < kHeadDim && o >= base && ((o - base) & 1) == 0;
  if (lead) {
    const int i = (o - base) >> 1;
    const float x0 = bf16f(z_s[o]), x1 = bf16f(z_s[o + 1]);
    const float c = cs_row[2 * i];
    const float s = cs_row[2 * i + 1];
    const float a = x0 * c, bb = x1 * s, cc = x0 * s, dd = x1 * c;
    r0 = f32_to_bf16(a - bb);
    r1 = f32_to_bf16(cc + dd);
  }
  __syncthreads();
  if (lead) {
    z_s[o] = r0;
    z_s[o + 1] = r1;
  }
  __syncthreads();

  if (f8) {
    // FP8 row: one e4m3 scale for the 128 values; every thread finds the
    // amax itself (LDS broadcast reads, no further barrier) and writes its
    // own code byte (and, with row_copy, the same byte of the row's 33-word
    // copy in LDS)
    if (o < kHeadDim && (dst || row_copy)) {
      uint32_t amax = 0;
      for (int j = 0; j < kHeadDim; ++j) {
        const uint32_t a = z_s[j] & 0x7fffu;
        amax = a > amax ? a : amax;
      }
      const int e = ue8m0_exponent_f8(bf16f(amax));
      const uint8_t code = (uint8_t)e4m3_code(z_s[o], e);
      const uint32_t scale = (uint32_t)(127 + e) << 23;
      if (dst) {
        dst[o] = code;
        if (o == 0) *reinterpret_cast<uint32_t*>(dst + 128) = scale;
      }
      if (row_copy) {
        reinterpret_cast<uint8_t*>(row_copy)[o] = code;
        if (o == 0) row_copy[32] = scale;
      }
    }
    return;
  }
  if (o < 4 && dst) {
    uint32_t xp[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) xp[i] = z_s[32 * o + 2 * i] | (z_s[32 * o + 2 * i + 1] << 16);
    uint32_t codes[4];
    const int e = quant_block32(xp, codes);
    uint32_t* dcodes = reinterpret_cast<uint32_t*>(dst + 16 * o);
#pragma unroll
    for (int i = 0; i < 4; ++i) dcodes[i] = codes[i];
    dst[64 + o] = (uint8_t)(e + 127);
    if (row_copy) {  // the same row in LDS (17 words), for a caller that scores it
#pragma unroll
      for (int i = 0; i < 4; ++i) row_copy[4 * o + i] = codes[i];
      reinterpret_cast<uint8_t*>(row_copy)[64 + o] = (uint8_t)(e + 127);
    }
  }
}

}  // namespace idx
