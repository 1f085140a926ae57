// quant.hip -- block-32 e2m1/e8m0 quantise-dequantise of 128-wide bf16 rows
// into 68-byte key rows ([IDX, forward: fp4_act_quant]; [CMP,
// fp4_quant_e8m0_inplace, to_e2m1_rne]; row size from [VLLM,
// _indexer_k_cache_head_dim]).
//
// One thread per block of 32 values: it reads 64 contiguous bytes, writes
// 16 code bytes, one scale byte and (optionally) 64 bytes of round trip.
// HBM-bound; 1 byte of scale per 32 values is written with a byte store.
#include "idx_common.hpp"

namespace idx {

__global__ __launch_bounds__(256) void fp4_quant_kernel(const uint16_t* __restrict__ x,
                                                        int64_t n_blocks,
                                                        uint8_t* __restrict__ rows,
                                                        uint16_t* __restrict__ rt) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  const int64_t row = blk >> 2;
  const int j = (int)(blk & 3);
  const uint4* src = reinterpret_cast<const uint4*>(x + blk * kBlock);
  uint32_t xp[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    xp[4 * i + 0] = v.x;
    xp[4 * i + 1] = v.y;
    xp[4 * i + 2] = v.z;
    xp[4 * i + 3] = v.w;
  }
  uint32_t codes[4];
  const int e = quant_block32(xp, codes);
  uint8_t* dst = rows + row * kRowBytes;
  uint32_t* dcodes = reinterpret_cast<uint32_t*>(dst + 16 * j);  // 4-byte aligned: 68*row + 16*j
#pragma unroll
  for (int i = 0; i < 4; ++i) dcodes[i] = codes[i];
  dst[64 + j] = (uint8_t)(e + 127);
  if (rt) {
    uint32_t out[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c0 = (codes[i / 4] >> (8 * (i % 4))) & 0xfu;
      const uint32_t c1 = (codes[i / 4] >> (8 * (i % 4) + 4)) & 0xfu;
      out[i] = e2m1_dequant_bf16(c0, e) | (e2m1_dequant_bf16(c1, e) << 16);
    }
    uint4* d = reinterpret_cast<uint4*>(rt + blk * kBlock);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
  }
}

}  // namespace idx

extern "C" idx_status idx_fp4_quant(const uint16_t* x, int64_t n_rows, uint8_t* rows68,
                                    uint16_t* roundtrip, void* stream) {
  if (n_rows < 0) return IDX_EINVAL;
  if (n_rows == 0) return IDX_OK;
  if (!x || !rows68) return IDX_EINVAL;
  const int64_t n_blocks = n_rows * 4;
  const int64_t grid = (n_blocks + 255) / 256;
  if (grid > 0x7fffffffLL) return IDX_EINVAL;
  hipLaunchKernelGGL(idx::fp4_quant_kernel, dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)stream, x, n_blocks, rows68, roundtrip);
  return idx_host::launch_status();
}
