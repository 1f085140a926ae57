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

// FP8 rows ([VLLM, _indexer_k_cache_head_dim]: 128 e4m3 bytes and one fp32
// ue8m0 scale per 128 values): four threads per row, 32 values each, the
// block's scale agreed between them (quant_block128_f8).
__global__ __launch_bounds__(256) void fp8_quant_kernel(const uint16_t* __restrict__ x,
                                                        int64_t n_quads,
                                                        uint8_t* __restrict__ rows,
                                                        uint16_t* __restrict__ rt) {
  const int64_t qd = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (qd >= n_quads) return;  // whole rows: the four lanes of a row leave together
  const int64_t row = qd >> 2;
  const int j = (int)(qd & 3);
  const uint4* src = reinterpret_cast<const uint4*>(x + qd * kBlock);
  uint32_t xp[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    xp[4 * i + 0] = v.x;
    xp[4 * i + 1] = v.y;
    xp[4 * i + 2] = v.z;
    xp[4 * i + 3] = v.w;
  }
  uint32_t codes[8];
  const int e = quant_block128_f8(xp, codes);
  uint32_t* dst = reinterpret_cast<uint32_t*>(rows + row * kRowBytesF8);  // 4-byte aligned
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[8 * j + i] = codes[i];
  if (j == 0) dst[32] = (uint32_t)(127 + e) << 23;  // the scale 2^e as fp32
  if (rt) {
    uint32_t out[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w = codes[i / 2] >> (16 * (i % 2));
      out[i] = e4m3_dequant_bf16(w & 0xffu, e) | (e4m3_dequant_bf16((w >> 8) & 0xffu, e) << 16);
    }
    uint4* d = reinterpret_cast<uint4*>(rt + qd * kBlock);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
  }
}

// The query step ([IDX, forward: the query heads' RoPE on the last rd dims
// at positions start_pos + s, fp4_act_quant, weights_proj(x) * softmax_scale
// * n_heads^-0.5]; [VLLM, fused_indexer_q_rope_quant] fuses the three).
//
// A workgroup takes 64 head rows (256 blocks of 32 values, 16 KB of bf16)
// and reads them in four passes of 16-byte words: in pass i lane t loads
// word 256i + t, so every load instruction is one contiguous 1 KB run.  That
// word is piece p = t & 3 (elements 8p..8p+7) of block j = (t >> 2) & 3 of
// row 16i + t/16.  The four lanes of a quad hold one block: each finds the
// largest sign-cleared pattern of its 8 values, two DPP quad permutes give
// all four the block's amax, and each lane converts its own 8 values into
// the block's code word p (the quantiser below, split four ways).
//
// Word m of a piece holds the pair (d, d + 1), d = 32j + 8p + 2m, a RoPE
// pair whenever d >= D - rd (pairs never straddle a piece: 8 and D - rd are
// even).  Rotation as the key publish: (x0*c - x1*s, x0*s + x1*c), every
// product and sum rounded in fp32 (the library is built with
// -ffp-contract=off), then bf16; then the quantiser.  The piece-0 lane of
// block 0 of each head also writes bf16(fp32(w_raw) * w_scale).  The 64
// rows leave through LDS in one coalesced run of words.
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
  return v > o ? v : o;
}

__global__ __launch_bounds__(256) void q_rope_quant_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ w_raw, float w_scale,
    const float* __restrict__ cos_sin, int rd, int S, int H, int start_pos, int64_t n_blocks,
    uint8_t* __restrict__ rows, uint16_t* __restrict__ rt, uint16_t* __restrict__ w_out) {
  const int t = threadIdx.x;
  const int p = t & 3, j = (t >> 2) & 3, w16 = t & 15;  // piece, block, 16-byte word of the row
  const int64_t rh0 = (int64_t)blockIdx.x * 64;  // first row of the workgroup
  const int64_t nrows = n_blocks >> 2;
  const int base = kHeadDim - rd;
  const uint4* src = reinterpret_cast<const uint4*>(q);
  // all four loads first; a row past the last reads row 0 and stores nothing
  // (a quad's four lanes share a row, so they agree on it)
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t rh = rh0 + 16 * i + (t >> 4);
    v[i] = src[(rh < nrows ? rh : 0) * 16 + w16];
  }
  // each row's position, one 64-bit division per row: lanes 0..63 of wave 0
  __shared__ int pos_l[64];
  __shared__ uint32_t stage[64 * 17];
  if (t < 64) {
    const int64_t rh = rh0 + t;
    pos_l[t] = start_pos + (int)(((rh < nrows ? rh : 0) / H) % S);
  }
  __syncthreads();
  // every (cos, sin) pair the lane may rotate, all sixteen loads in flight
  // together (a pair below D - rd takes entry 0 and is not used)
  float2 csv[4][4];
  if (rd > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2* cs =
          reinterpret_cast<const float2*>(cos_sin + (int64_t)pos_l[16 * i + (t >> 4)] * rd);  // [rd/2]
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int pi = (32 * j + 8 * p + 2 * m - base) >> 1;
        csv[i][m] = cs[pi > 0 ? pi : 0];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lrow = 16 * i + (t >> 4);
    const int64_t rh = rh0 + lrow;  // head row r * H + h
    const bool live = rh < nrows;
    uint32_t xp[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    if (rd > 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (32 * j + 8 * p + 2 * m >= base) {  // a RoPE pair
          const float x0 = bf16f(xp[m] & 0xffffu), x1 = bf16f(xp[m] >> 16);
          const float c = csv[i][m].x, sn = csv[i][m].y;
          const float a = x0 * c, bb = x1 * sn, cc = x0 * sn, dd = x1 * c;
          xp[m] = f32x2_to_bf16x2(a - bb, cc + dd);
        }
      }
    }
    // quant_block32's amax and codes, one piece per lane
    u16x2_t mx = __builtin_bit_cast(u16x2_t, xp[0] & 0x7fff7fffu);
#pragma unroll
    for (int m = 1; m < 4; ++m)
      mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2_t, xp[m] & 0x7fff7fffu));
    const uint32_t amax_bits = quad_max_u32(mx[0] > mx[1] ? mx[0] : mx[1]);
    const int e = e8m0_exponent(bf16f(amax_bits));
    const float scale = __uint_as_float((uint32_t)(127 + e) << 23);  // 2^e, e in [-126, 126]
    uint32_t word = 0;
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, xp[0]), scale, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, xp[1]), scale, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, xp[2]), scale, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, xp[3]), scale, 3);
    stage[lrow * 17 + w16] = word;  // bytes 16j + 4p of the row
    if (p == 0) reinterpret_cast<uint8_t*>(stage)[lrow * kRowBytes + 64 + j] = (uint8_t)(e + 127);
    if (rt && live) {
      uint32_t out[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        out[m] = e2m1_dequant_bf16((word >> (8 * m)) & 0xfu, e) |
                 (e2m1_dequant_bf16((word >> (8 * m + 4)) & 0xfu, e) << 16);
      reinterpret_cast<uint4*>(rt)[rh * 16 + w16] = make_uint4(out[0], out[1], out[2], out[3]);
    }
    if (w16 == 0 && live) w_out[rh] = (uint16_t)f32_to_bf16(bf16f(w_raw[rh]) * w_scale);
  }
  __syncthreads();
  const int nw = (int)((nrows - rh0 < 64 ? nrows - rh0 : 64) * 17);
  uint32_t* dst = reinterpret_cast<uint32_t*>(rows + rh0 * kRowBytes);
  for (int i = t; i < nw; i += 256) dst[i] = stage[i];
}

}  // namespace idx

extern "C" idx_status idx_q_rope_quant(const uint16_t* q, const uint16_t* w_raw, float w_scale,
                                       const float* cos_sin, int P, int B, int S, int H, int D,
                                       int rd, int start_pos, uint8_t* q_rows,
                                       uint16_t* q_roundtrip, uint16_t* w_out, void* stream) {
  if (B < 0 || S < 0 || H < 0 || D <= 0 || P < 0 || start_pos < 0) return IDX_EINVAL;
  if (D != idx::kHeadDim) return IDX_EUNSUPPORTED;
  if (rd < 0 || rd > D || (rd & 1)) return IDX_EINVAL;
  if ((int64_t)B * S * H == 0) return IDX_OK;
  if (!q || !w_raw || !q_rows || !w_out || (rd > 0 && !cos_sin)) return IDX_EINVAL;
  if (rd > 0 && (int64_t)start_pos + S - 1 >= P) return IDX_EINVAL;  // position not in the table
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(q_roundtrip) & 15) ||
      (reinterpret_cast<uintptr_t>(q_rows) & 3) || (reinterpret_cast<uintptr_t>(cos_sin) & 7))
    return IDX_EINVAL;
  const int64_t n_blocks = (int64_t)B * S * H * 4;
  const int64_t grid = (n_blocks + 255) / 256;
  if (grid > 0x7fffffffLL) return IDX_EINVAL;
  hipLaunchKernelGGL(idx::q_rope_quant_kernel, dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)stream, q, w_raw, w_scale, cos_sin, rd, S, H, start_pos,
                     n_blocks, q_rows, q_roundtrip, w_out);
  return idx_host::launch_status();
}

extern "C" idx_status idx_fp4_quant(const uint16_t* x, int64_t n_rows, uint8_t* rows68,
                                    uint16_t* roundtrip, void* stream) {
  if (n_rows < 0) return IDX_EINVAL;
  if (n_rows == 0) return IDX_OK;
  if (!x || !rows68) return IDX_EINVAL;
  // x and roundtrip move as 16-byte words, the rows as 4-byte words
  if (!idx_host::aligned(x, 16) || !idx_host::aligned(roundtrip, 16) ||
      !idx_host::aligned(rows68, 4))
    return IDX_EINVAL;
  const int64_t n_blocks = n_rows * 4;
  const int64_t grid = (n_blocks + 255) / 256;
  if (grid > 0x7fffffffLL) return IDX_EINVAL;
  hipLaunchKernelGGL(idx::fp4_quant_kernel, dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)stream, x, n_blocks, rows68, roundtrip);
  return idx_host::launch_status();
}

extern "C" idx_status idx_fp8_quant(const uint16_t* x, int64_t n_rows, uint8_t* rows132,
                                    uint16_t* roundtrip, void* stream) {
  if (n_rows < 0) return IDX_EINVAL;
  if (n_rows == 0) return IDX_OK;
  if (!x || !rows132) return IDX_EINVAL;
  if (!idx_host::aligned(x, 16) || !idx_host::aligned(roundtrip, 16) ||
      !idx_host::aligned(rows132, 4))
    return IDX_EINVAL;
  const int64_t n_quads = n_rows * 4;
  const int64_t grid = (n_quads + 255) / 256;
  if (grid > 0x7fffffffLL) return IDX_EINVAL;
  hipLaunchKernelGGL(idx::fp8_quant_kernel, dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)stream, x, n_quads, rows132, roundtrip);
  return idx_host::launch_status();
}
