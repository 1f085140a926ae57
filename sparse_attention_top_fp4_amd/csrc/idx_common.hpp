// idx_common.hpp -- device helpers shared by the gfx950 kernels of the
// DeepSeek-V4.1 Indexer hot path: bf16 conversion, the block-32 e2m1/e8m0
// quantiser, order-preserving score keys, and wave/block scans.
//
// Pages cited by page and section: [IDX] "DeepSeek V4.1" (class Indexer),
// [CMP] "Module compress" (CPU reference API), [VLLM] the vLLM
// "attention.py" patch (DeepseekV4Indexer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/idx.h"

namespace idx {

constexpr int kHeadDim = 128;   // index_head_dim
constexpr int kRowBytes = 68;   // [VLLM, _indexer_k_cache_head_dim]: 64 code bytes + 4 scale bytes
constexpr int kBlock = 32;      // values per e8m0 scale
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;  // order key of -inf

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round a finite fp32 to bf16, nearest-even.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two finite fp32 values to a pair of bf16 (a in the low half), nearest-even,
// in one conversion instruction of gfx950: equal to f32_to_bf16 on both for
// every finite input (idx_probe_bf16_convert checks all of them).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  const f32x2_v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// ------------------------------------------------------------- quantiser
// [CMP, fp4_quant_e8m0_inplace]: the scale is the power-of-two ceiling of
// amax/6 with amax raised to at least 6*2^-126.  Writing the (normal) amax as
// m*2^E with m in [1,2): 6*2^e >= m*2^E  <=>  e >= E-2 + log2(m/1.5), so the
// ceiling is e = E-2 when m <= 1.5 and E-1 otherwise.  Exact, no division.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  const float a = fmaxf(amax, 0x1.8p-124f);  // 6 * 2^-126
  const uint32_t u = __float_as_uint(a);
  const int E = (int)(u >> 23) - 127;
  return E - 2 + ((u & 0x7fffffu) > 0x400000u ? 1 : 0);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Quantise 32 bf16 values packed two per word (element 2i in the low half of
// word i).  Returns e; codes[j] holds elements 8j..8j+7, element 8j+m in
// nibble m, so the four words are bytes 16*block.. of the 68-byte row.
//   amax: the largest |x| as the largest sign-cleared bf16 pattern (the
//         patterns of non-negative finite values order like their values),
//         with packed 16-bit max;
//   codes: [CMP, to_e2m1_rne] -- nearest point of the e2m1 grid
//         {0,.5,1,1.5,2,3,4,6} to |x|/2^e, ties to the even code (the
//         midpoints .25 1.25 2.5 5 go down, .75 1.75 3.5 go up), sign kept.
//         gfx950's scaled bf16->fp4 conversion of x with scale 2^e rounds to
//         nearest-even and keeps the sign, which is this rule; the GPU tests
//         check it against the oracle on every finite bf16 at several scales.
__device__ __forceinline__ int quant_block32(const uint32_t (&xp)[16], uint32_t (&codes)[4]) {
  u16x2_t m = __builtin_bit_cast(u16x2_t, xp[0] & 0x7fff7fffu);
#pragma unroll
  for (int i = 1; i < 16; ++i)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, xp[i] & 0x7fff7fffu));
  const uint32_t amax_bits = m[0] > m[1] ? m[0] : m[1];
  const int e = e8m0_exponent(bf16f(amax_bits));
  const float scale = __uint_as_float((uint32_t)(127 + e) << 23);  // 2^e, e in [-126, 126]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t word = 0;
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, xp[4 * j + 0]), scale, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, xp[4 * j + 1]), scale, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, xp[4 * j + 2]), scale, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, xp[4 * j + 3]), scale, 3);
    codes[j] = word;
  }
  return e;
}

// Dequantised bf16 of a code at exponent e (exact: at most 2 significant
// bits; 0.5 * 2^-126 is a subnormal that fp32 and bf16 both hold).
__device__ __forceinline__ uint32_t e2m1_dequant_bf16(uint32_t code, int e) {
  const uint32_t m = code & 7u;
  // twice the grid value: 0 1 2 3 4 6 8 12
  const uint32_t tw = m < 4u ? m : (m == 4u ? 4u : (m == 5u ? 6u : (m == 6u ? 8u : 12u)));
  const float half_scale = __uint_as_float((uint32_t)(127 + e) << 23) * 0.5f;  // 2^(e-1)
  const float v = (float)tw * half_scale;
  return f32_to_bf16((code & 8u) ? -v : v);
}

// ------------------------------------------------------------ FP8 rows
// The FP8 indexer cache ([VLLM, _indexer_k_cache_head_dim]: 128 fp8 bytes and
// one fp32 scale per 128 values; [VLLM, DeepseekV4Indexer.__init__]:
// quant_block_size 128, scale_fmt "ue8m0"): bytes 0..127 the OCP e4m3 codes
// of elements 0..127 (bit 7 = sign), bytes 128..131 the scale 2^e as fp32.
constexpr int kRowBytesF8 = 132;

// e of the block scale: the smallest integer with 448 * 2^e >= amax, amax
// raised to at least 448 * 2^-126.  With amax = m * 2^E, m in [1, 2):
// 1.75 * 2^(8+e) >= m * 2^E  <=>  e = E - 8 when m <= 1.75, else E - 7.
__device__ __forceinline__ int ue8m0_exponent_f8(float amax) {
  const float a = fmaxf(amax, 0x1.cp-118f);  // 448 * 2^-126
  const uint32_t u = __float_as_uint(a);
  const int E = (int)(u >> 23) - 127;
  return E - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
}

// e4m3 code of the bf16 x at scale 2^e (|x| / 2^e <= 448): the nearest e4m3
// point, ties to the even code, sign in bit 7.  y = |x| * 2^-e is exact (a
// power-of-two scaling; a y that fp32 holds only as a subnormal rounds to
// code 0 either way).  Below 2^-6 the e4m3 points are the multiples of 2^-9
// (code = the multiple; 8 is the first normal, 2^-6); above, keeping the
// fp32 exponent and top three mantissa bits with a round-half-even carry
// gives the code after rebasing the exponent bias from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_code(uint32_t xb16, int e) {
  const float y = fabsf(bf16f(xb16)) * __uint_as_float((uint32_t)(127 - e) << 23);
  uint32_t code;
  if (y < 0x1p-6f) {
    code = (uint32_t)__builtin_rintf(y * 512.0f);
  } else {
    const uint32_t u = __float_as_uint(y);
    uint32_t r = u >> 20;
    const uint32_t low = u & 0xfffffu;
    r += (low > 0x80000u || (low == 0x80000u && (r & 1u))) ? 1u : 0u;
    code = r - (120u << 3);
  }
  return code | ((xb16 >> 8) & 0x80u);
}

// Dequantised bf16 of an e4m3 code at scale 2^e: (8 + m) * 2^(E - 10) for
// exponent field E > 0, m * 2^-9 for E = 0, times 2^e (exact in fp32; the
// bf16 rounding is the only one, and exact unless the value falls below
// bf16's subnormals).
__device__ __forceinline__ uint32_t e4m3_dequant_bf16(uint32_t code, int e) {
  const uint32_t E = (code >> 3) & 15u, m = code & 7u;
  const float v = E == 0u ? (float)m * 0x1p-9f
                          : (float)(8u + m) * __uint_as_float((E + 117u) << 23);
  const float sv = v * __uint_as_float((uint32_t)(127 + e) << 23);
  return f32_to_bf16((code & 0x80u) ? -sv : sv);
}

// Quantise 128 bf16 values spread over four consecutive lanes (this lane:
// 32 of them, packed two per word, element 2i in the low half of word i):
// the four lanes agree on the block's e (returned); codes[j] gets elements
// 4j..4j+3 of this lane's 32, element 4j+m in byte m.
__device__ __forceinline__ int quant_block128_f8(const uint32_t (&xp)[16], uint32_t (&codes)[8]) {
  u16x2_t m = __builtin_bit_cast(u16x2_t, xp[0] & 0x7fff7fffu);
#pragma unroll
  for (int i = 1; i < 16; ++i)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, xp[i] & 0x7fff7fffu));
  uint32_t amax_bits = m[0] > m[1] ? m[0] : m[1];
  // the four lanes of the block: exchange by xor 1 and 2 (all four active)
  uint32_t o = (uint32_t)__shfl_xor((int)amax_bits, 1, 64);
  amax_bits = o > amax_bits ? o : amax_bits;
  o = (uint32_t)__shfl_xor((int)amax_bits, 2, 64);
  amax_bits = o > amax_bits ? o : amax_bits;
  const int e = ue8m0_exponent_f8(bf16f(amax_bits));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w0 = xp[2 * j], w1 = xp[2 * j + 1];
    codes[j] = e4m3_code(w0 & 0xffffu, e) | (e4m3_code(w0 >> 16, e) << 8) |
               (e4m3_code(w1 & 0xffffu, e) << 16) | (e4m3_code(w1 >> 16, e) << 24);
  }
  return e;
}

// ---------------------------------------------------------- score keys
// Order-preserving key of a score: larger score -> larger key; -0 maps to +0.
// Integer form: negative floats have every bit flipped, the others only the
// sign bit (the arithmetic shift spreads the sign over the word).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  u = u == 0x80000000u ? 0u : u;
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// ------------------------------------------------------ wave/block scans
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS traffic):
// Hillis-Steele steps inside each row of 16 lanes (row_shr 1, 2, 4, 8), then
// row_bcast15 carries each row's total into the next row (rows 1 and 3) and
// row_bcast31 carries the first half-wave's total into rows 2 and 3.  Lanes
// whose source is outside the row read 0.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Sum over the wave (every lane active), by DPP scan: no LDS round trips.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_sum(v), 63);
}

// number of lanes below this one with the predicate set
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// v_writelane_b32: the result is `old` with lane `lane` set to the uniform
// `val`.  This compiler has no builtin for it, so the LLVM intrinsic is
// declared by name.
extern "C" __device__ int idx_writelane_i32(int val, int lane, int old) __asm(
    "llvm.amdgcn.writelane.i32");

// acc + lanes_below(mask), in the two mbcnt instructions
__device__ __forceinline__ uint32_t lanes_below_acc(uint64_t mask, uint32_t acc) {
  return (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mask, acc));
}

}  // namespace idx

// ------------------------------------------------------- host helpers
namespace idx_host {

// Block select from block maxima bmax[R][ld_b] (nb <= kSelectWaveMaxBlocks
// blocks of cbs positions; the rule of idx_select_candidate_blocks), one
// wave per row.  Defined in topk.hip.
constexpr int kSelectWaveMaxBlocks = 1024;
idx_status select_blocks_from_max(const float* bmax, int64_t ld_b, int R, int nb, int T,
                                  const int32_t* compress_lens, int cbs, int ctb, int32_t* ids,
                                  int64_t ld_ids, hipStream_t st);
// idx_score in candidate mode with slot v's score at slot_scores[r][v]
// (ld >= n_cand * cand_block_size) and no -inf fill; with l1_scores, extra
// workgroups of the launch also run kernel A of the split top-k of those
// level-one scores [R][l1_ld] (histogram l1_hist, workspace l1_ws, k_out
// l1_kout; T as the candidate rows').  Defined in score.hip.
idx_status score_candidates_compact(const uint16_t* q, const uint16_t* w, const uint8_t* k_cache,
                                    int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                                    const int32_t* compress_lens, const int32_t* cand_blocks,
                                    int n_cand, int cand_block_size, float* slot_scores,
                                    int64_t ld, uint32_t* key_hist, hipStream_t stream,
                                    const float* l1_scores = nullptr, int64_t l1_ld = 0,
                                    const uint32_t* l1_hist = nullptr, uint32_t* l1_ws = nullptr,
                                    int l1_kout = 0);
inline idx_status launch_status() {
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
}

// p is a multiple of `bytes` (a power of two); null counts as aligned.
inline bool aligned(const void* p, uintptr_t bytes) {
  return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0;
}
}  // namespace idx_host
