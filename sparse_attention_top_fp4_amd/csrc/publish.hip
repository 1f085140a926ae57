// publish.hip -- index-key publish of a key-owning Indexer layer
// ([IDX, forward: k = k_norm(wk(latent)), RoPE on the last rope_head_dim
// dims at the group's position, fp4 round trip, store at start_pos // ratio];
// [VLLM, DeepseekV4Indexer._produce_k / indexer_k_norm_rope_store]).
//
// One workgroup of 128 threads per (sequence, group); thread o owns output
// feature o.  Every floating-point step has a fixed order and explicit
// rounding (the library is built with -ffp-contract=off):
//   y_o  = bf16(sum_i fma(wk[o][i], latent[i]))      i ascending, from +0
//   ss   = sum_o fma(y_o, y_o)                        o ascending, from +0
//   inv  = 1 / sqrt(ss / 128 + eps)                   correctly rounded
//   z_o  = bf16((y_o * inv) * gamma_o)
//   RoPE on interleaved pairs of the last rd dims: (x0*c - x1*s, x0*s + x1*c)
//   then the block-32 e2m1/e8m0 quantiser and the 68-byte row store.
// Tiny and latency-bound (one row per sequence in decode); it must run
// before the score of the same step reads the cache, which the caller gets
// by issuing both on one stream.
#include "idx_common.hpp"
#include "publish_dev.hpp"

#include <math.h>

#include <atomic>

namespace idx {

constexpr int kPubPageRows = 64;  // compressed positions per page of a paged cache

__global__ __launch_bounds__(128) void publish_kernel(
    const uint16_t* __restrict__ latent, const uint16_t* __restrict__ wk,
    const float* __restrict__ gamma, const float* __restrict__ cos_sin, int Din, int rd, float eps,
    int start_pos, int ratio, int G, uint8_t* __restrict__ kc, int64_t kstride,
    const int32_t* __restrict__ bt, int64_t bt_stride, int64_t page_stride, int n_pages,
    bool f8) {
  const int rb = f8 ? kRowBytesF8 : kRowBytes;
  extern __shared__ __attribute__((aligned(16))) uint16_t lat_s[];  // Din bf16
  __shared__ float y_s[kHeadDim];
  __shared__ uint32_t z_s[kHeadDim];
  __shared__ float inv_s;
  const int bg = blockIdx.x;
  const int b = bg / G, g = bg % G;
  const int pos = start_pos == 0 ? g * ratio : start_pos + 1 - ratio;
  const int row = start_pos == 0 ? g : start_pos / ratio + g;
  const int o = threadIdx.x;

#pragma unroll 4
  for (int i = o; i < Din; i += kHeadDim) lat_s[i] = latent[(int64_t)bg * Din + i];
  __syncthreads();

  const float acc = publish_linear(o, lat_s, wk, Din);
  y_s[o] = bf16f(f32_to_bf16(acc));
  __syncthreads();
  // contiguous rows, or slot row % 64 of the sequence's page row / 64 (a
  // page id outside [0, n_pages) is not written)
  uint8_t* dst = nullptr;
  if (!bt) {
    dst = kc + ((int64_t)b * kstride + row) * rb;
  } else {
    const int page = bt[(int64_t)b * bt_stride + row / kPubPageRows];
    if (page >= 0 && page < n_pages)
      dst = kc + (int64_t)page * page_stride + (int64_t)(row % kPubPageRows) * rb;
  }
  publish_finish(threadIdx.x, y_s, z_s, &inv_s, gamma, cos_sin + (int64_t)pos * rd, rd, eps,
                 dst, f8);
}

// Many groups (the prompt's keys): one workgroup of kPubGroups * 128 threads
// publishes kPubGroups consecutive (sequence, group) slots, thread o of
// group i computing output o of slot i.  wk is staged once per workgroup in
// LDS as bf16 pairs with two pad words per row (rows 8-byte aligned for the
// chain's 8-byte reads, lane o's row on its own bank pair in each
// half-wave), the slots' latents as floats; every output is still the
// sequential fma chain over the input features, i ascending.  Din <= 512 and
// even (the LDS holds all of wk).
constexpr int kPubGroups = 8;
constexpr int kPubGroupsMaxDin = 512;

__global__ __launch_bounds__(kPubGroups * kHeadDim) void publish_groups_kernel(
    const uint16_t* __restrict__ latent, const uint16_t* __restrict__ wk,
    const float* __restrict__ gamma, const float* __restrict__ cos_sin, int Din, int rd, float eps,
    int start_pos, int ratio, int B, int G, uint8_t* __restrict__ kc, int64_t kstride,
    const int32_t* __restrict__ bt, int64_t bt_stride, int64_t page_stride, int n_pages,
    bool f8) {
  extern __shared__ __attribute__((aligned(16))) uint32_t pg_smem[];
  const int rb = f8 ? kRowBytesF8 : kRowBytes;
  // words per wk row: two pad words keep rows 8-byte aligned for the
  // 8-byte reads below, and the 64 lanes' rows start on distinct bank pairs
  // in each half-wave
  const int wpr = Din / 2 + 2;
  uint32_t* wk_s = pg_smem;                                           // [128][wpr]
  float* lat_s = reinterpret_cast<float*>(pg_smem + kHeadDim * wpr);  // [kPubGroups][Din]
  __shared__ float y_s[kPubGroups][kHeadDim];
  __shared__ uint32_t z_s[kPubGroups][kHeadDim];
  __shared__ float inv_s[kPubGroups];
  const int tid = threadIdx.x, gi = tid >> 7, o = tid & (kHeadDim - 1);
  const int64_t nslots = (int64_t)B * G;
  const int64_t bg0 = (int64_t)blockIdx.x * kPubGroups;

  // wk and the slots' latents into LDS, thread t taking column t % width of
  // every (NT / width)-th row: one division per thread, not per word (Din <=
  // 512, so a pass covers at least 4 wk rows and 2 latent rows).  The
  // latents are requested first, so that they arrive beside wk.
  constexpr int NT = kPubGroups * kHeadDim;
  const uint32_t* wk32 = reinterpret_cast<const uint32_t*>(wk);
  const int hw = Din / 2;
  {
    // at most kPubGroups / 2 slots per thread, all requested before any store
    constexpr int kLat = kPubGroups / 2;
    const int gpp = NT / Din, g0 = tid / Din, k = tid - g0 * Din;
    if (g0 < gpp) {
      uint16_t t[kLat];
#pragma unroll
      for (int u = 0; u < kLat; ++u) {
        const int64_t bg = bg0 + g0 + u * gpp;  // a slot past the end re-reads slot 0
        t[u] = latent[(g0 + u * gpp < kPubGroups && bg < nslots ? bg : bg0) * Din + k];
      }
#pragma unroll
      for (int u = 0; u < kLat; ++u) {
        const int g = g0 + u * gpp;
        if (g < kPubGroups) lat_s[g * Din + k] = bg0 + g < nslots ? bf16f(t[u]) : 0.0f;
      }
    }
  }
  if ((hw & 3) == 0 && (reinterpret_cast<uintptr_t>(wk) & 15) == 0) {  // uniform
    // 16-byte loads: thread t takes words [4q, 4q + 4) of rows r0, r0 + rpp,
    // ... (q = t % (hw / 4)), all requested before any LDS store (a store
    // right after each load would wait out every load's latency in turn); a
    // row past the end re-reads the last row and is not stored.  The rows'
    // LDS starts are 8-byte aligned: two 8-byte stores per load.
    const int qpr = hw >> 2, rpp = NT / qpr, r0 = tid / qpr, c = 4 * (tid - r0 * qpr);
    const uint4* wk128 = reinterpret_cast<const uint4*>(wk);
    if (r0 < rpp)
      for (int row0 = r0; row0 < kHeadDim; row0 += 8 * rpp) {
        uint4 t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = row0 + u * rpp;
          t[u] = wk128[((row < kHeadDim ? row : kHeadDim - 1) * hw + c) >> 2];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = row0 + u * rpp;
          if (row < kHeadDim) {
            uint2* d = reinterpret_cast<uint2*>(wk_s + row * wpr + c);
            d[0] = make_uint2(t[u].x, t[u].y);
            d[1] = make_uint2(t[u].z, t[u].w);
          }
        }
      }
  } else {
    // sixteen rows' loads in flight before their LDS stores; a row past the
    // end re-reads the last row and is not stored
    const int rpp = NT / hw, r0 = tid / hw, c = tid - r0 * hw;
    if (r0 < rpp)
      for (int row0 = r0; row0 < kHeadDim; row0 += 16 * rpp) {
        uint32_t t[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int row = row0 + u * rpp;
          t[u] = wk32[(row < kHeadDim ? row : kHeadDim - 1) * hw + c];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int row = row0 + u * rpp;
          if (row < kHeadDim) wk_s[row * wpr + c] = t[u];
        }
      }
  }
  __syncthreads();

  const uint32_t* wrow = wk_s + o * wpr;
  float acc = 0.0f;  // y_o of slot gi: sum_i fma(wk[o][i], latent[i]), i ascending
  if ((Din & 3) == 0) {  // uniform
    // four inputs per step: one 8-byte wk read and one 16-byte latent read
    // (the latent read is the same address in every lane), half the LDS
    // instructions of the two-input step, which bound this loop
    const uint2* w4 = reinterpret_cast<const uint2*>(wrow);
    const float4* l4 = reinterpret_cast<const float4*>(lat_s + gi * Din);
#pragma unroll 8
    for (int k4 = 0; k4 < Din / 4; ++k4) {
      const uint2 w = w4[k4];
      const float4 l = l4[k4];
      acc = __builtin_fmaf(bf16f(w.x & 0xffffu), l.x, acc);
      acc = __builtin_fmaf(bf16f(w.x >> 16), l.y, acc);
      acc = __builtin_fmaf(bf16f(w.y & 0xffffu), l.z, acc);
      acc = __builtin_fmaf(bf16f(w.y >> 16), l.w, acc);
    }
  } else {
    const float2* lrow = reinterpret_cast<const float2*>(lat_s + gi * Din);  // Din even
    // unrolled so the LDS reads of later pairs are in flight during the chain
#pragma unroll 16
    for (int k2 = 0; k2 < hw; ++k2) {
      const uint32_t w2 = wrow[k2];
      const float2 l2 = lrow[k2];
      acc = __builtin_fmaf(bf16f(w2 & 0xffffu), l2.x, acc);
      acc = __builtin_fmaf(bf16f(w2 >> 16), l2.y, acc);
    }
  }
  y_s[gi][o] = bf16f(f32_to_bf16(acc));
  __syncthreads();

  const int64_t bg = bg0 + gi;
  int pos = 0;
  uint8_t* dst = nullptr;
  if (bg < nslots) {
    const int64_t b = bg / G;
    const int g = (int)(bg - b * G);
    pos = start_pos == 0 ? g * ratio : start_pos + 1 - ratio;
    const int row = start_pos == 0 ? g : start_pos / ratio + g;
    if (!bt) {
      dst = kc + (b * kstride + row) * rb;
    } else {
      const int page = bt[b * bt_stride + row / kPubPageRows];
      if (page >= 0 && page < n_pages)
        dst = kc + (int64_t)page * page_stride + (int64_t)(row % kPubPageRows) * rb;
    }
  }
  publish_finish(o, y_s[gi], z_s[gi], &inv_s[gi], gamma, cos_sin + (int64_t)pos * rd, rd, eps,
                 dst, f8);
}

size_t publish_groups_lds(int Din) {
  return ((size_t)kHeadDim * (Din / 2 + 2) + (size_t)kPubGroups * Din) * 4u;
}

}  // namespace idx

namespace {
// The many-groups kernel uses more than 64 KB of dynamic LDS; the limit is a
// per-device function attribute, raised once on each device the library
// runs on.
bool set_groups_lds_limit() {
  static std::atomic<uint64_t> done_mask{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done_mask.load(std::memory_order_acquire) & bit)) return true;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&idx::publish_groups_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)idx::publish_groups_lds(idx::kPubGroupsMaxDin)) != hipSuccess)
    return false;
  if (bit) done_mask.fetch_or(bit, std::memory_order_acq_rel);
  return true;
}

// Shared by the contiguous and the paged entry points (bt null: contiguous
// rows of stride k_batch_stride_rows).
idx_status publish_impl(const uint16_t* latent, const uint16_t* wk, const float* gamma,
                        const float* cos_sin, int P, int B, int G, int Din, int D, int rd,
                        float eps, int start_pos, int ratio, uint8_t* k_cache,
                        int64_t k_batch_stride_rows, int Tcap, const int32_t* bt,
                        int64_t bt_stride, int64_t page_stride, int n_pages, void* stream,
                        bool f8 = false) {
  if (B < 0 || G < 0 || Din <= 0 || D <= 0 || ratio <= 0 || start_pos < 0 || P < 0 || Tcap < 0)
    return IDX_EINVAL;
  if (D != idx::kHeadDim) return IDX_EUNSUPPORTED;
  if (rd < 0 || rd > D || (rd & 1)) return IDX_EINVAL;
  if (!(eps >= 0.0f)) return IDX_EINVAL;
  if ((int64_t)B * G == 0) return IDX_OK;
  if (!latent || !wk || !gamma || !k_cache || (rd > 0 && !cos_sin)) return IDX_EINVAL;
  if (!bt && k_batch_stride_rows < Tcap) return IDX_EINVAL;
  // rows are written as 4-byte words
  if (!idx_host::aligned(k_cache, 4) || (bt && (page_stride & 3))) return IDX_EINVAL;
  int64_t max_pos, max_row;
  if (start_pos == 0) {
    max_pos = (int64_t)(G - 1) * ratio;
    max_row = G - 1;
  } else {
    if (G != 1) return IDX_EINVAL;
    max_pos = (int64_t)start_pos + 1 - ratio;
    if (max_pos < 0) return IDX_EINVAL;
    max_row = start_pos / ratio;
  }
  if (rd > 0 && max_pos >= P) return IDX_EINVAL;
  if (max_row >= Tcap) return IDX_EINVAL;
  if ((int64_t)B * G > 0x7fffffffLL) return IDX_EINVAL;
  if ((size_t)Din * 2 > 60 * 1024) return IDX_EUNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  // many groups: workgroups of kPubGroups slots sharing wk in LDS
  if ((int64_t)B * G >= idx::kPubGroups && Din <= idx::kPubGroupsMaxDin && (Din & 1) == 0 &&
      (reinterpret_cast<uintptr_t>(wk) & 3) == 0) {
    if (!set_groups_lds_limit()) return IDX_EHIP;
    const int64_t nwg = ((int64_t)B * G + idx::kPubGroups - 1) / idx::kPubGroups;
    hipLaunchKernelGGL(idx::publish_groups_kernel, dim3((unsigned)nwg),
                       dim3(idx::kPubGroups * idx::kHeadDim), idx::publish_groups_lds(Din), st,
                       latent, wk, gamma, cos_sin, Din, rd, eps, start_pos, ratio, B, G, k_cache,
                       k_batch_stride_rows, bt, bt_stride, page_stride, n_pages, f8);
    return idx_host::launch_status();
  }
  hipLaunchKernelGGL(idx::publish_kernel, dim3((unsigned)(B * G)), dim3(idx::kHeadDim),
                     (size_t)Din * 2, st, latent, wk, gamma, cos_sin, Din, rd, eps,
                     start_pos, ratio, G, k_cache, k_batch_stride_rows, bt, bt_stride,
                     page_stride, n_pages, f8);
  return idx_host::launch_status();
}
}  // namespace

extern "C" idx_status idx_publish_keys(const uint16_t* latent, const uint16_t* wk,
                                       const float* gamma, const float* cos_sin, int P, int B,
                                       int G, int Din, int D, int rd, float eps, int start_pos,
                                       int ratio, uint8_t* k_cache, int64_t k_batch_stride_rows,
                                       int Tcap, void* stream) {
  return publish_impl(latent, wk, gamma, cos_sin, P, B, G, Din, D, rd, eps, start_pos, ratio,
                      k_cache, k_batch_stride_rows, Tcap, nullptr, 0, 0, 0, stream);
}

extern "C" idx_status idx_publish_keys_fp8(const uint16_t* latent, const uint16_t* wk,
                                           const float* gamma, const float* cos_sin, int P, int B,
                                           int G, int Din, int D, int rd, float eps, int start_pos,
                                           int ratio, uint8_t* k_cache,
                                           int64_t k_batch_stride_rows, int Tcap, void* stream) {
  return publish_impl(latent, wk, gamma, cos_sin, P, B, G, Din, D, rd, eps, start_pos, ratio,
                      k_cache, k_batch_stride_rows, Tcap, nullptr, 0, 0, 0, stream, true);
}

extern "C" idx_status idx_publish_keys_paged(const uint16_t* latent, const uint16_t* wk,
                                             const float* gamma, const float* cos_sin, int P,
                                             int B, int G, int Din, int D, int rd, float eps,
                                             int start_pos, int ratio, uint8_t* k_pages,
                                             int64_t page_stride, int n_pages,
                                             const int32_t* block_table, int64_t bt_stride,
                                             int Tcap, void* stream) {
  if ((int64_t)B * G > 0) {
    if (!block_table || n_pages <= 0) return IDX_EINVAL;
    if (page_stride < (int64_t)idx::kPubPageRows * idx::kRowBytes) return IDX_EINVAL;
    if (bt_stride < ((int64_t)Tcap + idx::kPubPageRows - 1) / idx::kPubPageRows)
      return IDX_EINVAL;
  }
  return publish_impl(latent, wk, gamma, cos_sin, P, B, G, Din, D, rd, eps, start_pos, ratio,
                      k_pages, 0, Tcap, block_table, bt_stride, page_stride, n_pages, stream);
}

// Host-side YaRN RoPE table (the YaRN method of Peng et al., in the form of
// DeepSeek's precompute_freqs_cis that [CMP, yarn_freqs_cis] names).  Pair i
// has the plain frequency theta^(-2i/rd).  With orig_len > 0 and factor != 1
// it slides to plain/factor along a linear ramp in i: 0 up to the floor of
// the correction dimension of beta_fast rotations over orig_len, 1 from the
// ceiling of that of beta_slow rotations, both kept inside [0, rd - 1].
extern "C" idx_status idx_yarn_cos_sin(int P, int rd, double theta, double factor, int orig_len,
                                       double beta_fast, double beta_slow, float* out) {
  if (P < 0 || rd <= 0 || (rd & 1) || !(theta > 1.0) || !(factor > 0.0) || orig_len < 0)
    return IDX_EINVAL;
  if (P == 0) return IDX_OK;
  if (!out) return IDX_EINVAL;
  const int half = rd / 2;
  double freq[1024];
  if (half > 1024) return IDX_EUNSUPPORTED;
  for (int i = 0; i < half; ++i) freq[i] = pow(theta, -(2.0 * i) / rd);
  if (orig_len > 0 && factor != 1.0) {
    if (!(beta_fast > 0.0) || !(beta_slow > 0.0)) return IDX_EINVAL;
    // dimension whose pair turns `rotations` times over orig_len positions
    auto corr_dim = [&](double rotations) {
      return rd * log((double)orig_len / (rotations * 2.0 * M_PI)) / (2.0 * log(theta));
    };
    double lo = floor(corr_dim(beta_fast)), hi = ceil(corr_dim(beta_slow));
    lo = lo < 0.0 ? 0.0 : lo;
    hi = hi > rd - 1 ? rd - 1 : hi;
    if (hi == lo) hi += 0.001;
    for (int i = 0; i < half; ++i) {
      double t = (i - lo) / (hi - lo);
      t = t < 0.0 ? 0.0 : (t > 1.0 ? 1.0 : t);
      freq[i] = freq[i] * (1.0 - t) + freq[i] / factor * t;
    }
  }
  for (int64_t p = 0; p < P; ++p)
    for (int i = 0; i < half; ++i) {
      const double a = (double)p * freq[i];
      out[(p * half + i) * 2] = (float)cos(a);
      out[(p * half + i) * 2 + 1] = (float)sin(a);
    }
  return IDX_OK;
}
