// merge.hip -- the top-k of a row split along its positions (T-split): each
// slice's local top-k as (position, score) pairs, and the merge of the
// slices' pairs into the row's top-k.
//
// [IDX, forward]: keep min(index_topk, T) positions by score, re-sort them by
// position, t + offset where t < compress_lens and -1 otherwise; ties go to
// the lower position.  A position in the row's top k is beaten by fewer than
// k positions of the row, hence of its own slice, so it is in its slice's
// top k: the union of the slices' top-k lists holds the row's top k, and
// ranking that union by (score descending, position ascending) gives it.
// Slices in position order, each list ascending, concatenate to a list whose
// valid entries ascend, so "lowest position first" among equal scores is
// "lowest list slot first", which is the row ranking's own tie rule
// (row_topk.hpp) applied to the list as a virtual row.
#include "idx_common.hpp"
#include "row_topk.hpp"

#include <atomic>

namespace idx {

// compress_lens of the slice [start, start + Tg): clamp(cl - start, 0, Tg)
__global__ __launch_bounds__(256) void slice_lens_kernel(const int32_t* __restrict__ cl, int R,
                                                         int start, int Tg,
                                                         int32_t* __restrict__ out) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  const int64_t c = (int64_t)cl[r] - start;
  out[r] = (int32_t)(c < 0 ? 0 : (c > Tg ? Tg : c));
}

// Score of each listed position: pos[r][j] = start + t (t in [0, Tg)) or -1
__global__ __launch_bounds__(256) void pair_scores_kernel(const float* __restrict__ scores,
                                                          int64_t ld, int R, int kout, int start,
                                                          const int32_t* __restrict__ pos,
                                                          int64_t ld_out,
                                                          float* __restrict__ sc) {
  const int64_t n = (int64_t)R * kout;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / kout, j = i - r * kout;
    const int p = pos[r * ld_out + j];
    sc[r * ld_out + j] = p >= 0 ? scores[r * ld + (p - start)] : -__builtin_inff();
  }
}

constexpr int kMergeNT = 1024;
constexpr int kMergeMaxN = kMergeNT * 32;  // list entries per row (all slices)

// The row's list of G*n pairs as a virtual row: slot s = g*n + j is entry j
// of slice g's list, its score the pair's score, absent (NaN) for a -1
// position.  posl: N words of dynamic LDS, the position of every slot.
struct ListPos {
  const lds_i32* posl;
  __device__ __forceinline__ int operator()(int s) const { return posl[s]; }
};

// Largest / smallest float over the wave by DPP scan steps (the pattern of
// wave_inclusive_sum); lanes whose source lies outside the row read the
// identity.  NaN lanes are skipped (fmaxf / fminf return the other operand).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max_step(float v) {
  const int o = __builtin_amdgcn_update_dpp((int)0xff800000u, __float_as_int(v), CTRL, ROWS, 0xf,
                                            false);
  return fmaxf(v, __int_as_float(o));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_min_step(float v) {
  const int o = __builtin_amdgcn_update_dpp((int)0x7f800000u, __float_as_int(v), CTRL, ROWS, 0xf,
                                            false);
  return fminf(v, __int_as_float(o));
}
// row_shr:1, 2, 4, 8 inside each row of 16 lanes, then row_bcast:15 (rows 1
// and 3) and row_bcast:31 (rows 2 and 3): lane 63 holds the wave's result
__device__ __forceinline__ float wave_max_f32(float v) {
  v = dpp_max_step<0x111, 0xf>(v);
  v = dpp_max_step<0x112, 0xf>(v);
  v = dpp_max_step<0x114, 0xf>(v);
  v = dpp_max_step<0x118, 0xf>(v);
  v = dpp_max_step<0x142, 0xa>(v);
  v = dpp_max_step<0x143, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_min_f32(float v) {
  v = dpp_min_step<0x111, 0xf>(v);
  v = dpp_min_step<0x112, 0xf>(v);
  v = dpp_min_step<0x114, 0xf>(v);
  v = dpp_min_step<0x118, 0xf>(v);
  v = dpp_min_step<0x142, 0xa>(v);
  v = dpp_min_step<0x143, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Threshold search of the merge (the result as row_refine's).  The lists hold
// only the slices' top scores, which the fixed top 11 key bits would put in a
// handful of bins, so that the LDS atomics of a wave hit one address; the
// first digit here is (key >> s) - (kmin >> s) instead, for the least s that
// keeps the valid keys' span [kmin, kmax] within 2048 bins, so the bins
// follow the scores' own spread.  Bins are aligned to 2^s in key space, so
// each is a (prefix, shift) range of the key bits and the later digits are
// the next bits below it (at most 11 per pass).
template <int EPT>
__device__ __forceinline__ void merge_select(const float (&v)[EPT], float hi, float lo,
                                             uint32_t* hist, uint32_t* sh, uint32_t* wtot,
                                             uint32_t kout, uint32_t& prefix, int& shift,
                                             uint32_t& need, uint32_t& bin_count) {
  const int tid = threadIdx.x;
  const uint32_t kmax = score_key(hi), kmin = score_key(lo);
  int s = 0;
  while ((kmax >> s) - (kmin >> s) >= 2048u) ++s;  // s <= 21
  const uint32_t kb = kmin >> s;
  // (hist was cleared before the barrier that published the range)
  uint32_t one = 1u;  // the count in one register, not rebuilt per element
  asm volatile("" : "+v"(one));
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (v[e] == v[e]) atomicAdd(&hist[(score_key(v[e]) >> s) - kb], one);
  __syncthreads();
  uint32_t bin, krem, bcnt;
  select_bin_r<kMergeNT, 2048>(hist, kout, 0xffffffffu, 0u, sh, wtot, bin, krem, bcnt);
  prefix = kb + bin;
  shift = s;
  while (bcnt != krem && shift > 0) {  // uniform
    const int nshift = shift > 11 ? shift - 11 : 0;
    const uint32_t nbm = (1u << (shift - nshift)) - 1u;
    const uint32_t lo_key = prefix << shift;
    // the digits of a negative score are the complement of its bits
    const uint32_t flip = (lo_key & 0x80000000u) ? 0u : nbm;
    for (int i = tid; i < 2048; i += kMergeNT) hist[i] = 0u;
    __syncthreads();
    const KeyRange in(lo_key, lo_key | ((1u << shift) - 1u));
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const bool ge = v[e] >= in.f_lo, le = v[e] <= in.f_hi;
      if (ge & le) atomicAdd(&hist[(__float_as_uint(v[e]) >> nshift) & nbm], one);
    }
    __syncthreads();
    uint32_t k2;
    select_bin_r<kMergeNT, 2048>(hist, krem, 0xffffffffu, 0u, sh, wtot, bin, k2, bcnt, flip);
    prefix = (prefix << (shift - nshift)) | bin;
    shift = nshift;
    krem = k2;
  }
  need = krem;
  bin_count = bcnt;
}

template <int EPT>
__global__ __launch_bounds__(kMergeNT) void topk_merge_kernel(
    const int32_t* __restrict__ pos, const float* __restrict__ score, int G, int n,
    int64_t list_stride, int64_t ld, const int32_t* __restrict__ cl_arr, int T, int kout,
    int32_t offset, int32_t* __restrict__ out, int64_t ld_out) {
  extern __shared__ uint32_t dyn_lds[];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t mbuf[kMergeNT * EPT / 16];
  __shared__ uint32_t wtot[3 * (kMergeNT / 64)];
  __shared__ uint32_t sh[4];
  constexpr int NW = kMergeNT / 64;
  lds_i32* posl = (lds_i32*)dyn_lds;
  const int r = blockIdx.x, tid = threadIdx.x;
  int32_t* orow = out + (int64_t)r * ld_out;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  if (c <= kout) {  // the closed form, whatever the scores
    row_keep_prefix<kMergeNT>(c, kout, offset, orow);
    return;
  }
  const int N = G * n;  // 0 when the lists are empty (n == 0)
  const int wbase = row_base<EPT>();
  // Every pair is requested before any is used, with no branch between the
  // loads (a branch per element would make each load wait for the one
  // before): a slot past the list end re-reads the last pair, and is
  // dropped below.
  int pp[EPT];
  float ss[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    pp[e] = -1;
    ss[e] = 0.0f;
  }
  if (N > 0) {
    const int64_t rbase = (int64_t)r * ld;
    const int64_t o_last = (int64_t)(G - 1) * list_stride + rbase + (n - 1);
    if (n >= 64) {
      // slot wbase + 64e as (list g, entry j): one division, then steps of
      // 64 that wrap at most once
      int g = wbase / n, j = wbase - g * n;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int64_t o = wbase + 64 * e < N ? (int64_t)g * list_stride + rbase + j : o_last;
        pp[e] = pos[o];
        ss[e] = score[o];
        j += 64;
        const bool wrap = j >= n;
        j = wrap ? j - n : j;
        g += wrap ? 1 : 0;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int sl = wbase + 64 * e < N ? wbase + 64 * e : N - 1;
        const int g = sl / n, j = sl - g * n;
        const int64_t o = (int64_t)g * list_stride + rbase + j;
        pp[e] = pos[o];
        ss[e] = score[o];
      }
    }
  }
  float v[EPT];
  uint32_t nvalid = 0;
  float hi = -__builtin_inff(), lo = __builtin_inff();  // the valid scores' range
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int s = wbase + 64 * e;
    const int p = s < N ? pp[e] : -1;
    v[e] = p >= 0 ? ss[e] : __builtin_nanf("");
    nvalid += p >= 0 ? 1u : 0u;
    hi = fmaxf(hi, v[e]);
    lo = fminf(lo, v[e]);
    if (s < N) posl[s] = p;
  }
  // the valid count and the range over the block in one exchange; the same
  // barrier publishes posl and the cleared histogram
  {
    const int lane = tid & 63, w = tid >> 6;
    const uint32_t vw = wave_sum(nvalid);
    const float hw = wave_max_f32(hi), lw = wave_min_f32(lo);
    float* wf = reinterpret_cast<float*>(wtot);
    if (lane == 0) {
      wtot[w] = vw;
      wf[NW + w] = hw;
      wf[2 * NW + w] = lw;
    }
    for (int i = tid; i < 2048; i += kMergeNT) hist[i] = 0u;
    __syncthreads();
    nvalid = wave_sum(lane < NW ? wtot[lane] : 0u);
    hi = wave_max_f32(lane < NW ? wf[NW + lane] : -__builtin_inff());
    lo = wave_min_f32(lane < NW ? wf[2 * NW + lane] : __builtin_inff());
    __syncthreads();  // wtot is the scans' again
  }
  const uint32_t V = nvalid;
  int32_t* stage = kout <= 2048 ? reinterpret_cast<int32_t*>(hist) : nullptr;
  uint32_t prefix, need, bcnt;
  int shift;
  if (V >= (uint32_t)kout) {
    merge_select<EPT>(v, hi, lo, hist, sh, wtot, (uint32_t)kout, prefix, shift, need, bcnt);
  } else {
    // fewer valid pairs than k_out (lists that are not the slices' top-k
    // lists): every valid pair is taken, the rest of the row is -1
    if (stage)
      for (int i = tid; i < kout; i += kMergeNT) stage[i] = -1;
    else
      for (int i = tid; i < kout; i += kMergeNT) orow[i] = -1;
    __syncthreads();
    prefix = kKeyNegInf;  // taken: every score >= -inf, i.e. every valid pair
    shift = 0;
    need = 0;
    bcnt = 0;
  }
  // every listed position lies below compress_lens, so each taken slot is
  // written as its position + offset
  row_emit<kMergeNT, EPT>(v, prefix, shift, need, bcnt, c, kout, offset, wbase, mbuf, stage,
                          wtot, orow, ListPos{posl});
}

}  // namespace idx

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t merge_lds(int N) { return (size_t)N * 4u; }

// The merge kernels use more than 64 KB of dynamic LDS for the longest
// lists; the limit is a per-device function attribute, raised once on each
// device the library runs on.
bool set_merge_lds_limit() {
  static std::atomic<uint64_t> done_mask{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done_mask.load(std::memory_order_acquire) & bit)) return true;
  const int lim = (int)merge_lds(idx::kMergeMaxN);
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&idx::topk_merge_kernel<8>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lim) != hipSuccess ||
      hipFuncSetAttribute(reinterpret_cast<const void*>(&idx::topk_merge_kernel<16>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lim) != hipSuccess ||
      hipFuncSetAttribute(reinterpret_cast<const void*>(&idx::topk_merge_kernel<32>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lim) != hipSuccess)
    return false;
  if (bit) done_mask.fetch_or(bit, std::memory_order_acq_rel);
  return true;
}

}  // namespace

extern "C" size_t idx_topk_pairs_workspace_size(int R, int T_slice, int index_topk) {
  if (R <= 0 || T_slice <= 0 || index_topk <= 0) return 0;
  return align256((size_t)R * 4u) + idx_topk_workspace_size(R, T_slice, index_topk);
}

extern "C" idx_status idx_topk_pairs(const float* scores, int64_t ld, int R, int T_slice,
                                     int slice_start, const int32_t* compress_lens,
                                     uint32_t* key_hist, int index_topk, int32_t* pos_out,
                                     float* score_out, int64_t ld_out, int32_t* k_out, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (R < 0 || T_slice < 0 || slice_start < 0 || index_topk <= 0) return IDX_EINVAL;
  if ((int64_t)slice_start + T_slice > (int64_t)INT32_MAX) return IDX_EINVAL;
  const int kout = index_topk < T_slice ? index_topk : T_slice;
  if (R == 0 || T_slice == 0) {
    if (k_out) *k_out = kout;
    return IDX_OK;
  }
  if (!scores || !compress_lens || !pos_out || !score_out || !ws) return IDX_EINVAL;
  if (ld < T_slice || ld_out < kout) return IDX_EINVAL;
  if (ws_bytes < idx_topk_pairs_workspace_size(R, T_slice, index_topk)) return IDX_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  int32_t* lens = (int32_t*)ws;
  const size_t lens_bytes = align256((size_t)R * 4u);
  hipLaunchKernelGGL(idx::slice_lens_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, st,
                     compress_lens, R, slice_start, T_slice, lens);
  idx_status s = idx_host::launch_status();
  if (s != IDX_OK) return s;
  void* tws = (char*)ws + lens_bytes;
  s = idx_topk(scores, ld, R, T_slice, lens, key_hist, index_topk, slice_start, pos_out, ld_out,
               nullptr, tws, ws_bytes - lens_bytes, stream);
  if (s != IDX_OK) return s;
  const int64_t n = (int64_t)R * kout;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(idx::pair_scores_kernel, dim3((unsigned)blocks), dim3(256), 0, st, scores,
                     ld, R, kout, slice_start, pos_out, ld_out, score_out);
  s = idx_host::launch_status();
  if (s == IDX_OK && k_out) *k_out = kout;
  return s;
}

extern "C" idx_status idx_merge_topk(const int32_t* pos, const float* score, int G, int n,
                                     int64_t list_stride, int64_t ld, int R,
                                     const int32_t* compress_lens, int T, int index_topk,
                                     int32_t offset, int32_t* out, int64_t ld_out,
                                     int32_t* k_out, void* stream) {
  if (R < 0 || T < 0 || G < 1 || n < 0 || index_topk <= 0) return IDX_EINVAL;
  const int kout = index_topk < T ? index_topk : T;
  if ((int64_t)G * n > idx::kMergeMaxN) return IDX_EUNSUPPORTED;
  if (R == 0 || T == 0) {
    if (k_out) *k_out = kout;
    return IDX_OK;
  }
  const int N = G * n;
  if (!compress_lens || !out) return IDX_EINVAL;
  if (N > 0 && (!pos || !score)) return IDX_EINVAL;
  if (ld_out < kout || ld < n) return IDX_EINVAL;
  // the G lists of a row must not overlap: list g of row r at
  // g*list_stride + r*ld, entries [0, n)
  if (G > 1 && list_stride < (int64_t)(R - 1) * ld + n) return IDX_EINVAL;
  if (!set_merge_lds_limit()) return IDX_EHIP;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)R), blk(idx::kMergeNT);
  const size_t lds = merge_lds(N > 0 ? N : 1);
  // empty lists still launch: rows with compress_lens > k_out are then all -1
  if (N <= idx::kMergeNT * 8)
    hipLaunchKernelGGL(idx::topk_merge_kernel<8>, grid, blk, lds, st, pos, score, G, n,
                       list_stride, ld, compress_lens, T, kout, offset, out, ld_out);
  else if (N <= idx::kMergeNT * 16)
    hipLaunchKernelGGL(idx::topk_merge_kernel<16>, grid, blk, lds, st, pos, score, G, n,
                       list_stride, ld, compress_lens, T, kout, offset, out, ld_out);
  else
    hipLaunchKernelGGL(idx::topk_merge_kernel<32>, grid, blk, lds, st, pos, score, G, n,
                       list_stride, ld, compress_lens, T, kout, offset, out, ld_out);
  const idx_status s = idx_host::launch_status();
  if (s == IDX_OK && k_out) *k_out = kout;
  return s;
}
