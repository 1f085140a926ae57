// topk.hip -- per-row top-k in position order, and the level-one candidate
// block selection built on it.
//
// [IDX, forward]: keep min(index_topk, T) positions by score, re-sort them by
// position, emit t + offset where t < compress_lens and -1 otherwise.  Ties
// go to the lower position; positions t >= compress_lens count as -inf.
//
// Method: radix select on order-preserving 32-bit keys in three digit passes
// (bits 31..21, 20..10, 9..0) with LDS histograms, then a compaction in
// position order.  Each wave owns a contiguous run of positions and visits
// it in order (element e of lane l is position base + 64e + l), so a wave
// ballot plus mbcnt gives every selected element its output slot and the
// result comes out already sorted by position; the threshold ties are taken
// from the lowest positions by ranking equal keys the same way.
//
//  - single-workgroup path: one workgroup per row, the row held in
//    registers (up to 64*EPT*NW positions);
//  - multi-workgroup path for long rows: chunks of 4096 positions, the
//    three histograms and per-chunk counts in a device workspace, one launch
//    per pass (each workgroup re-derives the earlier thresholds from the
//    global histograms, so no launch depends on a single-workgroup step).
//
// Elements equal to -inf (masked positions) are counted with a wave ballot
// instead of an LDS atomic per element, so heavily masked rows do not
// serialise on one histogram bin.
#include "idx_common.hpp"

#include <stdlib.h>

namespace idx {

constexpr int kHist1 = 0, kHist2 = 2048, kHist3 = 4096, kCnt = 5120;  // workspace row layout (words)
constexpr int kChunkNW = 4, kChunkEPT = 16, kChunk = kChunkNW * 64 * kChunkEPT;  // 4096

__device__ __forceinline__ int pass_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ int pass_bins(int p) { return p == 2 ? 1024 : 2048; }
__device__ __forceinline__ int pass_match_shift(int p) { return p == 0 ? 32 : (p == 1 ? 21 : 10); }
__device__ __forceinline__ int pass_hist_offset(int p) { return p == 0 ? kHist1 : (p == 1 ? kHist2 : kHist3); }

template <int NT>
__device__ __forceinline__ uint32_t block_inclusive_sum(uint32_t v, uint32_t* wtot) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_sum(v);
  if (lane == 63) wtot[w] = x;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if (i < w) add += wtot[i];
  __syncthreads();
  return x + add;
}

// Threshold bin of a histogram (LDS or global): the bin b with
// count(bins > b) < krem <= count(bins >= b).  Returns b and the number of
// elements still to take inside bin b.  Every thread of the block calls it.
template <int NT>
__device__ __forceinline__ void select_bin(const uint32_t* hist, int nbins, uint32_t krem,
                                           uint32_t* sh, uint32_t* wtot, uint32_t& bin,
                                           uint32_t& krem_out) {
  const int tid = threadIdx.x;
  const int bpt = (nbins + NT - 1) / NT;
  const int hi = nbins - tid * bpt;  // my bins are [lo, hi), scanned from the top
  const int lo = hi - bpt < 0 ? 0 : hi - bpt;
  uint32_t mine = 0;
  for (int b = hi - 1; b >= lo; --b) mine += hist[b];
  const uint32_t incl = block_inclusive_sum<NT>(mine, wtot);
  const uint32_t excl = incl - mine;
  if (excl < krem && krem <= incl) {
    uint32_t cum = excl;
    for (int b = hi - 1; b >= lo; --b) {
      const uint32_t c = hist[b];
      if (cum + c >= krem) {
        sh[0] = (uint32_t)b;
        sh[1] = krem - cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  bin = sh[0];
  krem_out = sh[1];
  __syncthreads();
}

// Adds this block's elements to the LDS histogram of digit `pass`, among
// elements whose higher digits equal `prefix`.  Element e of a lane is
// present when 64e + lane < nvalid.  -inf elements are counted into
// *ninf_sh by ballot.
template <int EPT>
__device__ __forceinline__ void hist_pass(const uint32_t (&key)[EPT], int nvalid, int pass,
                                          uint32_t prefix, uint32_t* hist, uint32_t* ninf_sh) {
  const int lane = threadIdx.x & 63;
  const int shift = pass_shift(pass), ms = pass_match_shift(pass);
  const uint32_t mask = (uint32_t)pass_bins(pass) - 1u;
  uint32_t ninf = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint32_t k = key[e];
    const bool present = e * 64 + lane < nvalid;
    const bool match = present && (ms == 32 || (k >> ms) == prefix);
    const bool isinf = match && k == kKeyNegInf;
    if (match && !isinf) atomicAdd(&hist[(k >> shift) & mask], 1u);
    ninf += (uint32_t)__popcll(__ballot(isinf));
  }
  if (lane == 0 && ninf) atomicAdd(ninf_sh, ninf);
}

template <int EPT>
__device__ __forceinline__ void load_keys(const float* __restrict__ srow, int base, int T, int c,
                                          uint32_t (&key)[EPT]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int t = base + e * 64 + lane;
    key[e] = t < T ? (t < c ? score_key(srow[t]) : kKeyNegInf) : 0u;
  }
}

// Histogram one digit of the block's keys into LDS (ready after return).
template <int NT, int EPT>
__device__ __forceinline__ void block_hist(const uint32_t (&key)[EPT], int nvalid, int pass,
                                           uint32_t prefix, uint32_t* hist, uint32_t* ninf_sh) {
  const int nb = pass_bins(pass);
  for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0;
  if (threadIdx.x == 0) *ninf_sh = 0;
  __syncthreads();
  hist_pass<EPT>(key, nvalid, pass, prefix, hist, ninf_sh);
  __syncthreads();
  if (threadIdx.x == 0 && *ninf_sh) hist[(kKeyNegInf >> pass_shift(pass)) & (uint32_t)(nb - 1)] += *ninf_sh;
  __syncthreads();
}

__device__ __forceinline__ uint32_t extend_prefix(uint32_t prefix, int pass, uint32_t bin) {
  return pass == 0 ? bin : ((prefix << (pass == 1 ? 11 : 10)) | bin);
}

// Writes the selected elements of the block (keys > ustar, and keys ==
// ustar while their global equal-rank is below need) in position order.
// out_base / eq_base: selected and equal elements before this block.
template <int NW, int EPT>
__device__ __forceinline__ void block_emit(const uint32_t (&key)[EPT], int nvalid, int base,
                                           uint32_t ustar, uint32_t need, uint32_t out_base,
                                           uint32_t eq_base, int c, int32_t offset,
                                           int32_t* __restrict__ orow, uint32_t kout,
                                           uint32_t (*wcnt)[NW]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const bool present = e * 64 + lane < nvalid;
    gt += (uint32_t)__popcll(__ballot(present && key[e] > ustar));
    eq += (uint32_t)__popcll(__ballot(present && key[e] == ustar));
  }
  if (lane == 0) {
    wcnt[0][w] = gt;
    wcnt[1][w] = eq;
  }
  __syncthreads();
  uint32_t ob = out_base, eqb = eq_base;
  for (int i = 0; i < w; ++i) {
    const uint32_t ei = wcnt[1][i];
    const uint32_t take = need > eqb ? (ei < need - eqb ? ei : need - eqb) : 0u;
    ob += wcnt[0][i] + take;
    eqb += ei;
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const bool present = e * 64 + lane < nvalid;
    const bool g = present && key[e] > ustar;
    const bool q = present && key[e] == ustar;
    const uint64_t qm = __ballot(q);
    const uint32_t qrank = eqb + lanes_below(qm);
    const bool sel = g || (q && qrank < need);
    const uint64_t sm = __ballot(sel);
    const uint32_t slot = ob + lanes_below(sm);
    if (sel && slot < kout) {  // always true for a consistent selection; guards the row
      const int t = base + e * 64 + lane;
      orow[slot] = t < c ? t + offset : -1;
    }
    ob += (uint32_t)__popcll(sm);
    eqb += (uint32_t)__popcll(qm);
  }
}

// ------------------------------------------------ single-workgroup path
template <int NW, int EPT>
__global__ __launch_bounds__(NW * 64) void topk_row_kernel(const float* __restrict__ scores,
                                                           int64_t ld, int T,
                                                           const int32_t* __restrict__ cl_arr,
                                                           int kout, int32_t offset,
                                                           int32_t* __restrict__ out,
                                                           int64_t ld_out) {
  constexpr int NT = NW * 64, SEG = 64 * EPT;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wtot[NW];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t wcnt[2][NW];
  const int r = blockIdx.x, w = threadIdx.x >> 6;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  const int base = w * SEG;
  const int nvalid = T - base;
  uint32_t key[EPT];
  load_keys<EPT>(scores + (int64_t)r * ld, base, T, c, key);

  uint32_t prefix = 0, krem = (uint32_t)kout;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    block_hist<NT, EPT>(key, nvalid, pass, prefix, hist, &sh[2]);
    uint32_t bin, k2;
    select_bin<NT>(hist, pass_bins(pass), krem, sh, wtot, bin, k2);
    prefix = extend_prefix(prefix, pass, bin);
    krem = k2;
  }
  block_emit<NW, EPT>(key, nvalid, base, prefix, krem, 0u, 0u, c, offset,
                      out + (int64_t)r * ld_out, (uint32_t)kout, wcnt);
}

// ------------------------------------------------- multi-workgroup path
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// Re-derive the thresholds of passes [0, npass) from the global histograms.
template <int NT>
__device__ __forceinline__ void resolve_passes(const uint32_t* __restrict__ wrow, int npass,
                                               int kout, uint32_t* sh, uint32_t* wtot,
                                               uint32_t& prefix, uint32_t& krem) {
  prefix = 0;
  krem = (uint32_t)kout;
  for (int p = 0; p < npass; ++p) {
    uint32_t bin, k2;
    select_bin<NT>(wrow + pass_hist_offset(p), pass_bins(p), krem, sh, wtot, bin, k2);
    prefix = extend_prefix(prefix, p, bin);
    krem = k2;
  }
}

template <int PASS>
__global__ __launch_bounds__(kChunkNW * 64) void topk_chunk_hist_kernel(
    const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    int kout, uint32_t* __restrict__ ws, int64_t ws_row_words) {
  constexpr int NT = kChunkNW * 64, SEG = 64 * kChunkEPT;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wtot[kChunkNW];
  __shared__ uint32_t sh[4];
  const int r = blockIdx.y, w = threadIdx.x >> 6;
  uint32_t* wrow = ws + (int64_t)r * ws_row_words;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  uint32_t prefix, krem;
  resolve_passes<NT>(wrow, PASS, kout, sh, wtot, prefix, krem);
  const int base = blockIdx.x * kChunk + w * SEG;
  uint32_t key[kChunkEPT];
  load_keys<kChunkEPT>(scores + (int64_t)r * ld, base, T, c, key);
  block_hist<NT, kChunkEPT>(key, T - base, PASS, prefix, hist, &sh[2]);
  const int nb = pass_bins(PASS);
  for (int i = threadIdx.x; i < nb; i += NT)
    if (hist[i]) atomicAdd(&wrow[pass_hist_offset(PASS) + i], hist[i]);
}

// Per chunk: count of keys above the threshold and equal to it.
__global__ __launch_bounds__(kChunkNW * 64) void topk_chunk_count_kernel(
    const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    int kout, uint32_t* __restrict__ ws, int64_t ws_row_words) {
  constexpr int NT = kChunkNW * 64, SEG = 64 * kChunkEPT;
  __shared__ uint32_t wtot[kChunkNW];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t tot[2];
  const int r = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t* wrow = ws + (int64_t)r * ws_row_words;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  uint32_t ustar, need;
  resolve_passes<NT>(wrow, 3, kout, sh, wtot, ustar, need);
  const int base = blockIdx.x * kChunk + w * SEG;
  uint32_t key[kChunkEPT];
  load_keys<kChunkEPT>(scores + (int64_t)r * ld, base, T, c, key);
  if (threadIdx.x < 2) tot[threadIdx.x] = 0;
  __syncthreads();
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kChunkEPT; ++e) {
    const bool present = e * 64 + lane < T - base;
    gt += (uint32_t)__popcll(__ballot(present && key[e] > ustar));
    eq += (uint32_t)__popcll(__ballot(present && key[e] == ustar));
  }
  if (lane == 0) {
    atomicAdd(&tot[0], gt);
    atomicAdd(&tot[1], eq);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    wrow[kCnt + 2 * blockIdx.x] = tot[0];
    wrow[kCnt + 2 * blockIdx.x + 1] = tot[1];
  }
}

__global__ __launch_bounds__(kChunkNW * 64) void topk_chunk_emit_kernel(
    const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    int kout, int32_t offset, int32_t* __restrict__ out, int64_t ld_out,
    const uint32_t* __restrict__ ws, int64_t ws_row_words) {
  constexpr int NT = kChunkNW * 64, SEG = 64 * kChunkEPT;
  __shared__ uint32_t wtot[kChunkNW];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t wcnt[2][kChunkNW];
  __shared__ uint32_t bases[2];
  const int r = blockIdx.y, w = threadIdx.x >> 6;
  const uint32_t* wrow = ws + (int64_t)r * ws_row_words;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  uint32_t ustar, need;
  resolve_passes<NT>(wrow, 3, kout, sh, wtot, ustar, need);
  if (threadIdx.x == 0) {
    uint32_t ob = 0, eqb = 0;
    for (int i = 0; i < (int)blockIdx.x; ++i) {
      const uint32_t gi = wrow[kCnt + 2 * i], ei = wrow[kCnt + 2 * i + 1];
      const uint32_t take = need > eqb ? (ei < need - eqb ? ei : need - eqb) : 0u;
      ob += gi + take;
      eqb += ei;
    }
    bases[0] = ob;
    bases[1] = eqb;
  }
  const int base = blockIdx.x * kChunk + w * SEG;
  uint32_t key[kChunkEPT];
  load_keys<kChunkEPT>(scores + (int64_t)r * ld, base, T, c, key);
  __syncthreads();
  block_emit<kChunkNW, kChunkEPT>(key, T - base, base, ustar, need, bases[0], bases[1], c,
                                  offset, out + (int64_t)r * ld_out, (uint32_t)kout, wcnt);
}

// ----------------------------------------------------------- short rows
// index_topk >= T: every position is kept ([VLLM, _fill_short_context_topk_indices]
// closed form, plus the offset the Indexer adds).
__global__ __launch_bounds__(256) void topk_all_kernel(int T, const int32_t* __restrict__ cl_arr,
                                                       int32_t offset, int32_t* __restrict__ out,
                                                       int64_t ld_out) {
  const int r = blockIdx.x;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  for (int t = threadIdx.x; t < T; t += 256) out[(int64_t)r * ld_out + t] = t < c ? t + offset : -1;
}

// ------------------------------------------------------ candidate blocks
// Block score = maximum of the block's scores at positions < cl (-inf when
// none); also writes the per-row block count ceil(cl / cbs).
__global__ __launch_bounds__(256) void block_max_kernel(const float* __restrict__ scores, int64_t ld,
                                                        int T, const int32_t* __restrict__ cl_arr,
                                                        int cbs, int nb, float* __restrict__ bmax,
                                                        int32_t* __restrict__ clb) {
  const int r = blockIdx.y, lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  if (blockIdx.x == 0 && threadIdx.x == 0) clb[r] = (c + cbs - 1) / cbs;
  if (j >= nb) return;
  const float* srow = scores + (int64_t)r * ld;
  float m = -__builtin_inff();
  const int t1 = min((j + 1) * cbs, c);
  for (int t = j * cbs + lane; t < t1; t += 64) m = fmaxf(m, srow[t]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  if (lane == 0) bmax[(int64_t)r * nb + j] = m;
}

}  // namespace idx

// ------------------------------------------------------------ host side
namespace {

enum TopkPath { kAuto = 0, kSingle = 1, kChunked = 2 };

// IDX_TOPK_PATH=chunked forces the multi-workgroup path for rows longer
// than 1024 (read on every call; used by tests and tuning).
TopkPath topk_path_override() {
  const char* e = getenv("IDX_TOPK_PATH");
  return (e && e[0] == 'c') ? kChunked : kAuto;
}

int64_t n_chunks(int T) { return ((int64_t)T + idx::kChunk - 1) / idx::kChunk; }

int64_t ws_row_words(int T) { return idx::kCnt + 2 * n_chunks(T); }

size_t chunked_ws_bytes(int R, int T) { return (size_t)R * (size_t)ws_row_words(T) * 4u; }

bool needs_chunked(int R, int T) {
  const TopkPath o = topk_path_override();
  if (T > 32768) return true;
  if (o == kChunked && T > 1024) return true;
  (void)R;
  return false;
}

idx_status topk_launch(const float* scores, int64_t ld, int R, int T, const int32_t* cl, int k,
                       int32_t offset, int32_t* out, int64_t ld_out, void* ws, size_t ws_bytes,
                       hipStream_t st) {
  if (R == 0 || T == 0) return IDX_OK;
  const int kout = k < T ? k : T;
  if (k >= T) {
    hipLaunchKernelGGL(idx::topk_all_kernel, dim3((unsigned)R), dim3(256), 0, st, T, cl, offset,
                       out, ld_out);
    return idx_host::launch_status();
  }
  if (!needs_chunked(R, T)) {
    if (T <= 1024)
      hipLaunchKernelGGL((idx::topk_row_kernel<4, 4>), dim3((unsigned)R), dim3(256), 0, st, scores,
                         ld, T, cl, kout, offset, out, ld_out);
    else if (T <= 8192)
      hipLaunchKernelGGL((idx::topk_row_kernel<4, 32>), dim3((unsigned)R), dim3(256), 0, st,
                         scores, ld, T, cl, kout, offset, out, ld_out);
    else
      hipLaunchKernelGGL((idx::topk_row_kernel<16, 32>), dim3((unsigned)R), dim3(1024), 0, st,
                         scores, ld, T, cl, kout, offset, out, ld_out);
    return idx_host::launch_status();
  }
  if (R > 65535) return IDX_EUNSUPPORTED;
  const size_t need = chunked_ws_bytes(R, T);
  if (!ws || ws_bytes < need) return IDX_EINVAL;
  uint32_t* w = (uint32_t*)ws;
  const int64_t rw = ws_row_words(T);
  const int64_t zero_n = (int64_t)R * rw;
  const int64_t zg = (zero_n + 255) / 256 < 4096 ? (zero_n + 255) / 256 : 4096;
  hipLaunchKernelGGL(idx::zero_words_kernel, dim3((unsigned)zg), dim3(256), 0, st, w, zero_n);
  const dim3 grid((unsigned)n_chunks(T), (unsigned)R);
  const dim3 blk(idx::kChunkNW * 64);
  hipLaunchKernelGGL(idx::topk_chunk_hist_kernel<0>, grid, blk, 0, st, scores, ld, T, cl, kout, w,
                     rw);
  hipLaunchKernelGGL(idx::topk_chunk_hist_kernel<1>, grid, blk, 0, st, scores, ld, T, cl, kout, w,
                     rw);
  hipLaunchKernelGGL(idx::topk_chunk_hist_kernel<2>, grid, blk, 0, st, scores, ld, T, cl, kout, w,
                     rw);
  hipLaunchKernelGGL(idx::topk_chunk_count_kernel, grid, blk, 0, st, scores, ld, T, cl, kout, w,
                     rw);
  hipLaunchKernelGGL(idx::topk_chunk_emit_kernel, grid, blk, 0, st, scores, ld, T, cl, kout,
                     offset, out, ld_out, (const uint32_t*)w, rw);
  return idx_host::launch_status();
}

size_t topk_ws_bytes(int R, int T, int k) {
  if (R <= 0 || T <= 0 || k >= T || T <= 1024) return 0;
  return chunked_ws_bytes(R, T);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" size_t idx_topk_workspace_size(int R, int T, int index_topk) {
  return topk_ws_bytes(R, T, index_topk);
}

extern "C" idx_status idx_topk(const float* scores, int64_t ld, int R, int T,
                               const int32_t* compress_lens, int index_topk, int32_t offset,
                               int32_t* out, int64_t ld_out, void* ws, size_t ws_bytes,
                               void* stream) {
  if (R < 0 || T < 0 || index_topk <= 0) return IDX_EINVAL;
  if (R == 0 || T == 0) return IDX_OK;
  if (!scores || !compress_lens || !out) return IDX_EINVAL;
  const int kout = index_topk < T ? index_topk : T;
  if (ld < T || ld_out < kout) return IDX_EINVAL;
  return topk_launch(scores, ld, R, T, compress_lens, index_topk, offset, out, ld_out, ws, ws_bytes,
                     (hipStream_t)stream);
}

extern "C" size_t idx_select_workspace_size(int R, int T, int ctb, int cbs) {
  if (R <= 0 || T <= 0 || ctb <= 0 || cbs <= 0) return 0;
  const int nb = (int)(((int64_t)T + cbs - 1) / cbs);
  return align256((size_t)R * nb * 4u) + align256((size_t)R * 4u) + topk_ws_bytes(R, nb, ctb);
}

extern "C" idx_status idx_select_candidate_blocks(const float* scores, int64_t ld, int R, int T,
                                                  const int32_t* compress_lens,
                                                  int candidate_topk_blocks, int cand_block_size,
                                                  int32_t* block_ids, int64_t ld_ids, void* ws,
                                                  size_t ws_bytes, void* stream) {
  if (R < 0 || T < 0 || candidate_topk_blocks <= 0 || cand_block_size <= 0) return IDX_EINVAL;
  if (R == 0 || T == 0) return IDX_OK;
  if (!scores || !compress_lens || !block_ids) return IDX_EINVAL;
  const int nb = (int)(((int64_t)T + cand_block_size - 1) / cand_block_size);
  const int kk = candidate_topk_blocks < nb ? candidate_topk_blocks : nb;
  if (ld < T || ld_ids < kk) return IDX_EINVAL;
  if (R > 65535) return IDX_EUNSUPPORTED;
  const size_t need = idx_select_workspace_size(R, T, candidate_topk_blocks, cand_block_size);
  if (!ws || ws_bytes < need) return IDX_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  float* bmax = (float*)base;
  int32_t* clb = (int32_t*)(base + align256((size_t)R * nb * 4u));
  void* tws = base + align256((size_t)R * nb * 4u) + align256((size_t)R * 4u);
  const size_t tws_bytes = ws_bytes - align256((size_t)R * nb * 4u) - align256((size_t)R * 4u);
  hipLaunchKernelGGL(idx::block_max_kernel, dim3((unsigned)((nb + 3) / 4), (unsigned)R), dim3(256),
                     0, st, scores, ld, T, compress_lens, cand_block_size, nb, bmax, clb);
  const idx_status s = idx_host::launch_status();
  if (s != IDX_OK) return s;
  return topk_launch(bmax, nb, R, nb, clb, candidate_topk_blocks, 0, block_ids, ld_ids, tws,
                     tws_bytes, st);
}
