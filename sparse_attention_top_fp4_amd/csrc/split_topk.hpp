// split_topk.hpp -- the top-k of long rows over several workgroups per row
// ([IDX, forward]: top min(index_topk, T) of a row's scores, in position
// order), given the score kernel's first-digit histogram of each row.
#pragma once

#include "row_topk.hpp"

namespace idx {

// Rows of 8193..262144 positions.  Kernel A: one workgroup of 512 threads per
// 8192-position part of a row writes the part's "above the threshold bin"
// bit mask and the (key, position) list of the elements inside the bin, one
// list per wave.  Kernel B: one workgroup of 1024 threads per row resolves
// the remaining digits on the collected list in LDS, marks the selected
// list elements into the masks and compacts the row in position order.
constexpr int kPartNW = 8, kPartEPT = 16, kPart = kPartNW * 64 * kPartEPT;  // 8192
constexpr int kSplitMaxT = 262144;
constexpr int kSplitCandCap = 8192;  // list elements resolved in LDS

// LDS index of mask word w (one pad word per 32) and the padded length.
__host__ __device__ __forceinline__ int split_pad(int w) { return w + (w >> 5); }
__host__ __device__ __forceinline__ int split_padded_words(int nw) { return nw + (nw >> 5) + 1; }

struct SplitLayout {  // per-row workspace, in 32-bit words
  int64_t nwords;     // T/32 rounded up: above-mask words
  int64_t nparts;
  int64_t cand_off, cnt_off, state_off, row_words;
  __host__ __device__ SplitLayout(int T) {
    nwords = ((int64_t)T + 31) / 32;
    nparts = ((int64_t)T + kPart - 1) / kPart;
    cand_off = (nwords + 1) & ~(int64_t)1;               // [nparts][8 waves][1024] (key, pos)
    cnt_off = cand_off + nparts * kPartNW * 1024 * 2;    // [nparts][8 waves]
    state_off = cnt_off + nparts * kPartNW;              // b1, krem, histogram total
    row_words = (state_off + 3 + 3) & ~(int64_t)3;       // rows 16-byte aligned, lists 8
  }
};

// Kernel A's work on part `part` of row r, for a workgroup of NT threads
// (NT / 64 waves; each wave takes the part's 8 wave ranges w, w + NT / 64,
// ..., so the lists are those of 8 waves whatever NT is).  Every range's
// scores are requested before the threshold search, so their latency
// overlaps it.  hist: 2048 words of LDS; wtot: NT / 64 words; sh: 4.
template <int NT>
__device__ __forceinline__ void split_a_part(int r, int part, const float* __restrict__ scores,
                                             int64_t ld, int T, const int32_t* __restrict__ cl_arr,
                                             const uint32_t* __restrict__ key_hist, int kout,
                                             uint32_t* __restrict__ ws, uint32_t* hist,
                                             uint32_t* wtot, uint32_t* sh) {
  constexpr int NW = NT / 64, VPW = kPartNW / NW, SEG = 64 * kPartEPT;
  static_assert(VPW * NW == kPartNW, "whole wave ranges per wave");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const SplitLayout L(T);
  uint32_t* wrow = ws + (int64_t)r * L.row_words;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  // every lane loads (past-the-end lanes re-read position T - 1)
  const float* srow = scores + (int64_t)r * ld;
  const unsigned last = (unsigned)(T - 1);
  float v[VPW][kPartEPT];
#pragma unroll
  for (int i = 0; i < VPW; ++i)
#pragma unroll
    for (int e = 0; e < kPartEPT; ++e) {
      const unsigned t = (unsigned)(part * kPart + (w + NW * i) * SEG + e * 64 + lane);
      v[i][e] = srow[t < last ? t : last];
    }
  uint32_t b1, krem, total;
  {
    constexpr int HPT = 2048 / NT;
    uint32_t hv[HPT], mine = 0;
#pragma unroll
    for (int j = 0; j < HPT; ++j) hv[j] = key_hist[(int64_t)r * 2048 + threadIdx.x + j * NT];
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
      hist[threadIdx.x + j * NT] = hv[j];
      mine += hv[j];
    }
    total = block_sum<NT>(mine, wtot);  // its barriers also publish hist
    uint32_t bc;
    // positions the histogram does not count are -inf
    select_bin_r<NT, 2048>(hist, (uint32_t)kout, kInfBin, (uint32_t)T - total, sh, wtot, b1, krem,
                           bc);
  }
  if (part == 0 && threadIdx.x == 0) {
    wrow[L.state_off] = b1;
    wrow[L.state_off + 1] = krem;
    wrow[L.state_off + 2] = total;  // kernel B checks it against compress_lens
  }
  const float lo = b1 <= kInfBin ? -__builtin_inff() : key_to_float(b1 << 21);
  const bool top = b1 >= 2044u;
  const float hi = top ? __builtin_inff() : key_to_float((b1 + 1u) << 21);
#pragma unroll
  for (int i = 0; i < VPW; ++i) {
    const int vw = w + NW * i;  // this range's list
    const int base = part * kPart + vw * SEG;
    uint2* cand = reinterpret_cast<uint2*>(wrow + L.cand_off +
                                           ((int64_t)part * kPartNW + vw) * 1024 * 2);
    uint32_t run = 0;
    uint32_t myword = 0;  // lane 2e / 2e+1 collects the low / high half of step e's mask
#pragma unroll
    for (int e = 0; e < kPartEPT; ++e) {
      const int t = base + e * 64 + lane;
      const float x = t < T ? (t < c ? v[i][e] : -__builtin_inff()) : __builtin_nanf("");
      const bool above = !top && x >= hi;
      const bool isc = x >= lo && (top || x < hi);
      const uint64_t am = __ballot(above);
      const uint64_t cm = __ballot(isc);
      myword = lane == 2 * e ? (uint32_t)am : (lane == 2 * e + 1 ? (uint32_t)(am >> 32) : myword);
      if (isc) cand[run + lanes_below(cm)] = make_uint2(score_key(x), (uint32_t)t);
      run += (uint32_t)__popcll(cm);
    }
    // the range's 32 mask words in one store
    const int64_t word = (base >> 5) + lane;
    if (lane < 2 * kPartEPT && word < L.nwords) wrow[word] = myword;
    if (lane == 0) wrow[L.cnt_off + (int64_t)part * kPartNW + vw] = run;
  }
}

}  // namespace idx
