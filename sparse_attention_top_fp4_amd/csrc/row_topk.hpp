// row_topk.hpp -- one workgroup ranks one row whose order keys sit in
// registers: the threshold search of the Indexer's top-k and the
// position-ordered output ([IDX, forward]: keep min(index_topk, T) positions
// by score, re-sort them by position, t + offset where t < compress_lens and
// -1 otherwise; ties go to the lower position).
//
// Layout: wave w owns the positions [w*64*EPT, (w+1)*64*EPT); in step i its
// lane l holds the four consecutive positions w*64*EPT + i*256 + 4l + [0, 4),
// key[4i + j] for position +j.  Loads of that layout are contiguous per wave.
//
// Search: radix select on the order keys in digits of 11, 11 and 10 bits.
// Each pass histograms in LDS the next digit of the keys whose higher digits
// equal the threshold prefix found so far (the first digit may come from the
// score kernel instead), and the search stops as soon as every element of
// the prefix bin is taken.  Output: per step, a wave scan of the selected
// counts gives every selected position its slot in position order.
#pragma once

#include "idx_common.hpp"

namespace idx {

constexpr uint32_t kInfBin = kKeyNegInf >> 21;  // first-digit bin of -inf

// An int32 in LDS, addressed as such (32-bit LDS addresses, ds_* access)
// rather than through a generic pointer.
typedef __attribute__((address_space(3))) int32_t lds_i32;

// Exclusive sum of the wave totals of the waves below this one, read back
// from LDS after the barrier: a short loop for a few waves, otherwise one
// word per lane and a wave sum.
template <int NT>
__device__ __forceinline__ uint32_t waves_below(const uint32_t* wtot, int w) {
  constexpr int NW = NT / 64;
  uint32_t add = 0;
  if constexpr (NW <= 4) {
#pragma unroll
    for (int i = 0; i < NW; ++i)
      if (i < w) add += wtot[i];
  } else {
    const int lane = threadIdx.x & 63;
    const uint32_t t = lane < NW ? wtot[lane] : 0u;
    add = wave_sum(lane < w ? t : 0u);
  }
  return add;
}

template <int NT>
__device__ __forceinline__ uint32_t waves_total(const uint32_t* wtot) {
  constexpr int NW = NT / 64;
  uint32_t s = 0;
  if constexpr (NW <= 4) {
#pragma unroll
    for (int i = 0; i < NW; ++i) s += wtot[i];
  } else {
    const int lane = threadIdx.x & 63;
    s = wave_sum(lane < NW ? wtot[lane] : 0u);
  }
  return s;
}

template <int NT>
__device__ __forceinline__ uint32_t block_inclusive_sum(uint32_t v, uint32_t* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_sum(v);
  if (lane == 63) wtot[w] = x;
  __syncthreads();
  const uint32_t add = waves_below<NT>(wtot, w);
  __syncthreads();
  return x + add;
}

// Two independent inclusive scans over the block in one exchange (wtot: 2*NT/64 words).
template <int NT>
__device__ __forceinline__ void block_inclusive_sum2(uint32_t& a, uint32_t& b, uint32_t* wtot) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  a = wave_inclusive_sum(a);
  b = wave_inclusive_sum(b);
  if (lane == 63) {
    wtot[w] = a;
    wtot[NW + w] = b;
  }
  __syncthreads();
  const uint32_t ad = waves_below<NT>(wtot, w), bd = waves_below<NT>(wtot + NW, w);
  __syncthreads();
  a += ad;
  b += bd;
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* wtot) {
  const uint32_t x = wave_sum(v);
  if ((threadIdx.x & 63) == 0) wtot[threadIdx.x >> 6] = x;
  __syncthreads();
  const uint32_t s = waves_total<NT>(wtot);
  __syncthreads();
  return s;
}

// Threshold bin of an LDS histogram of NB bins, bins read into registers at
// once (thread i owns the bins [NB - (i+1)*BPT, NB - i*BPT), the top bins
// first): the bin b with count(bins > b) < krem <= count(bins >= b), where
// bin `xbin` counts `xcnt` more.  Also returns the count of bin b.
template <int NT, int NB>
__device__ __forceinline__ void select_bin_r(const uint32_t* hist, uint32_t krem, uint32_t xbin,
                                             uint32_t xcnt, uint32_t* sh, uint32_t* wtot,
                                             uint32_t& bin, uint32_t& krem_out,
                                             uint32_t& bin_count) {
  constexpr int BPT = NB / NT;
  static_assert(BPT * NT == NB && BPT >= 1, "whole bins per thread");
  const int hi = NB - (int)threadIdx.x * BPT;  // my bins are [hi - BPT, hi)
  uint32_t cnt[BPT];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int b = hi - 1 - j;
    cnt[j] = hist[b] + ((uint32_t)b == xbin ? xcnt : 0u);
    mine += cnt[j];
  }
  const uint32_t incl = block_inclusive_sum<NT>(mine, wtot);
  uint32_t cum = incl - mine;
  if (cum < krem && krem <= incl) {
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (cum < krem && cum + cnt[j] >= krem) {
        sh[0] = (uint32_t)(hi - 1 - j);
        sh[1] = krem - cum;
        sh[2] = cnt[j];
      }
      cum += cnt[j];
    }
  }
  __syncthreads();
  bin = sh[0];
  krem_out = sh[1];
  bin_count = sh[2];
  __syncthreads();
}

// Position of (step 0, element 0) for this thread.
template <int EPT>
__device__ __forceinline__ int row_base() {
  return (int)(threadIdx.x >> 6) * 64 * EPT + 4 * (int)(threadIdx.x & 63);
}

// A row with compress_lens c <= kout: every position below c ranks above
// every masked one, so the row keeps [0, c) and then the lowest masked
// positions, whatever the scores.
template <int NT>
__device__ __forceinline__ void row_keep_prefix(int c, int kout, int32_t offset,
                                                int32_t* __restrict__ orow) {
  for (int i = threadIdx.x; i < kout; i += NT) orow[i] = i < c ? i + offset : -1;
}

// Order keys of the loaded values: position >= T -> 0 (absent, below every
// key), position >= c -> the key of -inf.  A wave whose positions all lie
// below c (c <= T) takes the plain keys.  Otherwise validity is integer
// arithmetic (sign bit of t - c) kept out of the compiler's reach: compare
// masks hoisted above the loads would hold two scalar registers per element.
template <int EPT>
__device__ __forceinline__ void row_keys(const float (&v)[EPT], int wbase, int c, int T,
                                         uint32_t (&key)[EPT]) {
  const int wend = (__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) + 1) * 64 * EPT;
  if (wend <= c) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) key[e] = score_key(v[e]);
    return;
  }
#pragma unroll
  for (int i = 0; i < EPT / 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = wbase + 256 * i + j;
      uint32_t below_c = (uint32_t)(t - c) >> 31, below_t = (uint32_t)(t - T) >> 31;
      asm volatile("" : "+v"(below_c), "+v"(below_t));
      const uint32_t m = kKeyNegInf & (0u - below_t);
      const uint32_t k = score_key(v[4 * i + j]);
      key[4 * i + j] = m ^ ((k ^ m) & (0u - below_c));
    }
}

// Threshold search.  hist: LDS, 2048 words.  counted == 0xffffffff: the
// first digit is counted here (hist is scratch); otherwise hist already
// holds the first-digit counts of the row's finite positions, `counted` of
// them, and the other T - counted positions are -inf.  Result: the keys
// whose bits [shift, 32) exceed `prefix` are taken, and of those equal to
// it (bin_count keys) the `need` lowest positions.
template <int NT, int EPT>
__device__ __forceinline__ void row_select(const uint32_t (&key)[EPT], uint32_t* hist,
                                           uint32_t counted, int T, int kout, uint32_t* sh,
                                           uint32_t* wtot, uint32_t& prefix, int& shift,
                                           uint32_t& need, uint32_t& bin_count) {
  static_assert(EPT % 4 == 0 && 2048 % NT == 0 && 1024 % NT == 0, "shape");
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t b1, krem, bcnt;
  if (counted != 0xffffffffu) {
    select_bin_r<NT, 2048>(hist, (uint32_t)kout, kInfBin, (uint32_t)T - counted, sh, wtot, b1,
                           krem, bcnt);
  } else {
    for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
    if (tid == 0) sh[3] = 0u;
    __syncthreads();
    uint32_t ninf = 0;  // -inf keys are counted per thread, not by atomics
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint32_t k = key[e];
      if (k != 0u && k != kKeyNegInf) atomicAdd(&hist[k >> 21], 1u);
      ninf += k == kKeyNegInf ? 1u : 0u;
    }
    ninf = wave_sum(ninf);
    if (lane == 0 && ninf) atomicAdd(&sh[3], ninf);
    __syncthreads();
    select_bin_r<NT, 2048>(hist, (uint32_t)kout, kInfBin, sh[3], sh, wtot, b1, krem, bcnt);
  }

  // remaining digits, among the keys of the threshold prefix
  prefix = b1;
  shift = 21;  // the prefix holds the key bits [shift, 32)
  // the -inf bin holds only -inf keys (all equal); otherwise stop as soon as
  // every element of the prefix bin is taken
  bool done = b1 == kInfBin || bcnt == krem;
#pragma unroll
  for (int pass = 1; pass < 3; ++pass) {
    if (done) break;
    constexpr int kNb2 = 2048, kNb3 = 1024;
    const int nshift = pass == 1 ? 10 : 0;
    const uint32_t nbm = pass == 1 ? (uint32_t)kNb2 - 1u : (uint32_t)kNb3 - 1u;
    for (int i = tid; i <= (int)nbm; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint32_t k = key[e];
      if ((k >> shift) == prefix) atomicAdd(&hist[(k >> nshift) & nbm], 1u);
    }
    __syncthreads();
    uint32_t bin, k2;
    if (pass == 1)
      select_bin_r<NT, kNb2>(hist, krem, 0xffffffffu, 0u, sh, wtot, bin, k2, bcnt);
    else
      select_bin_r<NT, kNb3>(hist, krem, 0xffffffffu, 0u, sh, wtot, bin, k2, bcnt);
    prefix = (prefix << (shift - nshift)) | bin;
    shift = nshift;
    krem = k2;
    done = bcnt == k2;
  }
  need = krem;
  bin_count = bcnt;
}

// Identity map from a row's slot to its position.
struct SamePos {
  __device__ __forceinline__ int operator()(int v) const { return v; }
};

// Bits 0..7 of b moved to bits 0, 4, ..., 28.
__device__ __forceinline__ uint32_t spread4(uint32_t b) {
  b = (b | (b << 12)) & 0x000F000Fu;
  b = (b | (b << 6)) & 0x03030303u;
  return (b | (b << 3)) & 0x11111111u;
}

// Position-ordered output of the selection.  Keys above the prefix range
// [lo, lo + span] are taken, and of the keys inside it the `need` at the
// lowest positions (all of them when that is every tied key).
//
// Each wave ballots the taken keys (and, when only some tied keys are taken,
// the tied ones): mask (i, j) of wave w has bit l for position
// w*64*EPT + 256i + 4l + j.  The masks go to LDS (mbuf: NT*EPT/16 words).
// Then thread g owns the 32 positions [32g, 32g + 32): it gathers byte
// (g % 8) of its step's four masks into one position-ordered word, the block
// scans the word counts, and the thread writes its positions in order.
// stage: LDS of at least kout words to assemble the row in (it is then
// written out in one coalesced pass; its contents may be the search
// histogram, which is no longer needed), or null to write directly.  pos:
// maps a slot of the ranked row to its position (increasing), which is
// written as pos + offset below c and as -1 otherwise.
template <int NT, int EPT, class Pos = SamePos>
__device__ __forceinline__ void row_emit(const uint32_t (&key)[EPT], uint32_t prefix, int shift,
                                         uint32_t need, uint32_t bin_count, int c, int kout,
                                         int32_t offset, int wbase, uint32_t* mbuf,
                                         int32_t* stage, uint32_t* wtot,
                                         int32_t* __restrict__ orow, Pos pos = Pos()) {
  constexpr int NV = EPT / 4, NMW = NT * EPT / 64;  // masks per block
  static_assert(EPT % 4 == 0 && EPT <= 32, "shape");
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lo = prefix << shift;
  const uint32_t span = (1u << shift) - 1u;
  const uint32_t hi = lo + span;
  const bool all_eq = need >= bin_count;  // every tied key is taken
  // taken: key > cut (every tied key too when all are taken)
  const uint32_t cut = all_eq ? lo - 1u : hi;
  {
    uint32_t glo = 0, ghi = 0, qlo = 0, qhi = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint64_t m = __ballot(key[e] > cut);
      glo = (uint32_t)idx_writelane_i32((int)(uint32_t)m, e, (int)glo);
      ghi = (uint32_t)idx_writelane_i32((int)(uint32_t)(m >> 32), e, (int)ghi);
    }
    if (!all_eq) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const uint64_t m = __ballot(key[e] - lo <= span);
        qlo = (uint32_t)idx_writelane_i32((int)(uint32_t)m, e, (int)qlo);
        qhi = (uint32_t)idx_writelane_i32((int)(uint32_t)(m >> 32), e, (int)qhi);
      }
    }
    if (lane < EPT) {
      reinterpret_cast<uint2*>(mbuf)[w * EPT + lane] = make_uint2(glo, ghi);
      reinterpret_cast<uint2*>(mbuf)[NMW + w * EPT + lane] = make_uint2(qlo, qhi);
    }
  }
  __syncthreads();
  // thread g: step (g / 8) of the block (wave-major), lanes 8(g % 8) .. + 8
  constexpr int NG = NT * EPT / 32;
  const bool has = NG >= NT || tid < NG;
  uint32_t gw = 0, qw = 0;
  const int gstep = tid >> 3, gbyte = tid & 7;
  if (has) {
    const uint8_t* mb = reinterpret_cast<const uint8_t*>(mbuf);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      gw |= spread4(mb[(gstep * 4 + j) * 8 + gbyte]) << j;
      if (!all_eq) qw |= spread4(mb[(NMW + gstep * 4 + j) * 8 + gbyte]) << j;
    }
  }
  uint32_t gc = (uint32_t)__popc(gw), qc = (uint32_t)__popc(qw);
  block_inclusive_sum2<NT>(gc, qc, wtot);
  // gc, qc: inclusive; before this word
  const uint32_t gb = gc - (uint32_t)__popc(gw), qb = qc - (uint32_t)__popc(qw);
  uint32_t sel = gw;
  if (!all_eq && qw) {  // the first `need` tied keys of the row, by position
    uint32_t take = need > qb ? need - qb : 0u, rest = qw;
    while (take && rest) {
      const uint32_t low = rest & (0u - rest);
      sel |= low;
      rest ^= low;
      --take;
    }
  }
  uint32_t slot = gb + (need < qb ? need : qb);
  // position of bit b: the step's base + 4 * (8 * gbyte + l) + j = base + 32 gbyte + b
  const int v0 = (gstep / NV) * 64 * EPT + (gstep % NV) * 256 + 32 * gbyte;
  auto out = [&](auto* dst) {
    while (sel) {
      const int b = __ffs(sel) - 1;
      sel &= sel - 1u;
      const int t = pos(v0 + b);
      if (slot < (uint32_t)kout) dst[slot] = t < c ? t + offset : -1;
      ++slot;
    }
  };
  if (stage) {
    lds_i32* st = (lds_i32*)stage;
    out(st);
    __syncthreads();
    for (int i = tid; i < kout; i += NT) orow[i] = st[i];
  } else {
    out(orow);
  }
}

}  // namespace idx
