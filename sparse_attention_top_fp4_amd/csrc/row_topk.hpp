// row_topk.hpp -- one workgroup ranks one row whose scores sit in
// registers: the threshold search of the Indexer's top-k and the
// position-ordered output ([IDX, forward]: keep min(index_topk, T) positions
// by score, re-sort them by position, t + offset where t < compress_lens and
// -1 otherwise; ties go to the lower position).
//
// Layout: element e of lane l of wave w is position w*64*EPT + 64e + l
// (row_base), so every load instruction reads 64 consecutive words and the
// ballot of element e is the bit map of 64 consecutive positions.
//
// Search: radix select on the order keys in digits of 11, 11 and 10 bits.
// The first digit's histogram comes from the score kernel or is counted
// here; each later pass histograms in LDS the next digit of the scores whose
// higher digits equal the threshold prefix found so far, and the search stops
// as soon as every element of the prefix bin is taken.
//
// Output: the waves' ballots of the taken scores (and of the tied ones, when
// only some are taken) are written to LDS as position-ordered bit-map words;
// one thread per 32-position word then takes its first slot from a block scan
// of the word counts and writes its positions in order.
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

// A workgroup barrier for LDS traffic only: each wave waits for its own LDS
// operations, not for its global loads in flight (which the fence of
// __syncthreads drains as well).  For code in which no thread reads global
// memory another thread of the workgroup wrote.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <bool LDS_ONLY>
__device__ __forceinline__ void block_barrier() {
  if constexpr (LDS_ONLY)
    lds_barrier();
  else
    __syncthreads();
}

template <int NT, bool LDS_ONLY = false>
__device__ __forceinline__ uint32_t block_inclusive_sum(uint32_t v, uint32_t* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_sum(v);
  if (lane == 63) wtot[w] = x;
  block_barrier<LDS_ONLY>();
  const uint32_t add = waves_below<NT>(wtot, w);
  block_barrier<LDS_ONLY>();
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

// Threshold bin of NB bin counts held in registers, thread i owning the
// bins [NB - (i+1)*BPT, NB - i*BPT), the top bins first (cnt[j]: bin
// NB - 1 - i*BPT - j): the bin b with count(bins > b) < krem <=
// count(bins >= b).  Also returns the count of bin b and, when total is
// given, the sum of all the counts (the same in every thread).
template <int NT, int NB, bool LDS_ONLY = false>
__device__ __forceinline__ void select_bin_regs(const uint32_t (&cnt)[NB / NT], uint32_t krem,
                                                uint32_t* sh, uint32_t* wtot, uint32_t& bin,
                                                uint32_t& krem_out, uint32_t& bin_count,
                                                uint32_t* total = nullptr) {
  constexpr int BPT = NB / NT;
  static_assert(BPT * NT == NB && BPT >= 1, "whole bins per thread");
  const int hi = NB - (int)threadIdx.x * BPT;  // my bins are [hi - BPT, hi)
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) mine += cnt[j];
  const uint32_t incl = block_inclusive_sum<NT, LDS_ONLY>(mine, wtot);
  // the wave totals stay in wtot until the next scan, past a barrier below
  if (total) *total = waves_total<NT>(wtot);
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
  block_barrier<LDS_ONLY>();
  bin = sh[0];
  krem_out = sh[1];
  bin_count = sh[2];
  block_barrier<LDS_ONLY>();
}

// The same from an LDS histogram, where bin `xbin` counts `xcnt` more and
// bin b is stored at hist[b ^ flip].
template <int NT, int NB, bool LDS_ONLY = false>
__device__ __forceinline__ void select_bin_r(const uint32_t* hist, uint32_t krem, uint32_t xbin,
                                             uint32_t xcnt, uint32_t* sh, uint32_t* wtot,
                                             uint32_t& bin, uint32_t& krem_out,
                                             uint32_t& bin_count, uint32_t flip = 0u) {
  constexpr int BPT = NB / NT;
  const int hi = NB - (int)threadIdx.x * BPT;
  uint32_t cnt[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int b = hi - 1 - j;
    cnt[j] = hist[(uint32_t)b ^ flip] + ((uint32_t)b == xbin ? xcnt : 0u);
  }
  select_bin_regs<NT, NB, LDS_ONLY>(cnt, krem, sh, wtot, bin, krem_out, bin_count);
}

// Row layout: element e of lane l of wave w is position w*64*EPT + 64e + l,
// so each element's loads are 64 consecutive words and each element's
// ballot is a position-ordered 64-bit word of the row's bit map.  Returns
// the position of element 0.
template <int EPT>
__device__ __forceinline__ int row_base() {
  return (int)(threadIdx.x >> 6) * 64 * EPT + (int)(threadIdx.x & 63);
}

// A row with compress_lens c <= kout: every position below c ranks above
// every masked one, so the row keeps [0, c) and then the lowest masked
// positions, whatever the scores.
template <int NT>
__device__ __forceinline__ void row_keep_prefix(int c, int kout, int32_t offset,
                                                int32_t* __restrict__ orow) {
  for (int i = threadIdx.x; i < kout; i += NT) orow[i] = i < c ? i + offset : -1;
}

// ------------------------------------------------ keys as float ranges
// The search runs on order keys (score_key), but the scores stay floats in
// registers: a range of keys is the range of floats with those keys, so one
// float compare tests "key > cut" and two test "key in [lo, hi]", and the
// next digit of a key is read from the float's bits (within one first-digit
// bin every float has the same sign; -0 falls in the bin of +0 and has the
// same digits as +0).  Absent positions hold NaN, which no compare admits.
constexpr uint32_t kKeyPosInf = 0xFF800000u;  // order key of +inf

// Float whose key is k, for keys of non-NaN floats.
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Least float whose key is >= k (k <= kKeyPosInf): -inf below the key of
// -inf; +0 for the key 0x7fffffff, which no float has (-0 takes +0's key).
__device__ __forceinline__ float key_floor_float(uint32_t k) {
  if (k <= kKeyNegInf) return -__builtin_inff();
  return key_to_float(k == 0x7fffffffu ? 0x80000000u : k);
}

// Greatest float whose key is <= k (k >= kKeyNegInf).
__device__ __forceinline__ float key_ceil_float(uint32_t k) {
  if (k >= kKeyPosInf) return __builtin_inff();
  return key_to_float(k == 0x7fffffffu ? 0x7ffffffeu : k);
}

// Floats whose keys lie in [lo, hi]: x >= f_lo && x <= f_hi.
struct KeyRange {
  float f_lo, f_hi;
  __device__ __forceinline__ KeyRange(uint32_t lo, uint32_t hi) {
    if (hi < kKeyNegInf || lo > kKeyPosInf) {  // only NaN keys: empty
      f_lo = __builtin_inff();
      f_hi = -__builtin_inff();
    } else {
      f_lo = key_floor_float(lo);
      f_hi = key_ceil_float(hi);
    }
  }
  __device__ __forceinline__ bool has(float x) const { return x >= f_lo && x <= f_hi; }
};

// x >= key_above(cut)  <=>  key(x) > cut, for non-NaN x (NaN: never).
__device__ __forceinline__ float key_above(uint32_t cut) {
  if (cut >= kKeyPosInf) return __builtin_nanf("");
  return key_floor_float(cut + 1u);
}

// Scores of the positions: position >= T -> NaN (absent), position >= c ->
// -inf (c <= T).  A wave whose positions all lie below c keeps them as they
// are.  Otherwise element e (position wbase + 64e) is tested as 64e < c - wbase
// and 64e < T - wbase: two compares against constants and two selects.  The
// bounds take an empty asm that reads the last element, so the compares
// cannot be hoisted above the loads (a hoisted mask would hold two scalar
// registers per element).
template <int EPT>
__device__ __forceinline__ void row_vals(float (&v)[EPT], int wbase, int c, int T) {
  const int wend = (__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) + 1) * 64 * EPT;
  if (wend <= c) return;
  int rc = c - wbase, rt = T - wbase;
  asm volatile("" : "+v"(rc), "+v"(rt) : "v"(v[EPT - 1]));
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    v[e] = 64 * e < rt ? (64 * e < rc ? v[e] : -__builtin_inff()) : __builtin_nanf("");
}

// The remaining digits of the threshold search, among the scores whose
// first digit is b1 (krem of them still to take, bcnt in that bin):
// histograms in LDS of the next digit of the scores matching the prefix so
// far, stopping as soon as every element of the prefix bin is taken.  The
// -inf bin holds only -inf scores (all equal), so it needs no further digit.
// hist: 2048 words of LDS, already zero when hist_zeroed.  Result: the keys
// whose bits [shift, 32) exceed `prefix` are taken, and of those equal to
// it (bin_count keys) the `need` lowest positions.
template <int NT, int EPT>
__device__ __forceinline__ void row_refine(const float (&v)[EPT], uint32_t* hist,
                                           bool hist_zeroed, uint32_t* sh, uint32_t* wtot,
                                           uint32_t b1, uint32_t krem, uint32_t bcnt,
                                           uint32_t& prefix, int& shift, uint32_t& need,
                                           uint32_t& bin_count) {
  const int tid = threadIdx.x;
  prefix = b1;
  shift = 21;  // the prefix holds the key bits [shift, 32)
  // the digits of a negative score are the complement of its bits
  const uint32_t neg = (b1 & 0x400u) ? 0u : 0xffffffffu;
  bool done = b1 == kInfBin || bcnt == krem;
#pragma unroll
  for (int pass = 1; pass < 3; ++pass) {
    if (done) break;
    constexpr int kNb2 = 2048, kNb3 = 1024;
    const int nshift = pass == 1 ? 10 : 0;
    const uint32_t nbm = pass == 1 ? (uint32_t)kNb2 - 1u : (uint32_t)kNb3 - 1u;
    if (pass > 1 || !hist_zeroed) {
      for (int i = tid; i <= (int)nbm; i += NT) hist[i] = 0u;
      __syncthreads();
    }
    // counted by the digit of the bits (the key digit of a negative score is
    // its complement, applied when the bins are read)
    const KeyRange in(prefix << shift, (prefix << shift) | ((1u << shift) - 1u));
    // the count is a register the compiler cannot rebuild per element
    uint32_t one = 1u;
    asm volatile("" : "+v"(one));
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      // the two compares' masks ANDed as scalars give the lanes that count
      // (a wave-level test to skip empty elements cost more scalar issue
      // than the two vector instructions it saves)
      const bool ge = v[e] >= in.f_lo, le = v[e] <= in.f_hi;
      if (ge & le) atomicAdd(&hist[(__float_as_uint(v[e]) >> nshift) & nbm], one);
    }
    __syncthreads();
    uint32_t bin, k2;
    if (pass == 1)
      select_bin_r<NT, kNb2>(hist, krem, 0xffffffffu, 0u, sh, wtot, bin, k2, bcnt, neg & nbm);
    else
      select_bin_r<NT, kNb3>(hist, krem, 0xffffffffu, 0u, sh, wtot, bin, k2, bcnt, neg & nbm);
    prefix = (prefix << (shift - nshift)) | bin;
    shift = nshift;
    krem = k2;
    done = bcnt == k2;
  }
  need = krem;
  bin_count = bcnt;
}

// Threshold search.  hist: LDS, 2048 words.  counted == 0xffffffff: the
// first digit is counted here (hist is scratch); otherwise hist already
// holds the first-digit counts of the row's finite positions, `counted` of
// them, and the other T - counted positions are -inf.  Result as row_refine.
template <int NT, int EPT>
__device__ __forceinline__ void row_select(const float (&v)[EPT], uint32_t* hist,
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
    uint32_t ninf = 0;  // -inf scores are counted per thread, not by atomics
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const float x = v[e];
      if (x > -__builtin_inff()) atomicAdd(&hist[score_key(x) >> 21], 1u);  // not NaN, not -inf
      ninf += x == -__builtin_inff() ? 1u : 0u;
    }
    ninf = wave_sum(ninf);
    if (lane == 0 && ninf) atomicAdd(&sh[3], ninf);
    __syncthreads();
    select_bin_r<NT, 2048>(hist, (uint32_t)kout, kInfBin, sh[3], sh, wtot, b1, krem, bcnt);
  }
  row_refine<NT, EPT>(v, hist, false, sh, wtot, b1, krem, bcnt, prefix, shift, need, bin_count);
}

// Identity map from a row's slot to its position.
struct SamePos {
  __device__ __forceinline__ int operator()(int v) const { return v; }
};

// Position-ordered output of the selection.  Keys above the prefix range
// [lo, lo + span] are taken, and of the keys inside it the `need` at the
// lowest positions (all of them when that is every tied key).
//
// Each wave ballots the taken scores (and, when only some tied scores are
// taken, the tied ones): the ballot of element e is the bit map of the
// positions w*64*EPT + 64e + [0, 64).  The maps go to LDS (mbuf: NT*EPT/16
// words); then thread g takes the word of positions [32g, 32g + 32), the
// block scans the word counts, and the thread writes its positions in order.
// stage: LDS of at least kout words to assemble the row in (it is then
// written out in one coalesced pass; its contents may be the search
// histogram, which is no longer needed), or null to write directly.  pos:
// maps a slot of the ranked row to its position (increasing), which is
// written as pos + offset below c and as -1 otherwise.
template <int NT, int EPT, class Pos = SamePos>
__device__ __forceinline__ void row_emit(const float (&v)[EPT], uint32_t prefix, int shift,
                                         uint32_t need, uint32_t bin_count, int c, int kout,
                                         int32_t offset, int wbase, uint32_t* mbuf,
                                         int32_t* stage, uint32_t* wtot,
                                         int32_t* __restrict__ orow, Pos pos = Pos()) {
  constexpr int NMW = NT * EPT / 64;  // 64-bit masks per block
  static_assert(EPT <= 32 && NT * EPT < 65536, "shape (counts packed in 16 bits)");
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lo = prefix << shift;
  const uint32_t hi = lo | ((1u << shift) - 1u);
  const bool all_eq = need >= bin_count;  // every tied score is taken
  // taken: key > cut (every tied key too when all are taken)
  const float above = key_above(all_eq ? lo - 1u : hi);
  {
    uint32_t glo = 0, ghi = 0, qlo = 0, qhi = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint64_t m = __ballot(v[e] >= above);
      glo = (uint32_t)idx_writelane_i32((int)(uint32_t)m, e, (int)glo);
      ghi = (uint32_t)idx_writelane_i32((int)(uint32_t)(m >> 32), e, (int)ghi);
    }
    if (!all_eq) {
      const KeyRange tied(lo, hi);
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        // the two compares' masks ANDed as scalars (a ballot of their
        // conjunction costs a select and a third compare)
        const uint64_t m = __ballot(v[e] >= tied.f_lo) & __ballot(v[e] <= tied.f_hi);
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
  // thread g: the 32 positions [32g, 32g + 32)
  constexpr int NG = NT * EPT / 32;
  uint32_t gw = 0, qw = 0;
  if (NG >= NT || tid < NG) {
    gw = mbuf[tid];
    if (!all_eq) qw = mbuf[2 * NMW + tid];
  }
  // both counts in one scan: taken in the low 16 bits, tied in the high
  // (a block holds fewer than 65536 positions)
  const uint32_t gq = (uint32_t)__popc(gw) | ((uint32_t)__popc(qw) << 16);
  const uint32_t before = block_inclusive_sum<NT>(gq, wtot) - gq;
  const uint32_t gb = before & 0xffffu, qb = before >> 16;
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
  const int v0 = 32 * tid;  // position of bit 0
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
