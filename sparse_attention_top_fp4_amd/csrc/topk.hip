// topk.hip -- per-row top-k in position order, and the level-one candidate
// block selection built on it.
//
// [IDX, forward]: keep min(index_topk, T) positions by score, re-sort them by
// position, emit t + offset where t < compress_lens and -1 otherwise.  Ties
// go to the lower position; positions t >= compress_lens count as -inf.
//
// Method: radix select on order-preserving 32-bit keys in three digit passes
// (bits 31..21, 20..10, 9..0), then a compaction in position order.
//
// The first digit's histogram usually comes from the score kernel, which
// counts the top 11 key bits of every score it writes (positions it did not
// score are -inf in the top-k's view, so their count is T minus the
// histogram's total).  Given that histogram:
//
//  - single-workgroup path (rows up to 32768): the row is loaded once into
//    registers and ranked there (row_topk.hpp): the remaining digits are LDS
//    histograms of the scores in the threshold's range, and the selection is
//    written as two position-ordered bit masks in LDS (keys above the
//    threshold; keys equal to it), which one thread per 32-position word
//    turns into output slots with one block scan, taking equal keys from the
//    lowest positions.  Comparisons after the threshold search are done on
//    the float scores (the threshold key maps back to a float; -0 equals +0
//    there as in the key order).
//  - split path (rows of 32769..262144 positions with a score histogram,
//    split_topk.hpp): kernel A, one workgroup per 8192-position part, writes
//    the part's above-the-bin mask and the list of its elements inside the
//    threshold bin; kernel B, one workgroup per row, resolves the remaining
//    digits on the gathered list and compacts the row.
//  - chunked path (longer rows, and rows past 32768 without a histogram):
//    chunks of 4096 positions over many workgroups; the remaining digit
//    histograms and per-chunk counts live in a device workspace, one launch
//    per step, and each workgroup re-derives the earlier thresholds from the
//    global histograms.
//
// Without a score histogram the first digit is histogrammed here as well.
// Elements equal to -inf (masked positions) are counted with a wave ballot
// instead of an LDS atomic per element.
#include "idx_common.hpp"
#include "row_topk.hpp"
#include "split_topk.hpp"

#include <stdlib.h>

#include <atomic>
#include <mutex>

namespace idx {

constexpr int kHist1 = 0, kHist2 = 2048, kHist3 = 4096, kCnt = 5120;  // workspace row layout (words)
constexpr int kChunkNW = 4, kChunkEPT = 16, kChunk = kChunkNW * 64 * kChunkEPT;  // 4096

__device__ __forceinline__ int pass_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ int pass_bins(int p) { return p == 2 ? 1024 : 2048; }
__device__ __forceinline__ int pass_match_shift(int p) { return p == 0 ? 32 : (p == 1 ? 21 : 10); }
__device__ __forceinline__ int pass_hist_offset(int p) { return p == 0 ? kHist1 : (p == 1 ? kHist2 : kHist3); }


// Threshold bin of a histogram (LDS or global): the bin b with
// count(bins > b) < krem <= count(bins >= b), where bin `xbin` counts
// `xcnt` more elements than the array says.  Returns b and the number of
// elements still to take inside bin b.  Every thread of the block calls it.
template <int NT>
__device__ __forceinline__ void select_bin(const uint32_t* hist, int nbins, uint32_t krem,
                                           uint32_t xbin, uint32_t xcnt, uint32_t* sh,
                                           uint32_t* wtot, uint32_t& bin, uint32_t& krem_out) {
  const int tid = threadIdx.x;
  const int bpt = (nbins + NT - 1) / NT;
  const int hi = nbins - tid * bpt;  // my bins are [lo, hi), scanned from the top
  const int lo = hi - bpt < 0 ? 0 : hi - bpt;
  uint32_t mine = 0;
  for (int b = hi - 1; b >= lo; --b) mine += hist[b] + ((uint32_t)b == xbin ? xcnt : 0u);
  const uint32_t incl = block_inclusive_sum<NT>(mine, wtot);
  const uint32_t excl = incl - mine;
  if (excl < krem && krem <= incl) {
    uint32_t cum = excl;
    for (int b = hi - 1; b >= lo; --b) {
      const uint32_t cnt = hist[b] + ((uint32_t)b == xbin ? xcnt : 0u);
      if (cum + cnt >= krem) {
        sh[0] = (uint32_t)b;
        sh[1] = krem - cum;
        break;
      }
      cum += cnt;
    }
  }
  __syncthreads();
  bin = sh[0];
  krem_out = sh[1];
  __syncthreads();
}

// First-digit threshold from a score histogram (already in LDS): positions
// the histogram does not count (T minus its total) are -inf.
template <int NT>
__device__ __forceinline__ void select_first_bin(const uint32_t* h1, int T, uint32_t kout,
                                                 uint32_t* sh, uint32_t* wtot, uint32_t& bin,
                                                 uint32_t& krem) {
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < 2048 / NT; ++j) mine += h1[threadIdx.x + j * NT];
  const uint32_t total = block_sum<NT>(mine, wtot);
  select_bin<NT>(h1, 2048, kout, kInfBin, (uint32_t)T - total, sh, wtot, bin, krem);
}

// Copy n (a multiple of NT) words from global memory into LDS, all loads in
// flight together.
template <int NT, int N>
__device__ __forceinline__ void copy_to_lds(uint32_t* dst, const uint32_t* __restrict__ src) {
  uint32_t tmp[N / NT];
#pragma unroll
  for (int j = 0; j < N / NT; ++j) tmp[j] = src[threadIdx.x + j * NT];
#pragma unroll
  for (int j = 0; j < N / NT; ++j) dst[threadIdx.x + j * NT] = tmp[j];
}

__device__ __forceinline__ uint32_t extend_prefix(uint32_t prefix, int pass, uint32_t bin) {
  return pass == 0 ? bin : ((prefix << (pass == 1 ? 11 : 10)) | bin);
}

// ------------------------------------------------ register-resident keys
// Keys of a run of positions; a position past T gets key 0 (the key of a
// negative NaN, which no supported score produces), so "present" needs no
// mask of its own.  Every lane loads (past-the-end lanes re-read position
// T-1), so all loads are in flight together.
template <int EPT>
__device__ __forceinline__ void load_vals(const float* __restrict__ srow, int base, int T,
                                          float (&v)[EPT]) {
  const int lane = threadIdx.x & 63;
  const unsigned last = (unsigned)(T - 1);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const unsigned t = (unsigned)(base + e * 64 + lane);
    v[e] = srow[t < last ? t : last];
  }
}

template <int EPT>
__device__ __forceinline__ void vals_to_keys(const float (&v)[EPT], int base, int T, int c,
                                             uint32_t (&key)[EPT]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int t = base + e * 64 + lane;
    key[e] = t < T ? (t < c ? score_key(v[e]) : kKeyNegInf) : 0u;
  }
}

template <int EPT>
__device__ __forceinline__ void load_keys(const float* __restrict__ srow, int base, int T, int c,
                                          uint32_t (&key)[EPT]) {
  float v[EPT];
  load_vals<EPT>(srow, base, T, v);
  vals_to_keys<EPT>(v, base, T, c, key);
}

// Adds the block's keys to the LDS histogram of digit `pass`, among keys
// whose higher digits equal `prefix` (key 0 marks an absent element; it only
// lands in bin 0 of the first digit, which no supported key reaches).  -inf
// keys are counted into *ninf_sh by ballot.
template <int EPT>
__device__ __forceinline__ void hist_pass(const uint32_t (&key)[EPT], int pass, uint32_t prefix,
                                          uint32_t* hist, uint32_t* ninf_sh) {
  const int lane = threadIdx.x & 63;
  const int shift = pass_shift(pass), ms = pass_match_shift(pass);
  const uint32_t mask = (uint32_t)pass_bins(pass) - 1u;
  uint32_t ninf = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint32_t k = key[e];
    const bool match = ms == 32 ? k != 0u : (k >> ms) == prefix;
    const bool isinf = k == kKeyNegInf;
    if (match && !isinf) atomicAdd(&hist[(k >> shift) & mask], 1u);
    ninf += (uint32_t)__popcll(__ballot(match && isinf));
  }
  if (lane == 0 && ninf) atomicAdd(ninf_sh, ninf);
}

// Histogram one digit of the block's keys into LDS (ready after return).
template <int NT, int EPT>
__device__ __forceinline__ void block_hist(const uint32_t (&key)[EPT], int pass, uint32_t prefix,
                                           uint32_t* hist, uint32_t* ninf_sh) {
  const int nb = pass_bins(pass);
  for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0;
  if (threadIdx.x == 0) *ninf_sh = 0;
  __syncthreads();
  hist_pass<EPT>(key, pass, prefix, hist, ninf_sh);
  __syncthreads();
  if (threadIdx.x == 0 && *ninf_sh) hist[(kKeyNegInf >> pass_shift(pass)) & (uint32_t)(nb - 1)] += *ninf_sh;
  __syncthreads();
}

// Writes the selected elements of the block (keys > ustar, and keys ==
// ustar while their global equal-rank is below need) in position order.
// out_base / eq_base: selected and equal elements before this block.
template <int NW, int EPT>
__device__ __forceinline__ void block_emit(const uint32_t (&key)[EPT], int base,
                                           uint32_t ustar, uint32_t need, uint32_t out_base,
                                           uint32_t eq_base, int c, int32_t offset,
                                           int32_t* __restrict__ orow, uint32_t kout,
                                           uint32_t (*wcnt)[NW]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t gt = 0, eq = 0;  // absent elements (key 0) are below any threshold key
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    gt += (uint32_t)__popcll(__ballot(key[e] > ustar));
    eq += (uint32_t)__popcll(__ballot(key[e] == ustar));
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
    const bool g = key[e] > ustar;
    const bool q = key[e] == ustar;
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

// ------------------------------------------------ single-workgroup rows
// One workgroup of NT threads per row of at most NT*EPT positions; the keys
// stay in registers (layout and method in row_topk.hpp).  key_hist
// (optional) is the score kernel's first-digit histogram of the row: it is
// read once and reset to zero for the next score call.  Only positions below
// compress_lens are loaded; a row with compress_lens <= k keeps all of them
// and needs no scores at all.
template <int NT, int EPT>
__global__ __launch_bounds__(NT) void topk_rows_kernel(
    const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    uint32_t* __restrict__ key_hist, int kout, int32_t offset, int32_t* __restrict__ out,
    int64_t ld_out) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t mbuf[NT * EPT / 16];
  __shared__ uint32_t wtot[2 * (NT / 64)];
  __shared__ uint32_t sh[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  int32_t* orow = out + (int64_t)r * ld_out;
  uint32_t* hrow = key_hist ? key_hist + (int64_t)r * 2048 : nullptr;

  // the histogram and the row are requested before compress_lens is known
  // (every load is in bounds whatever it is), so the three latencies overlap.
  // The score histogram first: this thread's bins [hhi - HPT, hhi), top bin
  // first, straight into the threshold search
  constexpr int HPT = 2048 / NT;
  const int hhi = 2048 - tid * HPT;
  uint32_t hreg[HPT];
  if (hrow)
#pragma unroll
    for (int j = 0; j < HPT; ++j) hreg[j] = hrow[hhi - 1 - j];

  const float* srow = scores + (int64_t)r * ld;
  const int wbase = row_base<EPT>();
  float v[EPT];
  uint32_t prefix, need, bin_count;
  int shift, c;
  {
    // every load in bounds and none conditional: a wave reaching past T
    // reads position T - 1 there (positions >= c are masked by row_vals
    // whatever they read)
    const int wend = (__builtin_amdgcn_readfirstlane(tid >> 6) + 1) * 64 * EPT;
    if (wend <= T) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) v[e] = srow[wbase + 64 * e];
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int t = wbase + 64 * e;
        v[e] = srow[t < T ? t : T - 1];
      }
    }
    c = cl_arr[r];
    c = c < 0 ? 0 : (c > T ? T : c);
    if (c <= kout) {
      row_keep_prefix<NT>(c, kout, offset, orow);
      if (hrow)
        for (int i = tid; i < 2048; i += NT) hrow[i] = 0u;
      return;
    }
    uint32_t b1 = 0, krem = 0, bcnt = 0;
    bool hist_ok = false;
    if (hrow) {
      // first digit from the score histogram while the scores are in flight
#pragma unroll
      for (int j = 0; j < HPT; ++j) hrow[hhi - 1 - j] = 0u;  // ready for the next score call
      for (int i = tid; i < 2048; i += NT) hist[i] = 0u;     // the next digit's histogram
      // the -inf bin counts the T - c unscored positions; T bounds that,
      // which selects the same bin and remainder (only the returned count of
      // the -inf bin grows)
#pragma unroll
      for (int j = 0; j < HPT; ++j)
        if (hhi - 1 - j == (int)kInfBin) hreg[j] += (uint32_t)T;
      uint32_t total;
      select_bin_regs<NT, 2048>(hreg, (uint32_t)kout, sh, wtot, b1, krem, bcnt, &total);
      // a histogram of these scores counts exactly the c positions below
      // compress_lens; any other total (a stale or doubly filled histogram)
      // is not used: the row is then ranked from its scores alone
      hist_ok = total - (uint32_t)T == (uint32_t)c;
    }
    row_vals<EPT>(v, wbase, c, T);
    if (hist_ok) {
      row_refine<NT, EPT>(v, hist, true, sh, wtot, b1, krem, bcnt, prefix, shift, need, bin_count);
    } else {
      row_select<NT, EPT>(v, hist, 0xffffffffu, T, kout, sh, wtot, prefix, shift, need,
                          bin_count);
    }
  }
  row_emit<NT, EPT>(v, prefix, shift, need, bin_count, c, kout, offset, wbase, mbuf,
                    kout <= 2048 ? reinterpret_cast<int32_t*>(hist) : nullptr, wtot, orow);
}

// ------------------------------------------------ level-two rows
// A level-two row is finite only inside its candidate blocks (idx_score with
// cand_blocks writes -inf everywhere else).  With at least k_out finite
// candidates, the top k_out of the whole row are among them, so the row is
// ranked as the virtual row of its candidate positions: slot v is position
// ids[v / cbs] * cbs + v % cbs, increasing with v because the ids ascend.
// With fewer (the literal rule keeps -inf positions then, lowest first), the
// kept set is every finite position plus the lowest k_out - F others, which
// all lie below k_out; that case is resolved on an LDS bit map of the row.
constexpr int kCandMaxT = 65536;    // row width the fallback bit map covers
constexpr int kCandMaxIds = 2048;   // candidate ids per row held in LDS

template <int NT, int EPT>
__device__ __forceinline__ void cand_rank_row(
    int r, const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    const int32_t* __restrict__ cand, int n_cand, int cbs, uint32_t* __restrict__ key_hist,
    int kout, int32_t offset, int32_t* __restrict__ out, int64_t ld_out, int compact) {
  constexpr int WPT = (kCandMaxT / 32) / NT;
  __shared__ uint32_t hist[2048];
  __shared__ int32_t ids[kCandMaxIds];
  __shared__ uint32_t mbuf[NT * EPT / 16];
  __shared__ uint32_t wtot[2 * (NT / 64)];
  __shared__ uint32_t sh[4];
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t* hrow = key_hist ? key_hist + (int64_t)r * 2048 : nullptr;
  // the score histogram (level two: counts of the candidate positions below
  // compress_lens) is requested first, this thread's bins [hhi - HPT, hhi)
  constexpr int HPT = 2048 / NT;
  const int hhi = 2048 - tid * HPT;
  uint32_t hreg[HPT];
  if (hrow)
#pragma unroll
    for (int j = 0; j < HPT; ++j) hreg[j] = hrow[hhi - 1 - j];
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  const int nb = (T + cbs - 1) / cbs;
  const int V = n_cand * cbs;
  const float* srow = scores + (int64_t)r * ld;
  const int wbase = row_base<EPT>();
  float v[EPT];
  if (compact) {
    // slot scores in slot order (idx_score_topk_candidates): requested
    // beside the ids, not after them; slots past V read slot V - 1 (masked)
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int sv = wbase + 64 * e;
      v[e] = srow[sv < V ? sv : V - 1];
    }
  }
  for (int i = tid; i < n_cand; i += NT) {
    const int id = cand[(int64_t)r * n_cand + i];
    ids[i] = (id < 0 || id >= nb) ? -1 : id;
  }
  for (int i = tid; i < 2048; i += NT) hist[i] = 0u;  // the next digit's histogram
  __syncthreads();
  // slot v lies in candidate block v / cbs (a shift for the usual
  // power-of-two block size: the division is dozens of instructions)
  const bool pow2 = (cbs & (cbs - 1)) == 0;
  const int cshift = __builtin_ctz((unsigned)cbs);
  auto block_of = [&](int v) { return pow2 ? v >> cshift : v / cbs; };
  // position of slot v, or -1 (no such block, or past T)
  auto slot_pos = [&](int v) {
    if (v >= V) return -1;
    const int blk = block_of(v), id = ids[blk];
    if (id < 0) return -1;
    const int p = id * cbs + (v - blk * cbs);
    return p < T ? p : -1;
  };
  uint32_t nfin = 0;
  {
    // validity as integer arithmetic on the sign bits, kept out of the
    // compiler's reach (no per-element compare masks live across the loads)
    uint32_t okp[EPT], fin[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int p = slot_pos(wbase + 64 * e);
      uint32_t ok = (uint32_t)(~p) >> 31;                // p >= 0
      uint32_t below_c = ((uint32_t)(p - c) >> 31) & ok;  // 0 <= p < c
      asm volatile("" : "+v"(ok), "+v"(below_c));
      okp[e] = ok;
      fin[e] = below_c;
      if (!compact) v[e] = srow[p & ~(p >> 31)];
    }
    // no such slot: NaN (absent); at or past c: -inf
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint32_t m = 0xff800000u ^ (0x80400000u & (okp[e] - 1u));
      const uint32_t u = __float_as_uint(v[e]);
      v[e] = __uint_as_float(m ^ ((u ^ m) & (0u - fin[e])));
      nfin += fin[e];
    }
  }
  const uint32_t F = block_sum<NT>(nfin, wtot);
  if (hrow)
#pragma unroll
    for (int j = 0; j < HPT; ++j) hrow[hhi - 1 - j] = 0u;  // ready for the next score call
  int32_t* orow = out + (int64_t)r * ld_out;
  if (F >= (uint32_t)kout) {
    uint32_t prefix, need, bcnt;
    int shift;
    bool hist_ok = false;
    uint32_t b1, krem, bc1;
    if (hrow) {
      // the -inf slots number at most V (only the returned count of the
      // -inf bin grows, as in the rows kernel)
#pragma unroll
      for (int j = 0; j < HPT; ++j)
        if (hhi - 1 - j == (int)kInfBin) hreg[j] += (uint32_t)V;
      uint32_t total;
      select_bin_regs<NT, 2048>(hreg, (uint32_t)kout, sh, wtot, b1, krem, bc1, &total);
      // the level-two histogram counts exactly the F candidate positions
      // below compress_lens; any other total is not used
      hist_ok = total - (uint32_t)V == F;
    }
    if (hist_ok) {
      row_refine<NT, EPT>(v, hist, true, sh, wtot, b1, krem, bc1, prefix, shift, need, bcnt);
    } else {
      row_select<NT, EPT>(v, hist, 0xffffffffu, V, kout, sh, wtot, prefix, shift, need, bcnt);
    }
    struct CandPos {
      const int32_t* ids;
      int cbs, cshift;
      bool pow2;
      __device__ __forceinline__ int operator()(int v) const {
        const int blk = pow2 ? v >> cshift : v / cbs;
        return ids[blk] * cbs + (v - blk * cbs);
      }
    };
    row_emit<NT, EPT>(v, prefix, shift, need, bcnt, c, kout, offset, wbase, mbuf,
                      kout <= 2048 ? reinterpret_cast<int32_t*>(hist) : nullptr, wtot, orow,
                      CandPos{ids, cbs, cshift, pow2});
    return;
  }

  // ---- fewer finite scores than k_out: bit map of the finite positions
  uint32_t* fin = hist;  // kCandMaxT bits
  for (int i = tid; i < kCandMaxT / 32; i += NT) fin[i] = 0u;
  __syncthreads();
  int wb = wbase;
  asm volatile("" : "+v"(wb));
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (v[e] > -__builtin_inff()) {  // neither absent (NaN) nor -inf
      const int p = slot_pos(wb + 64 * e);
      atomicOr(&fin[p >> 5], 1u << (p & 31));
    }
  }
  __syncthreads();
  // thread i owns words [i*WPT, (i+1)*WPT): the kept positions are the
  // finite ones plus the non-finite ones whose rank among non-finite
  // positions is below k_out - F
  const int nw = (T + 31) / 32;
  uint32_t selw[WPT];
  uint32_t nf = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = tid * WPT + j;
    selw[j] = w < nw ? fin[w] : 0u;
    nf += (uint32_t)__popc(selw[j]);
  }
  const uint32_t fbefore = block_inclusive_sum<NT>(nf, wtot) - nf;  // finite before my words
  const uint32_t extra = (uint32_t)kout - F;
  uint32_t fb = fbefore, ns = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = tid * WPT + j;
    if (w < nw) {
      const int rem = T - 32 * w;
      const uint32_t valid = rem >= 32 ? 0xffffffffu : ((1u << rem) - 1u);
      uint32_t rest = valid & ~selw[j];
      const uint32_t rbefore = (uint32_t)(32 * w) - fb;  // non-finite positions before word w
      uint32_t take = extra > rbefore ? extra - rbefore : 0u;
      uint32_t kept = selw[j];
      while (take-- && rest) {  // the lowest non-finite positions of this word
        const uint32_t low = rest & (0u - rest);
        kept |= low;
        rest ^= low;
      }
      fb += (uint32_t)__popc(selw[j]);
      selw[j] = kept;
      ns += (uint32_t)__popc(kept);
    }
  }
  __syncthreads();  // fin is rewritten as the output stage below
  uint32_t slot = block_inclusive_sum<NT>(ns, wtot) - ns;
  int32_t* dst = kout <= 2048 ? reinterpret_cast<int32_t*>(hist) : orow;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    uint32_t bits = selw[j];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1u;
      const int t = (tid * WPT + j) * 32 + b;
      if (slot < (uint32_t)kout) dst[slot] = t < c ? t + offset : -1;
      ++slot;
    }
  }
  if (dst != orow) {
    __syncthreads();
    for (int i = tid; i < kout; i += NT) orow[i] = dst[i];
  }
  (void)lane;
}

template <int NT, int EPT>
__global__ __launch_bounds__(NT) void topk_cand_kernel(
    const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    const int32_t* __restrict__ cand, int n_cand, int cbs, uint32_t* __restrict__ key_hist,
    int kout, int32_t offset, int32_t* __restrict__ out, int64_t ld_out, int compact) {
  cand_rank_row<NT, EPT>((int)blockIdx.x, scores, ld, T, cl_arr, cand, n_cand, cbs, key_hist, kout,
                         offset, out, ld_out, compact);
}

// ------------------------------------------------ streaming one-row ranking
// One workgroup ranks a whole row by streaming its scores from memory in
// tiles of NT*EPT: three digit passes of LDS histograms over the row, then
// the position-ordered emission tile by tile (block_emit), carrying the
// counts of selected and tied keys from tile to tile.  Slow (the row is read
// four times) but needs no histogram from the caller: the split path falls
// back to it when the histogram it was given does not match the row.
template <int NT>
__device__ __noinline__ void stream_rank_row(const float* __restrict__ srow, int T, int c, int kout,
                                             int32_t offset, int32_t* __restrict__ orow,
                                             uint32_t* hist, uint32_t* sh, uint32_t* wtot,
                                             uint32_t (*wcnt)[NT / 64]) {
  constexpr int EPT = 4, NW = NT / 64, TILE = NT * EPT;
  const int wb0 = (int)(threadIdx.x >> 6) * 64 * EPT;
  uint32_t prefix = 0, krem = (uint32_t)kout;
  for (int pass = 0; pass < 3; ++pass) {
    uint32_t key[EPT];
    {
      const int nb = pass_bins(pass);
      for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0u;
      if (threadIdx.x == 0) sh[2] = 0u;
      __syncthreads();
      for (int base = 0; base < T; base += TILE) {
        load_keys<EPT>(srow, base + wb0, T, c, key);
        hist_pass<EPT>(key, pass, prefix, hist, &sh[2]);
      }
      __syncthreads();
      if (threadIdx.x == 0 && sh[2])
        hist[(kKeyNegInf >> pass_shift(pass)) & (uint32_t)(nb - 1)] += sh[2];
      __syncthreads();
      uint32_t bin, k2;
      select_bin<NT>(hist, nb, krem, 0xffffffffu, 0u, sh, wtot, bin, k2);
      prefix = extend_prefix(prefix, pass, bin);
      krem = k2;
    }
  }
  // keys above `prefix` are taken, and of those equal to it the `krem` at
  // the lowest positions
  uint32_t ob = 0, eqb = 0;
  for (int base = 0; base < T; base += TILE) {
    uint32_t key[EPT];
    load_keys<EPT>(srow, base + wb0, T, c, key);
    block_emit<NW, EPT>(key, base + wb0, prefix, krem, ob, eqb, c, offset, orow,
                        (uint32_t)kout, wcnt);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      gt += wcnt[0][i];
      eq += wcnt[1][i];
    }
    __syncthreads();  // every thread has read this tile's counts
    ob += gt + (krem > eqb ? (eq < krem - eqb ? eq : krem - eqb) : 0u);
    eqb += eq;
  }
}

// ---------------------------------------- split path (score histogram given)
// (kernel A's part and the workspace layout: split_topk.hpp)

__global__ __launch_bounds__(kPartNW * 64) void topk_split_a_kernel(
    const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    const uint32_t* __restrict__ key_hist, int kout, uint32_t* __restrict__ ws) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wtot[kPartNW];
  __shared__ uint32_t sh[4];
  split_a_part<kPartNW * 64>((int)blockIdx.y, (int)blockIdx.x, scores, ld, T, cl_arr, key_hist,
                             kout, ws, hist, wtot, sh);
}

#ifndef IDX_SPLIT_B_THREADS
#define IDX_SPLIT_B_THREADS 1024
#endif
constexpr int kSplitBThreads = IDX_SPLIT_B_THREADS;

__device__ __forceinline__ void split_b_row(
    int r, const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    uint32_t* __restrict__ key_hist, int kout, int32_t offset, int32_t* __restrict__ out,
    int64_t ld_out, const uint32_t* __restrict__ ws) {
  constexpr int NT = kSplitBThreads, NW = NT / 64;
  // sel[padded nwords] eq[padded nwords] ckey[cap] cpos[cap]; mask word w
  // lives at w + w/32, so threads owning consecutive runs of words hit
  // distinct banks
  extern __shared__ uint32_t dyn[];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t regions[kSplitMaxT / kPart * kPartNW + 1];  // prefix of list counts
  __shared__ uint32_t wtot[NW];
  __shared__ uint32_t wtot2[2 * NW];
  __shared__ uint32_t sh[4];
  const int tid = threadIdx.x;
  const SplitLayout L(T);
  const uint32_t* wrow = ws + (int64_t)r * L.row_words;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  const int nw = (int)L.nwords;
  uint32_t* sel = dyn;
  const int nwp = split_padded_words(nw);
  uint32_t* eqm = dyn + nwp;
  uint32_t* ckey = dyn + 2 * nwp;
  uint32_t* cpos = ckey + kSplitCandCap;
  const int nreg = (int)L.nparts * kPartNW;

  // Everything the ranking reads from kernel A's output is requested in one
  // round: the search state (b1, krem and the histogram's total), the list
  // counts (at most 256 regions), and the first 8 * tpr entries of every
  // region (tpr threads per region, eight entries each; a region holds up to
  // 1024, so these reads stay inside it whatever its count).
  static_assert(kSplitMaxT / kPart * kPartNW <= NT, "one region per thread");
  const uint32_t rc = tid < nreg ? wrow[L.cnt_off + tid] : 0u;
  const uint32_t b1 = wrow[L.state_off];
  uint32_t krem = wrow[L.state_off + 1];
  const uint32_t htotal = wrow[L.state_off + 2];
  const uint32_t inf_count = key_hist[(int64_t)r * 2048 + kInfBin];
  const int tpr = NT / nreg;  // at least 4
  const int sj = tid / tpr, sli = tid - sj * tpr;
  uint2 sv[8];
  {
    const uint2* src =
        reinterpret_cast<const uint2*>(wrow + L.cand_off + (int64_t)(sj < nreg ? sj : 0) * 1024 * 2);
#pragma unroll
    for (int u = 0; u < 8; ++u) sv[u] = src[sli + u * tpr];
  }
  // this thread's words of the above-threshold masks (kernel A's output),
  // requested in the same round as the state and the list: every barrier
  // waits for the loads in flight, so any later request would be waited
  // for on its own
  constexpr int kMaxWpt = (kSplitMaxT / 32 + NT - 1) / NT;
  static_assert(kMaxWpt % 4 == 0, "whole 16-byte words per thread");
  const int wpt = (nw + NT - 1) / NT;
  uint32_t aw[kMaxWpt];
  if ((wpt & 3) == 0 && (reinterpret_cast<uintptr_t>(wrow) & 15) == 0 && tid * wpt + wpt <= nw) {
    // whole 16-byte words (rows are 16-byte aligned in a 16-byte aligned
    // workspace): a quarter of the load instructions, each line read once;
    // 8-byte words when the thread's count is even
#pragma unroll
    for (int j = 0; j < kMaxWpt; j += 4) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (j < wpt) v = *reinterpret_cast<const uint4*>(wrow + tid * wpt + j);
      aw[j] = v.x;
      aw[j + 1] = v.y;
      aw[j + 2] = v.z;
      aw[j + 3] = v.w;
    }
  } else if ((wpt & 1) == 0 && (reinterpret_cast<uintptr_t>(wrow) & 7) == 0 &&
             tid * wpt + wpt <= nw) {
#pragma unroll
    for (int j = 0; j < kMaxWpt; j += 2) {
      uint2 v = make_uint2(0u, 0u);
      if (j < wpt) v = *reinterpret_cast<const uint2*>(wrow + tid * wpt + j);
      aw[j] = v.x;
      aw[j + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kMaxWpt; ++j) {
      const int word = tid * wpt + j;
      aw[j] = wrow[word < nw ? word : nw - 1];
    }
  }

  // The score histogram counts exactly the c positions below compress_lens
  // when it comes from idx_score on these scores.  Any other total (a stale
  // or doubly filled histogram; kernel A summed it) made kernel A's
  // threshold meaningless: the row is then ranked from its scores alone.
  if (htotal != (uint32_t)c) {
    __shared__ uint32_t wcnt[2][NW];
    stream_rank_row<NT>(scores + (int64_t)r * ld, T, c, kout, offset,
                        out + (int64_t)r * ld_out, hist, sh, wtot, wcnt);
    for (int i = tid; i < 2048; i += NT) key_hist[(int64_t)r * 2048 + i] = 0u;
    return;
  }

  for (int i = tid; i < nwp; i += NT) {
    sel[i] = 0u;
    eqm[i] = 0u;
  }
  // list counts -> region prefix, one block scan
  const uint32_t rincl = block_inclusive_sum<NT, true>(rc, wtot);
  if (tid < nreg) regions[tid + 1] = rincl;
  if (tid == 0) regions[0] = 0;
  lds_barrier();
  const uint32_t ncand = regions[nreg];
  const bool only_inf = b1 == kInfBin && inf_count == 0u;

  uint32_t ustar = kKeyNegInf;
  if (!only_inf) {
    const bool in_lds = ncand <= (uint32_t)kSplitCandCap;
    // list element i lives in region j with regions[j] <= i < regions[j+1]
    auto fetch = [&](uint32_t i, uint32_t& k, uint32_t& p) {
      int lo = 0, hi = nreg;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (regions[mid] <= i) lo = mid; else hi = mid;
      }
      const uint32_t* cl = wrow + L.cand_off + (int64_t)lo * 1024 * 2;
      const uint32_t j = i - regions[lo];
      k = cl[2 * j];
      p = cl[2 * j + 1];
    };
    if (in_lds) {
      // threads split evenly over the regions; each thread copies every
      // tpr-th element of its region: the first eight from the round above,
      // the rest eight loads in flight at a time
      const int j = sj, li = sli;
      if (j < nreg) {
        const uint32_t base = regions[j], cnt = regions[j + 1] - base;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t e = li + u * tpr;
          if (e < cnt) {
            ckey[base + e] = sv[u].x;
            cpos[base + e] = sv[u].y;
          }
        }
        const uint2* src = reinterpret_cast<const uint2*>(wrow + L.cand_off + (int64_t)j * 1024 * 2);
        for (uint32_t e0 = li + 8u * tpr; e0 < cnt; e0 += 8u * tpr) {
          uint2 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const uint32_t e = e0 + u * tpr;
            v[u] = src[e < cnt ? e : 0u];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const uint32_t e = e0 + u * tpr;
            if (e < cnt) {
              ckey[base + e] = v[u].x;
              cpos[base + e] = v[u].y;
            }
          }
        }
      }
      lds_barrier();
    }
    // every pass over the list runs one of two loops (from LDS, or fetched
    // from the workspace when the list does not fit)
    auto each = [&](auto&& body) {
      if (in_lds) {
        for (uint32_t i = tid; i < ncand; i += NT) body(ckey[i], cpos[i]);
      } else {
        for (uint32_t i = tid; i < ncand; i += NT) {
          uint32_t k, p;
          fetch(i, k, p);
          body(k, p);
        }
      }
    };
    uint32_t prefix = b1, bc = 0;
    for (int pass = 1; pass < 3; ++pass) {
      const int nb = pass_bins(pass), shift = pass_shift(pass), ms = pass_match_shift(pass);
      if (pass == 2 && bc <= 64u) {
        // few keys share the 22-bit prefix (bc of them): collect them, and
        // wave 0 finds the krem-th largest directly (lane i counts the keys
        // above its own and those at least its own), two barriers instead
        // of a histogram pass
        __shared__ uint32_t small[64];
        __shared__ uint32_t nsmall;
        if (tid == 0) nsmall = 0u;
        lds_barrier();
        each([&](uint32_t k, uint32_t) {
          if ((k >> ms) == prefix) small[atomicAdd(&nsmall, 1u)] = k;
        });
        lds_barrier();
        if (tid < 64) {
          const uint32_t mine = tid < (int)bc ? small[tid] : 0u;
          uint32_t gt = 0, ge = 0;
          for (uint32_t j = 0; j < bc; ++j) {
            const uint32_t o = small[j];
            gt += o > mine ? 1u : 0u;
            ge += o >= mine ? 1u : 0u;
          }
          if (tid < (int)bc && gt < krem && krem <= ge) {  // one key value: equal writes
            sh[0] = mine;
            sh[1] = krem - gt;
          }
        }
        lds_barrier();
        prefix = sh[0];  // the whole key
        krem = sh[1];
        lds_barrier();
        break;
      }
      for (int i = tid; i < nb; i += NT) hist[i] = 0;
      lds_barrier();
      each([&](uint32_t k, uint32_t) {
        if ((k >> ms) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1u);
      });
      lds_barrier();
      uint32_t bin, k2;
      if (pass == 1)
        select_bin_r<NT, 2048, true>(hist, krem, 0xffffffffu, 0u, sh, wtot, bin, k2, bc);
      else
        select_bin_r<NT, 1024, true>(hist, krem, 0xffffffffu, 0u, sh, wtot, bin, k2, bc);
      prefix = extend_prefix(prefix, pass, bin);
      krem = k2;
    }
    ustar = prefix;
    // mark the list elements above the threshold and equal to it
    each([&](uint32_t k, uint32_t p) {
      if (k > ustar) atomicOr(&sel[split_pad(p >> 5)], 1u << (p & 31));
      else if (k == ustar) atomicOr(&eqm[split_pad(p >> 5)], 1u << (p & 31));
    });
  }
  const uint32_t need = krem;
  lds_barrier();

  // compaction: thread i owns words [i*wpt, (i+1)*wpt), wpt <= kMaxWpt; the
  // mask words are loaded together, the output row is assembled in LDS (the
  // histogram is free now) and written out in one coalesced pass
  // above / equal words of this thread stay in registers for the output
  uint32_t qv[kMaxWpt];
  uint32_t ng = 0, nq = 0;
#pragma unroll
  for (int j = 0; j < kMaxWpt; ++j) {
    const int word = tid * wpt + j;
    qv[j] = 0u;
    if (j < wpt && word < nw) {
      uint32_t a = aw[j] | sel[split_pad(word)];
      uint32_t q = eqm[split_pad(word)];
      if (only_inf) {  // the equal elements are the -inf ones: present and not above
        const int rem = T - word * 32;
        const uint32_t present = rem >= 32 ? 0xffffffffu : ((1u << rem) - 1u);
        q = present & ~aw[j];
        a = aw[j];
      }
      aw[j] = a;
      qv[j] = q;
      ng += (uint32_t)__popc(a);
      nq += (uint32_t)__popc(q);
    } else {
      aw[j] = 0u;
    }
  }
  uint32_t gi = ng, qi = nq;
  block_inclusive_sum2<NT>(gi, qi, wtot2);
  uint32_t qbefore = qi - nq;
  uint32_t slot = (gi - ng) + (qbefore < need ? qbefore : need);
  int32_t* orow = out + (int64_t)r * ld_out;
  const bool stage = kout <= 2048;
  int32_t* dst = stage ? reinterpret_cast<int32_t*>(hist) : orow;
#pragma unroll
  for (int j = 0; j < kMaxWpt; ++j) {
    const uint32_t qw = qv[j];
    const uint32_t qn = (uint32_t)__popc(qw);
    uint32_t take = need > qbefore ? (need - qbefore < qn ? need - qbefore : qn) : 0u;
    qbefore += qn;
    uint32_t bits = aw[j], rest = qw;
    while (take--) {
      const uint32_t low = rest & (0u - rest);
      bits |= low;
      rest ^= low;
    }
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1u;
      const int t = (tid * wpt + j) * 32 + b;
      if (slot < (uint32_t)kout) dst[slot] = t < c ? t + offset : -1;
      ++slot;
    }
  }
  if (stage) {
    __syncthreads();
    for (int i = tid; i < kout; i += NT) orow[i] = dst[i];
  }
  // every thread read the histogram before the scans above: reset it for the
  // next score call
  for (int i = tid; i < 2048; i += NT) key_hist[(int64_t)r * 2048 + i] = 0u;
}

__global__ __launch_bounds__(kSplitBThreads) void topk_split_b_kernel(
    const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    uint32_t* __restrict__ key_hist, int kout, int32_t offset, int32_t* __restrict__ out,
    int64_t ld_out, const uint32_t* __restrict__ ws) {
  split_b_row((int)blockIdx.x, scores, ld, T, cl_arr, key_hist, kout, offset, out, ld_out, ws);
}

// The two rankings of a two-level step in one launch (idx_two_level_topk):
// workgroups [0, R) run kernel B on level one's rows, workgroups [R, 2R) the
// candidate top-k on level two's slot scores.  Neither reads what the other
// writes (each level has its own histogram), and each alone fills only R
// CUs, so side by side they take about as long as the longer of the two.
static_assert(kSplitBThreads == 1024, "the candidate rows run on 1024 threads");
constexpr int kTwoLevelMaxT = 131072;  // kernel B's LDS beside the candidate kernel's
__global__ __launch_bounds__(1024) void topk_split_b_cand_kernel(
    int R, const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    uint32_t* __restrict__ key_hist, int kout, int32_t offset, int32_t* __restrict__ out1,
    int64_t ld_out1, const uint32_t* __restrict__ ws, const float* __restrict__ slot_scores,
    int64_t ld2, const int32_t* __restrict__ cand, int n_cand, int cbs,
    uint32_t* __restrict__ key_hist2, int32_t* __restrict__ out2, int64_t ld_out2) {
  if ((int)blockIdx.x < R)
    split_b_row((int)blockIdx.x, scores, ld, T, cl_arr, key_hist, kout, offset, out1, ld_out1, ws);
  else
    cand_rank_row<1024, 8>((int)blockIdx.x - R, slot_scores, ld2, T, cl_arr, cand, n_cand, cbs,
                           key_hist2, kout, offset, out2, ld_out2, 1);
}

// ------------------------------------------------- multi-workgroup path
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// Re-derive the thresholds of passes [0, npass) from the global histograms
// (the first one from the score histogram when given), each copied into the
// LDS buffer lh (2048 words) first.
template <int NT>
__device__ __forceinline__ void resolve_passes(const uint32_t* __restrict__ wrow,
                                               const uint32_t* __restrict__ h1, int T, int npass,
                                               int kout, uint32_t* lh, uint32_t* sh,
                                               uint32_t* wtot, uint32_t& prefix, uint32_t& krem) {
  prefix = 0;
  krem = (uint32_t)kout;
  for (int p = 0; p < npass; ++p) {
    uint32_t bin, k2;
    if (p == 2)
      copy_to_lds<NT, 1024>(lh, wrow + pass_hist_offset(p));
    else
      copy_to_lds<NT, 2048>(lh, (p == 0 && h1) ? h1 : wrow + pass_hist_offset(p));
    __syncthreads();
    if (p == 0 && h1)
      select_first_bin<NT>(lh, T, krem, sh, wtot, bin, k2);
    else
      select_bin<NT>(lh, pass_bins(p), krem, 0xffffffffu, 0u, sh, wtot, bin, k2);
    prefix = extend_prefix(prefix, p, bin);
    krem = k2;
  }
}

template <int PASS>
__global__ __launch_bounds__(kChunkNW * 64) void topk_chunk_hist_kernel(
    const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    const uint32_t* __restrict__ key_hist, int kout, uint32_t* __restrict__ ws,
    int64_t ws_row_words) {
  constexpr int NT = kChunkNW * 64, SEG = 64 * kChunkEPT;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wtot[kChunkNW];
  __shared__ uint32_t sh[4];
  const int r = blockIdx.y, w = threadIdx.x >> 6;
  uint32_t* wrow = ws + (int64_t)r * ws_row_words;
  const uint32_t* h1 = key_hist ? key_hist + (int64_t)r * 2048 : nullptr;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  const int base = blockIdx.x * kChunk + w * SEG;
  float v[kChunkEPT];
  load_vals<kChunkEPT>(scores + (int64_t)r * ld, base, T, v);  // in flight during the resolve
  uint32_t prefix, krem;
  resolve_passes<NT>(wrow, h1, T, PASS, kout, hist, sh, wtot, prefix, krem);
  uint32_t key[kChunkEPT];
  vals_to_keys<kChunkEPT>(v, base, T, c, key);
  block_hist<NT, kChunkEPT>(key, PASS, prefix, hist, &sh[2]);
  const int nb = pass_bins(PASS);
  for (int i = threadIdx.x; i < nb; i += NT)
    if (hist[i]) atomicAdd(&wrow[pass_hist_offset(PASS) + i], hist[i]);
}

// Per chunk: count of keys above the threshold and equal to it.
__global__ __launch_bounds__(kChunkNW * 64) void topk_chunk_count_kernel(
    const float* __restrict__ scores, int64_t ld, int T, const int32_t* __restrict__ cl_arr,
    const uint32_t* __restrict__ key_hist, int kout, uint32_t* __restrict__ ws,
    int64_t ws_row_words) {
  constexpr int NT = kChunkNW * 64, SEG = 64 * kChunkEPT;
  __shared__ uint32_t lh[2048];
  __shared__ uint32_t wtot[kChunkNW];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t tot[2];
  const int r = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t* wrow = ws + (int64_t)r * ws_row_words;
  const uint32_t* h1 = key_hist ? key_hist + (int64_t)r * 2048 : nullptr;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  const int base = blockIdx.x * kChunk + w * SEG;
  float v[kChunkEPT];
  load_vals<kChunkEPT>(scores + (int64_t)r * ld, base, T, v);
  uint32_t ustar, need;
  resolve_passes<NT>(wrow, h1, T, 3, kout, lh, sh, wtot, ustar, need);
  uint32_t key[kChunkEPT];
  vals_to_keys<kChunkEPT>(v, base, T, c, key);
  if (threadIdx.x < 2) tot[threadIdx.x] = 0;
  __syncthreads();
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kChunkEPT; ++e) {
    gt += (uint32_t)__popcll(__ballot(key[e] > ustar));
    eq += (uint32_t)__popcll(__ballot(key[e] == ustar));
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
    const uint32_t* __restrict__ key_hist, int kout, int32_t offset, int32_t* __restrict__ out,
    int64_t ld_out, const uint32_t* __restrict__ ws, int64_t ws_row_words) {
  constexpr int NT = kChunkNW * 64, SEG = 64 * kChunkEPT;
  __shared__ uint32_t lh[2048];
  __shared__ uint32_t wtot[kChunkNW];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t wcnt[2][kChunkNW];
  __shared__ uint32_t bases[2];
  const int r = blockIdx.y, w = threadIdx.x >> 6;
  const uint32_t* wrow = ws + (int64_t)r * ws_row_words;
  const uint32_t* h1 = key_hist ? key_hist + (int64_t)r * 2048 : nullptr;
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  const int base = blockIdx.x * kChunk + w * SEG;
  float v[kChunkEPT];
  load_vals<kChunkEPT>(scores + (int64_t)r * ld, base, T, v);
  uint32_t ustar, need;
  resolve_passes<NT>(wrow, h1, T, 3, kout, lh, sh, wtot, ustar, need);
  // selected and equal elements in the chunks before this one: a scan of the
  // equal counts gives each chunk its share of the `need` equal elements
  const int nprev = (int)blockIdx.x, cpt = (nprev + NT - 1) / NT;
  uint32_t esum = 0;
  for (int j = 0; j < cpt; ++j) {
    const int ch = threadIdx.x * cpt + j;
    if (ch < nprev) esum += wrow[kCnt + 2 * ch + 1];
  }
  uint32_t eb = block_inclusive_sum<NT>(esum, wtot) - esum;
  uint32_t gsum = 0;
  for (int j = 0; j < cpt; ++j) {
    const int ch = threadIdx.x * cpt + j;
    if (ch < nprev) {
      const uint32_t gi = wrow[kCnt + 2 * ch], ei = wrow[kCnt + 2 * ch + 1];
      gsum += gi + (need > eb ? (ei < need - eb ? ei : need - eb) : 0u);
      eb += ei;
    }
  }
  const uint32_t out_before = block_sum<NT>(gsum, wtot);
  const uint32_t eq_before = block_sum<NT>(esum, wtot);
  if (threadIdx.x == 0) {
    bases[0] = out_before;
    bases[1] = eq_before;
  }
  uint32_t key[kChunkEPT];
  vals_to_keys<kChunkEPT>(v, base, T, c, key);
  __syncthreads();
  block_emit<kChunkNW, kChunkEPT>(key, base, ustar, need, bases[0], bases[1], c, offset,
                                  out + (int64_t)r * ld_out, (uint32_t)kout, wcnt);
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

// Block select of up to 64 * EPL blocks by one wave, no LDS: block j (lane
// j % 64, slot j / 64) ranks by its maximum's order key, blocks at or past
// ceil(cl / cbs) as -inf, ties to the lower id.  The kout-th largest key u
// is built bit by bit from the top (largest u with at least kout keys >= u),
// each count a sum of ballot popcounts; then every block above u is taken,
// and of those equal to u the kout - (#above) of lowest id, and the taken
// ids leave in ascending order (-1 for a taken block past the reachable
// ones), each slot a popcount of the lower taken ids.
template <int EPL>
__global__ __launch_bounds__(64) void select_wave_kernel(const float* __restrict__ bmax,
                                                         int64_t ld_b, int nb, int T,
                                                         const int32_t* __restrict__ cl_arr,
                                                         int cbs, int kout,
                                                         int32_t* __restrict__ ids,
                                                         int64_t ld_ids) {
  const int r = blockIdx.x, lane = threadIdx.x;
  // the maxima are requested beside compress_lens (one round trip); blocks
  // past the reachable ones are masked once both are in
  float bm[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int j = e * 64 + lane;
    bm[e] = bmax[(int64_t)r * ld_b + (j < nb ? j : 0)];
  }
  int c = cl_arr[r];
  c = c < 0 ? 0 : (c > T ? T : c);
  const int clb = (int)(((int64_t)c + cbs - 1) / cbs);
  uint32_t key[EPL];  // 0: no such block (below every real key)
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int j = e * 64 + lane;
    key[e] = j < nb ? (j < clb ? score_key(bm[e]) : kKeyNegInf) : 0u;
  }
  uint32_t u = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = u | (1u << bit);
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) cnt += (uint32_t)__popcll(__ballot(key[e] >= cand));
    if (cnt >= (uint32_t)kout) u = cand;
  }
  uint32_t above = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) above += (uint32_t)__popcll(__ballot(key[e] > u));
  const uint32_t need = (uint32_t)kout - above;
  uint32_t eq_run = 0, sel_run = 0;
  int32_t* orow = ids + (int64_t)r * ld_ids;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int j = e * 64 + lane;
    const uint64_t em = __ballot(key[e] == u);
    const bool take = key[e] > u || (key[e] == u && eq_run + lanes_below(em) < need);
    eq_run += (uint32_t)__popcll(em);
    const uint64_t tm = __ballot(take);
    if (take) orow[sel_run + lanes_below(tm)] = j < clb ? j : -1;
    sel_run += (uint32_t)__popcll(tm);
  }
}

}  // namespace idx

// ------------------------------------------------------------ host side
namespace {

// IDX_TOPK_PATH=chunked forces the multi-workgroup path for rows longer
// than 1024 (read on every call; used by tests and tuning).
bool chunked_forced() {
  const char* e = getenv("IDX_TOPK_PATH");
  return e && e[0] == 'c';
}

// Rows up to this width run in one workgroup (keys in registers).
constexpr int kRowsMaxT = 32768;

int64_t n_chunks(int T) { return ((int64_t)T + idx::kChunk - 1) / idx::kChunk; }

int64_t ws_row_words(int T) { return idx::kCnt + 2 * n_chunks(T); }

size_t chunked_ws_bytes(int R, int T) { return (size_t)R * (size_t)ws_row_words(T) * 4u; }


// Longer rows with a score histogram: several workgroups per row.
bool use_split(int T, const uint32_t* key_hist) {
  return key_hist && T > kRowsMaxT && T <= idx::kSplitMaxT && !chunked_forced();
}

size_t split_ws_bytes(int R, int T) {
  return (size_t)R * (size_t)idx::SplitLayout(T).row_words * 4u;
}

size_t split_b_lds(int T) {
  return ((size_t)2 * idx::split_padded_words((int)idx::SplitLayout(T).nwords) +
          2 * idx::kSplitCandCap) * 4u;
}

// Kernel B may use more than 64 KB of dynamic LDS; the limit is a per-device
// function attribute, raised once on each device the library runs on.
bool set_split_lds_limit() {
  static std::atomic<uint64_t> done_mask{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done_mask.load(std::memory_order_acquire) & bit)) return true;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&idx::topk_split_b_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)split_b_lds(idx::kSplitMaxT)) != hipSuccess)
    return false;
  if (bit) done_mask.fetch_or(bit, std::memory_order_acq_rel);
  return true;
}

void zero_hist(uint32_t* key_hist, int R, hipStream_t st) {
  const int64_t n = (int64_t)R * 2048;
  const int64_t g = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(idx::zero_words_kernel, dim3((unsigned)g), dim3(256), 0, st, key_hist, n);
}

idx_status topk_launch(const float* scores, int64_t ld, int R, int T, const int32_t* cl,
                       uint32_t* key_hist, int k, int32_t offset, int32_t* out,
                       int64_t ld_out, void* ws, size_t ws_bytes, hipStream_t st) {
  if (R == 0 || T == 0) return IDX_OK;
  const int kout = k < T ? k : T;
  if (k >= T) {
    hipLaunchKernelGGL(idx::topk_all_kernel, dim3((unsigned)R), dim3(256), 0, st, T, cl, offset,
                       out, ld_out);
    if (key_hist) zero_hist(key_hist, R, st);
    return idx_host::launch_status();
  }
  // rows up to 32768 in one workgroup; longer rows with a histogram over
  // several workgroups per row (split); the rest in chunks
  const bool forced = chunked_forced() && T > 1024;
  if (!forced && T <= kRowsMaxT) {
    const dim3 g((unsigned)R);
    if (T <= 2048)
      hipLaunchKernelGGL((idx::topk_rows_kernel<256, 8>), g, dim3(256), 0, st, scores, ld, T, cl,
                         key_hist, kout, offset, out, ld_out);
    else if (T <= 8192)
      hipLaunchKernelGGL((idx::topk_rows_kernel<256, 32>), g, dim3(256), 0, st, scores, ld, T, cl,
                         key_hist, kout, offset, out, ld_out);
    else
      hipLaunchKernelGGL((idx::topk_rows_kernel<1024, 32>), g, dim3(1024), 0, st, scores, ld, T,
                         cl, key_hist, kout, offset, out, ld_out);
    return idx_host::launch_status();
  }
  if (use_split(T, key_hist)) {
    if (R > 65535) return IDX_EUNSUPPORTED;
    if (!ws || ws_bytes < split_ws_bytes(R, T)) return IDX_EINVAL;
    const idx::SplitLayout L(T);
    if (!set_split_lds_limit()) return IDX_EHIP;
    hipLaunchKernelGGL(idx::topk_split_a_kernel, dim3((unsigned)L.nparts, (unsigned)R),
                       dim3(idx::kPartNW * 64), 0, st, scores, ld, T, cl, key_hist, kout,
                       (uint32_t*)ws);
    hipLaunchKernelGGL(idx::topk_split_b_kernel, dim3((unsigned)R), dim3(idx::kSplitBThreads),
                       split_b_lds(T), st, scores, ld, T, cl, key_hist, kout, offset, out, ld_out,
                       (const uint32_t*)ws);
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
  // the chunked path counts its own first digit, so a score histogram (which
  // it cannot check against the row without another pass) is only reset
  const uint32_t* h1 = nullptr;
  hipLaunchKernelGGL(idx::topk_chunk_hist_kernel<0>, grid, blk, 0, st, scores, ld, T, cl, h1,
                     kout, w, rw);
  hipLaunchKernelGGL(idx::topk_chunk_hist_kernel<1>, grid, blk, 0, st, scores, ld, T, cl, h1,
                     kout, w, rw);
  hipLaunchKernelGGL(idx::topk_chunk_hist_kernel<2>, grid, blk, 0, st, scores, ld, T, cl, h1,
                     kout, w, rw);
  hipLaunchKernelGGL(idx::topk_chunk_count_kernel, grid, blk, 0, st, scores, ld, T, cl, h1,
                     kout, w, rw);
  hipLaunchKernelGGL(idx::topk_chunk_emit_kernel, grid, blk, 0, st, scores, ld, T, cl, h1,
                     kout, offset, out, ld_out, (const uint32_t*)w, rw);
  if (key_hist) zero_hist(key_hist, R, st);
  return idx_host::launch_status();
}

size_t topk_ws_bytes(int R, int T, int k) {
  if (R <= 0 || T <= 0 || k >= T || T <= 1024) return 0;
  size_t n = chunked_ws_bytes(R, T);
  if (T > kRowsMaxT && T <= idx::kSplitMaxT) n = n > split_ws_bytes(R, T) ? n : split_ws_bytes(R, T);
  return n;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" size_t idx_topk_workspace_size(int R, int T, int index_topk) {
  return topk_ws_bytes(R, T, index_topk);
}

extern "C" idx_status idx_topk(const float* scores, int64_t ld, int R, int T,
                               const int32_t* compress_lens, uint32_t* key_hist,
                               int index_topk, int32_t offset, int32_t* out, int64_t ld_out,
                               int32_t* k_out, void* ws, size_t ws_bytes, void* stream) {
  if (R < 0 || T < 0 || index_topk <= 0) return IDX_EINVAL;
  const int kout = index_topk < T ? index_topk : T;
  if (R == 0 || T == 0) {
    if (k_out) *k_out = kout;
    return IDX_OK;
  }
  if (!scores || !compress_lens || !out) return IDX_EINVAL;
  if (ld < T || ld_out < kout) return IDX_EINVAL;
  if (k_out) *k_out = kout;
  return topk_launch(scores, ld, R, T, compress_lens, key_hist, index_topk, offset, out, ld_out,
                     ws, ws_bytes, (hipStream_t)stream);
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
  if (nb <= idx_host::kSelectWaveMaxBlocks)
    return idx_host::select_blocks_from_max(bmax, nb, R, nb, T, compress_lens, cand_block_size,
                                            candidate_topk_blocks, block_ids, ld_ids, st);
  return topk_launch(bmax, nb, R, nb, clb, nullptr, candidate_topk_blocks, 0, block_ids, ld_ids,
                     tws, tws_bytes, st);
}

// One wave per row ranks the block maxima (nb <= kSelectWaveMaxBlocks).
idx_status idx_host::select_blocks_from_max(const float* bmax, int64_t ld_b, int R, int nb, int T,
                                            const int32_t* compress_lens, int cbs, int ctb,
                                            int32_t* ids, int64_t ld_ids, hipStream_t st) {
  if (nb <= 0 || nb > kSelectWaveMaxBlocks || R <= 0) return IDX_EINVAL;
  const int kout = ctb < nb ? ctb : nb;
  if (nb <= 512)
    hipLaunchKernelGGL(idx::select_wave_kernel<8>, dim3((unsigned)R), dim3(64), 0, st, bmax, ld_b,
                       nb, T, compress_lens, cbs, kout, ids, ld_ids);
  else
    hipLaunchKernelGGL(idx::select_wave_kernel<16>, dim3((unsigned)R), dim3(64), 0, st, bmax,
                       ld_b, nb, T, compress_lens, cbs, kout, ids, ld_ids);
  return idx_host::launch_status();
}

namespace {
// idx_topk_candidates on full rows (compact = false) or on slot scores
// (compact = true: scores[r][v] is slot v's score, ld >= n_cand * cbs).
idx_status topk_candidates_impl(const float* scores, int64_t ld, int R, int T,
                                const int32_t* compress_lens, const int32_t* cand_blocks,
                                int n_cand, int cand_block_size, uint32_t* key_hist,
                                int index_topk, int32_t offset, int32_t* out, int64_t ld_out,
                                int32_t* k_out, hipStream_t st, bool compact, bool check_only) {
  if (R < 0 || T < 0 || index_topk <= 0 || n_cand <= 0 || cand_block_size <= 0) return IDX_EINVAL;
  const int kout = index_topk < T ? index_topk : T;
  if (R == 0 || T == 0) {
    if (k_out && !check_only) *k_out = kout;
    return IDX_OK;
  }
  if (!scores || !compress_lens || !cand_blocks || !out) return IDX_EINVAL;
  const int64_t V = (int64_t)n_cand * cand_block_size;
  if (ld < (compact ? V : (int64_t)T) || ld_out < kout) return IDX_EINVAL;
  if (index_topk < T && (T > idx::kCandMaxT || n_cand > idx::kCandMaxIds || V > 8192))
    return IDX_EUNSUPPORTED;
  if (check_only) return IDX_OK;
  if (k_out) *k_out = kout;
  if (index_topk >= T) {
    hipLaunchKernelGGL(idx::topk_all_kernel, dim3((unsigned)R), dim3(256), 0, st, T,
                       compress_lens, offset, out, ld_out);
    if (key_hist) zero_hist(key_hist, R, st);
    return idx_host::launch_status();
  }
  // few rows, each a latency chain: many threads per row, few keys each
  if (V <= 2048)
    hipLaunchKernelGGL((idx::topk_cand_kernel<256, 8>), dim3((unsigned)R), dim3(256), 0, st,
                       scores, ld, T, compress_lens, cand_blocks, n_cand, cand_block_size,
                       key_hist, kout, offset, out, ld_out, compact ? 1 : 0);
  else
    hipLaunchKernelGGL((idx::topk_cand_kernel<1024, 8>), dim3((unsigned)R), dim3(1024), 0, st,
                       scores, ld, T, compress_lens, cand_blocks, n_cand, cand_block_size,
                       key_hist, kout, offset, out, ld_out, compact ? 1 : 0);
  return idx_host::launch_status();
}
}  // namespace

extern "C" idx_status idx_topk_candidates(const float* scores, int64_t ld, int R, int T,
                                          const int32_t* compress_lens, const int32_t* cand_blocks,
                                          int n_cand, int cand_block_size, uint32_t* key_hist,
                                          int index_topk, int32_t offset, int32_t* out,
                                          int64_t ld_out, int32_t* k_out, void* stream) {
  return topk_candidates_impl(scores, ld, R, T, compress_lens, cand_blocks, n_cand,
                              cand_block_size, key_hist, index_topk, offset, out, ld_out, k_out,
                              (hipStream_t)stream, false, false);
}

extern "C" idx_status idx_score_topk_candidates(
    const uint16_t* q, const uint16_t* w, const uint8_t* k_cache, int64_t k_batch_stride_rows,
    int B, int S, int H, int D, int T, const int32_t* compress_lens, const int32_t* cand_blocks,
    int n_cand, int cand_block_size, float* slot_scores, int64_t ld, uint32_t* key_hist,
    int index_topk, int32_t offset, int32_t* out, int64_t ld_out, int32_t* k_out, void* stream) {
  if (B < 0 || S < 0) return IDX_EINVAL;
  const int64_t R = (int64_t)B * S;
  if (R > 0x7fffffffLL) return IDX_EINVAL;
  // the top-k's checks first: nothing launches on a call it would refuse
  const idx_status e = topk_candidates_impl(slot_scores, ld, (int)R, T, compress_lens,
                                            cand_blocks, n_cand, cand_block_size, key_hist,
                                            index_topk, offset, out, ld_out, k_out,
                                            (hipStream_t)stream, true, true);
  if (e != IDX_OK) return e;
  if (R == 0 || T == 0) {
    if (k_out) *k_out = index_topk < T ? index_topk : T;
    return IDX_OK;
  }
  const idx_status s = idx_host::score_candidates_compact(
      q, w, k_cache, k_batch_stride_rows, B, S, H, D, T, compress_lens, cand_blocks, n_cand,
      cand_block_size, slot_scores, ld, key_hist, (hipStream_t)stream);
  if (s != IDX_OK) return s;
  return topk_candidates_impl(slot_scores, ld, (int)R, T, compress_lens, cand_blocks, n_cand,
                              cand_block_size, key_hist, index_topk, offset, out, ld_out, k_out,
                              (hipStream_t)stream, true, false);
}

// The rest of a two-level step after the level-one select: the level-one
// top-k of `scores` and level two's candidate score and top-k.  On the
// split path (32768 < T <= kTwoLevelMaxT, histograms given, level two on
// the 1024-thread candidate kernel) it is two launches: the candidate score
// with kernel A of level one beside it, then kernel B and the candidate
// top-k side by side; otherwise idx_topk then idx_score_topk_candidates.
namespace {
bool set_two_level_lds_limit() {
  static std::atomic<uint64_t> done_mask{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done_mask.load(std::memory_order_acquire) & bit)) return true;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&idx::topk_split_b_cand_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)split_b_lds(idx::kTwoLevelMaxT)) != hipSuccess)
    return false;
  if (bit) done_mask.fetch_or(bit, std::memory_order_acq_rel);
  return true;
}
}  // namespace

extern "C" idx_status idx_two_level_topk(
    const float* scores, int64_t ld, uint32_t* key_hist, int32_t* out1, int64_t ld_out1, void* ws,
    size_t ws_bytes, const uint16_t* q, const uint16_t* w2, const uint8_t* k_cache,
    int64_t k_batch_stride_rows, int B, int S, int H, int D, int T, const int32_t* compress_lens,
    const int32_t* cand_blocks, int n_cand, int cand_block_size, float* slot_scores, int64_t ld2,
    uint32_t* key_hist2, int index_topk, int32_t offset, int32_t* out2, int64_t ld_out2,
    void* stream) {
  if (B < 0 || S < 0 || T < 0 || index_topk <= 0) return IDX_EINVAL;
  const int64_t R = (int64_t)B * S;
  if (R > 0x7fffffffLL) return IDX_EINVAL;
  if (R == 0 || T == 0) return IDX_OK;
  // every check of both levels before anything launches
  const int kout = index_topk < T ? index_topk : T;
  if (!scores || !compress_lens || !out1 || ld < T || ld_out1 < kout) return IDX_EINVAL;
  if (key_hist && key_hist == key_hist2) return IDX_EINVAL;  // one histogram per level
  {
    const idx_status e = topk_candidates_impl(slot_scores, ld2, (int)R, T, compress_lens,
                                              cand_blocks, n_cand, cand_block_size, key_hist2,
                                              index_topk, offset, out2, ld_out2, nullptr,
                                              (hipStream_t)stream, true, true);
    if (e != IDX_OK) return e;
  }
  hipStream_t st = (hipStream_t)stream;
  const int64_t V = (int64_t)n_cand * cand_block_size;
  const bool together = use_split(T, key_hist) && T <= idx::kTwoLevelMaxT && key_hist2 &&
                        index_topk < T && V > 2048 && R <= 65535;
  if (!together) {
    const idx_status e = topk_launch(scores, ld, (int)R, T, compress_lens, key_hist, index_topk,
                                     offset, out1, ld_out1, ws, ws_bytes, st);
    if (e != IDX_OK) return e;
    return idx_score_topk_candidates(q, w2, k_cache, k_batch_stride_rows, B, S, H, D, T,
                                     compress_lens, cand_blocks, n_cand, cand_block_size,
                                     slot_scores, ld2, key_hist2, index_topk, offset, out2, ld_out2,
                                     nullptr, stream);
  }
  if (!ws || ws_bytes < split_ws_bytes((int)R, T)) return IDX_EINVAL;
  if (!set_two_level_lds_limit()) return IDX_EHIP;
  // the candidate score, with level one's kernel A on extra workgroups
  const idx_status e = idx_host::score_candidates_compact(
      q, w2, k_cache, k_batch_stride_rows, B, S, H, D, T, compress_lens, cand_blocks, n_cand,
      cand_block_size, slot_scores, ld2, key_hist2, st, scores, ld, key_hist, (uint32_t*)ws, kout);
  if (e != IDX_OK) return e;
  hipLaunchKernelGGL(idx::topk_split_b_cand_kernel, dim3((unsigned)(2 * R)), dim3(1024),
                     split_b_lds(T), st, (int)R, scores, ld, T, compress_lens, key_hist, kout,
                     offset, out1, ld_out1, (const uint32_t*)ws, slot_scores, ld2, cand_blocks,
                     n_cand, cand_block_size, key_hist2, out2, ld_out2);
  return idx_host::launch_status();
}

// ------------------------------------------------- allocation-free top-k
// For callers that cannot allocate device memory: the workspace of
// idx_topk comes from this file-scope array instead of the caller.  Each
// device the library runs on holds its own copy until the process ends; its
// device address is looked up once per device (hipGetSymbolAddress) and
// only that address is handed to kernels.
namespace {
constexpr size_t kScratchBytes = (size_t)16 << 20;
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch array.
idx_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return IDX_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return IDX_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return IDX_EHIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return IDX_OK;
}
}  // namespace

extern "C" size_t idx_topk_noalloc_max_workspace(void) { return kScratchBytes; }

extern "C" idx_status idx_topk_noalloc(const float* scores, int64_t ld, int R, int T,
                                       const int32_t* compress_lens, uint32_t* key_hist,
                                       int index_topk, int32_t offset, int32_t* out,
                                       int64_t ld_out, int32_t* k_out, void* stream) {
  if (R < 0 || T < 0 || index_topk <= 0) return IDX_EINVAL;
  const size_t need = topk_ws_bytes(R, T, index_topk);
  if (need > kScratchBytes) return IDX_EUNSUPPORTED;
  void* ws = nullptr;
  if (need > 0 && R > 0 && T > 0 && scores && compress_lens && out) {
    const idx_status e = scratch_address(&ws);
    if (e != IDX_OK) return e;
  }
  return idx_topk(scores, ld, R, T, compress_lens, key_hist, index_topk, offset, out, ld_out,
                  k_out, ws, ws ? kScratchBytes : 0, stream);
}
