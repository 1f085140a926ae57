// score.hip -- the Indexer score on gfx950 scaled-fp4 MFMA
// ([IDX, forward: the einsum of fp4 q with index_k, relu, times weights, sum
// over heads, compress_lens mask, level-two candidate mask]).
//
// Work split: one workgroup (4 waves) per (query row r, chunk of key
// positions).  The workgroup quantises the row's H x 128 bf16 query into LDS
// (one thread per 32-value block), then each wave walks 64-key tiles:
//
//   - the contraction is v_mfma_scale_f32_32x32x64_f8f6f4 with both operands
//     e2m1 and e8m0 block scales: M = 32 heads, N = 32 keys, K = 64 dims (two
//     32-value scale blocks, one per half-wave).  A 64-key tile is
//     2 key tiles x H/32 head tiles x 2 K-steps of MFMA; the key bytes feed
//     the B operand straight from the 68-byte rows (lane n+32g loads the 16
//     code bytes of block g of key n, and the block's scale byte).
//   - query heads are assigned to M rows so that, in the 32x32 accumulator,
//     lanes 0..31 hold heads [0, H/2) and lanes 32..63 heads [H/2, H) of
//     their key.
//   - the head sum has one fixed association: each half-wave sums its own
//     half of the heads ascending, one fma(max(d, 0), w, acc) per head from
//     +0, so lane n and lane n+32 each run one chain per key tile on the
//     registers the MFMA left them; one v_permlane32_swap of the two tiles'
//     chains and one add then give lane l the score of key t0+l.
//
// The dot products are exact (integer-valued block sums times powers of two
// fit fp32 for the documented input range), so the only rounding is the
// fixed-order head sum, which the oracle performs identically.
#include "idx_common.hpp"
#include "publish_dev.hpp"
#include "row_topk.hpp"
#include "split_topk.hpp"

#include <hip/hip_ext.h>
#include <atomic>

namespace idx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

struct __attribute__((aligned(4))) u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Head carried by M-row m of head tile ht (32 heads per tile, HT tiles).
// The 32x32 f32 accumulator gives lane l, register i the row
// (i/4)*8 + (l/32)*4 + i%4, so rows with bit 2 clear sit in lanes 0..31 and
// rows with bit 2 set in lanes 32..63; this map makes register i of tile ht
// hold head 16*ht + i in the low half-wave and H/2 + 16*ht + i in the high
// half-wave, so each half-wave walks its half of the heads ascending by
// (ht, i).
template <int HT>
__device__ __forceinline__ int head_of_row(int ht, int m) {
  return ((m >> 2) & 1) * 16 * HT + ht * 16 + (m >> 3) * 4 + (m & 3);
}

constexpr int kMaxCand = 2048;  // candidate blocks per row held in LDS
#ifndef IDX_SCORE_TILE_SETS
#define IDX_SCORE_TILE_SETS 3
#endif
constexpr int kTileSets = IDX_SCORE_TILE_SETS;  // key tiles per wave held in registers

// fp4 rows: [key tile][K-step] 16 code bytes of block 2*step + lane/32, and
// the row's four scale bytes.  fp8 rows (F8): [key tile][K-step] 32 code
// bytes (two words of 16), K-half lane/32 of the step, and the row's fp32
// scale.
template <bool F8 = false>
struct KeyTileT {
  u32x4 c[2][2][F8 ? 2 : 1];
  uint32_t sc[2];
};
typedef KeyTileT<false> KeyTile;

// Virtual position v -> key position.  Plain mode scores positions
// [0, limit) directly; candidate mode (level two) walks the listed blocks.
template <bool CAND>
struct PosMap {
  const int32_t* cand;  // row's candidate block ids (in LDS), candidate mode
  int cbs;
  int nblk;   // ceil(T / cbs)
  int limit;  // positions must be < limit (= clamped compress_lens)
  int vlim;   // virtual positions must be < vlim
  __device__ __forceinline__ int pos(int v) const {  // -1 when not scored
    if (!CAND) return v < vlim ? v : -1;  // vlim <= limit
    if (v >= vlim) return -1;
    const int j = v / cbs;
    const int id = cand[j];
    if (id < 0 || id >= nblk) return -1;
    const int p = id * cbs + (v - j * cbs);
    return p < limit ? p : -1;
  }
};

// Loads are issued for every lane without branches, so the compiler can keep
// the next tile's loads in flight while the current tile computes.  A lane
// without a key reads zeros (plain mode) or row 0 of the sequence (candidate
// mode); its MFMA column is then simply not stored (columns of the
// accumulator depend only on their own key).
//
// Plain mode: v0 is uniform across the wave, so the tile's base address and
// the number of bytes left before vlim go into a buffer resource held in
// scalar registers; every lane's offset is then the same for every tile, and
// the hardware range check returns zeros for keys at or past vlim (without
// reading them).  No per-tile vector address arithmetic.
constexpr int kBufWord3 = 0x00020000;  // raw buffer, 32-bit data (gfx9 family)

// Paged key cache ([VLLM, DeepseekV4IndexerCache]: pages of 64 compressed
// positions): row t of a sequence lives in slot t % 64 of physical page
// bt_row[t / 64], page p at pages + p * page_stride bytes.  A 64-key tile of
// plain mode starts at a multiple of 64, so it is exactly one page.
constexpr int kPageRows = 64;  // compressed positions per page

struct PageMap {
  const int32_t* bt;    // [B][bt_stride] physical page ids, or null (contiguous rows)
  int64_t bt_stride;
  int64_t page_stride;  // bytes
  int n_pages;          // valid ids are [0, n_pages)
};

// Paged tiles take their page id from `page` (uniform; see the caller).
// Candidate mode on pages: bt_lds holds the row's page ids (in LDS).
template <bool CAND, bool F8 = false>
__device__ __forceinline__ KeyTileT<F8> load_tile(const uint8_t* __restrict__ kseq,
                                                  const PosMap<CAND>& pm, int v0, int lane,
                                                  bool paged = false, int page = -1,
                                                  int64_t page_stride = 0, int n_pages = 0,
                                                  const int32_t* bt_lds = nullptr) {
  KeyTileT<F8> kt;
  const int half = lane >> 5;
  if constexpr (F8) {
    // 132-byte rows: K-step s, K-half `half` is bytes 64s + 32 half of the
    // codes; the scale word sits at byte 128.  Plain mode streams through a
    // buffer resource as the fp4 path does; candidate mode maps per lane.
    if constexpr (!CAND) {
      const int left = pm.vlim - v0;
      const int nrec = left > 0 ? (left < 64 ? left : 64) * kRowBytesF8 : 0;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(kseq + (int64_t)v0 * kRowBytesF8), (short)0, nrec, kBufWord3);
      const int vs = (lane & 31) * kRowBytesF8, vc = vs + 32 * half;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int o = vc + 32 * kRowBytesF8 * t;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const auto c = __builtin_amdgcn_raw_buffer_load_b128(rs, o + 64 * st + 16 * q, 0, 0);
            kt.c[t][st][q] = u32x4{c[0], c[1], c[2], c[3]};
          }
        }
        kt.sc[t] = __builtin_amdgcn_raw_buffer_load_b32(rs, vs + 32 * kRowBytesF8 * t + 128, 0, 0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int p = pm.pos(v0 + 32 * t + (lane & 31));
        const uint8_t* row = kseq + (int64_t)(p < 0 ? 0 : p) * kRowBytesF8;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          kt.c[t][st][0] = ld16(row + 64 * st + 32 * half);
          kt.c[t][st][1] = ld16(row + 64 * st + 32 * half + 16);
        }
        kt.sc[t] = *reinterpret_cast<const uint32_t*>(row + 128);
      }
    }
    return kt;
  }
  if constexpr (!CAND) {
    const int left = pm.vlim - v0;
    int nrec = left > 0 ? (left < 64 ? left : 64) * kRowBytes : 0;
    const uint8_t* base = kseq + (int64_t)v0 * kRowBytes;
    if (paged) {
      // an id outside [0, n_pages) reads nothing (its keys read as zeros)
      const bool ok = page >= 0 && page < n_pages;
      base = kseq + (ok ? (int64_t)page * page_stride : 0);
      nrec = ok ? nrec : 0;
    }
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(base), (short)0, nrec, kBufWord3);
    const int vs = (lane & 31) * kRowBytes, vc = vs + 16 * half;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const auto c0 = __builtin_amdgcn_raw_buffer_load_b128(rs, vc + 32 * kRowBytes * t, 0, 0);
      const auto c1 = __builtin_amdgcn_raw_buffer_load_b128(rs, vc + 32 * kRowBytes * t + 32, 0, 0);
      kt.c[t][0][0] = u32x4{c0[0], c0[1], c0[2], c0[3]};
      kt.c[t][1][0] = u32x4{c1[0], c1[1], c1[2], c1[3]};
      kt.sc[t] = __builtin_amdgcn_raw_buffer_load_b32(rs, vs + 32 * kRowBytes * t + 64, 0, 0);
    }
    return kt;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int p = pm.pos(v0 + 32 * t + (lane & 31));
    const uint8_t* row = kseq + (int64_t)(p < 0 ? 0 : p) * kRowBytes;
    bool zero = false;
    if (bt_lds) {  // paged: slot p % 64 of page bt[p / 64]; an invalid id gives a zero row
      const int pgid = p < 0 ? 0 : bt_lds[p >> 6];
      zero = p >= 0 && (pgid < 0 || pgid >= n_pages);
      row = kseq + (zero || p < 0 ? 0 : (int64_t)pgid * page_stride + (int64_t)(p & 63) * kRowBytes);
    }
    kt.c[t][0][0] = ld16(row + 16 * half);
    kt.c[t][1][0] = ld16(row + 32 + 16 * half);
    kt.sc[t] = *reinterpret_cast<const uint32_t*>(row + 64);
    if (zero) {
      kt.c[t][0][0] = u32x4{0u, 0u, 0u, 0u};
      kt.c[t][1][0] = u32x4{0u, 0u, 0u, 0u};
      kt.sc[t] = 0u;
    }
  }
  return kt;
}

// relu on the bit pattern: non-negative floats are non-negative int32s and
// every negative float (and -0) is a negative int32, so max(bits, 0) is
// max(x, +0) in one integer instruction (no NaN canonicalisation).
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// One 64-key tile: 2 key tiles x HT head tiles x 2 K-steps of MFMA and the
// fixed-order head sum; returns the score of key v0 + lane for lane `lane`.
// wv[16*ht + i] is the weight of the head register i of tile ht holds in
// this lane's half-wave.  Lane n and lane n+32 sum the low and the high half
// of the heads of key n of each key tile (two chains, heads ascending, from
// +0); the swap hands the low half-wave the chains of key tile 0 and the
// high half-wave those of key tile 1, and score = low chain + high chain.
template <int HT, bool F8 = false>
__device__ __forceinline__ float head_sum_tile(const KeyTileT<F8>& kt, const v8i (&A)[HT][2],
                                               const int (&sA)[HT][2],
                                               const float (&wv)[16 * HT], int lane) {
  float ch[2] = {0.0f, 0.0f};  // this half-wave's chain for key tile 0 and 1
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      v16f acc = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
      if constexpr (F8) {
        // e4m3 operands (format code 0), 32 bytes a lane; one scale for the
        // whole row: the exponent byte of the fp32 scale is its e8m0 code
        const int scs = (int)((kt.sc[t] >> 23) & 0xffu);
        const u32x4 a0 = kt.c[t][0][0], a1 = kt.c[t][0][1], b0 = kt.c[t][1][0],
                    b1 = kt.c[t][1][1];
        const v8i B0 = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                           (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        const v8i B1 = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                           (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[ht][0], B0, acc, 0, 0, 0,
                                                              sA[ht][0], 0, scs);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[ht][1], B1, acc, 0, 0, 0,
                                                              sA[ht][1], 0, scs);
      } else {
        // the high half-wave's blocks are the odd ones: shift its scale bytes
        // down by one, then the MFMA's scale byte select (op_sel) picks byte 2s
        const int scs = (int)(kt.sc[t] >> (8 * (lane >> 5)));
        const u32x4 c0 = kt.c[t][0][0], c1 = kt.c[t][1][0];
        const v8i B0 = v8i{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, 0, 0, 0, 0};
        const v8i B1 = v8i{(int)c1.x, (int)c1.y, (int)c1.z, (int)c1.w, 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[ht][0], B0, acc, 4, 4, 0,
                                                              sA[ht][0], 0, scs);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[ht][1], B1, acc, 4, 4, 0,
                                                              sA[ht][1], 2, scs);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ch[t] = __builtin_fmaf(relu_bits(acc[i]), wv[16 * ht + i], ch[t]);
    }
  }
  // low half-wave: (low chain, high chain) of key tile 0; high half-wave:
  // the same of key tile 1
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ch[0]), __float_as_uint(ch[1]),
                                                   false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Score tile of the one-row kernel: staged in LDS, histogram in LDS.
template <int HT, bool CAND, bool F8 = false>
__device__ __forceinline__ void score_tile(const KeyTileT<F8>& kt, const v8i (&A)[HT][2],
                                           const int (&sA)[HT][2], const float (&wv)[16 * HT],
                                           const PosMap<CAND>& pm, float* __restrict__ sbuf, int v0,
                                           int vbeg, int lane, uint32_t* hist_s) {
  const float sc = head_sum_tile<HT, F8>(kt, A, sA, wv, lane);
  sbuf[v0 - vbeg + lane] = sc;  // staged in LDS, written out when the chunk is done
  if (hist_s) {
    // the head sum never yields -0 (two chains from +0, then their sum), so
    // the first key digit needs no -0 canonicalisation
    const uint32_t u = __float_as_uint(sc);
    const uint32_t bin = (u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u)) >> 21;
    // plain mode counts every lane: a lane past the chunk read a zero key and
    // scored exactly +0, and the caller removes those counts once
    if (!CAND || pm.pos(v0 + lane) >= 0) atomicAdd(&hist_s[bin], 1u);
  }
}

// Fused top-k of a row scored by one workgroup (rows up to kFusedMaxT).
struct FusedTopk {
  int kout;          // min(index_topk, T)
  int32_t offset;
  int32_t* out;      // [R][ld_out]
  int64_t ld_out;
};
constexpr int kFusedEPT = 32;                     // keys per thread in the fused ranking
constexpr int kFusedMaxT = 256 * kFusedEPT;       // 8192

// Ranks a row scored into LDS by one workgroup (limit > kout), with the
// row layout of row_topk.hpp over 256 * EPT >= limit positions.  Positions
// in [limit, 256 * EPT) rank as -inf and past T as absent; none of them can
// be taken, since the row has more than kout finite scores.  hist_lds holds
// the first-digit counts of the `limit` scores.
template <int EPT>
__device__ __forceinline__ void fused_rank(float* sbuf, uint32_t* hist_lds, uint32_t* sh,
                                           uint32_t* wtot, int limit, int T, const FusedTopk& tk,
                                           int32_t* orow) {
  const int tid = threadIdx.x;
  const int span = T < 256 * EPT ? T : 256 * EPT;
  const int wbase = row_base<EPT>();
  float v[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) v[e] = sbuf[wbase + 64 * e];
  // sh and wtot live at the end of the score buffer: every wave has its
  // scores in registers before any scan writes there
  __syncthreads();
  row_vals<EPT>(v, wbase, limit, span);  // whatever sbuf held past limit
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) mine += hist_lds[tid + 256 * j];
  const uint32_t counted = block_sum<256>(mine, wtot);
  uint32_t prefix, need, bcnt;
  int shift;
  row_select<256, EPT>(v, hist_lds, counted, span, tk.kout, sh, wtot, prefix, shift, need, bcnt);
  // the score buffer is free once the scores are in registers: it holds the
  // selection masks (the launch sizes it for them)
  row_emit<256, EPT>(v, prefix, shift, need, bcnt, limit, tk.kout, tk.offset, wbase,
                     reinterpret_cast<uint32_t*>(sbuf),
                     tk.kout <= 2048 ? reinterpret_cast<int32_t*>(hist_lds) : nullptr, wtot,
                     orow);
}

// A decode step's key publish inside its score launch (idx_publish_score;
// [IDX, forward]: the key-owning layer stores the completed group's key
// before the score reads the cache).  The new key is row T - 1, the last
// scored position, so one extra workgroup per sequence publishes it and
// scores it for the row itself, while the other workgroups score [0, T - 1)
// and never read that row: no workgroup waits for another.
struct PubFuse {
  const uint16_t* latent;  // [B][Din] bf16, one completed group per sequence
  const uint16_t* wk;      // [128][Din] bf16
  const float* gamma;      // [128] fp32
  const float* cos_sin;    // [P][rd/2][2] fp32
  uint8_t* kc;             // the key cache; row T - 1 of each sequence is written
  int Din, rd, pos;        // pos: the group's position, start_pos + 1 - ratio
  float eps;
  int on;                  // 0: no publish in this launch
};

// The query step inside the score launch ([IDX, forward]: RoPE on the query
// heads' last rd dims at position start_pos + s, then fp4_act_quant; the
// head weights times w_scale), value for value as idx_q_rope_quant computes
// it: the thread that quantises block g of head h first rotates the block's
// RoPE pairs (adjacent dims, so a pair never leaves the block), each
// product and sum rounded in fp32 and the pair to bf16; each weight is
// bf16(fp32(w) * w_scale).
struct QStep {
  const float* cos_sin;  // [P][rd/2] (cos, sin) pairs
  int rd;
  int start_pos;
  float w_scale;
  int on;  // 0: the query heads are used as given
};

// Extra outputs of the plain and candidate launches.  Plain mode: the
// maximum of each cbs-wide block of the chunk's scores (the block score of
// the candidate select), written when bmax is set; chunk starts are then
// multiples of bmax_cbs.  Candidate mode with compact: slot v's score goes
// to scores[r][v] (the slots in list order, one contiguous run per chunk)
// instead of to its position; slots without a reachable position hold
// whatever their lanes computed.
struct Epi {
  float* bmax;       // [R][bmax_ld], or null
  int64_t bmax_ld;
  int bmax_cbs;
  int compact;
  // candidate mode: the last l1_parts rows of the grid run kernel A of the
  // level-one top-k instead (split_a_part on the level-one scores): the two
  // are independent steps of a two-level step, and side by side they share
  // one launch
  int l1_parts;
  const float* l1_scores;
  int64_t l1_ld;
  const uint32_t* l1_hist;
  uint32_t* l1_ws;
  int l1_kout;
};

// The role of the extra workgroup of row r (sequence b, decode: one row per
// sequence).  It runs beside workgroups that stream the cache at full HBM
// rate, where every dependent memory round trip costs microseconds, so its
// loads are all issued up front: the latent (as fp32), the query row,
// gamma, the RoPE row and the head weights into LDS, then the whole wk
// matrix into registers, row o's first 256 values in thread o and the next
// 256 in thread o + 128 (more passes for Din > 512).  Row o's fma chain
// runs through thread o's segment and continues, through LDS, in thread
// o + 128's: the chain of the publish kernels, value for value.  Threads
// 128..255 quantise the query heads while the first segment runs.  After
// the key's publish steps, wave 0 scores the new key with the streaming
// path's own tile code (matrix-core dots and head sum) on a tile that
// holds only that key.  hist_lds: 2048 words; dyn: the score buffer, at
// least kRoleDynWords words (the fp32 latent, then the bf16 query row);
// qs: H quantised heads of 17 words (F8: 33).  F8: the key cache and the
// heads hold FP8 rows, as the fp8 score and the fp8 publish write them.
constexpr int kRoleSeg = 256;   // wk values per thread per pass
constexpr int kRoleMaxDin = 2048;
constexpr int kRoleDynWords = kRoleMaxDin + 64 * kHeadDim / 2;  // latent + query row

template <int HT, bool F8 = false>
__device__ __forceinline__ void publish_and_score_last(
    const PubFuse& pf, const PageMap& pg, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ w, int64_t kstride, int T, int r, int b, int limit, float* srow,
    uint32_t* key_hist, uint32_t* lds, float* dyn, uint32_t* qs) {
  constexpr int H = 32 * HT;
  constexpr int NW = kRoleSeg / 8;  // 16-byte words of a segment
  const int tid = threadIdx.x;
  const int o = tid & (kHeadDim - 1), half = tid >> 7;
  const int Din = pf.Din;
  float* y_s = reinterpret_cast<float*>(lds);                    // 128
  uint32_t* z_s = lds + 128;                                     // 128
  float* inv_s = reinterpret_cast<float*>(lds + 256);            // 1
  uint32_t* row = lds + (F8 ? 728 : 260);                        // 17 words (F8: 33): the new key
  float* acc_s = reinterpret_cast<float*>(lds + 280);            // 128: chains in flight
  float* gamma_s = reinterpret_cast<float*>(lds + 408);          // 128
  float* cs_s = reinterpret_cast<float*>(lds + 536);             // rd <= 128
  float* w_s = reinterpret_cast<float*>(lds + 664);              // H <= 64
  float* lat_f = dyn;                                             // Din <= 2048
  uint4* q_s = reinterpret_cast<uint4*>(dyn + kRoleMaxDin);       // H * 16 words of 16 bytes

  // the small inputs first: their LDS stores wait for them, not for wk
  const uint16_t* lat = pf.latent + (int64_t)b * Din;
  const bool lat_vec = (Din & 7) == 0 && (reinterpret_cast<uintptr_t>(lat) & 15) == 0;
  uint4 lv = uint4{0u, 0u, 0u, 0u};
  if (lat_vec && tid < Din / 8) lv = reinterpret_cast<const uint4*>(lat)[tid];  // Din <= 2048
  const float gm = tid < kHeadDim ? pf.gamma[tid] : 0.0f;
  const float csv = tid < pf.rd ? pf.cos_sin[(int64_t)pf.pos * pf.rd + tid] : 0.0f;
  const float wq = tid < H ? bf16f(w[(int64_t)r * H + tid]) : 0.0f;
  // the query row: H * 16 = 512 HT words of 16 bytes, 2 HT a thread
  constexpr int QV = H * kHeadDim / 8 / 256;
  static_assert(QV * 256 * 8 == H * kHeadDim, "whole words per thread");
  const uint4* qrow = reinterpret_cast<const uint4*>(q + (int64_t)r * H * kHeadDim);
  uint4 qv[QV];
#pragma unroll
  for (int i = 0; i < QV; ++i) qv[i] = qrow[tid + 256 * i];
  // keep wk's burst behind the small loads: their LDS stores below then
  // wait for them alone
  __builtin_amdgcn_sched_barrier(0);

  const bool vec = (Din & 7) == 0 && (reinterpret_cast<uintptr_t>(pf.wk) & 15) == 0;
  // segment g of the chain: values [256 g, min(256 (g + 1), Din)), read
  // through one range-checked resource over the whole matrix (words past
  // the segment's end are loaded, or read as zeros past the matrix, and
  // not used), so the loads need no branches
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(pf.wk), (short)0, kHeadDim * Din * 2, kBufWord3);
  auto load_seg = [&](int g, uint4 (&v)[NW]) {
    const int off = (o * Din + kRoleSeg * g) * 2;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const auto c = __builtin_amdgcn_raw_buffer_load_b128(wrs, off + 16 * j, 0, 0);
      v[j] = uint4{c[0], c[1], c[2], c[3]};
    }
  };
  // acc continued over segment g; step j + 1's latent values are read into
  // the other register set while step j computes.  The reads are issued
  // whatever the segment's length (past Din they read other words of dyn,
  // which holds kRoleDynWords >= 2048 + 8 floats, and go unused), so the
  // waits before a step's fmas cover its own reads only.
  auto run_seg = [&](int g, const uint4 (&v)[NW], float acc) {
    const int n4 = (min(kRoleSeg * (g + 1), Din) - kRoleSeg * g) / 8;
    const float4* l4 = reinterpret_cast<const float4*>(lat_f) + 2 * NW * g;
    float4 L[2][2];
    L[0][0] = l4[0];
    L[0][1] = l4[1];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      if (j + 1 < NW) {
        L[(j + 1) & 1][0] = l4[2 * j + 2];
        L[(j + 1) & 1][1] = l4[2 * j + 3];
      }
      if (j < n4) {
        const float4 la = L[j & 1][0], lb = L[j & 1][1];
        const float x[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
        const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc = __builtin_fmaf(bf16f(u[m] & 0xffffu), x[2 * m], acc);
          acc = __builtin_fmaf(bf16f(u[m] >> 16), x[2 * m + 1], acc);
        }
      }
      // one step at a time: the chain is serial anyway, and reads hoisted
      // further ahead would need the registers wk holds
      __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
  };

  uint4 wv[NW];
  if (vec) load_seg(half, wv);
  if (lat_vec) {
    if (tid < Din / 8) {
      const uint32_t u[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        lat_f[8 * tid + 2 * m] = bf16f(u[m] & 0xffffu);
        lat_f[8 * tid + 2 * m + 1] = bf16f(u[m] >> 16);
      }
    }
  } else {
    for (int i = tid; i < Din; i += 256) lat_f[i] = bf16f(lat[i]);
  }
  if (tid < kHeadDim) gamma_s[tid] = gm;
  if (tid < pf.rd) cs_s[tid] = csv;
  if (tid < H) w_s[tid] = wq;
#pragma unroll
  for (int i = 0; i < QV; ++i) q_s[tid + 256 * i] = qv[i];
  __syncthreads();

  // the query heads' quantisation from LDS, blocks (h, g) of 32 values, by
  // threads 128..255 (t = 0..127) beside the chain's first segment
  auto quant_q = [&](int t) {
    for (int blk = t; blk < 4 * H; blk += kHeadDim) {
      const int h = blk >> 2, g = blk & 3;
      const uint4* src = q_s + h * 16 + 4 * g;
      uint32_t xp[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = src[i];
        xp[4 * i] = v.x;
        xp[4 * i + 1] = v.y;
        xp[4 * i + 2] = v.z;
        xp[4 * i + 3] = v.w;
      }
      if constexpr (F8) {  // a head's four blocks sit in one quad of lanes
        uint32_t codes[8];
        const int e = quant_block128_f8(xp, codes);
#pragma unroll
        for (int i = 0; i < 8; ++i) qs[h * 33 + 8 * g + i] = codes[i];
        if (g == 0) qs[h * 33 + 32] = (uint32_t)(127 + e) << 23;
      } else {
        uint32_t codes[4];
        const int e = quant_block32(xp, codes);
#pragma unroll
        for (int i = 0; i < 4; ++i) qs[h * 17 + 4 * g + i] = codes[i];
        reinterpret_cast<uint8_t*>(qs)[h * kRowBytes + 64 + g] = (uint8_t)(e + 127);
      }
    }
  };

  if (vec) {
    const int nseg = (Din + kRoleSeg - 1) / kRoleSeg;
    const int npass = (nseg + 1) / 2;
    for (int p = 0; p < npass; ++p) {
      const int g0 = 2 * p, g1 = 2 * p + 1;
      if (half == 0) {
        acc_s[o] = run_seg(g0, wv, p == 0 ? 0.0f : acc_s[o]);
        if (p + 1 < npass) load_seg(g0 + 2, wv);
      } else if (p == 0) {
        quant_q(o);
      }
      __syncthreads();
      if (half == 1 && g1 < nseg) {
        acc_s[o] = run_seg(g1, wv, acc_s[o]);
        if (p + 1 < npass) load_seg(g1 + 2, wv);
      }
      __syncthreads();
    }
    if (tid < kHeadDim) y_s[tid] = bf16f(f32_to_bf16(acc_s[tid]));
  } else {  // element loads: one thread per chain, ascending from +0
    if (tid < kHeadDim) {
      const uint16_t* wrow = pf.wk + (int64_t)tid * Din;
      float acc = 0.0f;
      for (int i = 0; i < Din; ++i) acc = __builtin_fmaf(bf16f(wrow[i]), lat_f[i], acc);
      y_s[tid] = bf16f(f32_to_bf16(acc));
    } else {
      quant_q(tid - kHeadDim);
    }
  }
  // row T - 1: contiguous, or slot (T - 1) % 64 of its page; a page id
  // outside [0, n_pages) is not written, and the row is scored as the zero
  // row the paged score reads there
  uint8_t* dst;
  if (F8 || !pg.bt) {
    dst = pf.kc + ((int64_t)b * kstride + (T - 1)) * (F8 ? kRowBytesF8 : kRowBytes);
  } else {
    const int page = pg.bt[(int64_t)b * pg.bt_stride + (T - 1) / kPageRows];
    dst = page >= 0 && page < pg.n_pages
              ? pf.kc + (int64_t)page * pg.page_stride + (int64_t)((T - 1) % kPageRows) * kRowBytes
              : nullptr;
    if (!dst && tid < 17) row[tid] = 0u;
  }
  __syncthreads();
  publish_finish(tid, y_s, z_s, inv_s, gamma_s, cs_s, pf.rd, pf.eps, dst, F8, row);
  __syncthreads();
  if (tid < 64) {
    // the tile: key 0 of key tile 0 is the new row (lane 0 holds blocks 0
    // and 2, lane 32 blocks 1 and 3, both its scale word), every other key
    // is zero; operands and weights as the streaming workgroups hold them
    const int lane = tid;
    v8i A[HT][2];
    int sA[HT][2];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = head_of_row<HT>(ht, lane & 31);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if constexpr (F8) {  // K-step st, K-half lane/32: bytes 64 st + 32 (lane/32)
          const uint32_t* p = qs + h * 33 + 16 * st + 8 * (lane >> 5);
          A[ht][st] = v8i{(int)p[0], (int)p[1], (int)p[2], (int)p[3],
                          (int)p[4], (int)p[5], (int)p[6], (int)p[7]};
          sA[ht][st] = (int)((qs[h * 33 + 32] >> 23) & 0xffu);
        } else {
          const int g = 2 * st + (lane >> 5);
          const uint32_t* p = qs + h * 17 + 4 * g;
          A[ht][st] = v8i{(int)p[0], (int)p[1], (int)p[2], (int)p[3], 0, 0, 0, 0};
          sA[ht][st] = reinterpret_cast<const uint8_t*>(qs)[h * kRowBytes + 64 + g];
        }
      }
    }
    float wvh[16 * HT];
#pragma unroll
    for (int j = 0; j < 16 * HT; ++j) wvh[j] = w_s[(lane >> 5) * (H / 2) + j];
    KeyTileT<F8> kt;
    const u32x4 z4 = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < (F8 ? 2 : 1); ++u) kt.c[t][st][u] = z4;
      kt.sc[t] = 0u;  // scale 2^-127 on zero codes: zero dots
    }
    if ((lane & 31) == 0) {
      if constexpr (F8) {  // lane 0: bytes 64 st + 0..31, lane 32: 64 st + 32..63
        const int hw = 8 * (lane >> 5);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint32_t* p = row + 16 * st + hw;
          kt.c[0][st][0] = u32x4{p[0], p[1], p[2], p[3]};
          kt.c[0][st][1] = u32x4{p[4], p[5], p[6], p[7]};
        }
        kt.sc[0] = row[32];
      } else {
        const int hw = 4 * (lane >> 5);
        kt.c[0][0][0] = u32x4{row[hw], row[hw + 1], row[hw + 2], row[hw + 3]};
        kt.c[0][1][0] = u32x4{row[8 + hw], row[9 + hw], row[10 + hw], row[11 + hw]};
        kt.sc[0] = row[16];
      }
    }
    const float sc = head_sum_tile<HT, F8>(kt, A, sA, wvh, lane);
    if (lane == 0 && T - 1 < limit) {
      if (srow) srow[T - 1] = sc;
      if (key_hist) atomicAdd(&key_hist[(int64_t)r * 2048 + (score_key(sc) >> 21)], 1u);
    }
  }
}

// The fused kernel (TOPK) is sized for four workgroups per CU: two key
// tile sets per wave (at most 128 VGPRs) and 40 KB of LDS, the 8 KB
// histogram plus the 32 KB score buffer, which also holds the query rows
// until they are in registers and the ranking's scan words.
template <int HT, bool CAND, bool TOPK, bool F8 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TOPK ? 4 : (F8 ? 1 : 3)))) void
score_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ q4,
    const uint16_t* __restrict__ w, const uint8_t* __restrict__ kc, int64_t kstride, int S, int T,
    const int32_t* __restrict__ cl, const int32_t* __restrict__ cand, int n_cand, int cbs,
    float* __restrict__ scores, int64_t ld, uint32_t* __restrict__ key_hist, int keys_per_wg,
    FusedTopk tk, PageMap pg, PubFuse pf, Epi ep, QStep qst) {
  static_assert(!(F8 && TOPK), "the fp8 rows have no fused ranking");
  constexpr int H = 32 * HT;
  constexpr int kSets = TOPK ? 2 : kTileSets;  // key tile sets in registers
  constexpr int QW = F8 ? kRowBytesF8 / 4 : kRowBytes / 4;  // words of a quantised head
  // top-11-bit key digits of this workgroup's scores (the publish role's
  // scratch, read as 16-byte words there)
  __shared__ __attribute__((aligned(16))) uint32_t hist_lds[2048];
  __shared__ int32_t cand_s[CAND ? kMaxCand : 1];
  __shared__ uint32_t qs_own[TOPK ? 1 : H * QW];
  extern __shared__ __attribute__((aligned(16))) float sbuf[];  // this chunk's scores
  // H quantised query rows of 68 bytes; the fused kernel keeps them at the
  // start of its score buffer (kFusedMaxT words), free until the first tile
  // is scored
  uint32_t* qs = TOPK ? reinterpret_cast<uint32_t*>(sbuf) : qs_own;
  // the fused ranking's scan words: the last 16 words of the score buffer
  uint32_t* wtot = reinterpret_cast<uint32_t*>(sbuf) + kFusedMaxT - 16;
  uint32_t* sh = wtot + 8;
  // rows in reverse dispatch order: causal rows grow with their index, so the
  // longest start first and the short ones fill the end of the launch
  const int r = gridDim.x - 1 - blockIdx.x;
  const int b = r / S;
  int limit = cl[r];
  limit = limit < 0 ? 0 : (limit > T ? T : limit);

  if constexpr (CAND && !TOPK && !F8) {
    // uniform: a workgroup of level one's kernel A (see Epi)
    const int l1_first = (int)gridDim.y - ep.l1_parts;
    if (ep.l1_parts && (int)blockIdx.y >= l1_first) {
      split_a_part<256>(r, (int)blockIdx.y - l1_first, ep.l1_scores, ep.l1_ld, T, cl, ep.l1_hist,
                        ep.l1_kout, ep.l1_ws, hist_lds, qs_own, qs_own + 8);
      return;
    }
  }
  PosMap<CAND> pm;
  pm.cand = cand_s;
  pm.cbs = cbs;
  pm.nblk = CAND ? (T + cbs - 1) / cbs : 0;
  pm.limit = limit;
  if constexpr (!CAND && !TOPK) {
    // uniform: the publishing workgroup, dispatched ahead of the chunks
    if (pf.on && blockIdx.y == 0) {
      publish_and_score_last<HT, F8>(pf, pg, q, w, kstride, T, r, b, limit,
                                 scores ? scores + (int64_t)r * ld : nullptr, key_hist, hist_lds,
                                 sbuf, qs_own);
      return;
    }
  }
  // with a publish in the launch, row T - 1 is the publishing workgroup's
  const int vtotal = CAND ? n_cand * cbs : (pf.on && limit > T - 1 ? T - 1 : limit);
  const int vbeg = ((int)blockIdx.y - (pf.on ? 1 : 0)) * keys_per_wg;
  const int vend = min(vbeg + keys_per_wg, vtotal);
  // nothing to score, or (fused, scores not wanted) a row with at most kout
  // reachable positions: it keeps [0, limit) and then the lowest masked
  // positions, whatever the scores ([VLLM, _fill_short_context_topk_indices])
  if (vbeg >= vend || (TOPK && !scores && limit <= tk.kout)) {
    if (TOPK) row_keep_prefix<256>(limit, tk.kout, tk.offset, tk.out + (int64_t)r * tk.ld_out);
    return;
  }
  pm.vlim = vend;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // paged candidate mode: the row's page ids for positions < limit, in the
  // dynamic LDS after the chunk's scores
  int32_t* bt_lds = nullptr;
  if (CAND && pg.bt) {
    bt_lds = reinterpret_cast<int32_t*>(sbuf + keys_per_wg);
    const int np = (limit + kPageRows - 1) / kPageRows;
    for (int i = tid; i < np; i += 256) bt_lds[i] = pg.bt[(int64_t)b * pg.bt_stride + i];
  }
  if (CAND) {
    for (int i = tid; i < n_cand; i += 256) cand_s[i] = cand[(int64_t)r * n_cand + i];
    __syncthreads();
  }

  // The query row and the weights are requested first, then the first key
  // tiles: the query's latency overlaps the tiles' instead of queueing
  // behind them (a workgroup cannot start its loop before its query is
  // quantised).  Thread (h, g) = (tid / 4, tid % 4) loads block g of head h.
  uint4 qv[4] = {};
  uint32_t q4v[(H * 17 + 255) / 256] = {};
  if (q4) {  // uniform: the quantised rows are the LDS layout itself
    const uint32_t* src = reinterpret_cast<const uint32_t*>(q4 + (int64_t)r * H * kRowBytes);
#pragma unroll
    for (int k = 0; k < (H * 17 + 255) / 256; ++k)
      if (tid + 256 * k < H * 17) q4v[k] = src[tid + 256 * k];
  } else if (tid < 4 * H) {
    const uint4* src =
        reinterpret_cast<const uint4*>(q + ((int64_t)r * H + (tid >> 2)) * kHeadDim + 32 * (tid & 3));
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[i] = src[i];
  }
  // the query step's (cos, sin) of this thread's RoPE pairs: pair i of the
  // block is dims 32 g + 2 i and + 1, rotated when 32 g + 2 i >= D - rd
  float2 csv[16];
  const int rope_base = kHeadDim - qst.rd;
  const bool rope_blk = !F8 && !q4 && qst.on && tid < 4 * H && 32 * (tid & 3) + 32 > rope_base;
  if (rope_blk) {
    const float2* cs = reinterpret_cast<const float2*>(
        qst.cos_sin + (int64_t)(qst.start_pos + r % S) * qst.rd);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 32 * (tid & 3) + 2 * i;
      csv[i] = cs[d >= rope_base ? (d - rope_base) >> 1 : 0];
    }
  }
  // weights of the heads this lane's half-wave sums: wv[j] = w[r][H/2*half + j]
  float wv[16 * HT];
  {
    const uint16_t* wrow = w + (int64_t)r * H + (lane >> 5) * (H / 2);
#pragma unroll
    for (int j = 0; j < 16 * HT; ++j) wv[j] = bf16f(wrow[j]);
    if (qst.on)  // uniform
#pragma unroll
      for (int j = 0; j < 16 * HT; j += 2) {
        const uint32_t p = f32x2_to_bf16x2(wv[j] * qst.w_scale, wv[j + 1] * qst.w_scale);
        wv[j] = bf16f(p & 0xffffu);
        wv[j + 1] = bf16f(p >> 16);
      }
  }

  // kSets register sets of key tiles: while one tile computes, the next
  // kSets - 1 tiles of this wave are in flight
  // contiguous: the sequence's rows; paged: the page pool (plain mode only)
  const bool paged = !CAND && pg.bt;  // plain mode: pages by readlane (below)
  const uint8_t* kseq = paged ? kc : kc + (int64_t)b * kstride * (F8 ? kRowBytesF8 : kRowBytes);
  const int ntiles = (vend - vbeg + 63) >> 6;
  int j = __builtin_amdgcn_readfirstlane(wave);  // uniform: tile bases stay scalar
  // paged: lane i holds the page of this wave's i-th tile (tile j + 4i; a
  // chunk has at most 128 tiles, 32 per wave), read here once, so a tile
  // takes its page with a readlane instead of a memory access; the table is
  // read only for tiles with keys
  int pid_lane = -1;
  if (paged) {
    const int v0l = vbeg + 64 * (j + 4 * lane);
    if (v0l < vend) pid_lane = pg.bt[(int64_t)b * pg.bt_stride + (v0l >> 6)];
  }
  auto tile_page = [&](int i) {  // i: uniform tile count of this wave
    return paged ? __builtin_amdgcn_readlane(pid_lane, i < 63 ? i : 63) : -1;
  };
  int it = 0;  // tiles of this wave started
  KeyTileT<F8> buf[kSets];
#pragma unroll
  for (int i = 0; i < kSets - 1; ++i)
    buf[i] = load_tile<CAND, F8>(kseq, pm, vbeg + 64 * (j + 4 * i), lane, paged, tile_page(i),
                                 pg.page_stride, pg.n_pages, bt_lds);

  uint32_t* hist_s = (key_hist || TOPK) ? hist_lds : nullptr;
  if (hist_s)
    for (int i = tid; i < 2048; i += 256) hist_lds[i] = 0;

  // --- the query row in LDS: given quantised (q4: H rows of 68 bytes, the
  // LDS layout itself), or quantised here, thread (h, g) handling block g
  // of head h
  if constexpr (F8) {
    // fp8 heads: four threads per head (32 values each), one e4m3 scale for
    // the head's 128 values; qs holds H rows of 132 bytes
    if (tid < 4 * H) {
      const int h = tid >> 2, g = tid & 3;
      uint32_t xp[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = qv[i];
        xp[4 * i] = v.x;
        xp[4 * i + 1] = v.y;
        xp[4 * i + 2] = v.z;
        xp[4 * i + 3] = v.w;
      }
      uint32_t codes[8];
      const int e = quant_block128_f8(xp, codes);
#pragma unroll
      for (int i = 0; i < 8; ++i) qs[h * QW + 8 * g + i] = codes[i];
      if (g == 0) qs[h * QW + 32] = (uint32_t)(127 + e) << 23;
    }
  } else {
  if (q4) {  // uniform
#pragma unroll
    for (int k = 0; k < (H * 17 + 255) / 256; ++k)
      if (tid + 256 * k < H * 17) qs[tid + 256 * k] = q4v[k];
  } else if (tid < 4 * H) {
    const int h = tid >> 2, g = tid & 3;
    uint32_t xp[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = qv[i];
      xp[4 * i] = v.x;
      xp[4 * i + 1] = v.y;
      xp[4 * i + 2] = v.z;
      xp[4 * i + 3] = v.w;
    }
    if (rope_blk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (32 * g + 2 * i >= rope_base) {
          const float x0 = bf16f(xp[i] & 0xffffu), x1 = bf16f(xp[i] >> 16);
          const float c = csv[i].x, sn = csv[i].y;
          const float a = x0 * c, bb = x1 * sn, cc = x0 * sn, dd = x1 * c;
          xp[i] = f32x2_to_bf16x2(a - bb, cc + dd);
        }
      }
    }
    uint32_t codes[4];
    const int e = quant_block32(xp, codes);
#pragma unroll
    for (int i = 0; i < 4; ++i) qs[h * 17 + 4 * g + i] = codes[i];
    reinterpret_cast<uint8_t*>(qs)[h * kRowBytes + 64 + g] = (uint8_t)(e + 127);
  }
  }

  __syncthreads();

  // A operands: head tile ht, K-step s -> head head_of_row(ht, lane%32), block 2s + lane/32
  v8i A[HT][2];
  int sA[HT][2];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = head_of_row<HT>(ht, lane & 31);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (F8) {
        // K-step s, K-half lane/32: bytes 64s + 32 (lane/32) of the head
        const uint32_t* p = qs + h * QW + 16 * s + 8 * (lane >> 5);
        A[ht][s] = v8i{(int)p[0], (int)p[1], (int)p[2], (int)p[3],
                       (int)p[4], (int)p[5], (int)p[6], (int)p[7]};
        sA[ht][s] = (int)((qs[h * QW + 32] >> 23) & 0xffu);
      } else {
        const int g = 2 * s + (lane >> 5);
        const uint32_t* p = qs + h * 17 + 4 * g;
        A[ht][s] = v8i{(int)p[0], (int)p[1], (int)p[2], (int)p[3], 0, 0, 0, 0};
        sA[ht][s] = reinterpret_cast<const uint8_t*>(qs)[h * kRowBytes + 64 + g];
      }
    }
  }
  if (TOPK) __syncthreads();  // the query rows' words are score slots from here on

  float* srow = scores ? scores + (int64_t)r * ld : nullptr;
  // the loop body is unrolled over the sets so every set index is a
  // compile-time constant (the sets stay in distinct registers)
  while (true) {
#pragma unroll
    for (int u = 0; u < kSets; ++u) {
      buf[(u + kSets - 1) % kSets] =
          load_tile<CAND, F8>(kseq, pm, vbeg + 64 * (j + 4 * (kSets - 1)), lane, paged,
                              tile_page(it + kSets - 1), pg.page_stride, pg.n_pages, bt_lds);
      score_tile<HT, CAND, F8>(buf[u], A, sA, wv, pm, sbuf, vbeg + 64 * j, vbeg, lane, hist_s);
      j += 4;
      ++it;
      if (j >= ntiles) goto done;
    }
  }
done:
  // the chunk's scores leave in one coalesced pass: interleaving small score
  // stores with the key stream costs far more HBM time than one burst
  __syncthreads();
  const int n = vend - vbeg;
  // every wave scores at least one tile (a wave past the last tile scores a
  // tile of zero keys before the loop test), so max(ntiles, 4) tiles ran
  const int lanes_scored = (ntiles > 4 ? ntiles : 4) * 64;
  if (!CAND && hist_s && lanes_scored > n) {  // uniform
    // the lanes past the chunk end each counted one +0 score
    if (tid == 0) hist_lds[score_key(0.0f) >> 21] -= (uint32_t)(lanes_scored - n);
    __syncthreads();
  }
  if (TOPK && !srow) {
    // scores not wanted: only the ranking below
  } else if ((!CAND || ep.compact) && (((uintptr_t)(srow + vbeg)) & 15) == 0) {
    float4* dst = reinterpret_cast<float4*>(srow + vbeg);
    const float4* src = reinterpret_cast<const float4*>(sbuf);
    for (int i = tid; i < (n >> 2); i += 256) dst[i] = src[i];
    for (int i = (n & ~3) + tid; i < n; i += 256) srow[vbeg + i] = sbuf[i];
  } else if (CAND && ep.compact) {
    for (int i = tid; i < n; i += 256) srow[vbeg + i] = sbuf[i];
  } else {
    for (int i = tid; i < n; i += 256) {
      const int p = pm.pos(vbeg + i);
      if (p >= 0) srow[p] = sbuf[i];
    }
  }
  if (!CAND && !TOPK && ep.bmax) {
    // block maxima from the scores in LDS (cbs a power of two in [16, 1024]
    // dividing the chunk): run i of 16 positions per thread and pass, the
    // maximum of its positions before the chunk end, then a butterfly over
    // the cbs / 16 lanes of the block (all blocks at once); the block's
    // first lane writes it.  A block reaching past the chunk end stops there
    // (= at compress_lens, where the row's last chunk ends); blocks wholly
    // past compress_lens are not written (the select ranks them as -inf).
    const int rpb = ep.bmax_cbs >> 4;  // runs per block, 1..64
    const int b0 = vbeg / ep.bmax_cbs;
    // (cbs divides the chunk, so a block's runs sit in one wave and iterate
    // together: the butterfly's lanes are all active)
    for (int i = tid; 16 * i < keys_per_wg; i += 256) {
      float m = -__builtin_inff();
      const float4* src = reinterpret_cast<const float4*>(sbuf + 16 * i);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 v = src[q4];
        const int t = 16 * i + 4 * q4;
        m = t < n ? fmaxf(m, v.x) : m;
        m = t + 1 < n ? fmaxf(m, v.y) : m;
        m = t + 2 < n ? fmaxf(m, v.z) : m;
        m = t + 3 < n ? fmaxf(m, v.w) : m;
      }
      for (int d = 1; d < rpb; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
      if ((i & (rpb - 1)) == 0 && 16 * i < n)
        ep.bmax[(int64_t)r * ep.bmax_ld + b0 + i / rpb] = m;
    }
  }
  if (key_hist && !TOPK) {
    uint32_t* grow = key_hist + (int64_t)r * 2048;
    for (int i = tid; i < 2048; i += 256)
      if (hist_lds[i]) atomicAdd(&grow[i], hist_lds[i]);
  }
  if (TOPK) {
    // the whole row [0, T) is this workgroup's chunk: rank it from LDS
    int32_t* orow = tk.out + (int64_t)r * tk.ld_out;
    if (limit <= tk.kout) {
      row_keep_prefix<256>(limit, tk.kout, tk.offset, orow);
      return;
    }
    // the ranked layout only needs to cover [0, limit): 256 * EPT positions
    // with EPT sized to the row (the ranking's work is proportional to EPT)
    if (limit <= 256 * 4)
      fused_rank<4>(sbuf, hist_lds, sh, wtot, limit, T, tk, orow);
    else if (limit <= 256 * 8)
      fused_rank<8>(sbuf, hist_lds, sh, wtot, limit, T, tk, orow);
    else if (limit <= 256 * 16)
      fused_rank<16>(sbuf, hist_lds, sh, wtot, limit, T, tk, orow);
    else if (limit <= 256 * 24)
      fused_rank<24>(sbuf, hist_lds, sh, wtot, limit, T, tk, orow);
    else
      fused_rank<kFusedEPT>(sbuf, hist_lds, sh, wtot, limit, T, tk, orow);
  }
}

__global__ __launch_bounds__(256) void zero_hist_kernel(uint32_t* __restrict__ h, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    h[i] = 0u;
}

__global__ __launch_bounds__(256) void fill_neg_inf_kernel(float* __restrict__ scores, int64_t ld,
                                                           int T) {
  const int r = blockIdx.y;
  const int t0 = blockIdx.x * 2048 + threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (t0 + 256 * i < T) scores[(int64_t)r * ld + t0 + 256 * i] = -__builtin_inff();
}

}  // namespace idx

namespace {
// ------------------------------------------------------- launch timing
constexpr int kTimingSlots = 256;
hipEvent_t g_timing_ev[kTimingSlots][2] = {};
std::atomic<int> g_timing_armed{-1};  // slot of the next score launch, or -1

// Launches the score kernel, through hipExtLaunchKernel with the armed
// event pair when timing is armed.  Launches from other threads only read
// the flag, so they do not race with each other.
template <typename... Args, typename F>
idx_status launch_score(F kern, dim3 grid, size_t lds, hipStream_t st, Args... args) {
  const int slot =
      g_timing_armed.load(std::memory_order_relaxed) >= 0 ? g_timing_armed.exchange(-1) : -1;
  if (slot >= 0)
    hipExtLaunchKernelGGL(kern, grid, dim3(256), (uint32_t)lds, st, g_timing_ev[slot][0],
                          g_timing_ev[slot][1], 0u, args...);
  else
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, args...);
  return idx_host::launch_status();
}

constexpr int kMaxKeysPerWg = 8192;  // bounds the LDS score buffer (32 KB)
// paged candidate mode keeps the row's page ids in LDS too (2048 ids, 8 KB)
constexpr int kMaxPagedCandT = 131072;
// IDX_SCORE_KEYS_PER_WG (tuning): keys per workgroup, read once per process
int keys_per_wg_override() {
  static const int v = [] {
    const char* e = getenv("IDX_SCORE_KEYS_PER_WG");
    return e ? atoi(e) : 0;
  }();
  return v;
}

int pick_keys_per_wg(int64_t R, int vtotal, int slots = 256, int min_kpw = 1024) {
  if (keys_per_wg_override() > 0) {
    const int o = (keys_per_wg_override() + 255) / 256 * 256;
    return o < kMaxKeysPerWg ? o : kMaxKeysPerWg;
  }
  // about one workgroup per CU over the whole launch (256 CUs): measured on
  // the decode shapes, one workgroup of four waves per CU streams as fast as
  // two or more, and each workgroup pays the query load and quantisation
  // once; at least min_kpw keys per workgroup so that cost stays amortised
  // (1024; 512 for candidate slots, whose launches are latency-bound: on the
  // two-level workload 512 took the step from 56.9 to 55.3 us)
  // slots: the CUs left for the chunks (fewer when other workgroups of the
  // launch hold some of them)
  const int64_t total = R * (int64_t)vtotal;
  int64_t kpw = (total + slots - 1) / slots;
  if (kpw < min_kpw) kpw = min_kpw;
  if (kpw > vtotal) kpw = vtotal;
  if (kpw > kMaxKeysPerWg) kpw = kMaxKeysPerWg;
  if (kpw < 256) kpw = 256;
  return (int)((kpw + 255) / 256 * 256);
}
}  // namespace

extern "C" idx_status idx_clear_key_hist(uint32_t* key_hist, int R, void* stream) {
  if (R < 0) return IDX_EINVAL;
  if (R == 0) return IDX_OK;
  if (!key_hist) return IDX_EINVAL;
  const int64_t n = (int64_t)R * 2048;
  const int64_t g = (n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048;
  hipLaunchKernelGGL(idx::zero_hist_kernel, dim3((unsigned)g), dim3(256), 0, (hipStream_t)stream,
                     key_hist, n);
  return idx_host::launch_status();
}

namespace {
// Shared by the contiguous and the paged entry points: the key source is
// (k_cache, k_batch_stride_rows) when pg.bt is null, else the page pool.
idx_status score_impl(const uint16_t* q, const uint8_t* q4, const uint16_t* w,
                      const uint8_t* k_cache,
                      int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                      const int32_t* compress_lens, const int32_t* cand_blocks, int n_cand,
                      int cand_block_size, float* scores, int64_t ld, uint32_t* key_hist,
                      idx::PageMap pg, void* stream, bool f8 = false,
                      idx::Epi ep = idx::Epi{nullptr, 0, 0, 0},
                      idx::QStep qst = idx::QStep{nullptr, 0, 0, 1.0f, 0}) {
  if (B < 0 || S < 0 || T < 0 || H <= 0 || D <= 0) return IDX_EINVAL;
  if (D != idx::kHeadDim) return IDX_EUNSUPPORTED;
  if (H != 32 && H != 64) return IDX_EUNSUPPORTED;
  if ((int64_t)B * S == 0 || T == 0) return IDX_OK;
  if ((!q && !q4) || !w || !k_cache || !compress_lens || !scores) return IDX_EINVAL;
  // q moves as 16-byte words, quantised rows and key rows as 4-byte words
  if (!idx_host::aligned(q, 16) || !idx_host::aligned(q4, 4) || !idx_host::aligned(k_cache, 4) ||
      (pg.bt && (pg.page_stride & 3)))
    return IDX_EINVAL;
  if (cand_blocks && (n_cand <= 0 || cand_block_size <= 0)) return IDX_EINVAL;
  if (ep.compact && !cand_blocks) return IDX_EINVAL;
  // a compact row holds the n_cand * cbs slots; a full row the T positions
  const int64_t row_need = ep.compact ? (int64_t)n_cand * cand_block_size : T;
  if (ld < row_need || (!pg.bt && k_batch_stride_rows < T)) return IDX_EINVAL;
  if (cand_blocks && n_cand > idx::kMaxCand) return IDX_EUNSUPPORTED;
  const int64_t R = (int64_t)B * S;
  if (R > 0x7fffffffLL) return IDX_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  int64_t vtotal = T;
  if (cand_blocks) {
    vtotal = (int64_t)n_cand * cand_block_size;
    if (vtotal > 0x7fffffffLL) return IDX_EINVAL;
  }
  const int kpw = pick_keys_per_wg(R, (int)vtotal, 256, cand_blocks ? 512 : 1024);
  const int64_t nchunks = (vtotal + kpw - 1) / kpw;
  if (nchunks > 65535) return IDX_EINVAL;
  size_t lds = (size_t)kpw * sizeof(float);
  if (cand_blocks && pg.bt) {  // the row's page ids follow the scores in LDS
    if (T > kMaxPagedCandT) return IDX_EUNSUPPORTED;
    lds += (size_t)((T + idx::kPageRows - 1) / idx::kPageRows) * sizeof(int32_t);
  }
  if (ep.bmax && (cand_blocks || ep.bmax_cbs <= 0 || kpw % ep.bmax_cbs)) return IDX_EINVAL;
  if (cand_blocks) {
    if (R > 65535) return IDX_EUNSUPPORTED;
    // full rows: every position outside the listed blocks is -inf
    if (!ep.compact)
      hipLaunchKernelGGL(idx::fill_neg_inf_kernel, dim3((unsigned)((T + 2047) / 2048),
                                                        (unsigned)R),
                         dim3(256), 0, st, scores, ld, T);
  }
  if (ep.l1_parts && (!cand_blocks || !ep.compact || nchunks + ep.l1_parts > 65535))
    return IDX_EINVAL;
  dim3 grid((unsigned)R, (unsigned)(nchunks + ep.l1_parts));
  auto kern = H == 64 ? (cand_blocks ? idx::score_kernel<2, true, false>
                                     : idx::score_kernel<2, false, false>)
                      : (cand_blocks ? idx::score_kernel<1, true, false>
                                     : idx::score_kernel<1, false, false>);
  if (f8)
    kern = H == 64 ? (cand_blocks ? idx::score_kernel<2, true, false, true>
                                  : idx::score_kernel<2, false, false, true>)
                   : (cand_blocks ? idx::score_kernel<1, true, false, true>
                                  : idx::score_kernel<1, false, false, true>);
  return launch_score(kern, grid, lds, st, q, q4, w, k_cache,
                      k_batch_stride_rows, S, T, compress_lens, cand_blocks, n_cand,
                      cand_block_size, scores, ld, key_hist, kpw, idx::FusedTopk{0, 0, nullptr, 0},
                      pg, idx::PubFuse{}, ep, qst);
}

idx_status score_topk_impl(const uint16_t* q, const uint8_t* q4, const uint16_t* w,
                           const uint8_t* k_cache,
                           int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                           const int32_t* compress_lens, int index_topk, int32_t offset,
                           int32_t* out, int64_t ld_out, float* scores, int64_t ld,
                           idx::PageMap pg, void* stream,
                           idx::QStep qst = idx::QStep{nullptr, 0, 0, 1.0f, 0}) {
  if (B < 0 || S < 0 || T < 0 || H <= 0 || D <= 0 || index_topk <= 0) return IDX_EINVAL;
  if (D != idx::kHeadDim) return IDX_EUNSUPPORTED;
  if (H != 32 && H != 64) return IDX_EUNSUPPORTED;
  if (T > idx::kFusedMaxT) return IDX_EUNSUPPORTED;
  if ((int64_t)B * S == 0 || T == 0) return IDX_OK;
  if ((!q && !q4) || !w || !k_cache || !compress_lens || !out) return IDX_EINVAL;
  if (!idx_host::aligned(q, 16) || !idx_host::aligned(q4, 4) || !idx_host::aligned(k_cache, 4) ||
      (pg.bt && (pg.page_stride & 3)))
    return IDX_EINVAL;
  const int kout = index_topk < T ? index_topk : T;
  if ((!pg.bt && k_batch_stride_rows < T) || ld_out < kout || (scores && ld < T))
    return IDX_EINVAL;
  const int64_t R = (int64_t)B * S;
  if (R > 0x7fffffffLL) return IDX_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  // one workgroup scores and ranks each whole row
  // the score buffer spans the whole ranked layout (it then holds the
  // selection masks)
  const int kpw = (T + 255) / 256 * 256;
  const size_t lds = (size_t)idx::kFusedMaxT * sizeof(float);
  auto kern = H == 64 ? idx::score_kernel<2, false, true> : idx::score_kernel<1, false, true>;
  return launch_score(kern, dim3((unsigned)R, 1u), lds, st, q, q4, w, k_cache, k_batch_stride_rows, S,
                      T, compress_lens, (const int32_t*)nullptr, 0, 0, scores, ld,
                      (uint32_t*)nullptr, kpw, idx::FusedTopk{kout, offset, out, ld_out}, pg,
                      idx::PubFuse{}, idx::Epi{nullptr, 0, 0, 0}, qst);
}

// Page map arguments shared by the paged entry points.
idx_status page_map(const int32_t* block_table, int64_t bt_stride, int64_t page_stride,
                    int n_pages, int T, idx::PageMap& pg) {
  if (!block_table || n_pages <= 0) return IDX_EINVAL;
  if (page_stride < (int64_t)idx::kPageRows * idx::kRowBytes) return IDX_EINVAL;
  if (bt_stride < ((int64_t)T + idx::kPageRows - 1) / idx::kPageRows) return IDX_EINVAL;
  pg = idx::PageMap{block_table, bt_stride, page_stride, n_pages};
  return IDX_OK;
}
}  // namespace

extern "C" idx_status idx_score(const uint16_t* q, const uint16_t* w, const uint8_t* k_cache,
                                int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                                const int32_t* compress_lens, const int32_t* cand_blocks,
                                int n_cand, int cand_block_size, float* scores, int64_t ld,
                                uint32_t* key_hist, void* stream) {
  return score_impl(q, nullptr, w, k_cache, k_batch_stride_rows, B, S, H, D, T, compress_lens,
                    cand_blocks,
                    n_cand, cand_block_size, scores, ld, key_hist,
                    idx::PageMap{nullptr, 0, 0, 0}, stream);
}

// The candidate score with its slots written compactly (see Epi), and, when
// l1_scores is given, level one's split kernel A in the same launch.
idx_status idx_host::score_candidates_compact(const uint16_t* q, const uint16_t* w,
                                              const uint8_t* k_cache, int64_t k_batch_stride_rows,
                                              int B, int S, int H, int D, int T,
                                              const int32_t* compress_lens,
                                              const int32_t* cand_blocks, int n_cand,
                                              int cand_block_size, float* slot_scores, int64_t ld,
                                              uint32_t* key_hist, hipStream_t stream,
                                              const float* l1_scores, int64_t l1_ld,
                                              const uint32_t* l1_hist, uint32_t* l1_ws,
                                              int l1_kout) {
  if (!cand_blocks) return IDX_EINVAL;
  if (l1_scores) {
    const int parts = (int)idx::SplitLayout(T).nparts;
    return score_impl(q, nullptr, w, k_cache, k_batch_stride_rows, B, S, H, D, T, compress_lens,
                      cand_blocks, n_cand, cand_block_size, slot_scores, ld, key_hist,
                      idx::PageMap{nullptr, 0, 0, 0}, stream, false,
                      idx::Epi{nullptr, 0, 0, 1, parts, l1_scores, l1_ld, l1_hist, l1_ws, l1_kout});
  }
  return score_impl(q, nullptr, w, k_cache, k_batch_stride_rows, B, S, H, D, T, compress_lens,
                    cand_blocks, n_cand, cand_block_size, slot_scores, ld, key_hist,
                    idx::PageMap{nullptr, 0, 0, 0}, stream, false, idx::Epi{nullptr, 0, 0, 1});
}

extern "C" idx_status idx_score_select_blocks(const uint16_t* q, const uint16_t* w,
                                              const uint8_t* k_cache, int64_t k_batch_stride_rows,
                                              int B, int S, int H, int D, int T,
                                              const int32_t* compress_lens, float* scores,
                                              int64_t ld, uint32_t* key_hist,
                                              int candidate_topk_blocks, int cand_block_size,
                                              int32_t* block_ids, int64_t ld_ids, void* ws,
                                              size_t ws_bytes, void* stream) {
  // the select's argument checks first: nothing launches on a bad call
  if (B < 0 || S < 0 || T < 0 || candidate_topk_blocks <= 0 || cand_block_size <= 0)
    return IDX_EINVAL;
  const int64_t R = (int64_t)B * S;
  if (R == 0 || T == 0) return IDX_OK;
  if (!block_ids || !ws) return IDX_EINVAL;
  const int nb = (int)(((int64_t)T + cand_block_size - 1) / cand_block_size);
  const int kk = candidate_topk_blocks < nb ? candidate_topk_blocks : nb;
  if (ld_ids < kk) return IDX_EINVAL;
  if (ws_bytes < idx_select_workspace_size((int)R, T, candidate_topk_blocks, cand_block_size))
    return IDX_EINVAL;
  if (R > 65535) return IDX_EUNSUPPORTED;
  const int kpw = pick_keys_per_wg(R, T);
  const bool pow2 = (cand_block_size & (cand_block_size - 1)) == 0;
  if (nb > idx_host::kSelectWaveMaxBlocks || !pow2 || cand_block_size < 16 ||
      cand_block_size > 1024 || kpw % cand_block_size) {
    // chunks that split blocks, or more blocks than one wave ranks: the
    // two calls
    const idx_status e = idx_score(q, w, k_cache, k_batch_stride_rows, B, S, H, D, T,
                                   compress_lens, nullptr, 0, 0, scores, ld, key_hist, stream);
    if (e != IDX_OK) return e;
    return idx_select_candidate_blocks(scores, ld, (int)R, T, compress_lens, candidate_topk_blocks,
                                       cand_block_size, block_ids, ld_ids, ws, ws_bytes, stream);
  }
  float* bmax = (float*)ws;  // [R][nb], the select workspace's first region
  const idx_status e = score_impl(q, nullptr, w, k_cache, k_batch_stride_rows, B, S, H, D, T,
                                  compress_lens, nullptr, 0, 0, scores, ld, key_hist,
                                  idx::PageMap{nullptr, 0, 0, 0}, stream, false,
                                  idx::Epi{bmax, nb, cand_block_size, 0});
  if (e != IDX_OK) return e;
  return idx_host::select_blocks_from_max(bmax, nb, (int)R, nb, T, compress_lens, cand_block_size,
                                          candidate_topk_blocks, block_ids, ld_ids,
                                          (hipStream_t)stream);
}

namespace {
// idx_publish_score and idx_publish_score_fp8: the same two steps on fp4 or
// FP8 rows (f8: the key row as idx_publish_keys_fp8 writes it, the heads
// and the score as idx_score_fp8 computes them).
idx_status publish_score_impl(const uint16_t* latent, const uint16_t* wk, const float* gamma,
                              const float* cos_sin, int P, int Din, int rd, float eps,
                              int start_pos, int ratio, const uint16_t* q, const uint16_t* w,
                              uint8_t* k_cache, int64_t k_batch_stride_rows, int B, int H, int D,
                              int T, const int32_t* compress_lens, float* scores, int64_t ld,
                              uint32_t* key_hist, void* stream, bool f8) {
  // every argument of both steps is checked before either launches
  if (ratio <= 0 || start_pos < 0 || B < 0 || T < 0 || P < 0 || Din <= 0 || H <= 0 || D <= 0)
    return IDX_EINVAL;
  if (D != idx::kHeadDim || (H != 32 && H != 64)) return IDX_EUNSUPPORTED;
  if (rd < 0 || rd > D || (rd & 1) || !(eps >= 0.0f)) return IDX_EINVAL;
  if ((size_t)Din * 2 > 60 * 1024) return IDX_EUNSUPPORTED;
  if (B == 0) return IDX_OK;
  if (!latent || !wk || !gamma || !k_cache || (rd > 0 && !cos_sin) || !q || !w ||
      !compress_lens || !scores)
    return IDX_EINVAL;
  if (!idx_host::aligned(q, 16) || !idx_host::aligned(k_cache, 4)) return IDX_EINVAL;
  if (k_batch_stride_rows < T || ld < T) return IDX_EINVAL;
  const int64_t row = start_pos / ratio;  // the completed group's cache row
  const int pos = start_pos + 1 - ratio;  // its position
  if (start_pos > 0 && pos < 0) return IDX_EINVAL;
  if (rd > 0 && (start_pos > 0 ? pos : 0) >= P) return IDX_EINVAL;
  if (row >= k_batch_stride_rows) return IDX_EINVAL;
  const bool fuse = start_pos > 0 && row == (int64_t)T - 1 && Din <= idx::kRoleMaxDin;
  if (!fuse) {  // two launches in stream order: the key, then the score
    const int tcap = k_batch_stride_rows < 0x7fffffff ? (int)k_batch_stride_rows : 0x7fffffff;
    const idx_status e =
        (f8 ? idx_publish_keys_fp8 : idx_publish_keys)(latent, wk, gamma, cos_sin, P, B, 1, Din,
                                                       D, rd, eps, start_pos, ratio, k_cache,
                                                       k_batch_stride_rows, tcap, stream);
    if (e != IDX_OK) return e;
    return (f8 ? idx_score_fp8 : idx_score)(q, w, k_cache, k_batch_stride_rows, B, 1, H, D, T,
                                            compress_lens, nullptr, 0, 0, scores, ld, key_hist,
                                            stream);
  }
  // keys [0, T - 1) in chunks as idx_score would take them, and one more
  // workgroup per sequence for the published key T - 1; while those are
  // few, the chunks are sized to the CUs they leave (a CU streaming two
  // chunks would set the launch's length)
  const int kpw = pick_keys_per_wg(B, T - 1, B < 64 ? 256 - B : 256);
  const int nch = (T - 1 + kpw - 1) / kpw;
  if (nch + 1 > 65535) return IDX_EINVAL;
  auto kern = H == 64 ? idx::score_kernel<2, false, false> : idx::score_kernel<1, false, false>;
  if (f8)
    kern = H == 64 ? idx::score_kernel<2, false, false, true>
                   : idx::score_kernel<1, false, false, true>;
  // the publishing workgroup keeps the fp32 latent and the query row in
  // the score buffer
  const size_t lds = (size_t)(kpw > idx::kRoleDynWords ? kpw : idx::kRoleDynWords) * sizeof(float);
  return launch_score(kern, dim3((unsigned)B, (unsigned)(nch + 1)), lds,
                      (hipStream_t)stream, q, (const uint8_t*)nullptr, w,
                      (const uint8_t*)k_cache, k_batch_stride_rows, 1, T, compress_lens,
                      (const int32_t*)nullptr, 0, 0, scores, ld, key_hist, kpw,
                      idx::FusedTopk{0, 0, nullptr, 0}, idx::PageMap{nullptr, 0, 0, 0},
                      idx::PubFuse{latent, wk, gamma, cos_sin, k_cache, Din, rd, pos, eps, 1},
                      idx::Epi{nullptr, 0, 0, 0}, idx::QStep{nullptr, 0, 0, 1.0f, 0});
}
}  // namespace

extern "C" idx_status idx_publish_score(const uint16_t* latent, const uint16_t* wk,
                                        const float* gamma, const float* cos_sin, int P, int Din,
                                        int rd, float eps, int start_pos, int ratio,
                                        const uint16_t* q, const uint16_t* w, uint8_t* k_cache,
                                        int64_t k_batch_stride_rows, int B, int H, int D, int T,
                                        const int32_t* compress_lens, float* scores, int64_t ld,
                                        uint32_t* key_hist, void* stream) {
  return publish_score_impl(latent, wk, gamma, cos_sin, P, Din, rd, eps, start_pos, ratio, q, w,
                            k_cache, k_batch_stride_rows, B, H, D, T, compress_lens, scores, ld,
                            key_hist, stream, false);
}

extern "C" idx_status idx_publish_score_fp8(const uint16_t* latent, const uint16_t* wk,
                                            const float* gamma, const float* cos_sin, int P,
                                            int Din, int rd, float eps, int start_pos, int ratio,
                                            const uint16_t* q, const uint16_t* w,
                                            uint8_t* k_cache, int64_t k_batch_stride_rows, int B,
                                            int H, int D, int T, const int32_t* compress_lens,
                                            float* scores, int64_t ld, uint32_t* key_hist,
                                            void* stream) {
  return publish_score_impl(latent, wk, gamma, cos_sin, P, Din, rd, eps, start_pos, ratio, q, w,
                            k_cache, k_batch_stride_rows, B, H, D, T, compress_lens, scores, ld,
                            key_hist, stream, true);
}

extern "C" idx_status idx_publish_score_paged(
    const uint16_t* latent, const uint16_t* wk, const float* gamma, const float* cos_sin, int P,
    int Din, int rd, float eps, int start_pos, int ratio, const uint16_t* q, const uint16_t* w,
    uint8_t* k_pages, int64_t page_stride, int n_pages, const int32_t* block_table,
    int64_t bt_stride, int B, int H, int D, int T, const int32_t* compress_lens, float* scores,
    int64_t ld, uint32_t* key_hist, void* stream) {
  // every argument of both steps is checked before either launches
  if (ratio <= 0 || start_pos < 0 || B < 0 || T < 0 || P < 0 || Din <= 0 || H <= 0 || D <= 0)
    return IDX_EINVAL;
  if (D != idx::kHeadDim || (H != 32 && H != 64)) return IDX_EUNSUPPORTED;
  if (rd < 0 || rd > D || (rd & 1) || !(eps >= 0.0f)) return IDX_EINVAL;
  if ((size_t)Din * 2 > 60 * 1024) return IDX_EUNSUPPORTED;
  if (B == 0) return IDX_OK;
  if (!latent || !wk || !gamma || !k_pages || (rd > 0 && !cos_sin) || !q || !w ||
      !compress_lens || !scores)
    return IDX_EINVAL;
  if (!idx_host::aligned(q, 16) || !idx_host::aligned(k_pages, 4) || (page_stride & 3))
    return IDX_EINVAL;
  if (ld < T) return IDX_EINVAL;
  const int64_t row = start_pos / ratio;  // the completed group's cache row
  const int pos = start_pos + 1 - ratio;  // its position
  if (start_pos > 0 && pos < 0) return IDX_EINVAL;
  if (rd > 0 && (start_pos > 0 ? pos : 0) >= P) return IDX_EINVAL;
  // the block table covers the scored rows and the published one
  const int64_t rows = row + 1 > T ? row + 1 : T;
  if (rows > 0x7fffffffLL) return IDX_EINVAL;
  idx::PageMap pg{nullptr, 0, 0, 0};
  {
    const idx_status e = page_map(block_table, bt_stride, page_stride, n_pages, (int)rows, pg);
    if (e != IDX_OK) return e;
  }
  const bool fuse = start_pos > 0 && row == (int64_t)T - 1 && Din <= idx::kRoleMaxDin;
  if (!fuse) {  // two launches in stream order: the key, then the score
    const idx_status e = idx_publish_keys_paged(latent, wk, gamma, cos_sin, P, B, 1, Din, D, rd,
                                                eps, start_pos, ratio, k_pages, page_stride,
                                                n_pages, block_table, bt_stride, (int)rows, stream);
    if (e != IDX_OK) return e;
    return idx_score_paged(q, w, k_pages, page_stride, n_pages, block_table, bt_stride, B, 1, H,
                           D, T, compress_lens, nullptr, 0, 0, scores, ld, key_hist, stream);
  }
  // as idx_publish_score: keys [0, T - 1) in chunks, one more workgroup per
  // sequence for the published key T - 1
  const int kpw = pick_keys_per_wg(B, T - 1, B < 64 ? 256 - B : 256);
  const int nch = (T - 1 + kpw - 1) / kpw;
  if (nch + 1 > 65535) return IDX_EINVAL;
  auto kern = H == 64 ? idx::score_kernel<2, false, false> : idx::score_kernel<1, false, false>;
  const size_t lds = (size_t)(kpw > idx::kRoleDynWords ? kpw : idx::kRoleDynWords) * sizeof(float);
  return launch_score(kern, dim3((unsigned)B, (unsigned)(nch + 1)), lds,
                      (hipStream_t)stream, q, (const uint8_t*)nullptr, w,
                      (const uint8_t*)k_pages, 0, 1, T, compress_lens,
                      (const int32_t*)nullptr, 0, 0, scores, ld, key_hist, kpw,
                      idx::FusedTopk{0, 0, nullptr, 0}, pg,
                      idx::PubFuse{latent, wk, gamma, cos_sin, k_pages, Din, rd, pos, eps, 1},
                      idx::Epi{nullptr, 0, 0, 0}, idx::QStep{nullptr, 0, 0, 1.0f, 0});
}

extern "C" idx_status idx_score_fp8(const uint16_t* q, const uint16_t* w, const uint8_t* k_cache,
                                    int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                                    const int32_t* compress_lens, const int32_t* cand_blocks,
                                    int n_cand, int cand_block_size, float* scores, int64_t ld,
                                    uint32_t* key_hist, void* stream) {
  if (!q && (int64_t)B * S > 0 && T > 0) return IDX_EINVAL;
  return score_impl(q, nullptr, w, k_cache, k_batch_stride_rows, B, S, H, D, T, compress_lens,
                    cand_blocks, n_cand, cand_block_size, scores, ld, key_hist,
                    idx::PageMap{nullptr, 0, 0, 0}, stream, true);
}

extern "C" idx_status idx_score_topk(const uint16_t* q, const uint16_t* w, const uint8_t* k_cache,
                                     int64_t k_batch_stride_rows, int B, int S, int H, int D,
                                     int T, const int32_t* compress_lens, int index_topk,
                                     int32_t offset, int32_t* out, int64_t ld_out, float* scores,
                                     int64_t ld, void* stream) {
  return score_topk_impl(q, nullptr, w, k_cache, k_batch_stride_rows, B, S, H, D, T,
                         compress_lens, index_topk, offset, out, ld_out, scores, ld,
                         idx::PageMap{nullptr, 0, 0, 0}, stream);
}

namespace {
// The query step's arguments (as idx_q_rope_quant checks them).
idx_status qstep_args(const float* cos_sin, int P, int rd, int start_pos, int S, int D,
                      float w_scale, idx::QStep& qs) {
  if (P < 0 || start_pos < 0 || rd < 0 || rd > D || (rd & 1)) return IDX_EINVAL;
  if (rd > 0 && (!cos_sin || !idx_host::aligned(cos_sin, 8) ||
                 (int64_t)start_pos + S - 1 >= P))  // every position in the table
    return IDX_EINVAL;
  qs = idx::QStep{cos_sin, rd, start_pos, w_scale, 1};
  return IDX_OK;
}
}  // namespace

extern "C" idx_status idx_score_qrope(const uint16_t* q, const uint16_t* w_raw, float w_scale,
                                      const float* cos_sin, int P, int rd, int start_pos,
                                      const uint8_t* k_cache, int64_t k_batch_stride_rows, int B,
                                      int S, int H, int D, int T, const int32_t* compress_lens,
                                      float* scores, int64_t ld, uint32_t* key_hist,
                                      void* stream) {
  if (D != idx::kHeadDim && D > 0) return IDX_EUNSUPPORTED;
  idx::QStep qs;
  const idx_status e = qstep_args(cos_sin, P, rd, start_pos, S < 0 ? 0 : S, D, w_scale, qs);
  if (e != IDX_OK) return e;
  return score_impl(q, nullptr, w_raw, k_cache, k_batch_stride_rows, B, S, H, D, T, compress_lens,
                    nullptr, 0, 0, scores, ld, key_hist, idx::PageMap{nullptr, 0, 0, 0}, stream,
                    false, idx::Epi{nullptr, 0, 0, 0}, qs);
}

extern "C" idx_status idx_score_topk_qrope(const uint16_t* q, const uint16_t* w_raw,
                                           float w_scale, const float* cos_sin, int P, int rd,
                                           int start_pos, const uint8_t* k_cache,
                                           int64_t k_batch_stride_rows, int B, int S, int H, int D,
                                           int T, const int32_t* compress_lens, int index_topk,
                                           int32_t offset, int32_t* out, int64_t ld_out,
                                           float* scores, int64_t ld, void* stream) {
  if (D != idx::kHeadDim && D > 0) return IDX_EUNSUPPORTED;
  idx::QStep qs;
  const idx_status e = qstep_args(cos_sin, P, rd, start_pos, S < 0 ? 0 : S, D, w_scale, qs);
  if (e != IDX_OK) return e;
  return score_topk_impl(q, nullptr, w_raw, k_cache, k_batch_stride_rows, B, S, H, D, T,
                         compress_lens, index_topk, offset, out, ld_out, scores, ld,
                         idx::PageMap{nullptr, 0, 0, 0}, stream, qs);
}

extern "C" idx_status idx_score_paged(const uint16_t* q, const uint16_t* w, const uint8_t* k_pages,
                                      int64_t page_stride, int n_pages,
                                      const int32_t* block_table, int64_t bt_stride, int B, int S,
                                      int H, int D, int T, const int32_t* compress_lens,
                                      const int32_t* cand_blocks, int n_cand,
                                      int cand_block_size, float* scores, int64_t ld,
                                      uint32_t* key_hist, void* stream) {
  idx::PageMap pg{nullptr, 0, 0, 0};
  if (T > 0 && B > 0 && S > 0) {  // the page map matters only when there is work
    const idx_status e = page_map(block_table, bt_stride, page_stride, n_pages, T, pg);
    if (e != IDX_OK) return e;
  }
  return score_impl(q, nullptr, w, k_pages, 0, B, S, H, D, T, compress_lens, cand_blocks, n_cand,
                    cand_block_size, scores, ld, key_hist, pg, stream);
}

extern "C" idx_status idx_score_topk_paged(const uint16_t* q, const uint16_t* w,
                                           const uint8_t* k_pages, int64_t page_stride,
                                           int n_pages, const int32_t* block_table,
                                           int64_t bt_stride, int B, int S, int H, int D, int T,
                                           const int32_t* compress_lens, int index_topk,
                                           int32_t offset, int32_t* out, int64_t ld_out,
                                           float* scores, int64_t ld, void* stream) {
  idx::PageMap pg{nullptr, 0, 0, 0};
  if (T > 0 && B > 0 && S > 0) {  // the page map matters only when there is work
    const idx_status e = page_map(block_table, bt_stride, page_stride, n_pages, T, pg);
    if (e != IDX_OK) return e;
  }
  return score_topk_impl(q, nullptr, w, k_pages, 0, B, S, H, D, T, compress_lens, index_topk,
                         offset, out, ld_out, scores, ld, pg, stream);
}

extern "C" idx_status idx_score_q4(const uint8_t* q_rows, const uint16_t* w,
                                   const uint8_t* k_cache, int64_t k_batch_stride_rows, int B,
                                   int S, int H, int D, int T, const int32_t* compress_lens,
                                   const int32_t* cand_blocks, int n_cand, int cand_block_size,
                                   float* scores, int64_t ld, uint32_t* key_hist, void* stream) {
  return score_impl(nullptr, q_rows, w, k_cache, k_batch_stride_rows, B, S, H, D, T,
                    compress_lens, cand_blocks, n_cand, cand_block_size, scores, ld, key_hist,
                    idx::PageMap{nullptr, 0, 0, 0}, stream);
}

extern "C" idx_status idx_score_topk_q4(const uint8_t* q_rows, const uint16_t* w,
                                        const uint8_t* k_cache, int64_t k_batch_stride_rows,
                                        int B, int S, int H, int D, int T,
                                        const int32_t* compress_lens, int index_topk,
                                        int32_t offset, int32_t* out, int64_t ld_out,
                                        float* scores, int64_t ld, void* stream) {
  return score_topk_impl(nullptr, q_rows, w, k_cache, k_batch_stride_rows, B, S, H, D, T,
                         compress_lens, index_topk, offset, out, ld_out, scores, ld,
                         idx::PageMap{nullptr, 0, 0, 0}, stream);
}

extern "C" idx_status idx_timing_arm(int slot) {
  if (slot < 0 || slot >= kTimingSlots) return IDX_EINVAL;
  for (int i = 0; i < 2; ++i)
    if (!g_timing_ev[slot][i] && hipEventCreate(&g_timing_ev[slot][i]) != hipSuccess)
      return IDX_EHIP;
  g_timing_armed.store(slot);
  return IDX_OK;
}

extern "C" idx_status idx_timing_read(int slot, float* ms) {
  if (slot < 0 || slot >= kTimingSlots || !ms || !g_timing_ev[slot][1]) return IDX_EINVAL;
  if (hipEventSynchronize(g_timing_ev[slot][1]) != hipSuccess) return IDX_EHIP;
  return hipEventElapsedTime(ms, g_timing_ev[slot][0], g_timing_ev[slot][1]) == hipSuccess
             ? IDX_OK
             : IDX_EHIP;
}
