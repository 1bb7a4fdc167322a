// Per-query top-k selection, selection bitmask and tile classes (gfx950).
//
// Source: "DeepSeek3.2: Onboard sparse attention", Background (the top-k is a
// non-parametric choice of the keys each query attends to) and "What this PR
// does", item 1 (top-k indices and an index mask); "Support Ring Attention
// with DeepSeek DSA Sparse Indexer", Forward Flow (the index mask is
// [batch, S, S], shared by all heads, tiled into partial-mask blocks).
//
// Keys may be compressed blocks ("Add Flash Attention Support to Deepseek v4",
// Description): Sk keys per row, key s visible to query t when s <= (t + 1) /
// ratio - 1, so a row's keys are 0 .. L - 1 with L = (t + 1) / ratio, and the
// mask rows are ceil(Sk / 64) words. ratio 1 and Sk = S is token-level DSA;
// segment IDs come only with ratio 1.
//
// Selection rule: n = min(K, |valid(t)|) keys. Larger scores win. Among equal
// scores the smaller key position wins, and -0 equals +0.
//
// Three kernels by row length L = t + 1 (with segment IDs, by the span from
// the row's first same-segment key to t):
//   * L <= 4096: one wave per row, the row's keys in VGPRs (topk_wave_kernel);
//   * longer rows, one workgroup each: one read of the row that lists only the keys above a
//     sampled lower bound of the threshold (topk_stash_kernel);
//   * rows that list falls short for, and any row when K is too large for
//     the list: a multi-pass kernel that re-reads the row (topk_long_kernel).
// All of them find the K-th largest key T exactly, through a 2048-bin
// histogram that is monotone in the score (equal scores share a bin) and
// then the keys of T's bin; c_gt = #{key > T} and c_eq = K - c_gt ties at T
// are taken, lowest positions first. |valid| <= K takes every valid key; a
// causal-only row with L <= K never reads its scores. Each kernel emits the
// ascending index list and the row's u64 mask words together.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace dsa {

constexpr int kNB = 2048;  // histogram bins

// A score's bits in a 32-bit register (bf16 in the high half, as a float) and
// its value
template <typename ST> struct ScoreBits;
template <> struct ScoreBits<float> {
  __device__ static __forceinline__ uint32_t load(const float* p, int s) { return __float_as_uint(p[s]); }
  __device__ static __forceinline__ float value(uint32_t b) { return __uint_as_float(b); }
};
template <> struct ScoreBits<uint16_t> {
  __device__ static __forceinline__ uint32_t load(const uint16_t* p, int s) { return (uint32_t)p[s] << 16; }
  __device__ static __forceinline__ float value(uint32_t b) { return __uint_as_float(b & 0xffff0000u); }
};

template <typename ST> struct ScoreLoad;
template <> struct ScoreLoad<float> {
  __device__ static __forceinline__ float get(const float* p, int s) { return p[s]; }
};
template <> struct ScoreLoad<uint16_t> {
  __device__ static __forceinline__ float get(const uint16_t* p, int s) { return bf2f(p[s]); }
};

// inverse of fkey for a valid (non-zero) key
__device__ __forceinline__ float kfloat(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// first index-list entry of a row that topk_wave_kernel leaves to the long-row kernels
constexpr int32_t kLongRow = -2;

// Rows whose keys fit kWaveWords 64-key words from their first valid word go
// to topk_wave_kernel, one wave per row.
constexpr int kWaveWords = 64;

// First position s <= t whose segment ID is seg_t (t's own), by one wave: a
// forward scan over [0, t], 16 positions per lane and step (all loads of a
// step in flight together). With packed documents it is the start of t's
// document, and valid(t) lies in [first, t] for any segment IDs, so the
// selection only needs the words from first / 64 on.
__device__ int first_same_segment_wave(const int32_t* segb, int t, int seg_t) {
  const int lane = threadIdx.x & 63;
  constexpr int kStep = 16;
  for (int base = 0; base <= t; base += 64 * kStep) {
    int v[kStep];
#pragma unroll
    for (int j = 0; j < kStep; ++j) {
      const int p = base + 64 * j + lane;
      v[j] = p <= t ? segb[p] : 0;
    }
#pragma unroll
    for (int j = 0; j < kStep; ++j) {
      const uint64_t m = __ballot(base + 64 * j + lane <= t && v[j] == seg_t);
      if (m) return base + 64 * j + (int)__builtin_ctzll(m);
    }
  }
  return t;  // not reached: seg[t] == seg_t
}

// Per-wave scratch of topk_wave_kernel: a histogram and a candidate list
struct WaveTopkShared {
  uint32_t hist[kNB];
  uint32_t cand[64];
  uint64_t words[kWaveWords];
};

// Rows whose keys lie within kWaveWords words (4096 keys): one wave per row,
// four rows per workgroup, and no workgroup barrier. Lane l holds position l
// of each of the row's words, so a row's keys sit in 64 VGPRs per lane.
//   * The K-th largest key T: the keys (order-preserving integers, 0 for
//     invalid positions) are binned into 2048 bins over [min, max] by their
//     top bits in the wave's own LDS histogram; a suffix scan over the lanes
//     finds T's bin. A bin of at most 64 keys is ranked directly (each lane
//     one candidate, compared with every other through readlane); a crowded
//     bin is binned again over its own key interval, until one key is left.
//   * Compaction walks the words in order with running counts of the keys
//     above T and tied at T: a ballot per word gives its mask word, and
//     ballot/mbcnt give each selected key its slot. Ties at T go to the lowest
//     positions.
// Longest rows first. With segment IDs, a row's span from its first
// same-segment key must fit kWaveWords words; wider rows get kLongRow in
// their first index entry and are left to the long-row kernels.
template <typename ST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void topk_wave_kernel(const ST* __restrict__ scores, int64_t ld,
                                                        const int32_t* __restrict__ seg, int B, int S,
                                                        int Sk, int ratio, int K, int row0, int nrows, int nreg,
                                                        int32_t* __restrict__ idx,
                                                        uint64_t* __restrict__ bits) {
  __shared__ WaveTopkShared shw[4];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int item = (int)blockIdx.x * 4 + wid;
  if (item >= nreg * B) return;  // the whole wave: nothing in this kernel waits for other waves
  WaveTopkShared& sh = shw[wid];
  const int b = item % B, r = nreg - 1 - item / B;  // longest rows first
  const int t = row0 + r;
  const int tk = (t + 1) / ratio - 1, L = tk + 1;  // last visible key, row length
  const int W = (Sk + 63) / 64;
  int32_t* idx_row = idx + ((size_t)b * S + t) * K;
  uint64_t* bits_row = bits + ((size_t)b * S + t) * W;
  const ST* row = scores + ((size_t)b * nrows + r) * ld;
  const int32_t* segb = seg ? seg + (size_t)b * S : nullptr;

  if (!segb && L <= K) {
    // causal-only row with at most K keys: every key 0..t, no score read;
    // 16-byte stores when the rows are 16-byte aligned (K a multiple of 4)
    if ((K & 3) == 0) {
      for (int i = 4 * lane; i < K; i += 256)
        *(int4*)(idx_row + i) = make_int4(i < L ? i : -1, i + 1 < L ? i + 1 : -1, i + 2 < L ? i + 2 : -1,
                                          i + 3 < L ? i + 3 : -1);
    } else {
      for (int i = lane; i < K; i += 64) idx_row[i] = i < L ? i : -1;
    }
    for (int w = lane; w < W; w += 64)
      bits_row[w] = w < L / 64 ? ~0ull : (w == L / 64 && (L & 63) ? (1ull << (L & 63)) - 1ull : 0ull);
    return;
  }
  int wb = 0, seg_t = 0;
  if (segb) {
    seg_t = segb[t];
    wb = __builtin_amdgcn_readfirstlane(first_same_segment_wave(segb, t, seg_t) / 64);
    if (t / 64 - wb + 1 > kWaveWords) {
      if (lane == 0) idx_row[0] = kLongRow;
      return;
    }
  }
  const int nw = tk / 64 - wb + 1;  // the row's words from wb on
  const int s_lane = 64 * wb + lane;  // this lane's position in word wb
  // keys: 0 for positions that are not valid; first 1 for the valid ones
  uint32_t key[kWaveWords];
  uint32_t n_valid = 0;
  if (segb) {
#pragma unroll
    for (int j = 0; j < kWaveWords; ++j) key[j] = (j < nw && s_lane + 64 * j <= tk) ? (uint32_t)segb[s_lane + 64 * j] : 0u;
#pragma unroll
    for (int j = 0; j < kWaveWords; ++j) {
      key[j] = (j < nw && s_lane + 64 * j <= tk && (int)key[j] == seg_t) ? 1u : 0u;
      n_valid += (uint32_t)__popcll(__ballot(key[j] != 0u));
    }
  } else {  // only the last word can hold positions past t
#pragma unroll
    for (int j = 0; j < kWaveWords; ++j) key[j] = j < nw - 1 ? 1u : (j == nw - 1 && s_lane + 64 * j <= tk) ? 1u : 0u;
    n_valid = (uint32_t)L;
  }
  // the K-th largest key T, how many of the keys equal to T are taken
  // (c_eq), and how many there are (n_eq); a row that keeps every valid key
  // has T = 1 with all of its keys tied at T
  uint32_t T = 1, c_eq = n_valid, n_eq = n_valid;
  if (n_valid > (uint32_t)K) {
    // the scores of the valid positions, all loads in flight at once, into
    // the key registers as raw bits; positions that are not valid hold
    // 0xffffffff, a NaN pattern no (finite) score has
#pragma unroll
    for (int j = 0; j < kWaveWords; ++j)
      key[j] = (j < nw && key[j]) ? ScoreBits<ST>::load(row, s_lane + 64 * j) : 0xffffffffu;
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < kWaveWords; ++j) {
      const uint32_t kk = key[j] != 0xffffffffu ? fkey(ScoreBits<ST>::value(key[j])) : 0u;
      key[j] = kk;
      kmin = min(kmin, kk - 1u);  // 0 (not valid) wraps to the largest value
      kmax = max(kmax, kk);
    }
    kmin = wave_umin(kmin) + 1u;
    kmax = wave_umax(kmax);
    uint32_t klo = kmin, khi = kmax, need = (uint32_t)K;
    n_eq = 0;
    while (klo != khi) {
      const uint32_t span = khi - klo;
      const int nbits = 32 - __clz(span);
      const int shift = nbits > 11 ? nbits - 11 : 0;
#pragma unroll
      for (int i = 0; i < kNB / 256; ++i) *(u32x4*)&sh.hist[4 * (64 * i + lane)] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < kWaveWords; ++j) {
        const uint32_t d = key[j] - klo;  // keys outside [klo, khi] (and 0) wrap above span
        if (d <= span) atomicAdd(&sh.hist[d >> shift], 1u);
      }
      // lane l holds bins [32l, 32l+32); counts above a lane's bins by a
      // scan over the lanes, then the lane walks its own bins downwards
      // (read again from LDS, so no bin counts stay in registers)
      uint32_t tot = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4 x = *(const u32x4*)&sh.hist[32 * lane + 4 * i];
        tot += x[0] + x[1] + x[2] + x[3];
      }
      const uint32_t pre = wave_incl_scan(tot);
      uint32_t running = __builtin_amdgcn_readlane(pre, 63) - pre;  // keys in bins of higher lanes
      int fb = -1;
      uint32_t fab = 0, fcnt = 0;
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        const u32x4 x = *(const u32x4*)&sh.hist[32 * lane + 4 * i];
#pragma unroll
        for (int r = 3; r >= 0; --r) {
          if (running < need && running + x[r] >= need) {
            fb = 32 * lane + 4 * i + r;
            fab = running;
            fcnt = x[r];
          }
          running += x[r];
        }
      }
      const int src = (int)__builtin_ctzll(__ballot(fb >= 0));
      const uint32_t bstar = (uint32_t)__builtin_amdgcn_readlane(fb, src);
      need -= (uint32_t)__builtin_amdgcn_readlane((int)fab, src);
      const uint32_t cnt = (uint32_t)__builtin_amdgcn_readlane((int)fcnt, src);
      const uint32_t nlo = klo + (bstar << shift);
      const uint32_t nhi = shift == 0 ? nlo : min(khi, nlo + ((1u << shift) - 1u));
      n_eq = cnt;  // the bin's keys, all equal once the bin is one value
      if (nlo != nhi && cnt <= 64u) {
        // rank the bin's keys directly: the candidate with #greater < need <=
        // #greater + #equal is T
        uint32_t nc = 0;
#pragma unroll
        for (int j = 0; j < kWaveWords; ++j) {
          const bool inb = key[j] - nlo <= nhi - nlo;
          const uint64_t m = __ballot(inb);
          if (inb) sh.cand[nc + lanes_below(m)] = key[j];
          nc += (uint32_t)__popcll(m);
        }
        const uint32_t ki = lane < (int)nc ? sh.cand[lane] : 0u;
        uint32_t gt = 0, eq = 0;
        for (uint32_t jj = 0; jj < nc; ++jj) {
          const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)ki, (int)jj);
          gt += kj > ki;
          eq += kj == ki;
        }
        const int hit = (int)__builtin_ctzll(__ballot(lane < (int)nc && gt < need && need <= gt + eq));
        klo = khi = (uint32_t)__builtin_amdgcn_readlane((int)ki, hit);
        need -= (uint32_t)__builtin_amdgcn_readlane((int)gt, hit);
        n_eq = (uint32_t)__builtin_amdgcn_readlane((int)eq, hit);
        break;
      }
      klo = nlo;
      khi = nhi;
    }
    if (kmin == kmax) n_eq = n_valid;  // every valid key is the same value
    T = klo;
    c_eq = need;
  }

  // compaction, words in order with running counts of selected keys; when
  // every key tied at T is taken a key is selected iff key >= T, else the
  // ties at T go to the lowest positions
  uint32_t nsel = 0, eb = 0;
  // the mask words go to the wave's LDS slice, then out in one store
  auto put_word = [&](int j, uint64_t m) {
    if (lane == 0) sh.words[j] = m;
  };
  if (n_eq == c_eq) {
#pragma unroll
    for (int j = 0; j < kWaveWords; ++j) {
      if (j < nw) {  // wave-uniform
        const bool sel = key[j] >= T;
        const uint64_t selm = __ballot(sel);
        if (sel) idx_row[nsel + lanes_below(selm)] = s_lane + 64 * j;
        put_word(j, selm);
        nsel += (uint32_t)__popcll(selm);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kWaveWords; ++j) {
      if (j < nw) {  // wave-uniform
        const bool eq = key[j] == T;
        const uint64_t eqm = __ballot(eq);
        const bool sel = key[j] > T || (eq && eb + lanes_below(eqm) < c_eq);
        const uint64_t selm = __ballot(sel);
        if (sel) idx_row[nsel + lanes_below(selm)] = s_lane + 64 * j;
        put_word(j, selm);
        nsel += (uint32_t)__popcll(selm);
        eb += (uint32_t)__popcll(eqm);
      }
    }
  }
  if (lane < nw) bits_row[wb + lane] = sh.words[lane];
  for (int w = lane; w < wb; w += 64) bits_row[w] = 0ull;
  for (int w = wb + nw + lane; w < W; w += 64) bits_row[w] = 0ull;
  for (int i = (int)nsel + lane; i < K; i += 64) idx_row[i] = -1;
}

// ---- multi-pass selection of a long row (any K; the rows the single-read
// kernel below leaves): one workgroup per row, the row's scores read from
// global memory in every pass. Wave w walks one contiguous range of the row's
// 64-key words in order, lane = key position in the word, so every count it
// needs is a running scalar: no per-word arrays.
//   1. The histogram's value range comes from a strided sample of 1024 valid
//      scores. Values outside it go to the edge bins, so the bins stay
//      monotone in the value (equal scores share a bin) and the result stays
//      exact; a badly placed range only makes step 3 take its slow branch.
//   2. A 2048-bin histogram over the sampled range locates the bin b* of the
//      K-th largest score.
//   3. One pass counts, per wave, the keys in bins above b*, and collects the
//      keys of bin b* (key and position). The K-th largest key T is found by
//      ranking them directly; the candidates above or at T are then added to
//      their waves' counts. A crowded b* (more candidates than the list
//      holds) falls back to radix passes over the key interval of b*, and one
//      more pass counts each wave's keys above and at T.
//   4. An exclusive prefix over the waves' counts gives each wave its first
//      slot; the last pass walks the words in order and writes the ascending
//      index list (ties at T from the lowest positions) and, 64 words per
//      store, the mask words.
constexpr int kMaxLW = 16;        // most waves per workgroup
constexpr int kLCand = 256;       // candidates ranked directly (one per thread)
constexpr int kSample = 1024;     // scores sampled for the histogram range

struct LongShared {
  uint32_t hist[kNB + 1];         // + a bin that invalid positions count into
  uint32_t cand_key[kLCand];
  uint32_t cand_pos[kLCand];
  uint32_t red_u[2 * kMaxLW];
  float red_f[2 * kMaxLW];
  uint32_t wave_g[kMaxLW], wave_e[kMaxLW];
  uint32_t found_bin, found_above, ncand, thresh, thresh_above;
};

template <int NW> __device__ __forceinline__ void block_minmax_f(float& mn, float& mx, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) { red[wid] = mn; red[NW + wid] = mx; }
  __syncthreads();
  mn = red[0];
  mx = red[NW];
#pragma unroll
  for (int i = 1; i < NW; ++i) { mn = fminf(mn, red[i]); mx = fmaxf(mx, red[NW + i]); }
  __syncthreads();
}
template <int NW> __device__ __forceinline__ void block_minmax_u(uint32_t& mn, uint32_t& mx, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  mn = wave_umin(mn);
  mx = wave_umax(mx);
  if (lane == 0) { red[wid] = mn; red[NW + wid] = mx; }
  __syncthreads();
  mn = red[0];
  mx = red[NW];
#pragma unroll
  for (int i = 1; i < NW; ++i) { mn = min(mn, red[i]); mx = max(mx, red[NW + i]); }
  __syncthreads();
}

// Largest bin b of hist[0..kNB) with count(bins >= b) >= need, for NT threads;
// writes b and count(bins > b). Needs count(all bins) >= need >= 1.
template <int NT>
__device__ __forceinline__ void find_bin_n(const uint32_t* hist, uint32_t need, uint32_t* red, uint32_t& found_bin,
                           uint32_t& found_above, uint32_t* total = nullptr) {
  constexpr int PER = kNB / NT, NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t c[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) { c[i] = hist[PER * tid + i]; tot += c[i]; }
  // suffix sum over the lanes at or above this one (they hold higher bins)
  const uint32_t pre = wave_incl_scan(tot);
  const uint32_t incl = __builtin_amdgcn_readlane(pre, 63) - pre + tot;
  if (lane == 0) red[wid] = incl;  // wave total
  __syncthreads();
  uint32_t running = incl - tot;  // keys in bins above this thread's chunk
  for (int w2 = wid + 1; w2 < NW; ++w2) running += red[w2];
  if (total) {
    uint32_t all = 0;
    for (int w2 = 0; w2 < NW; ++w2) all += red[w2];
    *total = all;
  }
  __syncthreads();
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) {
    if (running < need && running + c[i] >= need) {
      found_bin = PER * tid + i;
      found_above = running;
    }
    running += c[i];
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

// One row t of one batch row: scores `row` (positions 0..t), segment IDs
// `segb` of that batch row (SEG), outputs idx_row / bits_row. sh and segw
// (one u64 per 64-key word, SEG) are the workgroup's LDS.
template <typename ST, bool SEG, int NW>
__device__ void multipass_row(const ST* __restrict__ row, const int32_t* __restrict__ segb, int W, int K, int t,
                              int L, int32_t* __restrict__ idx_row, uint64_t* __restrict__ bits_row, LongShared& sh,
                              uint64_t* segw) {
  constexpr int NT = 64 * NW;
  constexpr int kU = 8;  // words per step: all of their reads issued first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = (L + 63) / 64;  // the row's keys are 0 .. L - 1, its mask row W words
  // this wave's words [wa, wb)
  const int nwp = (nw + NW - 1) / NW;
  const int wa = min(nw, wid * nwp), wb = min(nw, wa + nwp);

  if (!SEG && L <= K) {
    // causal-only row with at most K keys: every key 0..t, no score read
    for (int i = tid; i < K; i += NT) idx_row[i] = i < L ? i : -1;
    for (int w = tid; w < W; w += NT)
      bits_row[w] = w < L / 64 ? ~0ull : (w == L / 64 && (L & 63) ? (1ull << (L & 63)) - 1ull : 0ull);
    return;
  }
  uint32_t n_valid = (uint32_t)L;
  if (SEG) {
    const int seg_t = segb[t];
    uint32_t c = 0;
    for (int w = wa; w < wb; ++w) {
      const int s = 64 * w + lane;
      const uint64_t m = __ballot(s < L && segb[s] == seg_t);
      if (lane == 0) segw[w] = m;
      c += popc64(m);
    }
    if (lane == 0) sh.red_u[wid] = c;
    __syncthreads();
    n_valid = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) n_valid += sh.red_u[i];
    __syncthreads();
  }
  // is this lane's position in word w valid (w < nw)
  auto valid = [&](int w) -> bool {
    if (SEG) return (segw[w] >> lane) & 1ull;
    return 64 * w + lane < L;
  };
  const bool take_all = n_valid <= (uint32_t)K;

  auto score = [&](int s) -> float { return ScoreLoad<ST>::get(row, s); };
  // scores of words w0 .. w0 + kU - 1 (those below wb), every read issued
  // before any use; positions past t are not read
  auto load_words = [&](int w0, float (&x)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int w = w0 + u, s = 64 * w + lane;
      x[u] = 0.f;
      if (w < wb && s < L) x[u] = score(s);
    }
  };

  uint32_t T = 0, c_eq = 0;
  float Tf = 0.f;
  if (!take_all) {
    // 1. histogram range from a strided sample of valid scores
    float mn = INFINITY, mx = -INFINITY;
    for (int i = tid; i < kSample; i += NT) {
      const int s = (int)(((int64_t)i * L) / kSample);
      const bool v = SEG ? ((segw[s >> 6] >> (s & 63)) & 1ull) : true;
      if (v) {
        const float x = score(s);
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
    }
    block_minmax_f<NW>(mn, mx, sh.red_f);
    if (!(mn <= mx)) {  // no valid key sampled: the whole row
      for (int w = wa; w < wb; ++w)
        if (valid(w)) {
          const float x = score(64 * w + lane);
          mn = fminf(mn, x);
          mx = fmaxf(mx, x);
        }
      block_minmax_f<NW>(mn, mx, sh.red_f);
    }
    // a single sampled value: a huge scale puts it in bin 0, larger scores in the top bin
    const float inv = mx > mn ? (float)kNB / (mx - mn) : 1e30f;
    auto bin_of = [&](float x) -> int { return (int)fminf(fmaxf((x - mn) * inv, 0.f), (float)(kNB - 1)); };
    // 2. histogram
    for (int i = tid; i <= kNB; i += NT) sh.hist[i] = 0;
    if (tid == 0) sh.ncand = 0;
    __syncthreads();
    for (int w0 = wa; w0 < wb; w0 += kU) {
      float x[kU];
      load_words(w0, x);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int w = w0 + u;
        if (w < wb) atomicAdd(&sh.hist[valid(w) ? bin_of(x[u]) : kNB], 1u);
      }
    }
    __syncthreads();
    find_bin_n<NT>(sh.hist, (uint32_t)K, sh.red_u, sh.found_bin, sh.found_above);
    const int bstar = (int)sh.found_bin;
    uint32_t need = (uint32_t)K - sh.found_above;
    // 3. this wave's keys in bins above b*, and the keys of b*
    uint32_t klo = 0xffffffffu, khi = 0u, gw = 0u;
    for (int w0 = wa; w0 < wb; w0 += kU) {
      float x[kU];
      load_words(w0, x);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int w = w0 + u;
        if (w >= wb) break;  // wave-uniform
        const int bn = valid(w) ? bin_of(x[u]) : -1;
        gw += popc64(__ballot(bn > bstar));
        if (bn == bstar) {
          const uint32_t k = fkey(x[u]);
          klo = min(klo, k);
          khi = max(khi, k);
          const uint32_t slot = atomicAdd(&sh.ncand, 1u);
          if (slot < (uint32_t)kLCand) {
            sh.cand_key[slot] = k;
            sh.cand_pos[slot] = (uint32_t)(64 * w + lane);
          }
        }
      }
    }
    if (lane == 0) {
      sh.wave_g[wid] = gw;
      sh.wave_e[wid] = 0u;
    }
    block_minmax_u<NW>(klo, khi, sh.red_u);  // its barrier also publishes the candidates
    const uint32_t nc = sh.ncand;
    if (nc <= (uint32_t)kLCand) {
      // candidate i is T when #greater < need <= #greater + #equal
      if (tid < (int)nc) {
        const uint32_t ki = sh.cand_key[tid];
        uint32_t gt = 0, eq = 0;
        for (uint32_t j = 0; j < nc; ++j) {
          const uint32_t kj = sh.cand_key[j];
          gt += kj > ki;
          eq += kj == ki;
        }
        if (gt < need && need <= gt + eq) {
          sh.thresh = ki;  // every thread that writes holds the same key
          sh.thresh_above = gt;
        }
      }
      __syncthreads();
      T = sh.thresh;
      c_eq = need - sh.thresh_above;
      if (tid < (int)nc) {
        const uint32_t k = sh.cand_key[tid], wi = (sh.cand_pos[tid] >> 6) / (uint32_t)nwp;
        if (k > T) atomicAdd(&sh.wave_g[wi], 1u);
        else if (k == T) atomicAdd(&sh.wave_e[wi], 1u);
      }
    } else {
      // crowded b*: radix passes over its key interval [klo, khi]
      while (klo != khi) {
        const uint32_t span = khi - klo;
        const int nbits = 32 - __clz(span);
        const int shift = nbits > 11 ? nbits - 11 : 0;
        for (int i = tid; i < kNB; i += NT) sh.hist[i] = 0;
        __syncthreads();
        for (int w = wa; w < wb; ++w)
          if (valid(w)) {
            const uint32_t k = fkey(score(64 * w + lane));
            if (k >= klo && k <= khi) atomicAdd(&sh.hist[(k - klo) >> shift], 1u);
          }
        __syncthreads();
        find_bin_n<NT>(sh.hist, need, sh.red_u, sh.found_bin, sh.found_above);
        need -= sh.found_above;
        const uint32_t nlo = klo + (sh.found_bin << shift);
        const uint32_t nhi = shift == 0 ? nlo : min(khi, nlo + ((1u << shift) - 1u));
        klo = nlo;
        khi = nhi;
      }
      T = klo;
      c_eq = need;
      uint32_t g2 = 0, e2 = 0;
      for (int w = wa; w < wb; ++w) {
        const bool v = valid(w);
        const uint32_t k = v ? fkey(score(64 * w + lane)) : 0u;
        g2 += popc64(__ballot(v && k > T));
        e2 += popc64(__ballot(v && k == T));
      }
      if (lane == 0) {
        sh.wave_g[wid] = g2;
        sh.wave_e[wid] = e2;
      }
    }
    Tf = kfloat(T);
  } else {
    uint32_t g2 = 0;
    for (int w = wa; w < wb; ++w) g2 += popc64(__ballot(valid(w)));
    if (lane == 0) {
      sh.wave_g[wid] = g2;
      sh.wave_e[wid] = 0u;
    }
  }
  __syncthreads();

  // 4. this wave's first slot, then its words in order
  uint32_t gb = 0, eb = 0;
  for (int w2 = 0; w2 < wid; ++w2) {
    gb += sh.wave_g[w2];
    eb += sh.wave_e[w2];
  }
  gb = __builtin_amdgcn_readfirstlane(gb);
  eb = __builtin_amdgcn_readfirstlane(eb);
  uint32_t mlo = 0, mhi = 0;  // lane j: mask word wa + 64 * (k / 64) + j
  for (int w0 = wa; w0 < wb; w0 += kU) {
    float x[kU];
    if (take_all) {
#pragma unroll
      for (int u = 0; u < kU; ++u) x[u] = 0.f;
    } else {
      load_words(w0, x);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int w = w0 + u;
      if (w >= wb) break;  // wave-uniform
      const bool v = valid(w);
      const bool gt = v && (take_all || x[u] > Tf);
      const bool eq = v && !take_all && x[u] == Tf;
      const uint64_t eqm = __ballot(eq);
      const bool sel = gt || (eq && eb + lanes_below(eqm) < c_eq);
      const uint64_t selm = __ballot(sel);
      const uint32_t pos = gb + min(eb, c_eq) + lanes_below(selm);
      if (sel && pos < (uint32_t)K) idx_row[pos] = 64 * w + lane;
      gb += popc64(__ballot(gt));
      eb += popc64(eqm);
      const int j = (w - wa) & 63;
      if (lane == j) {
        mlo = (uint32_t)selm;
        mhi = (uint32_t)(selm >> 32);
      }
      if (j == 63 || w == wb - 1) {  // wave-uniform: store the collected mask words
        if (lane <= j) bits_row[w - j + lane] = ((uint64_t)mhi << 32) | mlo;
      }
    }
  }
  for (int w = nw + tid; w < W; w += NT) bits_row[w] = 0ull;
  const int n = take_all ? (int)n_valid : K;
  for (int i = n + tid; i < K; i += NT) idx_row[i] = -1;
}

template <typename ST, bool SEG, int NW>
__global__ __launch_bounds__(64 * NW) void topk_long_kernel(const ST* __restrict__ scores, int64_t ld,
                                                            const int32_t* __restrict__ seg, int B, int S,
                                                            int Sk, int ratio, int K, int row0, int nrows, int rbeg,
                                                            int rcount, int32_t* __restrict__ idx,
                                                            uint64_t* __restrict__ bits) {
  __shared__ LongShared sh;
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  const int b = blockIdx.x % B;
  const int r = rbeg + rcount - 1 - (int)(blockIdx.x / B);  // longest rows first
  const int t = row0 + r;
  // with segment IDs, topk_wave_kernel (run before) marks the rows it leaves
  if (SEG && idx[((size_t)b * S + t) * K] != kLongRow) return;
  const int W = (Sk + 63) / 64;
  multipass_row<ST, SEG, NW>(scores + ((size_t)b * nrows + r) * ld, SEG ? seg + (size_t)b * S : nullptr, W, K, t,
                             (t + 1) / ratio, idx + ((size_t)b * S + t) * K, bits + ((size_t)b * S + t) * W, sh,
                             (uint64_t*)dyn);
}

// ---- rows longer than 64 * kWaveWords keys, read once
//
// A strided sample of the row (32 runs of 64 consecutive keys) gives a lower
// bound lo on the threshold, chosen so that about 2K of the row's keys are at
// or above it. One pass over the row (16-byte loads, every score read once)
// lists each key >= lo; every other key costs one compare. A 2048-bin
// histogram over [lo, sampled max] is then built from the list. Any
// lo for which at least K keys are listed gives the exact result: every key
// in a bin above the K-th largest's bin is listed, and so are the largest
// keys of that bin. The K-th largest key T is then found by ranking the
// listed keys of its bin (their scores re-read by position), ties at T are
// ordered by position, and the selected positions are set in a per-word LDS
// mask that is turned into the index list and the mask words, one word per
// thread. A row whose list comes out short, or longer than the LDS list
// holds, is finished by the multi-pass selection in the same workgroup.
//
// In the pass, each lane reads kSU 16-byte blocks per stage, with the next
// stage in flight (two register buffers in turn). Each wave lists into its own region of
// the list, at slots from the ballot of each score slot: no atomics on the
// list, and no waits inside the pass.
constexpr int kStash = 6656;     // list slots (kStash / NW per wave)
constexpr int kStashUse = 6144;  // listed keys a row can rely on: kStash minus 64 per wave of 8
constexpr int kChunks = 32;      // sample: runs of 64 consecutive keys
constexpr int kSB = 256;         // sample histogram bins
constexpr int kSU = 2;           // 16-byte blocks per lane and stage (two stages in flight)
constexpr uint32_t kHole = 0xffffffffu;  // a list slot whose key is not valid (other segment)

struct StashShared {
  uint32_t hist[kNB];
  uint32_t shist[kSB];
  uint32_t cand_key[kLCand];
  uint32_t cand_pos[kLCand];
  uint32_t red_u[2 * kMaxLW];
  float red_f[2 * kMaxLW];
  uint32_t wave_g[kMaxLW];   // per wave: listed keys, then selected keys of a word chunk
  uint32_t samp_n[kMaxLW];   // per wave: valid sampled scores
  uint32_t found_bin, found_above, ncand, thresh, thresh_above;
};

// order-preserving 16-bit key of a bfloat16 score (its bits); -0 maps like +0
__device__ __forceinline__ uint32_t bkey16(uint32_t h) {
  h &= 0xffffu;
  if (h == 0x8000u) h = 0u;
  return (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
}

// dynamic LDS of topk_stash_kernel: the list, which the selection mask
// reuses once the list has been read into registers, then the
// segment-validity words. Sharing keeps a 128K row's workgroup at 36 KB of
// LDS, four per CU.
static size_t stash_list_bytes(int nw_max) {
  return (size_t)nw_max * 8 > (size_t)kStash * 4 ? (size_t)nw_max * 8 : (size_t)kStash * 4;
}
static size_t stash_lds_bytes(int nw_max, bool seg) {
  return stash_list_bytes(nw_max) + (seg ? (size_t)nw_max * 8 : 0);
}

// Held to 64 VGPRs, so that four workgroups (eight waves per SIMD) share a
// CU. Only the multi-pass fallback, an out-of-line call, spills at that budget.
template <typename ST, bool SEG>
constexpr int stash_waves_per_simd() { return 8; }

template <typename ST, bool SEG, int NW>
__global__ __launch_bounds__(64 * NW, (stash_waves_per_simd<ST, SEG>())) void topk_stash_kernel(const ST* __restrict__ scores, int64_t ld,
                                                             const int32_t* __restrict__ seg, int B, int S, int Sk,
                                                             int ratio, int K, int row0, int nrows, int rbeg,
                                                             int rcount, int nw_max,
                                                             int32_t* __restrict__ idx,
                                                             uint64_t* __restrict__ bits) {
  constexpr int NT = 64 * NW;
  constexpr int EPB = 16 / (int)sizeof(ST);  // scores per 16-byte block
  constexpr int CPW = kChunks / NW;          // sample runs per wave
  constexpr int kCapW = kStash / NW;         // list entries per wave
  constexpr int kSPT = kStash / NT;          // list slots per thread
  __shared__ StashShared sh;
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  uint32_t* stash = dyn;                         // the list
  uint64_t* selw = (uint64_t*)dyn;               // per word: the selected positions (after the list)
  // per word: same-segment positions <= t
  uint64_t* segw = (uint64_t*)(dyn + (nw_max * 2 > kStash ? nw_max * 2 : kStash));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x % B;
  const int r = rbeg + rcount - 1 - (int)(blockIdx.x / B);  // longest rows first
  const int t = row0 + r;
  const int W = (Sk + 63) / 64;
  const int L = (t + 1) / ratio, nw = (L + 63) / 64;
  const ST* row = scores + ((size_t)b * nrows + r) * ld;
  int32_t* idx_row = idx + ((size_t)b * S + t) * K;
  uint64_t* bits_row = bits + ((size_t)b * S + t) * W;

  // with segment IDs, topk_wave_kernel (run before) marks the rows it leaves
  if (SEG && idx_row[0] != kLongRow) return;
  if (!SEG && L <= K) {
    // causal-only row with at most K keys: every key 0..t, no score read
    for (int i = tid; i < K; i += NT) idx_row[i] = i < L ? i : -1;
    for (int w = tid; w < W; w += NT)
      bits_row[w] = w < L / 64 ? ~0ull : (w == L / 64 && (L & 63) ? (1ull << (L & 63)) - 1ull : 0ull);
    return;
  }
  uint32_t n_valid = (uint32_t)L;
  if (SEG) {
    const int32_t* segb = seg + (size_t)b * S;
    const int seg_t = segb[t];
    uint32_t c = 0;
    for (int w = wid; w < nw; w += NW) {
      const int s = 64 * w + lane;
      const uint64_t m = __ballot(s < L && segb[s] == seg_t);
      if (lane == 0) segw[w] = m;
      c += popc64(m);
    }
    if (lane == 0) sh.red_u[wid] = c;
    __syncthreads();
    n_valid = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) n_valid += sh.red_u[i];
    __syncthreads();
  }
  auto valid_pos = [&](int p) -> bool {  // 0 <= p < L
    if (SEG) return (segw[p >> 6] >> (p & 63)) & 1ull;
    return true;
  };
  const bool take_all = n_valid <= (uint32_t)K;

  // The sample's loads are issued first, then the first stage of the pass,
  // which reads the 16-byte blocks [ra, ra + 16 * nblk) and stays in flight
  // during the sample.
  const uintptr_t rs = (uintptr_t)row, ra = rs & ~(uintptr_t)15;
  const int nblk = (int)((rs + (uintptr_t)L * sizeof(ST) - ra + 15) / 16);
  const int p_ra = -(int)((rs - ra) / sizeof(ST));  // position of the first block's first score
  // derived from the row pointer, so the loads stay global (flat loads would
  // also count against the LDS wait counter)
  const u32x4* blk = (const u32x4*)((const char*)row - (rs - ra));
  // Stage st reads blocks [st * kSU * NT, (st + 1) * kSU * NT): wave w takes
  // block (st * kSU + u) * NT + 64 * w + lane, u < kSU. A score's index in
  // its wave's own sequence, ((st * kSU + u) * 64 + lane) * EPB + e, stays
  // below 2^16. Loads past the row re-read its last block.
  const int nstage = (nblk + kSU * NT - 1) / (kSU * NT);
  auto load_stage = [&](int st, u32x4 (&v)[kSU]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kSU; ++u) v[u] = blk[min((st * kSU + u) * NT + tid, nblk - 1)];
  };
  float sx[CPW];
  bool sv[CPW];
  u32x4 vb0[kSU], vb1[kSU];  // stages st and st + 1 (two in turn)
  if (!take_all) {
    // sample: run c starts at c * (L - 64) / (kChunks - 1)
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int c = wid + NW * j;
      const int p = (int)(((int64_t)c * (L - 64)) / (kChunks - 1)) + lane;
      sv[j] = valid_pos(p);
      sx[j] = sv[j] ? ScoreLoad<ST>::get(row, p) : 0.f;
    }
    load_stage(0, vb0);
  }

  bool fail = false;
  if (take_all) {
    for (int w = tid; w < nw; w += NT) selw[w] = segw[w];
  } else {
    for (int i = tid; i < kNB; i += NT) sh.hist[i] = 0;
    for (int i = tid; i < kSB; i += NT) sh.shist[i] = 0;
    if (tid == 0) sh.ncand = 0;
    float mn = INFINITY, mx = -INFINITY;
    uint32_t nvs = 0;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      if (sv[j]) {
        mn = fminf(mn, sx[j]);
        mx = fmaxf(mx, sx[j]);
      }
      nvs += popc64(__ballot(sv[j]));
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
      sh.red_f[wid] = mn;
      sh.red_f[NW + wid] = mx;
      sh.samp_n[wid] = nvs;
    }
    __syncthreads();
    nvs = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      mn = fminf(mn, sh.red_f[i]);
      mx = fmaxf(mx, sh.red_f[NW + i]);
      nvs += sh.samp_n[i];
    }
    // the same in every lane (read from LDS): readfirstlane keeps them, the
    // branches on them and the pass's list counts in scalar registers
    mn = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mn)));
    mx = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mx)));
    nvs = __builtin_amdgcn_readfirstlane(nvs);
    float lo = mn;
    if (nvs < 64) {
      fail = true;  // uniform: too few valid keys sampled
    } else if (mx > mn) {
      // lo: the lower edge of the sample-histogram bin holding the ks-th
      // largest sample, ks sized so that about 2K of the row's valid keys
      // lie at or above it
      const float inv_s = (float)kSB / (mx - mn);
#pragma unroll
      for (int j = 0; j < CPW; ++j)
        if (sv[j]) atomicAdd(&sh.shist[(int)fminf(fmaxf((sx[j] - mn) * inv_s, 0.f), (float)(kSB - 1))], 1u);
      __syncthreads();
      if (wid == 0) {
        const uint32_t ks =
            (uint32_t)min((uint64_t)nvs, max((uint64_t)1, ((uint64_t)nvs * 2 * K + n_valid - 1) / n_valid));
        constexpr int PER = kSB / 64;
        uint32_t c[PER], tot = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          c[i] = sh.shist[PER * lane + i];
          tot += c[i];
        }
        // samples in the bins of this lane and the lanes above
        const uint32_t pre = wave_incl_scan(tot);
        const uint32_t incl = __builtin_amdgcn_readlane(pre, 63) - pre + tot;
        uint32_t running = incl - tot;
#pragma unroll
        for (int i = PER - 1; i >= 0; --i) {
          if (running < ks && running + c[i] >= ks) sh.found_bin = PER * lane + i;
          running += c[i];
        }
      }
      __syncthreads();
      lo = mn + (float)__builtin_amdgcn_readfirstlane(sh.found_bin) / inv_s;
    }
    if (!fail) {
      // bins: fp32 scores, linear in the value over [lo, max]; bf16 scores,
      // one bin per value from the largest bf16 value below lo (exact while
      // the listed values span fewer than 2047 of them)
      // The pass lists this wave's scores >= lo in its region of the list.
      // An entry is (position << 11) | bin for fp32 scores; for bf16 it is the
      // score's 16-bit key in the high half (its raw bits when lo > 0, since
      // then every listed score is positive) and its index in the wave's own
      // sequence in the low half. Per score slot: one compare, whose ballot is
      // the slot's listing mask, a lane prefix from mbcnt, and the entry.
      // Bins, segment validity and the histogram are taken afterwards from the
      // list, so their cost follows the list, not the row. A row whose wave
      // listed more than its region holds less 64 is finished by the
      // multi-pass selection.
      const bool posk = sizeof(ST) == 2 && lo > 0.f;
      const float inv = mx > lo ? fminf((float)kNB / (mx - lo), 1e30f) : 1.f;
      const uint32_t klo16 = bkey16(__float_as_uint(lo) >> 16);
      const uint32_t kb16 = klo16 > 0 ? klo16 - 1 : 0;
      uint32_t listed = 0;  // this wave's listed scores so far (uniform)
      static_assert(kSU == 2, "the stage scan takes two blocks per lane");
      auto scan = [&](auto chk, auto pos, int st, u32x4 v0, u32x4 v1) __attribute__((always_inline)) {
        constexpr bool CHK = decltype(chk)::value, POS = decltype(pos)::value;
#pragma unroll
        for (int u = 0; u < kSU; ++u) {
          const u32x4 vu = u ? v1 : v0;
          const uint32_t r = (uint32_t)(((st * kSU + u) * 64 + lane) * EPB);  // index in the wave's sequence
          const int pb = p_ra + ((st * kSU + u) * NT + tid) * EPB;             // position of the block
          const uint32_t pr11 = (uint32_t)pb << 11;
#pragma unroll
          for (int e = 0; e < EPB; ++e) {
            uint32_t xb;  // the score's bits as a float (bf16 in the high half)
            if constexpr (sizeof(ST) == 4) xb = vu[e];
            else xb = (e & 1) ? (vu[e >> 1] & 0xffff0000u) : (vu[e >> 1] << 16);
            const float x = __uint_as_float(xb);
            bool c = x >= lo;
            if constexpr (CHK) c = c && (uint32_t)(pb + e) < (uint32_t)L;
            const uint64_t m = __ballot(c);
            uint32_t ent;
            if constexpr (sizeof(ST) == 4) {
              ent = pr11 + ((uint32_t)e << 11) +
                    (uint32_t)__builtin_amdgcn_fmed3f((x - lo) * inv, 0.f, (float)(kNB - 1));
            } else {
              uint32_t xk = xb;  // POS: the bits are the key (sign bit clear)
              if constexpr (!POS) xk = x < 0.f ? (xb ^ 0xffff0000u) : (xb | 0x80000000u);  // -0 as +0
              ent = xk + r + (uint32_t)e;
            }
            // past kCapW - 64 listed keys the slots repeat the region's last
            // 64; such a wave sends its row to the multi-pass selection
            const uint32_t base = wid * kCapW + min(listed, (uint32_t)(kCapW - 64));
            if (c) stash[base + lanes_below(m)] = ent;
            listed = __builtin_amdgcn_readfirstlane(listed + popc64(m));  // uniform: keep it scalar
          }
        }
      };
      auto scan_stage = [&](auto pos, int st, u32x4 v0, u32x4 v1) __attribute__((always_inline)) {
        if (st >= nstage) return;  // wave-uniform
        const int pa = p_ra + st * kSU * NT * EPB;  // the stage's first position
        if (pa < 0 || pa + kSU * NT * EPB > L) scan(std::true_type{}, pos, st, v0, v1);
        else scan(std::false_type{}, pos, st, v0, v1);
      };
      // loads one stage ahead; past the last stage they re-read the last block
      auto pass = [&](auto pos) __attribute__((always_inline)) {
        for (int st = 0; st < nstage; st += 2) {
          load_stage(st + 1, vb1);
          scan_stage(pos, st, vb0[0], vb0[1]);
          load_stage(st + 2, vb0);
          scan_stage(pos, st + 1, vb1[0], vb1[1]);
        }
      };
      if (posk) pass(std::true_type{});
      else pass(std::false_type{});
      if (lane == 0) sh.wave_g[wid] = listed;
      __syncthreads();  // the list is complete
      bool over = false;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) over |= sh.wave_g[w2] > (uint32_t)(kCapW - 64);
      // Each wave takes its own region back: slot lane + 64 * q of it, up to
      // its own count (listed, still in a scalar register), as (position <<
      // 11) | bin; keys of other segments become holes, the rest count into
      // the histogram. bf16 bins: bkey16 of the score minus kb16, one bin per
      // bf16 value.
      static_assert(kSPT * 64 == kCapW, "a wave's region is kSPT slots per lane");
      uint32_t ent[kSPT];
#pragma unroll
      for (int q = 0; q < kSPT; ++q) {
        ent[q] = kHole;
        if (over || (uint32_t)(64 * q) >= listed) continue;  // uniform
        const uint32_t jr = (uint32_t)(lane + 64 * q);
        if (jr < listed) {
          uint32_t e = stash[wid * kCapW + jr];
          if constexpr (sizeof(ST) == 2) {
            const uint32_t k16 = posk ? (e >> 16) | 0x8000u : e >> 16;
            const uint32_t r = e & 0xffffu, g = r / EPB;  // (st * kSU + u) * 64 + lane
            const uint32_t pq = (uint32_t)(p_ra + (int)(((g >> 6) * NT + wid * 64 + (g & 63)) * EPB + r % EPB));
            e = (pq << 11) | min(k16 - kb16, (uint32_t)(kNB - 1));
          }
          if (SEG && !valid_pos((int)(e >> 11))) {
            e = kHole;
          } else {
            atomicAdd(&sh.hist[e & (kNB - 1)], 1u);
          }
          ent[q] = e;
        }
      }
      __syncthreads();  // the histogram is complete
      uint32_t nst = 0;  // valid listed keys: the histogram's total
      find_bin_n<NT>(sh.hist, (uint32_t)K, sh.red_u, sh.found_bin, sh.found_above, &nst);
      if (over || nst < (uint32_t)K) {
        fail = true;
      } else {
        // every thread holds its list slots (find_bin_n passed barriers since):
        // the mask takes over the list's LDS
        for (int w = tid; w < nw; w += NT) selw[w] = 0ull;
        __syncthreads();
        const uint32_t bstar = __builtin_amdgcn_readfirstlane(sh.found_bin);
        const uint32_t need = (uint32_t)K - __builtin_amdgcn_readfirstlane(sh.found_above);
#pragma unroll
        for (int q = 0; q < kSPT; ++q) {
          if ((uint32_t)(64 * q) >= listed) continue;  // uniform: past the wave's listed keys
          if (ent[q] == kHole) continue;
          const uint32_t bn = ent[q] & (kNB - 1), p = ent[q] >> 11;
          if (bn == bstar) {
            const uint32_t slot = atomicAdd(&sh.ncand, 1u);
            if (slot < (uint32_t)kLCand) sh.cand_pos[slot] = p;
          } else if (bn > bstar) {
            atomicOr((unsigned long long*)&selw[p >> 6], 1ull << (p & 63));
          }
        }
        __syncthreads();
        const uint32_t nc = sh.ncand;
        if (nc > (uint32_t)kLCand) {
          fail = true;
        } else if (sizeof(ST) == 2 && bstar < (uint32_t)(kNB - 1)) {
          // bf16, exact bin: every candidate equals T; the need lowest positions are taken
          if (tid < (int)nc) {
            const uint32_t p = sh.cand_pos[tid];
            bool sel = true;
            if (need < nc) {
              uint32_t below = 0;
              for (uint32_t j = 0; j < nc; ++j) below += sh.cand_pos[j] < p;
              sel = below < need;
            }
            if (sel) atomicOr((unsigned long long*)&selw[p >> 6], 1ull << (p & 63));
          }
        } else {
          if (tid < (int)nc) sh.cand_key[tid] = fkey(ScoreLoad<ST>::get(row, (int)sh.cand_pos[tid]));
          __syncthreads();
          // candidate i is T when #greater < need <= #greater + #equal
          if (tid < (int)nc) {
            const uint32_t ki = sh.cand_key[tid];
            uint32_t gt = 0, eq = 0;
            for (uint32_t j = 0; j < nc; ++j) {
              const uint32_t kj = sh.cand_key[j];
              gt += kj > ki;
              eq += kj == ki;
            }
            if (gt < need && need <= gt + eq) {
              sh.thresh = ki;  // every thread that writes holds the same key
              sh.thresh_above = gt;
            }
          }
          __syncthreads();
          const uint32_t T = sh.thresh, c_eq = need - sh.thresh_above;
          if (tid < (int)nc) {
            const uint32_t k = sh.cand_key[tid], p = sh.cand_pos[tid];
            bool sel = k > T;
            if (k == T) {  // ties at T: the lowest positions
              uint32_t below = 0;
              for (uint32_t j = 0; j < nc; ++j) below += sh.cand_key[j] == T && sh.cand_pos[j] < p;
              sel = below < c_eq;
            }
            if (sel) atomicOr((unsigned long long*)&selw[p >> 6], 1ull << (p & 63));
          }
        }
      }
    }
  }
  if (fail) {  // uniform: the multi-pass selection, its state in the list's LDS
    static_assert(sizeof(LongShared) <= kStash * 4, "multi-pass state must fit the list");
    __syncthreads();
    multipass_row<ST, SEG, NW>(row, SEG ? seg + (size_t)b * S : nullptr, W, K, t, L, idx_row, bits_row,
                               *reinterpret_cast<LongShared*>(stash), segw);
    return;
  }
  __syncthreads();

  // ordered output, one mask word per thread: an exclusive scan of the
  // words' counts gives each word its first slot
  uint32_t base = 0;  // selected keys in the words before this chunk
  for (int c0 = 0; c0 < nw; c0 += NT) {
    const int w = c0 + tid;
    const uint64_t m = w < nw ? selw[w] : 0ull;
    const uint32_t cnt = popc64(m);
    const uint32_t incl = wave_incl_scan(cnt);
    if (lane == 63) sh.wave_g[wid] = incl;
    __syncthreads();
    uint32_t pos = base + incl - cnt, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const uint32_t c = sh.wave_g[w2];
      if (w2 < wid) pos += c;
      tot += c;
    }
    __syncthreads();
    if (w < nw) bits_row[w] = m;
    for (uint64_t mm = m; mm; mm &= mm - 1) idx_row[pos++] = 64 * w + __builtin_ctzll(mm);
    base += tot;
  }
  for (int w = nw + tid; w < W; w += NT) bits_row[w] = 0ull;
  const int n = take_all ? (int)n_valid : K;
  for (int i = n + tid; i < K; i += NT) idx_row[i] = -1;
}

// Bits of caller-given index lists: one workgroup per row, the row's words
// assembled in LDS with atomic ORs, then written out whole.
__global__ __launch_bounds__(256) void build_bits_kernel(const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ seg, int B,
                                                         int S, int Sk, int ratio, int K,
                                                         uint64_t* __restrict__ bits) {
  extern __shared__ unsigned long long words[];
  const int W = (Sk + 63) / 64;
  const int b = blockIdx.x % B, t = blockIdx.x / B;
  const int tk = (t + 1) / ratio - 1;  // last visible key
  for (int w = threadIdx.x; w < W; w += 256) words[w] = 0ull;
  __syncthreads();
  const int32_t* row = idx + ((size_t)b * S + t) * K;
  const int seg_t = seg ? seg[(size_t)b * S + t] : 0;
  for (int i = threadIdx.x; i < K; i += 256) {
    const int s = row[i];
    if (s >= 0 && s <= tk && (!seg || seg[(size_t)b * S + s] == seg_t))
      atomicOr(&words[s >> 6], 1ull << (s & 63));
  }
  __syncthreads();
  uint64_t* out = bits + ((size_t)b * S + t) * W;
  for (int w = threadIdx.x; w < W; w += 256) out[w] = words[w];
}

// Tile classes of query tiles [qt0, qt1): a workgroup per (query tile, 64
// key tiles). Lane = key tile (one mask word per row), wave w takes rows
// t0 + 32w .. t0 + 32w + 31 of the query tile, and the four waves' OR and AND
// of their words are combined in LDS.
__global__ __launch_bounds__(256) void tile_class_kernel(const uint64_t* __restrict__ bits, int S, int Sk, int qt0,
                                                         uint8_t* __restrict__ cls) {
  __shared__ uint64_t s_or[4][64], s_and[4][64];
  const int W = (Sk + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int kt = blockIdx.x * 64 + lane;
  const int qt = qt0 + blockIdx.y, b = blockIdx.z;
  const int t0 = qt * 128, t1 = min(S, t0 + 128);
  const int ta = t0 + 32 * wv, tb = min(t1, ta + 32);
  uint64_t o = 0ull, a = ~0ull;
  if (kt < NK) {
    const uint64_t* col = bits + ((size_t)b * S) * W + kt;
#pragma unroll 8
    for (int t = ta; t < tb; ++t) {
      const uint64_t w = col[(size_t)t * W];
      o |= w;
      a &= w;
    }
  }
  s_or[wv][lane] = o;
  s_and[wv][lane] = a;
  __syncthreads();
  if (wv == 0 && kt < NK) {
    o = s_or[0][lane] | s_or[1][lane] | s_or[2][lane] | s_or[3][lane];
    a = s_and[0][lane] & s_and[1][lane] & s_and[2][lane] & s_and[3][lane];
    const bool keys_in_range = (kt + 1) * 64 <= Sk;
    cls[((size_t)b * NQ + qt) * NK + kt] = o == 0ull ? 0 : ((keys_in_range && a == ~0ull) ? 2 : 1);
  }
}

// words of the longest row among rows [rbeg, rbeg + rcount) of the slab
static int longest_row_words(int row0, int rbeg, int rcount, int ratio) {
  return ((row0 + rbeg + rcount) / ratio + 63) / 64;
}
template <typename ST, bool SEG, int NW>
static hipError_t launch_multipass(const ST* scores, int64_t ld, const int32_t* seg, int B, int S, int Sk, int ratio,
                                   int K, int row0, int nrows, int rbeg, int rcount, int32_t* idx, uint64_t* bits,
                                   hipStream_t st) {
  const int nw_max = longest_row_words(row0, rbeg, rcount, ratio);
  const size_t shm = SEG ? (size_t)nw_max * 8 : 0;
  if (shm + sizeof(LongShared) > 160 * 1024) return hipErrorInvalidValue;
  const void* fn = (const void*)topk_long_kernel<ST, SEG, NW>;
  if (shm > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((topk_long_kernel<ST, SEG, NW>), dim3((unsigned)((size_t)rcount * B)), dim3(64 * NW),
                     shm, st, scores, ld, seg, B, S, Sk, ratio, K, row0, nrows, rbeg, rcount, idx, bits);
  return hipGetLastError();
}
template <typename ST, bool SEG, int NW>
static hipError_t launch_stash(const ST* scores, int64_t ld, const int32_t* seg, int B, int S, int Sk, int ratio,
                               int K, int row0, int nrows, int rbeg, int rcount, int32_t* idx, uint64_t* bits,
                               hipStream_t st) {
  const int nw_max = longest_row_words(row0, rbeg, rcount, ratio);
  const size_t shm = stash_lds_bytes(nw_max, SEG);
  if (shm + sizeof(StashShared) > 160 * 1024) return hipErrorInvalidValue;
  const void* fn = (const void*)topk_stash_kernel<ST, SEG, NW>;
  if (shm > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((topk_stash_kernel<ST, SEG, NW>), dim3((unsigned)((size_t)rcount * B)), dim3(64 * NW), shm,
                     st, scores, ld, seg, B, S, Sk, ratio, K, row0, nrows, rbeg, rcount, nw_max, idx, bits);
  return hipGetLastError();
}
// rows [rbeg, rbeg + rcount) of the slab, all longer than 64 * kWaveWords keys
template <typename ST, bool SEG>
static hipError_t launch_long_rows(const ST* scores, int64_t ld, const int32_t* seg, int B, int S, int Sk, int ratio,
                                   int K, int row0, int nrows, int rbeg, int rcount, int32_t* idx, uint64_t* bits,
                                   hipStream_t st) {
  if (2 * K > kStashUse)  // the listed keys could not hold the selection: multi-pass only
    return launch_multipass<ST, SEG, 16>(scores, ld, seg, B, S, Sk, ratio, K, row0, nrows, rbeg, rcount, idx, bits,
                                         st);
  return launch_stash<ST, SEG, 8>(scores, ld, seg, B, S, Sk, ratio, K, row0, nrows, rbeg, rcount, idx, bits, st);
}

// Rows are routed by length L = (t + 1) / ratio (longest first): up to 64 *
// kWaveWords keys in one wave's VGPRs; longer rows are read once into a short
// list of their largest keys, with the multi-pass selection behind for rows
// where the list misses.
// With segment IDs a row's keys lie in [first, t], first its segment's first
// position: every row goes to the one-wave kernel, which leaves the rows whose
// span is wider than its registers hold to the long-row kernels (it marks them
// in their first index entry, and those kernels skip every other row), so
// packed documents of up to 4096 keys never take the long path.
template <typename ST>
static hipError_t launch_topk_t(const void* scores, int64_t ld, const int32_t* seg, int B, int S, int Sk, int ratio,
                                int K, int row0, int nrows, int32_t* idx, uint64_t* bits, hipStream_t st) {
  const ST* sc = (const ST*)scores;
  const int l_reg = 64 * kWaveWords;
  // rows with L > l_reg, i.e. t >= ratio * (l_reg + 1) - 1, start here
  const int n_long_from = (int)max((int64_t)0, min((int64_t)nrows, (int64_t)ratio * (l_reg + 1) - 1 - row0));
  const int n_reg = seg ? nrows : n_long_from;  // rows the one-wave kernel looks at
  hipError_t e = hipSuccess;
  // the one-wave kernel first: with segment IDs it marks the rows it leaves
  if (n_reg > 0) {
    hipLaunchKernelGGL((topk_wave_kernel<ST>), dim3((unsigned)(((size_t)n_reg * B + 3) / 4)), dim3(256), 0, st,
                       sc, ld, seg, B, S, Sk, ratio, K, row0, nrows, n_reg, idx, bits);
    e = hipGetLastError();
  }
  if (e == hipSuccess && nrows > n_long_from)
    e = seg ? launch_long_rows<ST, true>(sc, ld, seg, B, S, Sk, ratio, K, row0, nrows, n_long_from,
                                         nrows - n_long_from, idx, bits, st)
            : launch_long_rows<ST, false>(sc, ld, seg, B, S, Sk, ratio, K, row0, nrows, n_long_from,
                                          nrows - n_long_from, idx, bits, st);
  return e;
}

hipError_t launch_topk(const void* scores, bool score_bf16, int64_t ld, const int32_t* seg, int B, int S, int Sk,
                       int ratio, int K, int row0, int nrows, int32_t* idx, uint64_t* bits, hipStream_t st) {
  return score_bf16 ? launch_topk_t<uint16_t>(scores, ld, seg, B, S, Sk, ratio, K, row0, nrows, idx, bits, st)
                    : launch_topk_t<float>(scores, ld, seg, B, S, Sk, ratio, K, row0, nrows, idx, bits, st);
}

hipError_t launch_build_bits(const int32_t* idx, const int32_t* seg, int B, int S, int Sk, int ratio, int K,
                             uint64_t* bits, hipStream_t st) {
  const size_t shm = (size_t)mask_words(Sk) * 8;
  hipLaunchKernelGGL(build_bits_kernel, dim3((unsigned)((size_t)B * S)), dim3(256), shm, st, idx,
                     seg, B, S, Sk, ratio, K, bits);
  return hipGetLastError();
}

hipError_t launch_tile_classes(const uint64_t* bits, int B, int S, int Sk, int qt0, int qt1, uint8_t* cls,
                               hipStream_t st) {
  if (qt1 <= qt0) return hipSuccess;
  dim3 grid((unsigned)((n_ktiles(Sk) + 63) / 64), (unsigned)(qt1 - qt0), (unsigned)B);
  hipLaunchKernelGGL(tile_class_kernel, grid, dim3(256), 0, st, bits, S, Sk, qt0, cls);
  return hipGetLastError();
}

}  // namespace dsa
