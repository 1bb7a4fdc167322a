// Per-query top-k selection, selection bitmask and tile classes (gfx950).
//
// Source: "DeepSeek3.2: Onboard sparse attention", Background (the top-k is a
// non-parametric choice of the keys each query attends to) and "What this PR
// does", item 1 (top-k indices and an index mask); "Support Ring Attention
// with DeepSeek DSA Sparse Indexer", Forward Flow (the index mask is
// [batch, S, S], shared by all heads, tiled into partial-mask blocks).
//
// Selection rule: n = min(K, |valid(t)|) keys. Larger scores win. Among equal
// scores the smaller key position wins, and -0 equals +0.
//
// One workgroup (4 waves) per query row. Rows short enough keep their keys in
// LDS after one coalesced read; longer ones re-read global memory per pass.
//   * |valid| <= K: every valid key is taken and the scores are never read.
//   * otherwise the K-th largest key T is found exactly:
//       1. min/max of the row's valid scores;
//       2. a 2048-bin histogram that is linear in the score value. Bins are
//          monotone in the value, so equal scores share a bin. Scores of a row
//          are spread out, so few lanes collide on one LDS counter. The bin
//          holding the K-th largest score is then a contiguous range of the
//          order-preserving u32 keys [klo, khi];
//       3. radix passes over (key - klo) >> shift with at most 2048 bins each,
//          until the range is a single key T.
//     Then c_gt = #{key > T} and c_eq = K - c_gt ties at T are taken,
//     lowest positions first.
//   * compaction walks the row in 64-key words, one word per wave step:
//     ballot gives the word's selection bits (the bitmask word itself),
//     and mbcnt over the ballots gives each selected lane its ascending slot
//     in the index list. A first walk counts per wave; a second one writes.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

constexpr int kNB = 2048;  // histogram bins

template <typename ST> struct ScoreLoad;
template <> struct ScoreLoad<float> {
  __device__ static __forceinline__ float get(const float* p, int s) { return p[s]; }
};
template <> struct ScoreLoad<uint16_t> {
  __device__ static __forceinline__ float get(const uint16_t* p, int s) { return bf2f(p[s]); }
};

constexpr int kCand = 256;  // candidates ranked directly (one per thread)

struct TopkShared {
  uint32_t hist[kNB];
  uint32_t red_u[8];
  float red_f[8];
  uint32_t found_bin, found_above;
  uint32_t wave_gt[4], wave_eq[4];
  uint32_t ncand, thresh;
  uint32_t cand[kCand];
};

__device__ __forceinline__ uint32_t block_sum(uint32_t x, TopkShared& sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  x = wave_sum(x);
  if (lane == 0) sh.red_u[wid] = x;
  __syncthreads();
  const uint32_t r = sh.red_u[0] + sh.red_u[1] + sh.red_u[2] + sh.red_u[3];
  __syncthreads();
  return r;
}
__device__ __forceinline__ void block_minmax(float& mn, float& mx, TopkShared& sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) { sh.red_f[wid] = mn; sh.red_f[4 + wid] = mx; }
  __syncthreads();
  mn = fminf(fminf(sh.red_f[0], sh.red_f[1]), fminf(sh.red_f[2], sh.red_f[3]));
  mx = fmaxf(fmaxf(sh.red_f[4], sh.red_f[5]), fmaxf(sh.red_f[6], sh.red_f[7]));
  __syncthreads();
}
__device__ __forceinline__ void block_uminmax(uint32_t& mn, uint32_t& mx, TopkShared& sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  mn = wave_umin(mn);
  mx = wave_umax(mx);
  if (lane == 0) { sh.red_u[wid] = mn; sh.red_u[4 + wid] = mx; }
  __syncthreads();
  mn = min(min(sh.red_u[0], sh.red_u[1]), min(sh.red_u[2], sh.red_u[3]));
  mx = max(max(sh.red_u[4], sh.red_u[5]), max(sh.red_u[6], sh.red_u[7]));
  __syncthreads();
}

// Given the histogram in sh.hist[0..kNB), find the largest bin b with
// count(bins >= b) >= need. Writes b and count(bins > b) to sh. Needs
// count(all bins) >= need >= 1.
__device__ void find_bin(TopkShared& sh, uint32_t need) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // thread i owns bins [8i, 8i+8); scan in descending bin order: thread order
  // reversed, so thread j = 255 - i covers the j-th chunk from the top
  const int j = 255 - tid;
  uint32_t c[8];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) { c[i] = sh.hist[8 * tid + i]; tot += c[i]; }
  // inclusive prefix over j (descending bins) within the wave: lanes ordered by j
  // j = 255 - tid, so within a wave, lower j is higher lane. Use a suffix scan
  // over lanes: incl = sum of tot over lanes >= this lane.
  uint32_t incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_down(incl, o);
    if (lane + o < 64) incl += y;
  }
  if (lane == 0) sh.red_u[wid] = incl;  // wave total
  __syncthreads();
  // waves with larger wid hold higher bins
  uint32_t above_waves = 0;
  for (int w2 = wid + 1; w2 < 4; ++w2) above_waves += sh.red_u[w2];
  __syncthreads();
  uint32_t running = above_waves + incl - tot;  // count of bins above this thread's chunk
  (void)j;
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    if (running < need && running + c[i] >= need) {
      sh.found_bin = 8 * tid + i;
      sh.found_above = running;
    }
    running += c[i];
  }
  __syncthreads();
}

// inverse of fkey for a valid (non-zero) key
__device__ __forceinline__ float kfloat(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One workgroup per row. All passes work on order-preserving u32 keys, with
// key 0 marking a position outside valid(t) (every finite score maps above
// 0x007fffff). With IN_LDS the row's keys are built once from one coalesced
// read of the scores and every later pass reads LDS; otherwise (rows too long
// for LDS) each pass recomputes them from global memory.
template <typename ST, bool IN_LDS>
__global__ __launch_bounds__(256) void topk_kernel(const ST* __restrict__ scores, int64_t ld,
                                                   const int32_t* __restrict__ seg, int B, int S,
                                                   int K, int row0, int nrows,
                                                   int32_t* __restrict__ idx,
                                                   uint64_t* __restrict__ bits) {
  __shared__ TopkShared sh;
  extern __shared__ uint32_t rowkeys[];  // IN_LDS: keys of positions [0, 64 * nw)
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x % B;
  const int r = nrows - 1 - (int)(blockIdx.x / B);  // longest rows first
  const int t = row0 + r;
  const int W = (S + 63) / 64;
  const ST* row = scores + ((size_t)b * nrows + r) * ld;
  const int32_t* segb = seg ? seg + (size_t)b * S : nullptr;
  const int seg_t = seg ? segb[t] : 0;
  const int L = t + 1;
  const int nw = (L + 63) / 64;

  auto gkey = [&](int s) -> uint32_t {  // key from global memory (0 if not valid)
    if (s >= L || (segb && segb[s] != seg_t)) return 0u;
    return fkey(ScoreLoad<ST>::get(row, s));
  };
  auto key = [&](int s) -> uint32_t {
    if constexpr (IN_LDS) return rowkeys[s];
    else return gkey(s);
  };

  int32_t* idx_row = idx + ((size_t)b * S + t) * K;
  uint64_t* bits_row = bits + ((size_t)b * S + t) * W;
  if (!segb && L <= K) {
    // causal-only row with at most K keys: every key 0..t, no score read
    for (int i = tid; i < K; i += 256) idx_row[i] = i < L ? i : -1;
    for (int w = tid; w < W; w += 256)
      bits_row[w] = w < L / 64 ? ~0ull : (w == L / 64 && (L & 63) ? (1ull << (L & 63)) - 1ull : 0ull);
    return;
  }
  uint32_t n_valid = (uint32_t)L;
  if (segb) {
    uint32_t c = 0;
    for (int s = tid; s < L; s += 256) c += (segb[s] == seg_t);
    n_valid = block_sum(c, sh);
  }
  const bool take_all = n_valid <= (uint32_t)K;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  if constexpr (IN_LDS) {
    // take-all rows never read scores: their keys only mark validity
    for (int s = tid; s < 64 * nw; s += 256) {
      const uint32_t kk = take_all ? ((s < L && (!segb || segb[s] == seg_t)) ? 1u : 0u) : gkey(s);
      rowkeys[s] = kk;
      if (kk) {
        kmin = min(kmin, kk);
        kmax = max(kmax, kk);
      }
    }
    __syncthreads();  // the row's keys are visible to every wave
  }
  uint32_t T = 0, c_eq = 0;
  if (!take_all) {
    if constexpr (!IN_LDS) {
      for (int s = tid; s < L; s += 256) {
        const uint32_t kk = key(s);
        if (kk) {
          kmin = min(kmin, kk);
          kmax = max(kmax, kk);
        }
      }
    }
    block_uminmax(kmin, kmax, sh);
    uint32_t need = (uint32_t)K;
    uint32_t klo, khi;
    if (kmin == kmax) {
      klo = khi = kmax;
    } else {
      // value-linear bins: monotone in the score, so equal scores share a bin
      const float mn = kfloat(kmin), mx = kfloat(kmax);
      const float inv = (float)kNB / (mx - mn);
      for (int i = tid; i < kNB; i += 256) sh.hist[i] = 0;
      __syncthreads();
      for (int s = tid; s < L; s += 256) {
        const uint32_t kk = key(s);
        if (kk) {
          const int bin = (int)fminf(fmaxf((kfloat(kk) - mn) * inv, 0.f), (float)(kNB - 1));
          atomicAdd(&sh.hist[bin], 1u);
        }
      }
      __syncthreads();
      find_bin(sh, need);
      const int bstar = (int)sh.found_bin;
      need -= sh.found_above;
      // the keys in bin b* form one contiguous key interval; collect them, and
      // when few, take the need-th largest by direct ranking
      if (tid == 0) sh.ncand = 0;
      __syncthreads();
      klo = 0xffffffffu;
      khi = 0u;
      for (int s = tid; s < L; s += 256) {
        const uint32_t kk = key(s);
        if (kk) {
          const int bin = (int)fminf(fmaxf((kfloat(kk) - mn) * inv, 0.f), (float)(kNB - 1));
          if (bin == bstar) {
            klo = min(klo, kk);
            khi = max(khi, kk);
            const uint32_t slot = atomicAdd(&sh.ncand, 1u);
            if (slot < (uint32_t)kCand) sh.cand[slot] = kk;
          }
        }
      }
      block_uminmax(klo, khi, sh);
      const uint32_t nc = sh.ncand;
      if (nc <= (uint32_t)kCand) {
        // candidate i is the threshold when #greater < need <= #greater + #equal
        if (tid < (int)nc) {
          const uint32_t ki = sh.cand[tid];
          uint32_t gt = 0, eq = 0;
          for (uint32_t j = 0; j < nc; ++j) {
            const uint32_t kj = sh.cand[j];
            gt += kj > ki;
            eq += kj == ki;
          }
          if (gt < need && need <= gt + eq) {
            sh.thresh = ki;  // every thread that writes holds the same key
            sh.found_above = gt;
          }
        }
        __syncthreads();
        klo = khi = sh.thresh;
        need -= sh.found_above;
      }
    }
    // radix refinement on the key interval [klo, khi]
    while (klo != khi) {
      const uint32_t span = khi - klo;
      const int nbits = 32 - __clz(span);
      const int shift = nbits > 11 ? nbits - 11 : 0;
      for (int i = tid; i < kNB; i += 256) sh.hist[i] = 0;
      __syncthreads();
      for (int s = tid; s < L; s += 256) {
        const uint32_t kk = key(s);
        if (kk >= klo && kk <= khi) atomicAdd(&sh.hist[(kk - klo) >> shift], 1u);
      }
      __syncthreads();
      find_bin(sh, need);
      need -= sh.found_above;
      const uint32_t nlo = klo + (sh.found_bin << shift);
      const uint32_t nhi = shift == 0 ? nlo : min(khi, nlo + ((1u << shift) - 1u));
      klo = nlo;
      khi = nhi;
    }
    T = klo;
    c_eq = need;
  }

  // ---- compaction: ascending index list and bitmask words
  const int wpw = (nw + 3) / 4;
  const int wa = wid * wpw, wb = min(nw, wa + wpw);
  auto classify = [&](int s, bool& gt, bool& eq) {
    const uint32_t kk = (IN_LDS || s < L) ? key(s) : 0u;
    if (take_all) {
      gt = kk != 0u;
      eq = false;
    } else {
      gt = kk != 0u && kk > T;
      eq = kk != 0u && kk == T;
    }
  };
  uint32_t my_gt = 0, my_eq = 0;
  for (int w = wa; w < wb; ++w) {
    bool gt, eq;
    classify(64 * w + lane, gt, eq);
    my_gt += __popcll(__ballot(gt));
    my_eq += __popcll(__ballot(eq));
  }
  if (lane == 0) { sh.wave_gt[wid] = my_gt; sh.wave_eq[wid] = my_eq; }
  __syncthreads();
  uint32_t eq_before = 0, sel_before = 0;
  for (int w2 = 0; w2 < wid; ++w2) {
    const uint32_t take_eq = eq_before >= c_eq ? 0u : min(sh.wave_eq[w2], c_eq - eq_before);
    sel_before += sh.wave_gt[w2] + take_eq;
    eq_before += sh.wave_eq[w2];
  }
  for (int w = wa; w < wb; ++w) {
    const int s = 64 * w + lane;
    bool gt, eq;
    classify(s, gt, eq);
    const uint64_t eqm = __ballot(eq);
    const uint32_t eq_rank = eq_before + lanes_below(eqm);
    const bool sel = gt || (eq && eq_rank < c_eq);
    const uint64_t selm = __ballot(sel);
    const uint32_t pos = sel_before + lanes_below(selm);
    if (sel && pos < (uint32_t)K) idx_row[pos] = s;
    if (lane == 0) bits_row[w] = selm;
    eq_before += __popcll(eqm);
    sel_before += __popcll(selm);
  }
  for (int w = nw + tid; w < W; w += 256) bits_row[w] = 0ull;
  const int n = take_all ? (int)n_valid : K;
  for (int i = n + tid; i < K; i += 256) idx_row[i] = -1;
}

// Rows of at most 64 * 4 * kRegWords keys: the row's keys stay in VGPRs.
// Wave w holds 64-key words w, w+4, w+8, ... (lane = position in the word), so
// every pass is register work, and the compaction handles all words in
// parallel: per-word counts of the "greater" and "tied" keys go to LDS, one
// wave-wide prefix scan gives every word its first slot, and ballot/mbcnt
// place the keys inside a word. One workgroup per row, longest rows first.
constexpr int kRegWords = 16;

template <typename ST>
__global__ __launch_bounds__(256) void topk_reg_kernel(const ST* __restrict__ scores, int64_t ld,
                                                       const int32_t* __restrict__ seg, int B, int S,
                                                       int K, int row0, int nrows,
                                                       int32_t* __restrict__ idx,
                                                       uint64_t* __restrict__ bits) {
  __shared__ TopkShared sh;
  __shared__ uint32_t wgt[64], weq[64];  // per 64-key word: keys above T, keys equal to T
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int W = (S + 63) / 64;
  // row of work item i (longest rows first), and whether it reads scores
  auto row_of = [&](int i, int& b, int& r) {
    b = i % B;
    r = nrows - 1 - i / B;
  };
  auto reads_scores = [&](int t) { return seg != nullptr || t + 1 > K; };
  // raw scores of a row's positions held by this lane (positions >= L are not read)
  ST raw[kRegWords];
  auto load_row = [&](int i) {
    int b, r;
    row_of(i, b, r);
    const int t = row0 + r;
    if (!reads_scores(t)) return;
    const ST* row = scores + ((size_t)b * nrows + r) * ld;
#pragma unroll
    for (int j = 0; j < kRegWords; ++j) {
      const int s = 64 * (4 * j + wid) + lane;
      if (s <= t) raw[j] = row[s];
    }
  };
  {
    const int item = blockIdx.x;
    int b, r;
    row_of(item, b, r);
    const int t = row0 + r;
    const int32_t* segb = seg ? seg + (size_t)b * S : nullptr;
    const int seg_t = seg ? segb[t] : 0;
    const int L = t + 1;
    const int nw = (L + 63) / 64;
    int32_t* idx_row = idx + ((size_t)b * S + t) * K;
    uint64_t* bits_row = bits + ((size_t)b * S + t) * W;
    if (!reads_scores(t)) {
      // causal-only row with at most K keys: every key 0..t, no score read
      for (int i = tid; i < K; i += 256) idx_row[i] = i < L ? i : -1;
      for (int w = tid; w < W; w += 256)
        bits_row[w] = w < L / 64 ? ~0ull : (w == L / 64 && (L & 63) ? (1ull << (L & 63)) - 1ull : 0ull);
      return;
    }
    load_row(item);  // all of the row's score loads in flight at once
    // keys of the valid positions (0 = not valid); take-all rows only need validity
    uint32_t nv = 0;
#pragma unroll
    for (int j = 0; j < kRegWords; ++j) {
      const int s = 64 * (4 * j + wid) + lane;
      nv += __popcll(__ballot(s < L && (!segb || segb[s] == seg_t)));
    }
    __syncthreads();  // the previous row is done with the shared state
    if (lane == 0) sh.red_u[wid] = nv;
    __syncthreads();
    const uint32_t n_valid = sh.red_u[0] + sh.red_u[1] + sh.red_u[2] + sh.red_u[3];
    const bool take_all = n_valid <= (uint32_t)K;
    uint32_t key[kRegWords];
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < kRegWords; ++j) {
      const int s = 64 * (4 * j + wid) + lane;
      const bool valid = s < L && (!segb || segb[s] == seg_t);
      uint32_t kk = 0u;
      if (valid) kk = take_all ? 1u : fkey(ScoreLoad<ST>::get(&raw[j], 0));
      key[j] = kk;
      if (kk) {
        kmin = min(kmin, kk);
        kmax = max(kmax, kk);
      }
    }
    uint32_t T = 0, c_eq = 0;
    if (!take_all) {
      __syncthreads();  // red_u is reused
      block_uminmax(kmin, kmax, sh);
      uint32_t need = (uint32_t)K;
      uint32_t klo, khi;
      if (kmin == kmax) {
        klo = khi = kmax;
      } else {
        // value-linear bins: monotone in the score, so equal scores share a bin
        const float mn = kfloat(kmin), mx = kfloat(kmax);
        const float inv = (float)kNB / (mx - mn);
        for (int i = tid; i < kNB; i += 256) sh.hist[i] = 0;
        __syncthreads();
        auto bin_of = [&](uint32_t kk) {
          return (int)fminf(fmaxf((kfloat(kk) - mn) * inv, 0.f), (float)(kNB - 1));
        };
#pragma unroll
        for (int j = 0; j < kRegWords; ++j)
          if (key[j]) atomicAdd(&sh.hist[bin_of(key[j])], 1u);
        __syncthreads();
        find_bin(sh, need);
        const int bstar = (int)sh.found_bin;
        need -= sh.found_above;
        if (tid == 0) sh.ncand = 0;
        __syncthreads();
        klo = 0xffffffffu;
        khi = 0u;
#pragma unroll
        for (int j = 0; j < kRegWords; ++j)
          if (key[j] && bin_of(key[j]) == bstar) {
            klo = min(klo, key[j]);
            khi = max(khi, key[j]);
            const uint32_t slot = atomicAdd(&sh.ncand, 1u);
            if (slot < (uint32_t)kCand) sh.cand[slot] = key[j];
          }
        block_uminmax(klo, khi, sh);
        const uint32_t nc = sh.ncand;
        if (nc <= (uint32_t)kCand) {
          // candidate i is the threshold when #greater < need <= #greater + #equal
          if (tid < (int)nc) {
            const uint32_t ki = sh.cand[tid];
            uint32_t gt = 0, eq = 0;
            for (uint32_t jj = 0; jj < nc; ++jj) {
              const uint32_t kj = sh.cand[jj];
              gt += kj > ki;
              eq += kj == ki;
            }
            if (gt < need && need <= gt + eq) {
              sh.thresh = ki;  // every thread that writes holds the same key
              sh.found_above = gt;
            }
          }
          __syncthreads();
          klo = khi = sh.thresh;
          need -= sh.found_above;
        }
      }
      // radix refinement on the key interval [klo, khi] (crowded threshold bins)
      while (klo != khi) {
        const uint32_t span = khi - klo;
        const int nbits = 32 - __clz(span);
        const int shift = nbits > 11 ? nbits - 11 : 0;
        for (int i = tid; i < kNB; i += 256) sh.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kRegWords; ++j)
          if (key[j] >= klo && key[j] <= khi) atomicAdd(&sh.hist[(key[j] - klo) >> shift], 1u);
        __syncthreads();
        find_bin(sh, need);
        need -= sh.found_above;
        const uint32_t nlo = klo + (sh.found_bin << shift);
        const uint32_t nhi = shift == 0 ? nlo : min(khi, nlo + ((1u << shift) - 1u));
        klo = nlo;
        khi = nhi;
      }
      T = klo;
      c_eq = need;
    }

    // ---- compaction: per-word counts, one scan, then every word in parallel
    auto is_gt = [&](uint32_t kk) { return take_all ? kk != 0u : (kk != 0u && kk > T); };
    auto is_eq = [&](uint32_t kk) { return !take_all && kk != 0u && kk == T; };
#pragma unroll
    for (int j = 0; j < kRegWords; ++j) {
      const uint32_t cg = (uint32_t)__popcll(__ballot(is_gt(key[j])));
      const uint32_t ce = (uint32_t)__popcll(__ballot(is_eq(key[j])));
      const int w = 4 * j + wid;
      if (lane == 0 && w < 64) {
        wgt[w] = cg;
        weq[w] = ce;
      }
    }
    __syncthreads();
    // exclusive prefix over the row's words (lane = word), in every wave
    const uint32_t g = lane < nw ? wgt[lane] : 0u, e = lane < nw ? weq[lane] : 0u;
    uint32_t gi = g, ei = e;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t gy = __shfl_up(gi, o), ey = __shfl_up(ei, o);
      if (lane >= o) {
        gi += gy;
        ei += ey;
      }
    }
    const uint32_t gx = gi - g, ex = ei - e;  // keys above T / ties in the words before
#pragma unroll
    for (int j = 0; j < kRegWords; ++j) {
      const int w = 4 * j + wid;
      if (w >= nw) continue;  // wave-uniform
      const int s = 64 * w + lane;
      const uint32_t gb = __builtin_amdgcn_readlane(gx, w), eb = __builtin_amdgcn_readlane(ex, w);
      const bool gt = is_gt(key[j]), eq = is_eq(key[j]);
      const uint32_t eq_rank = eb + lanes_below(__ballot(eq));
      const bool sel = gt || (eq && eq_rank < c_eq);
      const uint64_t selm = __ballot(sel);
      const uint32_t pos = gb + min(eb, c_eq) + lanes_below(selm);
      if (sel && pos < (uint32_t)K) idx_row[pos] = s;
      if (lane == 0) bits_row[w] = selm;
    }
    for (int w = nw + tid; w < W; w += 256) bits_row[w] = 0ull;
    const int n = take_all ? (int)n_valid : K;
    for (int i = n + tid; i < K; i += 256) idx_row[i] = -1;
  }
}

// Bits of caller-given index lists: one workgroup per row, the row's words
// assembled in LDS with atomic ORs, then written out whole.
__global__ __launch_bounds__(256) void build_bits_kernel(const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ seg, int B,
                                                         int S, int K, uint64_t* __restrict__ bits) {
  extern __shared__ unsigned long long words[];
  const int W = (S + 63) / 64;
  const int b = blockIdx.x % B, t = blockIdx.x / B;
  for (int w = threadIdx.x; w < W; w += 256) words[w] = 0ull;
  __syncthreads();
  const int32_t* row = idx + ((size_t)b * S + t) * K;
  const int seg_t = seg ? seg[(size_t)b * S + t] : 0;
  for (int i = threadIdx.x; i < K; i += 256) {
    const int s = row[i];
    if (s >= 0 && s <= t && (!seg || seg[(size_t)b * S + s] == seg_t))
      atomicOr(&words[s >> 6], 1ull << (s & 63));
  }
  __syncthreads();
  uint64_t* out = bits + ((size_t)b * S + t) * W;
  for (int w = threadIdx.x; w < W; w += 256) out[w] = words[w];
}

// Tile classes of query tiles [qt0, qt1): thread per key tile (one mask word).
__global__ __launch_bounds__(256) void tile_class_kernel(const uint64_t* __restrict__ bits, int B,
                                                         int S, int qt0, uint8_t* __restrict__ cls) {
  const int W = (S + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int kt = blockIdx.x * 256 + threadIdx.x;
  const int qt = qt0 + blockIdx.y, b = blockIdx.z;
  if (kt >= NK) return;
  const int t0 = qt * 128, t1 = min(S, t0 + 128);
  uint64_t o = 0ull, a = ~0ull;
  for (int t = t0; t < t1; ++t) {
    const uint64_t w = bits[((size_t)b * S + t) * W + kt];
    o |= w;
    a &= w;
  }
  const bool keys_in_range = (kt + 1) * 64 <= S;
  cls[((size_t)b * NQ + qt) * NK + kt] = o == 0ull ? 0 : ((keys_in_range && a == ~0ull) ? 2 : 1);
}

// rows whose keys fit this much dynamic LDS keep them there
constexpr size_t kTopkLdsMax = 128 * 1024;

template <typename ST>
static hipError_t launch_topk_t(const void* scores, int64_t ld, const int32_t* seg, int B, int S, int K,
                                int row0, int nrows, int32_t* idx, uint64_t* bits, hipStream_t st) {
  const size_t nrow_all = (size_t)nrows * B;
  dim3 grid((unsigned)nrow_all), block(256);
  if (S <= 64 * 4 * kRegWords) {
    hipLaunchKernelGGL((topk_reg_kernel<ST>), grid, block, 0, st, (const ST*)scores, ld, seg, B, S, K, row0,
                       nrows, idx, bits);
    return hipGetLastError();
  }
  const size_t shm = (size_t)mask_words(S) * 64 * sizeof(uint32_t);
  if (shm <= kTopkLdsMax) {
    if (shm > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<ST, true>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((topk_kernel<ST, true>), grid, block, shm, st, (const ST*)scores, ld, seg, B, S, K,
                       row0, nrows, idx, bits);
  } else {
    hipLaunchKernelGGL((topk_kernel<ST, false>), grid, block, 0, st, (const ST*)scores, ld, seg, B, S, K,
                       row0, nrows, idx, bits);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const void* scores, bool score_bf16, int64_t ld, const int32_t* seg,
                       int B, int S, int K, int row0, int nrows, int32_t* idx, uint64_t* bits,
                       hipStream_t st) {
  return score_bf16 ? launch_topk_t<uint16_t>(scores, ld, seg, B, S, K, row0, nrows, idx, bits, st)
                    : launch_topk_t<float>(scores, ld, seg, B, S, K, row0, nrows, idx, bits, st);
}

hipError_t launch_build_bits(const int32_t* idx, const int32_t* seg, int B, int S, int K,
                             uint64_t* bits, hipStream_t st) {
  const size_t shm = (size_t)mask_words(S) * 8;
  hipLaunchKernelGGL(build_bits_kernel, dim3((unsigned)((size_t)B * S)), dim3(256), shm, st, idx,
                     seg, B, S, K, bits);
  return hipGetLastError();
}

hipError_t launch_tile_classes(const uint64_t* bits, int B, int S, int qt0, int qt1, uint8_t* cls,
                               hipStream_t st) {
  if (qt1 <= qt0) return hipSuccess;
  dim3 grid((unsigned)((n_ktiles(S) + 255) / 256), (unsigned)(qt1 - qt0), (unsigned)B);
  hipLaunchKernelGGL(tile_class_kernel, grid, dim3(256), 0, st, bits, B, S, qt0, cls);
  return hipGetLastError();
}

}  // namespace dsa
