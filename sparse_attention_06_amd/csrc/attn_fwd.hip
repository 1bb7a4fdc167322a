// Block-sparse flash-attention forward over the DSA selection mask (gfx950).
//
// Source: "Support Ring Attention with DeepSeek DSA Sparse Indexer", Forward
// Flow (one [batch, S, S] index mask for all heads, combined with causal; on
// kept entries the logit is the scaled query-key product, others drop out);
// "Integrate DeepSeek Sparse Attention with Tokamax Flash Attention",
// Description (flash attention driven by a dynamic 3-D index mask).
//
// MFMA kernel (bf16, Dqk = 192, Dv = 128). A workgroup is one (b, h, 256-query
// block) with 8 waves of 32 queries each, two waves per SIMD. It walks the
// 64-key tiles up to the diagonal. Tiles that are EMPTY for both of its
// 128-query tiles are skipped outright. A wave whose own tile is EMPTY, or
// whose 32 queries keep no key of the tile, idles on it. PARTIAL tiles read
// one u64 selection word per query.
//   S^T = K Q^T: keys on MFMA rows, queries on columns, so each lane owns one
//   query and 32 of the tile's 64 logits. The online-softmax max and sum are
//   in-lane, with one exchange between lane halves. Q stays in VGPRs.
//   O^T += V^T P^T: the probabilities go straight from the S^T accumulator
//   into the B operand. The key order inside each 16-wide k step is permuted
//   to match the accumulator layout. V^T comes from the natural V tile in LDS
//   through the gfx950 transposing LDS read, with the same permutation.
// The tile walk reads the workgroup's tile-class rows from LDS, where they are
// staged at start. K/V tiles are double buffered and filled by direct
// global->LDS copies; the next tile's copies are issued right after the
// barrier and land while the current tile is computed. The per-query
// selection word of the next tile is loaded before those copies, so waiting
// for it never waits for them.
// LDS pitches: K rows 400 B (b128 reads of 16 consecutive rows hit distinct
// banks), V rows 320 B (the four rows of a transposing read cover all 64
// banks). exp2 is the hardware v_exp_f32, with the scale folded in
// (scale * log2 e). O is rescaled only when a tile max passes the reference
// max by more than 2^8.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

namespace fwd {
constexpr int DQK = 192, DV = 128, TK = 64;
constexpr int NW = 8;                // waves per workgroup: 2 per SIMD
constexpr int QW = 32 * NW;          // queries per workgroup (two 128-query tiles)
constexpr int KS = DQK / 16;         // k steps of S^T
constexpr int NB = 2;                // K/V tile buffers
constexpr int KSL = DQK / 8 + 1;     // 16-byte slots per LDS K row (one pad slot): 400 B
constexpr int VSL = DV / 8 + 4;      // ... per V row (four pad slots): 320 B
constexpr int KP = KSL * 8;          // LDS pitch of a K row (elements)
constexpr int VP = VSL * 8;          // LDS pitch of a V row
constexpr int KBLK = TK * KSL / 64;  // 1 KB blocks per K tile (25)
constexpr int VBLK = TK * VSL / 64;  // ... per V tile (20)
constexpr int KI = (KBLK + NW - 1) / NW, VI = (VBLK + NW - 1) / NW;  // blocks per wave
static_assert(TK * KSL % 64 == 0 && TK * VSL % 64 == 0, "tiles must be whole 1 KB blocks");
}  // namespace fwd

// Scores phase of one 64-key tile for a wave's 32 queries: S^T into sacc,
// masked (dropped keys become -inf), and the tile max of each query in log2
// units. This lane's keys are kb*32 + 8i + 4*half + r (i, r in 0..3); with
// the query word shifted right by 4*half, the bit of accumulator register r of
// half kb sits at position 32*kb + 8*(r/4) + r%4.
__device__ __forceinline__ float fwd_scores(const uint16_t* sK, const u32x4 (&qf)[fwd::KS], uint64_t mw,
                                            bool full, float scale_log2, f32x16 (&sacc)[2]) {
  using namespace fwd;
  const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 a = *(const u32x4*)(sK + (kb * 32 + col) * KP + ks * 16 + 8 * half);
      sacc[kb] = mfma32(a, qf[ks], sacc[kb]);
    }
  float tm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  if (full) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tm[r & 3] = fmaxf(tm[r & 3], sacc[kb][r]);
  } else {
    const uint64_t mwh = mw >> (4 * half);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t w = (uint32_t)(mwh >> (32 * kb));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // keep ? x : -inf as a bit select on an all-ones / all-zeros field
        const int keep = __builtin_amdgcn_sbfe((int)w, 8 * (r >> 2) + (r & 3), 1);
        const float x = __int_as_float((keep & __float_as_int(sacc[kb][r])) | (~keep & (int)0xff800000u));
        sacc[kb][r] = x;
        tm[r & 3] = fmaxf(tm[r & 3], x);
      }
    }
  }
  const float tmax = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
  return half_max(tmax) * scale_log2;  // scale > 0 commutes with max
}

// Update phase: online-softmax step with the masked logits of fwd_scores and
// the PV MFMAs against the tile's V. Lazy rescaling: probabilities are taken
// relative to a reference max m that only moves when the tile max exceeds it
// by more than 8 (log2 units), so p <= 2^8. O and l share the reference, so
// the result is unchanged; the O rescale (64 accumulator multiplies) is rare.
__device__ __forceinline__ void fwd_update(const uint16_t* sV, const f32x16 (&sacc)[2], float tmax,
                                           float scale_log2, float& m, float& l, f32x16 (&oacc)[4]) {
  using namespace fwd;
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const bool bump = tmax > m + 8.f;
  if (__ballot(bump)) {
    const float m_new = bump ? tmax : m;
    const float alpha = bump ? fast_exp2(m - m_new) : 1.f;  // m = -inf on a first bump: alpha = 0
    l *= alpha;
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[eb][i] *= alpha;
    m = m_new;
  }
  const float neg_m = m == -INFINITY ? 0.f : -m;
  // O^T[e, q] += V^T[e, key] P^T[key, q]; V^T fragments read transposed from the V tile,
  // keys permuted inside each 16-key step to match the S^T accumulator rows
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
      float pv8[8];
#pragma unroll
      for (int c8 = 0; c8 < 8; ++c8) {
        pv8[c8] = fast_exp2(fmaf(sacc[kb][8 * p2 + c8], scale_log2, neg_m));
        ls[c8 & 3] += pv8[c8];
      }
      const u32x4 pb = u32x4{pack_bf2(pv8[0], pv8[1]), pack_bf2(pv8[2], pv8[3]), pack_bf2(pv8[4], pv8[5]),
                             pack_bf2(pv8[6], pv8[7])};
      const int r0 = kb * 32 + 16 * p2 + 4 * half;
#pragma unroll
      for (int eb = 0; eb < 4; ++eb) oacc[eb] = mfma32(lds_tr_frag(sV, VP, r0, r0 + 8, eb * 32), pb, oacc[eb]);
    }
  l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
}

__global__ __launch_bounds__(fwd::NW * 64) void attn_fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint64_t* __restrict__ bits, const uint8_t* __restrict__ cls, int B, int S, int H,
    float scale_log2, uint16_t* __restrict__ o, float* __restrict__ lse) {
  using namespace fwd;
  __shared__ __attribute__((aligned(1024))) uint16_t smK[NB][TK * KP];
  __shared__ __attribute__((aligned(1024))) uint16_t smV[NB][TK * VP];
  __shared__ uint8_t scls[2][kMaxTiles];  // tile classes of the workgroup's two 128-query tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so per-wave data is scalar
  const int half = lane >> 5, col = lane & 31;
  const int W = (S + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int NQW = (S + QW - 1) / QW;
  // the query blocks of a (b, h) on one XCD (they share K/V), costliest first
  int bh, qw;
  grouped_order(xcd_remap((int)blockIdx.x, (int)gridDim.x), NQW, B * H, bh, qw);
  const int b = bh / H, h = bh % H;
  const int tq = qw * QW + wid * 32 + col;  // this lane's query
  const bool qvalid = tq < S;
  const int qt_w = min(NQ - 1, (qw * QW + wid * 32) / 128);  // this wave's 128-query tile
  const int qt0 = qw * QW / 128, qt1 = min(NQ - 1, qt0 + 1);
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;  // token strides
  const uint16_t* kbase = k + (size_t)b * S * rs_qk + (size_t)h * DQK;
  const uint16_t* vbase = v + (size_t)b * S * rs_v + (size_t)h * DV;

  // this wave's 1 KB blocks of a tile: block j covers slots 64j .. 64j+63 of the
  // padded [64 rows][KSL or VSL slots] layout; pad slots copy a harmless chunk.
  // Row and chunk of each slot are fixed, so byte offsets within the tile's
  // rows are computed once.
  uint32_t koff[KI], voff[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int slot = (wid + i * NW) * 64 + lane;
    koff[i] = (uint32_t)(((slot / KSL) * rs_qk + min(slot % KSL, KSL - 2) * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int slot = (wid + i * NW) * 64 + lane;
    voff[i] = (uint32_t)(((slot / VSL) * rs_v + min(slot % VSL, DV / 8 - 1) * 8) * 2);
  }
  auto issue = [&](int kt, int buf) {
    const char* kt_base = (const char*)(kbase + (size_t)kt * TK * rs_qk);
    const char* vt_base = (const char*)(vbase + (size_t)kt * TK * rs_v);
    const int lim = S - 1 - kt * TK;  // last in-range row of the tile
    if (lim >= TK - 1) {
#pragma unroll
      for (int i = 0; i < KI; ++i)
        if (wid + i * NW < KBLK) g2lds16(kt_base + koff[i], (char*)smK[buf] + (wid + i * NW) * 1024);
#pragma unroll
      for (int i = 0; i < VI; ++i)
        if (wid + i * NW < VBLK) g2lds16(vt_base + voff[i], (char*)smV[buf] + (wid + i * NW) * 1024);
    } else {  // ragged last tile: rows past S copy row S-1
#pragma unroll
      for (int i = 0; i < KI; ++i)
        if (wid + i * NW < KBLK) {
          const int row = ((wid + i * NW) * 64 + lane) / KSL;
          const int dr = row - min(row, lim);
          g2lds16(kt_base + koff[i] - (size_t)dr * rs_qk * 2, (char*)smK[buf] + (wid + i * NW) * 1024);
        }
#pragma unroll
      for (int i = 0; i < VI; ++i)
        if (wid + i * NW < VBLK) {
          const int row = ((wid + i * NW) * 64 + lane) / VSL;
          const int dr = row - min(row, lim);
          g2lds16(vt_base + voff[i] - (size_t)dr * rs_v * 2, (char*)smV[buf] + (wid + i * NW) * 1024);
        }
    }
  };

  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qvalid) z = *(const u32x4*)(q + ((size_t)b * S + tq) * rs_qk + (size_t)h * DQK + ks * 16 + 8 * half);
    qf[ks] = z;
  }

  float m = -INFINITY, l = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[eb][i] = 0.f;

  const int kt_last = min(S - 1, qw * QW + QW - 1) / TK;
  stage_bytes(scls[0], cls + ((size_t)b * NQ + qt0) * NK, kt_last + 1);
  stage_bytes(scls[1], cls + ((size_t)b * NQ + qt1) * NK, kt_last + 1);
  const uint8_t* cls0 = scls[0];
  const uint8_t* cls1 = scls[1];
  const uint8_t* clsw = scls[qt_w - qt0];
  const uint64_t* bits_q = bits + ((size_t)b * S + (qvalid ? tq : 0)) * W;
  auto next_tile = [&](int kt) {
    int n = kt + 1;
    while (n <= kt_last && cls0[n] == 0 && cls1[n] == 0) ++n;
    return n;
  };
  // this lane's selection word of tile kt (FULL: all ones; EMPTY: none)
  auto word = [&](int kt) -> uint64_t {
    const int c = clsw[kt];
    if (!qvalid || c == 0) return 0ull;
    return c == 2 ? ~0ull : bits_q[kt];
  };

  f32x16 sacc[2];
  __syncthreads();  // class rows staged
  int kt = next_tile(-1);
  if (kt <= kt_last) issue(kt, 0);
  uint64_t mw = kt <= kt_last ? word(kt) : 0ull;
  int buf = 0;
  while (kt <= kt_last) {
    const int kn = next_tile(kt);
    const int c = clsw[kt];
    wait_vmem();
    __syncthreads();  // tile kt visible in `buf`; every wave is done with the other buffer
    const uint64_t mw_n = kn <= kt_last ? word(kn) : 0ull;
    if (kn <= kt_last) issue(kn, buf ^ 1);
    if (c != 0 && __ballot(mw != 0ull)) {
      const float tmax = fwd_scores(smK[buf], qf, mw, c == 2, scale_log2, sacc);
      fwd_update(smV[buf], sacc, tmax, scale_log2, m, l, oacc);
    }
    mw = mw_n;
    buf ^= 1;
    kt = kn;
  }

  const float l_tot = half_sum(l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    uint16_t* orow = o + ((size_t)b * S + tq) * rs_v + (size_t)h * DV;
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = eb * 32 + 8 * g + 4 * half;
        u32x2 pk2 = {pack_bf2(oacc[eb][4 * g] * inv, oacc[eb][4 * g + 1] * inv),
                     pack_bf2(oacc[eb][4 * g + 2] * inv, oacc[eb][4 * g + 3] * inv)};
        *(u32x2*)(orow + e) = pk2;
      }
    if (half == 0)
      lse[((size_t)b * H + h) * S + tq] =
          l_tot > 0.f ? m * 0.69314718055994530942f + logf(l_tot) : -INFINITY;
  }
}

// Plain kernel for any head dims <= 256 and fp32 or bf16: one wave per
// (b, t, h), 64 keys (one mask word) per step. Lanes own keys for the logits
// and head-dim slots for the output.
template <typename T>
__global__ __launch_bounds__(256) void attn_fwd_plain_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const uint64_t* __restrict__ bits, int B, int S, int H, int Dqk, int Dv, float scale,
    T* __restrict__ o, float* __restrict__ lse) {
  __shared__ float qs[4][256];
  __shared__ float ps[4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + wid;  // (b, t, h) flattened
  if (row >= (size_t)B * S * H) return;             // whole wave leaves together
  const int h = (int)(row % H);
  const int t = (int)((row / H) % S);
  const int b = (int)(row / ((size_t)H * S));
  const int W = (S + 63) / 64;
  const T* qrow = q + ((size_t)b * S + t) * H * Dqk + (size_t)h * Dqk;
  for (int d = lane; d < Dqk; d += 64) qs[wid][d] = Elem<T>::load(qrow + d);
  __builtin_amdgcn_wave_barrier();
  float m = -INFINITY, l = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const uint64_t* brow = bits + ((size_t)b * S + t) * W;
  for (int w = 0; w <= t / 64; ++w) {
    const uint64_t word = brow[w];
    if (word == 0ull) continue;
    const int s = 64 * w + lane;
    float x = -INFINITY;
    if ((word >> lane) & 1ull) {
      const T* krow = k + ((size_t)b * S + s) * H * Dqk + (size_t)h * Dqk;
      float dot = 0.f;
      for (int d = 0; d < Dqk; ++d) dot = fmaf(qs[wid][d], Elem<T>::load(krow + d), dot);
      x = dot * scale;
    }
    const float m_new = fmaxf(m, wave_max(x));
    const float alpha = expf(m - m_new);
    const float p = (x == -INFINITY) ? 0.f : expf(x - m_new);
    l = l * alpha + wave_sumf(p);
    m = m_new;
    ps[wid][lane] = p;
    __builtin_amdgcn_wave_barrier();
    for (int j = 0; j < 4; ++j) acc[j] *= alpha;
    for (int jj = 0; jj < 64; ++jj) {
      if (!((word >> jj) & 1ull)) continue;
      const float pj = ps[wid][jj];
      const T* vrow = v + ((size_t)b * S + 64 * w + jj) * H * Dv + (size_t)h * Dv;
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (e < Dv) acc[j] = fmaf(pj, Elem<T>::load(vrow + e), acc[j]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  T* orow = o + ((size_t)b * S + t) * H * Dv + (size_t)h * Dv;
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < Dv) Elem<T>::store(orow + e, acc[j] * inv);
  }
  if (lane == 0) lse[((size_t)b * H + h) * S + t] = l > 0.f ? m + logf(l) : -INFINITY;
}

hipError_t launch_attn_fwd_mfma(const void* q, const void* k, const void* v, const uint64_t* bits,
                                const uint8_t* cls, int B, int S, int H, float scale, void* o,
                                float* lse, hipStream_t st) {
  const size_t nblk = (size_t)((S + fwd::QW - 1) / fwd::QW) * B * H;
  hipLaunchKernelGGL(attn_fwd_mfma_kernel, dim3((unsigned)nblk), dim3(fwd::NW * 64), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, bits, cls, B, S, H,
                     scale * 1.4426950408889634f, (uint16_t*)o, lse);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_plain(const void* q, const void* k, const void* v, const uint64_t* bits,
                                 int B, int S, int H, int Dqk, int Dv, float scale, bool bf16,
                                 void* o, float* lse, hipStream_t st) {
  const size_t nblk = ((size_t)B * S * H + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL(attn_fwd_plain_kernel<uint16_t>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, bits, B, S, H,
                       Dqk, Dv, scale, (uint16_t*)o, lse);
  else
    hipLaunchKernelGGL(attn_fwd_plain_kernel<float>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, bits, B, S, H, Dqk, Dv,
                       scale, (float*)o, lse);
  return hipGetLastError();
}

}  // namespace dsa
