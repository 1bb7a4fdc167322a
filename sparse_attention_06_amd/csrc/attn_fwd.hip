// Block-sparse flash-attention forward over the DSA selection mask (gfx950).
//
// Source: "Support Ring Attention with DeepSeek DSA Sparse Indexer", Forward
// Flow (one [batch, S, S] index mask for all heads, combined with causal; on
// kept entries the logit is the scaled query-key product, others drop out);
// "Integrate DeepSeek Sparse Attention with Tokamax Flash Attention",
// Description (flash attention driven by a dynamic 3-D index mask).
//
// MFMA kernel (bf16, Dqk = 192, Dv = 128). A workgroup is one (b, h, 256-query
// block) with 8 waves (two per SIMD) of 32 queries each. It walks the 64-key
// tiles up to the diagonal. Tiles that are EMPTY for both of its 128-query
// tiles are skipped outright. A wave whose tile is EMPTY idles. PARTIAL tiles
// read one u64 selection word per query.
//   S^T = K Q^T: keys on MFMA rows, queries on columns, so each lane owns one
//   query and 32 of the tile's 64 logits. The online-softmax max and sum are
//   in-lane, with one exchange between lane halves. Q stays in VGPRs.
//   O^T += V^T P^T: the probabilities go straight from the S^T accumulator
//   into the B operand. The key order inside each 16-wide k step is permuted
//   to match the accumulator layout. V^T comes from the natural V tile in LDS
//   through the gfx950 transposing LDS read, with the same permutation.
// K/V tiles are double buffered in LDS and filled by direct global->LDS copies
// (no staging registers). The next non-empty tile's copies are issued before
// the current tile is computed. exp2 is the hardware
// v_exp_f32, with the scale folded in (scale * log2 e). O is rescaled only when
// a tile max passes the reference max by more than 2^8.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

namespace fwd {
constexpr int DQK = 192, DV = 128, TK = 64;
constexpr int NW = 8;                // waves per workgroup: 2 per SIMD
constexpr int QW = 32 * NW;          // queries per workgroup (two 128-query tiles)
constexpr int KS = DQK / 16;         // k steps of S^T
constexpr int KSL = DQK / 8 + 1;     // 16-byte slots per LDS K row (one pad slot): 400 B
constexpr int VSL = DV / 8 + 1;      // ... per V row: 272 B
constexpr int KP = KSL * 8;          // LDS pitch of a K row (elements)
constexpr int VP = VSL * 8;          // LDS pitch of a V row
constexpr int KBLK = TK * KSL / 64;  // 1 KB blocks per K tile (25)
constexpr int VBLK = TK * VSL / 64;  // ... per V tile (17)
constexpr int KI = (KBLK + NW - 1) / NW, VI = (VBLK + NW - 1) / NW;  // blocks per wave
static_assert(TK * KSL % 64 == 0 && TK * VSL % 64 == 0, "tiles must be whole 1 KB blocks");
}  // namespace fwd

// One 64-key tile of the online softmax for a wave's 32 queries. Keys whose
// selection bit is clear drop out (FULL tiles pass all-ones words). This
// lane's keys are kb*32 + 8i + 4*half + r (i, r in 0..3); its query word is
// passed pre-shifted by 4*half and split into halves, so each bit sits at the
// constant position 8i + r of word kb.
__device__ __forceinline__ void fwd_tile(const uint16_t* sK, const uint16_t* sV, const u32x4 (&qf)[fwd::KS],
                                         uint32_t w0, uint32_t w1, float scale_log2, float& m, float& l,
                                         f32x16 (&oacc)[4]) {
  using namespace fwd;
  const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
  f32x16 sacc[2];
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

  // masked max over raw logits (the scale is positive, so it commutes with max)
  float tm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t w = kb ? w1 : w0;
      const float x = ((w >> (8 * (r >> 2) + (r & 3))) & 1u) ? sacc[kb][r] : -INFINITY;
      sacc[kb][r] = x;
      tm[r & 3] = fmaxf(tm[r & 3], x);
    }
  float tmax = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * scale_log2;

  // Lazy rescaling: probabilities are taken relative to a reference max m that
  // only moves when the tile max exceeds it by more than 8 (log2 units), so
  // p <= 2^8. O and l share the reference, so the result is unchanged; the
  // O rescale (64 accumulator multiplies) becomes rare.
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
  // double-buffered natural-layout K and V tiles, filled by direct global->LDS
  // copies; V^T fragments come from ds_read_b64_tr_b16 on the V tile
  __shared__ __attribute__((aligned(1024))) uint16_t smK[2][TK * KP];
  __shared__ __attribute__((aligned(1024))) uint16_t smV[2][TK * VP];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int W = (S + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int NQW = (S + QW - 1) / QW;
  // all query blocks of one (b, h) on one XCD (they share K/V), longest first
  const int Lb = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int bh = Lb / NQW;
  const int qw = NQW - 1 - Lb % NQW;
  const int b = bh / H, h = bh % H;
  const int tq = qw * QW + wid * 32 + col;  // this lane's query
  const bool qvalid = tq < S;
  const int qt_w = min(NQ - 1, (qw * QW + wid * 32) / 128);  // this wave's 128-query tile
  const int qt0 = qw * QW / 128, qt1 = min(NQ - 1, qt0 + 1);
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;  // token strides
  const uint16_t* kbase = k + (size_t)b * S * rs_qk + (size_t)h * DQK;
  const uint16_t* vbase = v + (size_t)b * S * rs_v + (size_t)h * DV;

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
  const uint8_t* cls0 = cls + ((size_t)b * NQ + qt0) * NK;
  const uint8_t* cls1 = cls + ((size_t)b * NQ + qt1) * NK;
  const uint8_t* clsw = cls + ((size_t)b * NQ + qt_w) * NK;
  const uint64_t* bits_q = bits + ((size_t)b * S + (qvalid ? tq : 0)) * W;
  auto next_tile = [&](int kt) {
    int n = kt + 1;
    while (n <= kt_last && cls0[n] == 0 && cls1[n] == 0) ++n;
    return n;
  };
  // this wave's 1 KB blocks of a tile: block j covers slots 64j .. 64j+63 of the
  // padded [64 rows][KSL or VSL slots] layout; pad slots copy a harmless chunk
  auto issue = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int j = wid + i * NW;
      if (j < KBLK) {
        const int slot = j * 64 + lane, row = slot / KSL, c = min(slot % KSL, KSL - 2);
        const int s = min(kt * TK + row, S - 1);
        g2lds16(kbase + (size_t)s * rs_qk + c * 8, (char*)smK[buf] + j * 1024);
      }
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int j = wid + i * NW;
      if (j < VBLK) {
        const int slot = j * 64 + lane, row = slot / VSL, c = min(slot % VSL, VSL - 2);
        const int s = min(kt * TK + row, S - 1);
        g2lds16(vbase + (size_t)s * rs_v + c * 8, (char*)smV[buf] + j * 1024);
      }
    }
  };

  int kt = next_tile(-1);
  if (kt <= kt_last) issue(kt, 0);
  int buf = 0;
  while (kt <= kt_last) {
    const int c = clsw[kt];
    uint64_t mw = (qvalid && c == 2) ? ~0ull : 0ull;
    if (c == 1 && qvalid) mw = bits_q[kt];
    wait_vmem();
    __syncthreads();  // tile kt visible in `buf`; every wave is done with the other buffer
    const int kn = next_tile(kt);
    if (kn <= kt_last) issue(kn, buf ^ 1);  // lands while this tile is computed
    if (c != 0 && __ballot(mw != 0ull))
      fwd_tile(smK[buf], smV[buf], qf, (uint32_t)(mw >> (4 * half)), (uint32_t)(mw >> (32 + 4 * half)),
               scale_log2, m, l, oacc);
    buf ^= 1;
    kt = kn;
  }

  const float l_tot = l + __shfl_xor(l, 32);
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
