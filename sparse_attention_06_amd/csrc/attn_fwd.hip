// Block-sparse flash-attention forward over the DSA selection mask (gfx950).
//
// Source: "Support Ring Attention with DeepSeek DSA Sparse Indexer", Forward
// Flow (one [batch, S, S] index mask for all heads, combined with causal; on
// kept entries the logit is the scaled query-key product, others drop out);
// "Integrate DeepSeek Sparse Attention with Tokamax Flash Attention",
// Description (flash attention driven by a dynamic 3-D index mask).
//
// MFMA kernel (bf16, Dqk = 192, Dv = 128). A workgroup is one (b, h, 128-query
// tile) with 4 waves of 32 queries each. It walks the 64-key tiles up to the
// diagonal. Tiles of class EMPTY are skipped outright. FULL tiles use no mask.
// PARTIAL tiles read one u64 selection word per query.
//   S^T = K Q^T: keys on MFMA rows, queries on columns, so each lane owns one
//   query and 32 of the tile's 64 logits. The online-softmax max and sum are
//   in-lane, with one exchange between lane halves. Q stays in VGPRs.
//   O^T += V^T P^T: the probabilities go straight from the S^T accumulator
//   into the B operand. The key order inside each 16-wide k step is permuted
//   to match the accumulator layout, and V^T is read from LDS with the same
//   permutation.
// exp2 with the scale folded in (scale * log2 e).
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

namespace fwd {
constexpr int DQK = 192, DV = 128, TK = 64;
constexpr int KS = DQK / 16;         // k steps of S^T
constexpr int KROW = DQK * 2 + 16;   // bytes per K row in LDS (padded)
constexpr int VTROW = TK * 2 + 16;   // bytes per V^T row (64 keys) in LDS (padded)
}  // namespace fwd

__global__ __launch_bounds__(256) void attn_fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint64_t* __restrict__ bits, const uint8_t* __restrict__ cls, int B, int S, int H,
    float scale_log2, uint16_t* __restrict__ o, float* __restrict__ lse) {
  using namespace fwd;
  __shared__ __attribute__((aligned(16))) unsigned char smK[TK * KROW];
  __shared__ __attribute__((aligned(16))) unsigned char smVT[DV * VTROW];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int W = (S + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int qt = NQ - 1 - (int)(blockIdx.x / (B * H));  // longest tiles first
  const int bh = blockIdx.x % (B * H);
  const int b = bh / H, h = bh % H;
  const int tq = qt * 128 + wid * 32 + col;  // this lane's query
  const bool qvalid = tq < S;
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;  // token strides

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

  const int kt_last = min(S - 1, qt * 128 + 127) / TK;
  const uint8_t* cls_row = cls + ((size_t)b * NQ + qt) * NK;
  const uint64_t* bits_q = bits + ((size_t)b * S + (qvalid ? tq : 0)) * W;

  for (int kt = 0; kt <= kt_last; ++kt) {
    const int c = cls_row[kt];
    if (c == 0) continue;  // uniform over the workgroup
    __syncthreads();       // previous tile's LDS reads are done
    // K tile [64][192] -> LDS rows
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int ci = tid + i * 256;
      const int row = ci / 24, cc = ci % 24;
      const int s = kt * TK + row;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (s < S) z = *(const u32x4*)(k + ((size_t)b * S + s) * rs_qk + (size_t)h * DQK + cc * 8);
      *(u32x4*)(smK + row * KROW + cc * 16) = z;
    }
    // V tile [64][128] -> LDS transposed V^T[e][key], two keys per 32-bit store
    {
      const int kp = tid & 31, ec = tid >> 5;  // keys 2kp, 2kp+1; e = 16 ec .. 16 ec + 15
      const int s0 = kt * TK + 2 * kp;
      u32x4 a0 = {0u, 0u, 0u, 0u}, a1 = a0, b0 = a0, b1 = a0;
      if (s0 < S) {
        const uint16_t* p = v + ((size_t)b * S + s0) * rs_v + (size_t)h * DV + ec * 16;
        a0 = *(const u32x4*)p;
        a1 = *(const u32x4*)(p + 8);
      }
      if (s0 + 1 < S) {
        const uint16_t* p = v + ((size_t)b * S + s0 + 1) * rs_v + (size_t)h * DV + ec * 16;
        b0 = *(const u32x4*)p;
        b1 = *(const u32x4*)(p + 8);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t wa = e < 8 ? a0[(e & 7) >> 1] : a1[(e & 7) >> 1];
        const uint32_t wb = e < 8 ? b0[(e & 7) >> 1] : b1[(e & 7) >> 1];
        const uint32_t lo = (e & 1) ? (wa >> 16) : (wa & 0xffffu);
        const uint32_t hi = (e & 1) ? (wb >> 16) : (wb & 0xffffu);
        *(uint32_t*)(smVT + (ec * 16 + e) * VTROW + kp * 4) = lo | (hi << 16);
      }
    }
    __syncthreads();

    uint64_t mw = ~0ull;
    if (c == 1) {
      mw = qvalid ? bits_q[kt] : 0ull;
      if (__ballot(mw != 0ull) == 0ull) continue;  // no selected key for this wave
    }

    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *(const u32x4*)(smK + (kb * 32 + col) * KROW + (ks * 16 + 8 * half) * 2);
        sacc[kb] = mfma32(a, qf[ks], sacc[kb]);
      }

    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[kb][r] * scale_log2;
        if (c == 1 && !((mw >> (kb * 32 + acc_row(r, half))) & 1ull)) x = -INFINITY;
        sacc[kb][r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[eb][i] *= alpha;

    u32x4 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        float pv[8];
#pragma unroll
        for (int c8 = 0; c8 < 8; ++c8) {
          pv[c8] = exp2f(sacc[kb][8 * p2 + c8] - m_use);
          l += pv[c8];
        }
        pb[kb][p2] = u32x4{pack_bf2(pv[0], pv[1]), pack_bf2(pv[2], pv[3]), pack_bf2(pv[4], pv[5]),
                           pack_bf2(pv[6], pv[7])};
      }
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          const unsigned char* base = smVT + (eb * 32 + col) * VTROW + (kb * 32 + 16 * p2 + 4 * half) * 2;
          const u32x2 lo = *(const u32x2*)base;
          const u32x2 hi = *(const u32x2*)(base + 16);
          oacc[eb] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[kb][p2], oacc[eb]);
        }
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
        u32x2 pk = {pack_bf2(oacc[eb][4 * g] * inv, oacc[eb][4 * g + 1] * inv),
                    pack_bf2(oacc[eb][4 * g + 2] * inv, oacc[eb][4 * g + 3] * inv)};
        *(u32x2*)(orow + e) = pk;
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
  const size_t nblk = (size_t)n_qtiles(S) * B * H;
  hipLaunchKernelGGL(attn_fwd_mfma_kernel, dim3((unsigned)nblk), dim3(256), 0, st,
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
