// Plain (VALU) backward kernels over the DSA selection mask: fp32, and bf16
// with head dims the MFMA kernels do not take (any dims <= 256).
//
// Source: "Support Ring Attention with DeepSeek DSA Sparse Indexer", Backward
// Flow (dQ = dP K, dK = dP^T Q, dV = P^T dO on the kept entries; dK/dV
// key-major). D(t) = dO(t) . O(t) and the base-2 log-sum-exp are computed
// first, by attn_bwd_prep_kernel, into the backward workspace.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

// ---------------------------------------------------------------------------
// Backward prologue: D(b,h,t) = sum_e dO(b,t,h,e) O(b,t,h,e) and
// lse(b,h,t) * log2(e), as two float32 [B,H,S] arrays at the workspace start.
// 16 lanes per (b, t, h) row, 8 elements per lane per pass.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                            const float* __restrict__ lse, int B, int S, int H,
                                                            int Dv, float* __restrict__ ws) {
  const int sub = threadIdx.x & 15;
  const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b, t, h) flattened
  const bool valid = row < (size_t)B * S * H;
  float acc = 0.f;
  if (valid) {
    const T* orow = o + row * Dv;
    const T* drow = dout + row * Dv;
    for (int e0 = sub * 8; e0 < Dv; e0 += 128) {
      if (sizeof(T) == 2 && e0 + 8 <= Dv && (Dv & 7) == 0) {
        const u32x4 a = *(const u32x4*)(orow + e0), g = *(const u32x4*)(drow + e0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc = fmaf(__uint_as_float(a[j] << 16), __uint_as_float(g[j] << 16), acc);
          acc = fmaf(__uint_as_float(a[j] & 0xffff0000u), __uint_as_float(g[j] & 0xffff0000u), acc);
        }
      } else {
        for (int e = e0; e < min(Dv, e0 + 8); ++e) acc = fmaf(Elem<T>::load(orow + e), Elem<T>::load(drow + e), acc);
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m, 16);
  if (valid && sub == 0) {
    const int h = (int)(row % H);
    const int t = (int)((row / H) % S);
    const int b = (int)(row / ((size_t)H * S));
    const size_t i = ((size_t)b * H + h) * S + t;
    ws[i] = acc;
    ws[(size_t)B * H * S + i] = lse[i] * 1.4426950408889634f;
  }
}

hipError_t launch_attn_bwd_prep(const void* o, const void* dout, const float* lse, int B, int S, int H, int Dv,
                                bool bf16, float* ws, hipStream_t st) {
  const size_t nblk = ((size_t)B * S * H + 15) / 16;
  if (bf16)
    hipLaunchKernelGGL(attn_bwd_prep_kernel<uint16_t>, dim3((unsigned)nblk), dim3(256), 0, st, (const uint16_t*)o,
                       (const uint16_t*)dout, lse, B, S, H, Dv, ws);
  else
    hipLaunchKernelGGL(attn_bwd_prep_kernel<float>, dim3((unsigned)nblk), dim3(256), 0, st, (const float*)o,
                       (const float*)dout, lse, B, S, H, Dv, ws);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plain kernels (any dims <= 256, fp32 or bf16).
// dq: one wave per (b, t, h), lanes over the keys of one mask word.
// dk/dv: one wave per (b, s, h), lanes over 64 queries at a time (t >= s),
//        reading bit (s % 64) of each query's word s / 64.
// Keys may be compressed blocks ("Add Flash Attention Support to Deepseek v4",
// Description): Sk keys of `ratio` tokens, key s visible to t when
// ratio*s + ratio - 1 <= t; mask rows are ceil(Sk / 64) words. ratio 1 and
// Sk = S is token-level DSA.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_dq_plain_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ D,
    const uint64_t* __restrict__ bits, int B, int S, int Sk, int ratio, int H, int Dqk, int Dv, float scale,
    T* __restrict__ dq) {
  __shared__ float qs[4][256], os[4][256], dss[4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + wid;
  if (row >= (size_t)B * S * H) return;
  const int h = (int)(row % H);
  const int t = (int)((row / H) % S);
  const int b = (int)(row / ((size_t)H * S));
  const int W = (Sk + 63) / 64;
  const int tk = (t + 1) / ratio - 1;  // last visible key
  for (int d = lane; d < Dqk; d += 64) qs[wid][d] = Elem<T>::load(q + row * Dqk + d);
  for (int d = lane; d < Dv; d += 64) os[wid][d] = Elem<T>::load(dout + row * Dv + d);
  __builtin_amdgcn_wave_barrier();
  const float L = lse[((size_t)b * H + h) * S + t];
  const float Dt = D[((size_t)b * H + h) * S + t];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const uint64_t* brow = bits + ((size_t)b * S + t) * W;
  for (int w = 0; w < (tk + 64) / 64; ++w) {
    const uint64_t word = brow[w];
    if (word == 0ull) continue;
    const int s = 64 * w + lane;
    float dsv = 0.f;
    if ((word >> lane) & 1ull) {
      const T* krow = k + (((size_t)b * Sk + s) * H + h) * Dqk;
      const T* vrow = v + (((size_t)b * Sk + s) * H + h) * Dv;
      float dot = 0.f, dp = 0.f;
      for (int d = 0; d < Dqk; ++d) dot = fmaf(qs[wid][d], Elem<T>::load(krow + d), dot);
      for (int e = 0; e < Dv; ++e) dp = fmaf(os[wid][e], Elem<T>::load(vrow + e), dp);
      const float p = expf(dot * scale - L);
      dsv = p * (dp - Dt);
    }
    dss[wid][lane] = dsv;
    __builtin_amdgcn_wave_barrier();
    for (int jj = 0; jj < 64; ++jj) {
      if (!((word >> jj) & 1ull)) continue;
      const float g = dss[wid][jj];
      const T* krow = k + (((size_t)b * Sk + 64 * w + jj) * H + h) * Dqk;
      for (int j = 0; j < 4; ++j) {
        const int d = lane + 64 * j;
        if (d < Dqk) acc[j] = fmaf(g, Elem<T>::load(krow + d), acc[j]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  for (int j = 0; j < 4; ++j) {
    const int d = lane + 64 * j;
    if (d < Dqk) Elem<T>::store(dq + row * Dqk + d, acc[j] * scale);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_plain_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ D, const uint64_t* __restrict__ bits, int B,
    int S, int Sk, int ratio, int H, int Dqk, int Dv, float scale, T* __restrict__ dk, T* __restrict__ dv) {
  __shared__ float ks_[4][256], vs_[4][256], ps[4][64], dss[4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + wid;  // (b, s, h), s one of the Sk keys
  if (row >= (size_t)B * Sk * H) return;
  const int h = (int)(row % H);
  const int s = (int)((row / H) % Sk);
  const int b = (int)(row / ((size_t)H * Sk));
  const int W = (Sk + 63) / 64;
  for (int d = lane; d < Dqk; d += 64) ks_[wid][d] = Elem<T>::load(k + row * Dqk + d);
  for (int d = lane; d < Dv; d += 64) vs_[wid][d] = Elem<T>::load(v + row * Dv + d);
  __builtin_amdgcn_wave_barrier();
  float ak[4] = {0.f, 0.f, 0.f, 0.f}, av[4] = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = ratio * s + ratio - 1; t0 < S; t0 += 64) {  // the first query that sees key s
    const int t = t0 + lane;
    float p = 0.f, dsv = 0.f;
    bool kept = false;
    if (t < S) kept = (bits[((size_t)b * S + t) * W + (s >> 6)] >> (s & 63)) & 1ull;
    if (kept) {
      const T* qrow = q + (((size_t)b * S + t) * H + h) * Dqk;
      const T* orow = dout + (((size_t)b * S + t) * H + h) * Dv;
      float dot = 0.f, dp = 0.f;
      for (int d = 0; d < Dqk; ++d) dot = fmaf(Elem<T>::load(qrow + d), ks_[wid][d], dot);
      for (int e = 0; e < Dv; ++e) dp = fmaf(Elem<T>::load(orow + e), vs_[wid][e], dp);
      p = expf(dot * scale - lse[((size_t)b * H + h) * S + t]);
      dsv = p * (dp - D[((size_t)b * H + h) * S + t]);
    }
    const uint64_t km = __ballot(kept);
    ps[wid][lane] = p;
    dss[wid][lane] = dsv;
    __builtin_amdgcn_wave_barrier();
    for (int jj = 0; jj < 64; ++jj) {
      if (!((km >> jj) & 1ull)) continue;
      const size_t trow = ((size_t)b * S + t0 + jj) * H + h;
      const float pj = ps[wid][jj], gj = dss[wid][jj];
      for (int j = 0; j < 4; ++j) {
        const int d = lane + 64 * j;
        if (d < Dqk) ak[j] = fmaf(gj, Elem<T>::load(q + trow * Dqk + d), ak[j]);
        if (d < Dv) av[j] = fmaf(pj, Elem<T>::load(dout + trow * Dv + d), av[j]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  for (int j = 0; j < 4; ++j) {
    const int d = lane + 64 * j;
    if (d < Dqk) Elem<T>::store(dk + row * Dqk + d, ak[j] * scale);
    if (d < Dv) Elem<T>::store(dv + row * Dv + d, av[j]);
  }
}

hipError_t launch_attn_bwd_dq_plain(const void* q, const void* k, const void* v,
                                    const void* dout, const float* lse, const float* D, const uint64_t* bits,
                                    int B, int S, int Sk, int ratio, int H, int Dqk, int Dv, float scale,
                                    bool bf16, void* dq, hipStream_t st) {
  const size_t nblk = ((size_t)B * S * H + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL(attn_bwd_dq_plain_kernel<uint16_t>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dout, lse, D, bits, B, S, Sk, ratio, H, Dqk, Dv, scale, (uint16_t*)dq);
  else
    hipLaunchKernelGGL(attn_bwd_dq_plain_kernel<float>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v,
                       (const float*)dout, lse, D, bits, B, S, Sk, ratio, H, Dqk, Dv, scale, (float*)dq);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv_plain(const void* q, const void* k, const void* v, const void* dout,
                                      const float* lse, const float* D, const uint64_t* bits, int B,
                                      int S, int Sk, int ratio, int H, int Dqk, int Dv, float scale, bool bf16,
                                      void* dk, void* dv, hipStream_t st) {
  const size_t nblk = ((size_t)B * Sk * H + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL(attn_bwd_dkdv_plain_kernel<uint16_t>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                       lse, D, bits, B, S, Sk, ratio, H, Dqk, Dv, scale, (uint16_t*)dk, (uint16_t*)dv);
  else
    hipLaunchKernelGGL(attn_bwd_dkdv_plain_kernel<float>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, (const float*)dout, lse, D,
                       bits, B, S, Sk, ratio, H, Dqk, Dv, scale, (float*)dk, (float*)dv);
  return hipGetLastError();
}

}  // namespace dsa
