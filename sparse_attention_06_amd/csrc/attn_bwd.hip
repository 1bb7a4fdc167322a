// Block-sparse flash-attention backward over the DSA selection mask (gfx950).
//
// Source: "Support Ring Attention with DeepSeek DSA Sparse Indexer", Backward
// Flow: the forward runs query-major while dK/dV run key-major. Each uses the
// same index mask, dQ = dP K, dK = dP^T Q and dV = P^T dO.
//
//   D(t)   = sum_e dO(t,e) O(t,e)       (computed by the query-major kernel,
//                                         which runs first and stores it)
//   P      = exp(scale q.k - LSE(t)) on kept (t, s)
//   dP     = dO(t) . v(s),   dS = P (dP - D(t))
//   dV(s) += P dO(t),        dK(s) += scale dS q(t)      (key-major kernel)
//   dQ(t)  = scale sum_s dS k(s)                         (query-major kernel)
// Both MFMA kernels recompute P from LSE. Neither uses atomics, so the result
// is deterministic. The key-major kernel reads the same row-major selection
// words as the forward. A lane owns one key, so the bit it needs sits at a
// fixed position of each query's word, and no transposed copy of the mask is
// needed.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

namespace bwd {
constexpr int DQK = 192, DV = 128;
constexpr int QC = 32;                 // queries per chunk (key-major kernel)
constexpr int QROW = DQK * 2 + 16;     // natural Q row in LDS
constexpr int DOROW = DV * 2 + 16;     // natural dO row
constexpr int TROW = QC * 2 + 16;      // transposed rows (32 queries)
constexpr int TK = 64;                 // keys per tile (query-major kernel)
constexpr int KROW = DQK * 2 + 16;
constexpr int VROW = DV * 2 + 16;
constexpr int KTROW = TK * 2 + 16;     // K^T rows (64 keys)
}  // namespace bwd

// transpose-store 8 bf16 values (one 16-byte chunk of row `qi`, columns
// c0..c0+7) into a [col][query] LDS array with row pitch `pitch` bytes.
__device__ __forceinline__ void tstore8(unsigned char* base, int pitch, int c0, int qi, u32x4 val) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = val[e >> 1];
    const uint16_t x = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
    *(uint16_t*)(base + (c0 + e) * pitch + qi * 2) = x;
  }
}

// ---------------------------------------------------------------------------
// dK / dV, key-major. Workgroup = (b, h, 128 keys), wave = 32 keys. Walks
// 32-query chunks from the first key to the end.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ D,
    const uint64_t* __restrict__ bits, const uint8_t* __restrict__ cls, int B, int S, int H,
    float scale, float scale_log2, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  using namespace bwd;
  __shared__ __attribute__((aligned(16))) unsigned char smQ[QC * QROW];
  __shared__ __attribute__((aligned(16))) unsigned char smQT[DQK * TROW];
  __shared__ __attribute__((aligned(16))) unsigned char smdO[QC * DOROW];
  __shared__ __attribute__((aligned(16))) unsigned char smdOT[DV * TROW];
  __shared__ float smL[QC], smD[QC];
  __shared__ uint64_t smW[2][QC];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int W = (S + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int nkb = (S + 127) / 128;
  const int kblk = (int)(blockIdx.x % nkb);  // short key blocks (late keys) last
  const int bh = (int)(blockIdx.x / nkb);
  const int b = bh / H, h = bh % H;
  const int kb0 = kblk * 128;
  const int s0 = kb0 + wid * 32;  // this wave's first key
  const int sk = s0 + col;        // this lane's key
  const bool kvalid = sk < S;
  const int kt_w = s0 / 64;        // this wave's 64-key tile
  const int kt_lo = kb0 / 64;      // workgroup's first key tile
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;

  u32x4 kf[DQK / 16], vf[DV / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (kvalid) z = *(const u32x4*)(k + ((size_t)b * S + sk) * rs_qk + (size_t)h * DQK + ks * 16 + 8 * half);
    kf[ks] = z;
  }
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (kvalid) z = *(const u32x4*)(v + ((size_t)b * S + sk) * rs_v + (size_t)h * DV + ks * 16 + 8 * half);
    vf[ks] = z;
  }
  f32x16 dkacc[DQK / 32], dvacc[DV / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dkacc[i][j] = 0.f;
#pragma unroll
  for (int i = 0; i < DV / 32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dvacc[i][j] = 0.f;

  const int bitpos = sk & 63;
  const int nchunks = (S + QC - 1) / QC;
  for (int qc = kb0 / QC; qc < nchunks; ++qc) {
    const int q0 = qc * QC;
    const int qt = q0 / 128;
    const uint8_t c_lo = cls[((size_t)b * NQ + qt) * NK + kt_lo];
    const uint8_t c_hi = (kt_lo + 1 < NK) ? cls[((size_t)b * NQ + qt) * NK + kt_lo + 1] : 0;
    if (c_lo == 0 && c_hi == 0) continue;  // uniform
    __syncthreads();
    // stage Q chunk (natural + transposed), dO chunk (natural + transposed)
    for (int ci = tid; ci < QC * 24; ci += 256) {
      const int qi = ci / 24, cc = ci % 24;
      const int t = q0 + qi;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (t < S) z = *(const u32x4*)(q + ((size_t)b * S + t) * rs_qk + (size_t)h * DQK + cc * 8);
      *(u32x4*)(smQ + qi * QROW + cc * 16) = z;
      tstore8(smQT, TROW, cc * 8, qi, z);
    }
    for (int ci = tid; ci < QC * 16; ci += 256) {
      const int qi = ci / 16, cc = ci % 16;
      const int t = q0 + qi;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (t < S) z = *(const u32x4*)(dout + ((size_t)b * S + t) * rs_v + (size_t)h * DV + cc * 8);
      *(u32x4*)(smdO + qi * DOROW + cc * 16) = z;
      tstore8(smdOT, TROW, cc * 8, qi, z);
    }
    if (tid < QC) {
      const int t = q0 + tid;
      smL[tid] = t < S ? lse[((size_t)b * H + h) * S + t] * 1.4426950408889634f : INFINITY;
      smD[tid] = t < S ? D[((size_t)b * H + h) * S + t] : 0.f;
    } else if (tid < 3 * QC) {
      const int qi = (tid - QC) % QC, which = (tid - QC) / QC;
      const int t = q0 + qi, kt = kt_lo + which;
      smW[which][qi] = (t < S && kt < NK) ? bits[((size_t)b * S + t) * W + kt] : 0ull;
    }
    __syncthreads();

    const uint8_t cw = (kt_w == kt_lo) ? c_lo : c_hi;
    if (cw == 0 || s0 > q0 + QC - 1) continue;  // empty tile or all keys after the chunk

    // S = Q K^T : rows = queries, columns = keys (lane's key)
    f32x16 sacc, dpacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks) {
      const u32x4 a = *(const u32x4*)(smQ + col * QROW + (ks * 16 + 8 * half) * 2);
      sacc = mfma32(a, kf[ks], sacc);
    }
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) {
      const u32x4 a = *(const u32x4*)(smdO + col * DOROW + (ks * 16 + 8 * half) * 2);
      dpacc = mfma32(a, vf[ks], dpacc);
    }
    const uint64_t* mwv = smW[kt_w - kt_lo];
    float p[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = acc_row(r, half);
      const bool keep = cw == 2 ? (q0 + qi < S) : (((mwv[qi] >> bitpos) & 1ull) != 0ull);
      const float pr = keep ? exp2f(sacc[r] * scale_log2 - smL[qi]) : 0.f;
      p[r] = pr;
      ds[r] = pr * (dpacc[r] - smD[qi]);
    }
    u32x4 pb[2], db[2];
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
      pb[p2] = u32x4{pack_bf2(p[8 * p2], p[8 * p2 + 1]), pack_bf2(p[8 * p2 + 2], p[8 * p2 + 3]),
                     pack_bf2(p[8 * p2 + 4], p[8 * p2 + 5]), pack_bf2(p[8 * p2 + 6], p[8 * p2 + 7])};
      db[p2] = u32x4{pack_bf2(ds[8 * p2], ds[8 * p2 + 1]), pack_bf2(ds[8 * p2 + 2], ds[8 * p2 + 3]),
                     pack_bf2(ds[8 * p2 + 4], ds[8 * p2 + 5]), pack_bf2(ds[8 * p2 + 6], ds[8 * p2 + 7])};
    }
    // dV^T[e, s] += dO^T[e, q] P[q, s];  dK^T[d, s] += Q^T[d, q] dS[q, s]
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
#pragma unroll
      for (int eb = 0; eb < DV / 32; ++eb) {
        const unsigned char* base = smdOT + (eb * 32 + col) * TROW + (16 * p2 + 4 * half) * 2;
        const u32x2 lo = *(const u32x2*)base;
        const u32x2 hi = *(const u32x2*)(base + 16);
        dvacc[eb] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[p2], dvacc[eb]);
      }
#pragma unroll
      for (int db2 = 0; db2 < DQK / 32; ++db2) {
        const unsigned char* base = smQT + (db2 * 32 + col) * TROW + (16 * p2 + 4 * half) * 2;
        const u32x2 lo = *(const u32x2*)base;
        const u32x2 hi = *(const u32x2*)(base + 16);
        dkacc[db2] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, db[p2], dkacc[db2]);
      }
    }
  }

  if (kvalid) {
    uint16_t* dkrow = dk + ((size_t)b * S + sk) * rs_qk + (size_t)h * DQK;
    uint16_t* dvrow = dv + ((size_t)b * S + sk) * rs_v + (size_t)h * DV;
#pragma unroll
    for (int i = 0; i < DQK / 32; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = i * 32 + 8 * g + 4 * half;
        *(u32x2*)(dkrow + d) = u32x2{pack_bf2(dkacc[i][4 * g] * scale, dkacc[i][4 * g + 1] * scale),
                                     pack_bf2(dkacc[i][4 * g + 2] * scale, dkacc[i][4 * g + 3] * scale)};
      }
#pragma unroll
    for (int i = 0; i < DV / 32; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = i * 32 + 8 * g + 4 * half;
        *(u32x2*)(dvrow + e) = u32x2{pack_bf2(dvacc[i][4 * g], dvacc[i][4 * g + 1]),
                                     pack_bf2(dvacc[i][4 * g + 2], dvacc[i][4 * g + 3])};
      }
  }
}

// ---------------------------------------------------------------------------
// dQ, query-major. Workgroup = (b, h, 128 queries), wave = 32 queries. Walks
// 64-key tiles up to the diagonal, skipping EMPTY tiles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ D, const uint64_t* __restrict__ bits, const uint8_t* __restrict__ cls, int B,
    int S, int H, float scale, float scale_log2, uint16_t* __restrict__ dq) {
  using namespace bwd;
  __shared__ __attribute__((aligned(16))) unsigned char smK[TK * KROW];
  __shared__ __attribute__((aligned(16))) unsigned char smKT[DQK * KTROW];
  __shared__ __attribute__((aligned(16))) unsigned char smV[TK * VROW];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int W = (S + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int qt = NQ - 1 - (int)(blockIdx.x / (B * H));
  const int bh = blockIdx.x % (B * H);
  const int b = bh / H, h = bh % H;
  const int tq = qt * 128 + wid * 32 + col;
  const bool qvalid = tq < S;
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;

  u32x4 qf[DQK / 16], of[DV / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qvalid) z = *(const u32x4*)(q + ((size_t)b * S + tq) * rs_qk + (size_t)h * DQK + ks * 16 + 8 * half);
    qf[ks] = z;
  }
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qvalid) z = *(const u32x4*)(dout + ((size_t)b * S + tq) * rs_v + (size_t)h * DV + ks * 16 + 8 * half);
    of[ks] = z;
  }
  const float Lq = qvalid ? lse[((size_t)b * H + h) * S + tq] * 1.4426950408889634f : INFINITY;
  // D(t) = dO(t) . O(t): this lane holds half of dO(t) as MFMA fragments; the
  // matching half of O(t) is read here and the halves are summed across lanes
  float Dq = 0.f;
  if (qvalid) {
    const uint16_t* orow = o + ((size_t)b * S + tq) * rs_v + (size_t)h * DV;
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) {
      const u32x4 ov = *(const u32x4*)(orow + ks * 16 + 8 * half);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wo = ov[e >> 1], wd = of[ks][e >> 1];
        const uint16_t xo = (e & 1) ? (uint16_t)(wo >> 16) : (uint16_t)(wo & 0xffffu);
        const uint16_t xd = (e & 1) ? (uint16_t)(wd >> 16) : (uint16_t)(wd & 0xffffu);
        Dq = fmaf(bf2f(xo), bf2f(xd), Dq);
      }
    }
  }
  Dq += __shfl_xor(Dq, 32);
  if (qvalid && half == 0) D[((size_t)b * H + h) * S + tq] = Dq;
  f32x16 dqacc[DQK / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dqacc[i][j] = 0.f;

  const int kt_last = min(S - 1, qt * 128 + 127) / TK;
  const uint8_t* cls_row = cls + ((size_t)b * NQ + qt) * NK;
  const uint64_t* bits_q = bits + ((size_t)b * S + (qvalid ? tq : 0)) * W;

  for (int kt = 0; kt <= kt_last; ++kt) {
    const int c = cls_row[kt];
    if (c == 0) continue;
    __syncthreads();
    for (int ci = tid; ci < TK * 24; ci += 256) {
      const int row = ci / 24, cc = ci % 24;
      const int s = kt * TK + row;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (s < S) z = *(const u32x4*)(k + ((size_t)b * S + s) * rs_qk + (size_t)h * DQK + cc * 8);
      *(u32x4*)(smK + row * KROW + cc * 16) = z;
      tstore8(smKT, KTROW, cc * 8, row, z);
    }
    for (int ci = tid; ci < TK * 16; ci += 256) {
      const int row = ci / 16, cc = ci % 16;
      const int s = kt * TK + row;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (s < S) z = *(const u32x4*)(v + ((size_t)b * S + s) * rs_v + (size_t)h * DV + cc * 8);
      *(u32x4*)(smV + row * VROW + cc * 16) = z;
    }
    __syncthreads();

    uint64_t mw = ~0ull;
    if (c == 1) {
      mw = qvalid ? bits_q[kt] : 0ull;
      if (__ballot(mw != 0ull) == 0ull) continue;
    }
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) { sacc[kb][i] = 0.f; dpacc[kb][i] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *(const u32x4*)(smK + (kb * 32 + col) * KROW + (ks * 16 + 8 * half) * 2);
        sacc[kb] = mfma32(a, qf[ks], sacc[kb]);
      }
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *(const u32x4*)(smV + (kb * 32 + col) * VROW + (ks * 16 + 8 * half) * 2);
        dpacc[kb] = mfma32(a, of[ks], dpacc[kb]);
      }
    u32x4 db[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        float dsv[8];
#pragma unroll
        for (int c8 = 0; c8 < 8; ++c8) {
          const int r = 8 * p2 + c8;
          const int key = kb * 32 + acc_row(r, half);
          const bool keep = c == 2 ? qvalid : (((mw >> key) & 1ull) != 0ull);
          const float pr = keep ? exp2f(sacc[kb][r] * scale_log2 - Lq) : 0.f;
          dsv[c8] = pr * (dpacc[kb][r] - Dq);
        }
        db[kb][p2] = u32x4{pack_bf2(dsv[0], dsv[1]), pack_bf2(dsv[2], dsv[3]), pack_bf2(dsv[4], dsv[5]),
                           pack_bf2(dsv[6], dsv[7])};
      }
    // dQ^T[d, q] += K^T[d, s] dS^T[s, q]
#pragma unroll
    for (int i = 0; i < DQK / 32; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          const unsigned char* base = smKT + (i * 32 + col) * KTROW + (kb * 32 + 16 * p2 + 4 * half) * 2;
          const u32x2 lo = *(const u32x2*)base;
          const u32x2 hi = *(const u32x2*)(base + 16);
          dqacc[i] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, db[kb][p2], dqacc[i]);
        }
  }
  if (qvalid) {
    uint16_t* dqrow = dq + ((size_t)b * S + tq) * rs_qk + (size_t)h * DQK;
#pragma unroll
    for (int i = 0; i < DQK / 32; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = i * 32 + 8 * g + 4 * half;
        *(u32x2*)(dqrow + d) = u32x2{pack_bf2(dqacc[i][4 * g] * scale, dqacc[i][4 * g + 1] * scale),
                                     pack_bf2(dqacc[i][4 * g + 2] * scale, dqacc[i][4 * g + 3] * scale)};
      }
  }
}

// ---------------------------------------------------------------------------
// Plain kernels (any dims <= 256, fp32 or bf16).
// dq: one wave per (b, t, h), lanes over the keys of one mask word.
// dk/dv: one wave per (b, s, h), lanes over 64 queries at a time (t >= s),
//        reading bit (s % 64) of each query's word s / 64.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_dq_plain_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ o,
    const T* __restrict__ dout, const float* __restrict__ lse, float* __restrict__ D,
    const uint64_t* __restrict__ bits, int B, int S, int H, int Dqk, int Dv, float scale,
    T* __restrict__ dq) {
  __shared__ float qs[4][256], os[4][256], dss[4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + wid;
  if (row >= (size_t)B * S * H) return;
  const int h = (int)(row % H);
  const int t = (int)((row / H) % S);
  const int b = (int)(row / ((size_t)H * S));
  const int W = (S + 63) / 64;
  for (int d = lane; d < Dqk; d += 64) qs[wid][d] = Elem<T>::load(q + row * Dqk + d);
  for (int d = lane; d < Dv; d += 64) os[wid][d] = Elem<T>::load(dout + row * Dv + d);
  __builtin_amdgcn_wave_barrier();
  const float L = lse[((size_t)b * H + h) * S + t];
  float Dt = 0.f;
  for (int e = lane; e < Dv; e += 64) Dt = fmaf(Elem<T>::load(o + row * Dv + e), os[wid][e], Dt);
  Dt = wave_sumf(Dt);
  if (lane == 0) D[((size_t)b * H + h) * S + t] = Dt;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const uint64_t* brow = bits + ((size_t)b * S + t) * W;
  for (int w = 0; w <= t / 64; ++w) {
    const uint64_t word = brow[w];
    if (word == 0ull) continue;
    const int s = 64 * w + lane;
    float dsv = 0.f;
    if ((word >> lane) & 1ull) {
      const T* krow = k + (((size_t)b * S + s) * H + h) * Dqk;
      const T* vrow = v + (((size_t)b * S + s) * H + h) * Dv;
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
      const T* krow = k + (((size_t)b * S + 64 * w + jj) * H + h) * Dqk;
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
    int S, int H, int Dqk, int Dv, float scale, T* __restrict__ dk, T* __restrict__ dv) {
  __shared__ float ks_[4][256], vs_[4][256], ps[4][64], dss[4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + wid;  // (b, s, h)
  if (row >= (size_t)B * S * H) return;
  const int h = (int)(row % H);
  const int s = (int)((row / H) % S);
  const int b = (int)(row / ((size_t)H * S));
  const int W = (S + 63) / 64;
  for (int d = lane; d < Dqk; d += 64) ks_[wid][d] = Elem<T>::load(k + row * Dqk + d);
  for (int d = lane; d < Dv; d += 64) vs_[wid][d] = Elem<T>::load(v + row * Dv + d);
  __builtin_amdgcn_wave_barrier();
  float ak[4] = {0.f, 0.f, 0.f, 0.f}, av[4] = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = s; t0 < S; t0 += 64) {
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

hipError_t launch_attn_bwd_dq_mfma(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, float* D, const uint64_t* bits,
                                   const uint8_t* cls, int B, int S, int H, float scale, void* dq,
                                   hipStream_t st) {
  const size_t nq = (size_t)n_qtiles(S) * B * H;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)nq), dim3(256), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o, (const uint16_t*)dout, lse,
                     D, bits, cls, B, S, H, scale, scale * 1.4426950408889634f, (uint16_t*)dq);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv_mfma(const void* q, const void* k, const void* v, const void* dout,
                                     const float* lse, const float* D, const uint64_t* bits,
                                     const uint8_t* cls, int B, int S, int H, float scale, void* dk,
                                     void* dv, hipStream_t st) {
  const size_t nkv = (size_t)((S + 127) / 128) * B * H;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)nkv), dim3(256), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse, D, bits, cls, B,
                     S, H, scale, scale * 1.4426950408889634f, (uint16_t*)dk, (uint16_t*)dv);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dq_plain(const void* q, const void* k, const void* v, const void* o,
                                    const void* dout, const float* lse, float* D, const uint64_t* bits,
                                    int B, int S, int H, int Dqk, int Dv, float scale, bool bf16,
                                    void* dq, hipStream_t st) {
  const size_t nblk = ((size_t)B * S * H + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL(attn_bwd_dq_plain_kernel<uint16_t>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o,
                       (const uint16_t*)dout, lse, D, bits, B, S, H, Dqk, Dv, scale, (uint16_t*)dq);
  else
    hipLaunchKernelGGL(attn_bwd_dq_plain_kernel<float>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, (const float*)o,
                       (const float*)dout, lse, D, bits, B, S, H, Dqk, Dv, scale, (float*)dq);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv_plain(const void* q, const void* k, const void* v, const void* dout,
                                      const float* lse, const float* D, const uint64_t* bits, int B,
                                      int S, int H, int Dqk, int Dv, float scale, bool bf16, void* dk,
                                      void* dv, hipStream_t st) {
  const size_t nblk = ((size_t)B * S * H + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL(attn_bwd_dkdv_plain_kernel<uint16_t>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                       lse, D, bits, B, S, H, Dqk, Dv, scale, (uint16_t*)dk, (uint16_t*)dv);
  else
    hipLaunchKernelGGL(attn_bwd_dkdv_plain_kernel<float>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, (const float*)dout, lse, D,
                       bits, B, S, H, Dqk, Dv, scale, (float*)dk, (float*)dv);
  return hipGetLastError();
}

}  // namespace dsa
