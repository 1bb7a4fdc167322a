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
// needed. Operands that the MFMAs need transposed (Q^T and dO^T for dK/dV, K^T
// for dQ) come from the natural LDS tiles through ds_read_b64_tr_b16. Tiles
// are double buffered, and the next tile's global loads are issued before the
// current tile is computed.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

namespace bwd {
constexpr int DQK = 192, DV = 128;
constexpr int QC = 32;              // queries per chunk (key-major kernel)
constexpr int TK = 64;              // keys per tile (query-major kernel)
constexpr int QP = DQK + 8;         // LDS pitch (elements) of q / k rows
constexpr int OP = DV + 8;          // LDS pitch of dO / v rows
constexpr int QCH = QC * DQK / 8 / 256;  // 16-byte chunks per thread: Q chunk (3)
constexpr int OCH = QC * DV / 8 / 256;   // dO chunk (2)
constexpr int KCH = TK * DQK / 8 / 256;  // K tile (6)
constexpr int VCH = TK * DV / 8 / 256;   // V tile (4)
}  // namespace bwd

__device__ __forceinline__ u32x4 pack8(const float* x) {
  return u32x4{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])};
}

// ---------------------------------------------------------------------------
// dK / dV, key-major. Workgroup = (b, h, 128 keys), wave = 32 keys held in
// registers (K, V fragments and the dK, dV accumulators). Walks the 32-query
// chunks from the first key to the end, skipping chunks whose tiles are EMPTY.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ D,
    const uint64_t* __restrict__ bits, const uint8_t* __restrict__ cls, int B, int S, int H,
    float scale, float scale_log2, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  using namespace bwd;
  __shared__ __attribute__((aligned(16))) uint16_t smQ[2][QC * QP];
  __shared__ __attribute__((aligned(16))) uint16_t smO[2][QC * OP];
  __shared__ float smL[2][QC], smD[2][QC];
  __shared__ uint64_t smW[2][2][QC];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int W = (S + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int nkb = (S + 127) / 128;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);  // a (b, h)'s key blocks share an XCD
  const int kblk = L % nkb;
  const int bh = L / nkb;
  const int b = bh / H, h = bh % H;
  const int kb0 = kblk * 128;
  const int s0 = kb0 + wid * 32;  // this wave's first key
  const int sk = s0 + col;        // this lane's key
  const bool kvalid = sk < S;
  const int kt_w = s0 / 64;       // this wave's 64-key tile
  const int kt_lo = kb0 / 64;     // workgroup's first key tile
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;
  const uint16_t* qbase = q + (size_t)b * S * rs_qk + (size_t)h * DQK;
  const uint16_t* obase = dout + (size_t)b * S * rs_v + (size_t)h * DV;
  const float* lrow = lse + ((size_t)b * H + h) * S;
  const float* drow = D + ((size_t)b * H + h) * S;

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
  auto chunk_cls = [&](int qc, int which) -> int {
    const int kt = kt_lo + which;
    return kt < NK ? cls[((size_t)b * NQ + (qc * QC) / 128) * NK + kt] : 0;
  };
  auto next_chunk = [&](int qc) {
    int n = qc + 1;
    while (n < nchunks && chunk_cls(n, 0) == 0 && chunk_cls(n, 1) == 0) ++n;
    return n;
  };

  u32x4 pq[QCH], po[OCH];
  float pl = 0.f, pd = 0.f;
  uint64_t pw = 0ull;
  auto gload = [&](int qc) {
    const int q0 = qc * QC;
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int ci = tid + i * 256, row = ci / 24, cc = ci % 24, t = q0 + row;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (t < S) z = *(const u32x4*)(qbase + (size_t)t * rs_qk + cc * 8);
      pq[i] = z;
    }
#pragma unroll
    for (int i = 0; i < OCH; ++i) {
      const int ci = tid + i * 256, row = ci / 16, cc = ci % 16, t = q0 + row;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (t < S) z = *(const u32x4*)(obase + (size_t)t * rs_v + cc * 8);
      po[i] = z;
    }
    if (tid < QC) {
      const int t = q0 + tid;
      pl = t < S ? lrow[t] * 1.4426950408889634f : INFINITY;
      pd = t < S ? drow[t] : 0.f;
    } else if (tid < 3 * QC) {
      const int qi = (tid - QC) % QC, which = (tid - QC) / QC;
      const int t = q0 + qi, kt = kt_lo + which;
      pw = (t < S && kt < NK) ? bits[((size_t)b * S + t) * W + kt] : 0ull;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int ci = tid + i * 256, row = ci / 24, cc = ci % 24;
      *(u32x4*)(&smQ[buf][row * QP + cc * 8]) = pq[i];
    }
#pragma unroll
    for (int i = 0; i < OCH; ++i) {
      const int ci = tid + i * 256, row = ci / 16, cc = ci % 16;
      *(u32x4*)(&smO[buf][row * OP + cc * 8]) = po[i];
    }
    if (tid < QC) {
      smL[buf][tid] = pl;
      smD[buf][tid] = pd;
    } else if (tid < 3 * QC) {
      smW[buf][(tid - QC) / QC][(tid - QC) % QC] = pw;
    }
  };

  int qc = kb0 / QC;
  if (chunk_cls(qc, 0) == 0 && chunk_cls(qc, 1) == 0) qc = next_chunk(qc);
  if (qc < nchunks) gload(qc);
  int buf = 0;
  while (qc < nchunks) {
    const int q0 = qc * QC;
    const int cw = chunk_cls(qc, kt_w - kt_lo);
    lstore(buf);
    __syncthreads();  // chunk qc visible; the other buffer is free
    const int qn = next_chunk(qc);
    if (qn < nchunks) gload(qn);  // in flight while this chunk is computed

    if (cw != 0 && s0 <= q0 + QC - 1) {
      const uint16_t* sQ = smQ[buf];
      const uint16_t* sO = smO[buf];
      // S = Q K^T and dP = dO V^T: rows = queries, columns = keys (lane's key)
      f32x16 sacc, dpacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < DQK / 16; ++ks)
        sacc = mfma32(*(const u32x4*)(sQ + col * QP + ks * 16 + 8 * half), kf[ks], sacc);
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks)
        dpacc = mfma32(*(const u32x4*)(sO + col * OP + ks * 16 + 8 * half), vf[ks], dpacc);
      // this lane's bit of query qi's word: one 32-bit half, constant bit offset
      const uint32_t* mw32 = (const uint32_t*)smW[buf][kt_w - kt_lo] + (bitpos >> 5);
      const int bsh = bitpos & 31;
      // dV^T[e, s] += dO^T[e, q] P[q, s];  dK^T[d, s] += Q^T[d, q] dS[q, s]
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        float p[8], ds[8];
#pragma unroll
        for (int c8 = 0; c8 < 8; ++c8) {
          const int r = 8 * p2 + c8;
          const int qi = acc_row(r, half);
          const bool keep = (mw32[2 * qi] >> bsh) & 1u;  // FULL tiles have every in-range bit set
          const float pr = keep ? fast_exp2(sacc[r] * scale_log2 - smL[buf][qi]) : 0.f;
          p[c8] = pr;
          ds[c8] = pr * (dpacc[r] - smD[buf][qi]);
        }
        const u32x4 pb = pack8(p), db = pack8(ds);
        const int r0 = 16 * p2 + 4 * half;
#pragma unroll
        for (int eb = 0; eb < DV / 32; ++eb)
          dvacc[eb] = mfma32(lds_tr_frag(sO, OP, r0, r0 + 8, eb * 32), pb, dvacc[eb]);
#pragma unroll
        for (int d2 = 0; d2 < DQK / 32; ++d2)
          dkacc[d2] = mfma32(lds_tr_frag(sQ, QP, r0, r0 + 8, d2 * 32), db, dkacc[d2]);
      }
    }
    buf ^= 1;
    qc = qn;
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
// dQ, query-major; also computes D. Workgroup = (b, h, 256 queries) with 8
// waves (two per SIMD) of 32 queries. Walks the non-empty 64-key tiles up to
// the diagonal; K and V tiles are double buffered in natural layout and filled
// by direct global->LDS copies. Each tile is processed as two 32-key halves to
// bound the live accumulators.
// ---------------------------------------------------------------------------
namespace dqk {
constexpr int NW = 8, QW = 32 * NW;
constexpr int KSL = bwd::DQK / 8 + 1, VSL = bwd::DV / 8 + 1;  // 16-byte slots per padded row
constexpr int KBLK = bwd::TK * KSL / 64, VBLK = bwd::TK * VSL / 64;
constexpr int KI = (KBLK + NW - 1) / NW, VI = (VBLK + NW - 1) / NW;
static_assert(KSL * 8 == bwd::QP && VSL * 8 == bwd::OP, "pitches");
}  // namespace dqk

__global__ __launch_bounds__(dqk::NW * 64) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ D, const uint64_t* __restrict__ bits, const uint8_t* __restrict__ cls, int B,
    int S, int H, float scale, float scale_log2, uint16_t* __restrict__ dq) {
  using namespace bwd;
  using dqk::NW;
  using dqk::QW;
  __shared__ __attribute__((aligned(1024))) uint16_t smK[2][TK * QP];
  __shared__ __attribute__((aligned(1024))) uint16_t smV[2][TK * OP];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int W = (S + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int NQW = (S + QW - 1) / QW;
  const int Lb = xcd_remap((int)blockIdx.x, (int)gridDim.x);  // a (b, h)'s query blocks share an XCD
  const int bh = Lb / NQW;
  const int qw = NQW - 1 - Lb % NQW;
  const int b = bh / H, h = bh % H;
  const int tq = qw * QW + wid * 32 + col;
  const bool qvalid = tq < S;
  const int qt_w = min(NQ - 1, (qw * QW + wid * 32) / 128);
  const int qt0 = qw * QW / 128, qt1 = min(NQ - 1, qt0 + 1);
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;
  const uint16_t* kbase = k + (size_t)b * S * rs_qk + (size_t)h * DQK;
  const uint16_t* vbase = v + (size_t)b * S * rs_v + (size_t)h * DV;

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
  auto issue = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < dqk::KI; ++i) {
      const int j = wid + i * NW;
      if (j < dqk::KBLK) {
        const int slot = j * 64 + lane, row = slot / dqk::KSL, c = min(slot % dqk::KSL, dqk::KSL - 2);
        const int s = min(kt * TK + row, S - 1);
        g2lds16(kbase + (size_t)s * rs_qk + c * 8, (char*)smK[buf] + j * 1024);
      }
    }
#pragma unroll
    for (int i = 0; i < dqk::VI; ++i) {
      const int j = wid + i * NW;
      if (j < dqk::VBLK) {
        const int slot = j * 64 + lane, row = slot / dqk::VSL, c = min(slot % dqk::VSL, dqk::VSL - 2);
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
    __syncthreads();
    const int kn = next_tile(kt);
    if (kn <= kt_last) issue(kn, buf ^ 1);

    if (c != 0 && __ballot(mw != 0ull)) {
      const uint16_t* sK = smK[buf];
      const uint16_t* sV = smV[buf];
      // this lane's keys are kb*32 + 8i + 4*half + r: pre-shift the word by 4*half
      const uint64_t mwh = mw >> (4 * half);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t w = (uint32_t)(mwh >> (32 * kb));
        f32x16 sacc, dpacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks)
          sacc = mfma32(*(const u32x4*)(sK + (kb * 32 + col) * QP + ks * 16 + 8 * half), qf[ks], sacc);
#pragma unroll
        for (int ks = 0; ks < DV / 16; ++ks)
          dpacc = mfma32(*(const u32x4*)(sV + (kb * 32 + col) * OP + ks * 16 + 8 * half), of[ks], dpacc);
        // dQ^T[d, q] += K^T[d, s] dS^T[s, q], keys permuted inside each 16-key step
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          float dsv[8];
#pragma unroll
          for (int c8 = 0; c8 < 8; ++c8) {
            const int r = 8 * p2 + c8;
            const bool keep = (w >> (8 * (r >> 2) + (r & 3))) & 1u;
            const float pr = keep ? fast_exp2(fmaf(sacc[r], scale_log2, -Lq)) : 0.f;
            dsv[c8] = pr * (dpacc[r] - Dq);
          }
          const u32x4 db = pack8(dsv);
          const int r0 = kb * 32 + 16 * p2 + 4 * half;
#pragma unroll
          for (int i = 0; i < DQK / 32; ++i)
            dqacc[i] = mfma32(lds_tr_frag(sK, QP, r0, r0 + 8, i * 32), db, dqacc[i]);
        }
      }
    }
    buf ^= 1;
    kt = kn;
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

hipError_t launch_attn_bwd_dq_mfma(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, float* D, const uint64_t* bits,
                                   const uint8_t* cls, int B, int S, int H, float scale, void* dq,
                                   hipStream_t st) {
  const size_t nq = (size_t)((S + dqk::QW - 1) / dqk::QW) * B * H;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)nq), dim3(dqk::NW * 64), 0, st, (const uint16_t*)q,
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

}  // namespace dsa
