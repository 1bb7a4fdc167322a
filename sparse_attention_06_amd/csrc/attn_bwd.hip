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
constexpr int KCH = TK * DQK / 8 / 256;  // K tile (6)
constexpr int VCH = TK * DV / 8 / 256;   // V tile (4)
}  // namespace bwd

__device__ __forceinline__ u32x4 pack8(const float* x) {
  return u32x4{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])};
}

// ---------------------------------------------------------------------------
// dK / dV, key-major. Workgroup = (b, h, 128 keys) with 8 waves in two roles,
// two waves per SIMD:
//   waves 0-3 ("A", 32 keys each, K/V fragments in VGPRs): S = Q K^T,
//     dP = dO V^T, P, dS, and dV^T += dO^T P. A hands dS to its partner
//     through LDS.
//   waves 4-7 ("B", the same 32 keys as wave w-4): dK^T += Q^T dS, one
//     32-query chunk behind A.
// So B's MFMAs run while A does its softmax-gradient VALU work, and no MFMA is
// done twice. Chunks with EMPTY tiles for the workgroup's keys are skipped.
// Q chunks are triple buffered (B reads the previous one); dO and dS are
// double buffered. All are filled by direct global->LDS copies.
// ---------------------------------------------------------------------------
namespace dkv {
constexpr int NW = 8;
constexpr int QSL = bwd::DQK / 8 + 1, OSL = bwd::DV / 8 + 1;    // 16-byte slots per padded row
constexpr int QBLK = (bwd::QC * QSL + 63) / 64;                 // 1 KB blocks per Q chunk (13)
constexpr int OBLK = (bwd::QC * OSL + 63) / 64;                 // ... per dO chunk (9)
constexpr int QI = (QBLK + NW - 1) / NW, OI = (OBLK + NW - 1) / NW;
static_assert(QSL * 8 == bwd::QP && OSL * 8 == bwd::OP, "pitches");
}  // namespace dkv

__global__ __launch_bounds__(dkv::NW * 64) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ D,
    const uint64_t* __restrict__ bits, const uint8_t* __restrict__ cls, int B, int S, int H,
    float scale, float scale_log2, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  using namespace bwd;
  using dkv::NW;
  __shared__ __attribute__((aligned(1024))) unsigned char smQ[3][dkv::QBLK * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char smO[2][dkv::OBLK * 1024];
  __shared__ __attribute__((aligned(16))) u32x4 smS[2][4][2][64];  // dS, B-operand layout, per A wave
  __shared__ __attribute__((aligned(16))) float smL[2][QC];
  __shared__ __attribute__((aligned(16))) float smD[2][QC];
  // mask words of the chunk's queries for the workgroup's two key tiles, split
  // into 32-bit halves: [buf][tile][half][query]
  __shared__ __attribute__((aligned(16))) uint32_t smW[2][2][2][QC];
  // tile classes of the workgroup's two key tiles for every 128-query tile
  __shared__ uint8_t scls[2][kMaxS / 128];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so per-wave data is scalar
  const int half = lane >> 5, col = lane & 31;
  const bool roleA = wid < 4;
  const int kw = wid & 3;
  const int W = (S + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int nkb = (S + 127) / 128;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);  // a (b, h)'s key blocks share an XCD
  const int kblk = L % nkb;
  const int bh = L / nkb;
  const int b = bh / H, h = bh % H;
  const int kb0 = kblk * 128;
  const int s0 = kb0 + kw * 32;   // this wave pair's first key
  const int sk = s0 + col;        // this lane's key
  const bool kvalid = sk < S;
  const int kt_w = s0 / 64;       // the pair's 64-key tile
  const int kt_lo = kb0 / 64;     // workgroup's first key tile
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;
  const uint16_t* qbase = q + (size_t)b * S * rs_qk + (size_t)h * DQK;
  const uint16_t* obase = dout + (size_t)b * S * rs_v + (size_t)h * DV;
  const float* lrow = lse + ((size_t)b * H + h) * S;
  const float* drow = D + ((size_t)b * H + h) * S;

  const int nchunks = (S + QC - 1) / QC;
  for (int i = tid; i < 2 * NQ; i += blockDim.x) {
    const int which = i / NQ, qt = i % NQ, kt = kt_lo + which;
    scls[which][qt] = kt < NK ? cls[((size_t)b * NQ + qt) * NK + kt] : 0;
  }
  __syncthreads();  // class column staged
  auto chunk_cls = [&](int qc, int which) -> int { return scls[which][(qc * QC) / 128]; };
  auto next_chunk = [&](int qc) {
    int n = qc + 1;
    while (n < nchunks && chunk_cls(n, 0) == 0 && chunk_cls(n, 1) == 0) ++n;
    return n;
  };
  // chunk qc's Q / dO rows into buffers (qb, ob); slots past the chunk copy a harmless chunk
  auto issue = [&](int qc, int qb, int ob) {
    const int q0 = qc * QC;
#pragma unroll
    for (int i = 0; i < dkv::QI; ++i) {
      const int j = wid + i * NW;
      if (j < dkv::QBLK) {
        const int slot = j * 64 + lane;
        const bool in = slot < QC * dkv::QSL;
        const int row = in ? slot / dkv::QSL : 0, c = in ? min(slot % dkv::QSL, dkv::QSL - 2) : 0;
        const int t = min(q0 + row, S - 1);
        g2lds16(qbase + (size_t)t * rs_qk + c * 8, smQ[qb] + j * 1024);
      }
    }
#pragma unroll
    for (int i = 0; i < dkv::OI; ++i) {
      const int j = wid + i * NW;
      if (j < dkv::OBLK) {
        const int slot = j * 64 + lane;
        const bool in = slot < QC * dkv::OSL;
        const int row = in ? slot / dkv::OSL : 0, c = in ? min(slot % dkv::OSL, dkv::OSL - 2) : 0;
        const int t = min(q0 + row, S - 1);
        g2lds16(obase + (size_t)t * rs_v + c * 8, smO[ob] + j * 1024);
      }
    }
  };
  // per-query scalars of chunk qc: LSE (log2 units), D, and the two mask words
  float pl = 0.f, pd = 0.f;
  uint64_t pw = 0ull;
  auto load_small = [&](int qc) {
    const int q0 = qc * QC;
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
  auto store_small = [&](int sb) {
    if (tid < QC) {
      smL[sb][tid] = pl;
      smD[sb][tid] = pd;
    } else if (tid < 3 * QC) {
      const int which = (tid - QC) / QC, qi = (tid - QC) % QC;
      smW[sb][which][0][qi] = (uint32_t)pw;
      smW[sb][which][1][qi] = (uint32_t)(pw >> 32);
    }
  };
  auto active = [&](int qc) { return chunk_cls(qc, kt_w - kt_lo) != 0 && s0 <= qc * QC + QC - 1; };

  int qc = kb0 / QC;
  if (chunk_cls(qc, 0) == 0 && chunk_cls(qc, 1) == 0) qc = next_chunk(qc);
  if (qc < nchunks) {
    issue(qc, 0, 0);
    load_small(qc);
  }

  if (roleA) {
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
    f32x16 dvacc[DV / 32];
#pragma unroll
    for (int i = 0; i < DV / 32; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) dvacc[i][j] = 0.f;
    for (int it = 0; qc < nchunks; ++it) {
      store_small(it & 1);
      wait_vmem();
      __syncthreads();  // chunk qc visible in buffers (it%3, it%2)
      const int qn = next_chunk(qc);
      if (qn < nchunks) {
        issue(qn, (it + 1) % 3, (it + 1) & 1);
        load_small(qn);
      }
      if (active(qc)) {
        const int q0 = qc * QC;
        const uint16_t* sQ = (const uint16_t*)smQ[it % 3];
        const uint16_t* sO = (const uint16_t*)smO[it & 1];
        f32x16 sacc, dpacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks)
          sacc = mfma32(*(const u32x4*)(sQ + col * QP + ks * 16 + 8 * half), kf[ks], sacc);
#pragma unroll
        for (int ks = 0; ks < DV / 16; ++ks)
          dpacc = mfma32(*(const u32x4*)(sO + col * OP + ks * 16 + 8 * half), vf[ks], dpacc);
        // per-row scalars of this lane's 16 query rows (rows 8i + 4*half + r are
        // 4-aligned runs): LSE, D and this wave's 32-bit half of each mask word
        // (the half is fixed per wave: keys s0..s0+31 sit in one half).
        // FULL tiles have every in-range bit set.
        const int bsh = sk & 31;
        const uint32_t* wrow = smW[it & 1][kt_w - kt_lo][(s0 >> 5) & 1];
        (void)q0;
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          float Lr[8], Dr[8];
          uint32_t Wr[8];
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2) {
            const int r0 = 8 * (2 * p2 + i2) + 4 * half;
            const f32x4 l4 = *(const f32x4*)&smL[it & 1][r0];
            const f32x4 d4 = *(const f32x4*)&smD[it & 1][r0];
            const u32x4 w4 = *(const u32x4*)&wrow[r0];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              Lr[4 * i2 + j] = l4[j];
              Dr[4 * i2 + j] = d4[j];
              Wr[4 * i2 + j] = w4[j];
            }
          }
          float p[8], ds[8];
#pragma unroll
          for (int c8 = 0; c8 < 8; ++c8) {
            const int r = 8 * p2 + c8;
            const bool keep = (Wr[c8] >> bsh) & 1u;
            const float pr = keep ? fast_exp2(fmaf(sacc[r], scale_log2, -Lr[c8])) : 0.f;
            p[c8] = pr;
            ds[c8] = pr * (dpacc[r] - Dr[c8]);
          }
          smS[it & 1][kw][p2][lane] = pack8(ds);  // to the partner wave, in B-operand layout
          const u32x4 pb = pack8(p);
          const int r0 = 16 * p2 + 4 * half;
#pragma unroll
          for (int eb = 0; eb < DV / 32; ++eb)
            dvacc[eb] = mfma32(lds_tr_frag(sO, OP, r0, r0 + 8, eb * 32), pb, dvacc[eb]);
        }
      }
      qc = qn;
    }
    __syncthreads();  // matches the partner's final barrier
    if (kvalid) {
      uint16_t* dvrow = dv + ((size_t)b * S + sk) * rs_v + (size_t)h * DV;
#pragma unroll
      for (int i = 0; i < DV / 32; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int e = i * 32 + 8 * g + 4 * half;
          *(u32x2*)(dvrow + e) = u32x2{pack_bf2(dvacc[i][4 * g], dvacc[i][4 * g + 1]),
                                       pack_bf2(dvacc[i][4 * g + 2], dvacc[i][4 * g + 3])};
        }
    }
  } else {
    f32x16 dkacc[DQK / 32];
#pragma unroll
    for (int i = 0; i < DQK / 32; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) dkacc[i][j] = 0.f;
    // dK^T[d, s] += Q^T[d, q] dS[q, s] for the chunk of iteration `it`
    auto dk_update = [&](int it) {
      const uint16_t* sQ = (const uint16_t*)smQ[it % 3];
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        const u32x4 db = smS[it & 1][kw][p2][lane];
        const int r0 = 16 * p2 + 4 * half;
#pragma unroll
        for (int d2 = 0; d2 < DQK / 32; ++d2)
          dkacc[d2] = mfma32(lds_tr_frag(sQ, QP, r0, r0 + 8, d2 * 32), db, dkacc[d2]);
      }
    };
    bool prev = false;
    int it = 0;
    for (; qc < nchunks; ++it) {
      store_small(it & 1);
      wait_vmem();
      __syncthreads();
      const int qn = next_chunk(qc);
      if (qn < nchunks) {
        issue(qn, (it + 1) % 3, (it + 1) & 1);
        load_small(qn);
      }
      if (prev) dk_update(it - 1);  // the chunk A finished before this barrier
      prev = active(qc);
      qc = qn;
    }
    __syncthreads();  // A's dS of the last chunk is visible
    if (prev) dk_update(it - 1);
    if (kvalid) {
      uint16_t* dkrow = dk + ((size_t)b * S + sk) * rs_qk + (size_t)h * DQK;
#pragma unroll
      for (int i = 0; i < DQK / 32; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = i * 32 + 8 * g + 4 * half;
          *(u32x2*)(dkrow + d) = u32x2{pack_bf2(dkacc[i][4 * g] * scale, dkacc[i][4 * g + 1] * scale),
                                       pack_bf2(dkacc[i][4 * g + 2] * scale, dkacc[i][4 * g + 3] * scale)};
        }
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

  // this lane's selection word of tile kt (FULL: all ones; EMPTY: none)
  auto word = [&](int kt) -> uint64_t {
    const int c = clsw[kt];
    if (!qvalid || c == 0) return 0ull;
    return c == 2 ? ~0ull : bits_q[kt];
  };
  __syncthreads();  // class rows staged
  int kt = next_tile(-1);
  if (kt <= kt_last) issue(kt, 0);
  uint64_t mw = kt <= kt_last ? word(kt) : 0ull;
  int buf = 0;
  while (kt <= kt_last) {
    const int c = clsw[kt];
    const int kn = next_tile(kt);
    wait_vmem();
    __syncthreads();  // tile kt visible in `buf`; every wave is done with the other buffer
    // the next selection word is loaded before the tile copies are issued, so
    // that waiting for it does not wait for them
    const uint64_t mw_n = kn <= kt_last ? word(kn) : 0ull;
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
    mw = mw_n;
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
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)nkv), dim3(dkv::NW * 64), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse, D, bits, cls, B,
                     S, H, scale, scale * 1.4426950408889634f, (uint16_t*)dk, (uint16_t*)dv);
  return hipGetLastError();
}

}  // namespace dsa
