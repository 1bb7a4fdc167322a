// Block-sparse flash-attention backward over the DSA selection mask (gfx950).
//
// Source: "Support Ring Attention with DeepSeek DSA Sparse Indexer", Backward
// Flow: the forward runs query-major while dK/dV run key-major. Each uses the
// same index mask, dQ = dP K, dK = dP^T Q and dV = P^T dO.
//
//   D(t)   = sum_e dO(t,e) O(t,e)       (a prologue kernel stores it, with the
//                                         base-2 LSE, in the workspace)
//   P      = exp(scale q.k - LSE(t)) on kept (t, s)
//   dP     = dO(t) . v(s),   dS = P (dP - D(t))
//   dV(s) += P dO(t),        dK(s) += scale dS q(t)      (key-major kernel)
//   dQ(t)  = scale sum_s dS k(s)                         (query-major kernel)
// The key-major kernel runs first: it recomputes P from LSE, forms dS, and
// (when the workspace has room for them) also stores dS^T as MFMA B-operand
// fragments, which the query-major kernel then contracts with K; nothing is
// recomputed there. Without that room the query-major kernel recomputes P and
// dS itself, in the same operations, so both routes give the same dQ.
// Neither uses atomics, so the result is deterministic. The key-major kernel
// reads the same row-major selection words as the forward: a lane owns one
// query and 16 keys of its word, so no transposed copy of the mask is needed.
// Operands that the MFMAs need transposed (Q^T, dO^T, P and dS for dK/dV, K^T
// for dQ) come from natural row-major LDS tiles through ds_read_b64_tr_b16. Tiles are double (or more)
// buffered, and later tiles' copies are issued before the current tile is
// computed.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

namespace bwd {
constexpr int DQK = 192, DV = 128;
constexpr int QC = 32;              // queries per chunk (key-major kernel)
constexpr int TK = 64;              // keys per tile (query-major kernel)
constexpr int QP = DQK + 32;        // LDS pitch (elements) of K rows (query-major kernel): 448 B
}  // namespace bwd

// ---------------------------------------------------------------------------
// dK / dV, key-major. Workgroup = (b, h, 128 keys) with 8 waves in two roles;
// wave w and wave w+4 share a SIMD:
//   waves 0-3 ("A", K/V fragments of 32 keys in VGPRs, raised issue priority):
//     S^T = K Q^T and dP^T = V dO^T for a 32-query chunk, then P and
//     dS = P (dP - D). In the transposed orientation a lane holds one query
//     (so one LSE, one D and one mask word per lane) and 16 keys, which is
//     exactly the dQ kernel's B-operand fragment of dS^T: A stores it to the
//     workspace straight from registers. P and dS also go to LDS as
//     [32 queries][32 keys] tiles (4-key groups swizzled, see dkv::TP).
//   waves 4-7 ("B", dV^T and dK^T accumulators): dV^T += dO^T P and
//     dK^T += Q^T dS, one chunk behind A, with P and dS read transposed. A B
//     wave owns 64 keys (two A waves' P and dS tiles) and half of their ten
//     32-row blocks of dK^T / dV^T, so every transposed Q^T or dO^T fragment
//     it reads feeds two MFMAs.
// Each wave issues 20 MFMAs per chunk. A's softmax-gradient VALU work hides
// under B's MFMAs: A has priority, so its MFMAs issue first after a barrier
// and B's fill the matrix pipe while A works on P and dS. Chunks with EMPTY
// tiles for the workgroup's keys are skipped.
// A chunk's operands -- Q and dO rows, LSE and D, and the 32-bit halves of the
// mask words of the workgroup's two key tiles -- all reach LDS through direct
// global->LDS copies, issued by the B waves only, right after the barrier: a
// wave stalls while the copy path accepts its copies, and every other
// placement measured (on A, on both roles, later in B's update) was slower.
// A chunk is only ~1.3k
// MFMA cycles of work, less than a global load's latency, so copies run two
// chunks ahead: four chunk buffers (B reads the previous chunk, A the current
// one, one is in flight, one being issued). Each B wave issues a fixed number
// of copies per chunk, so a counted vmcnt wait finds the current chunk
// complete while the next one is still in flight. P and dS are double
// buffered. The Q and dO tiles use the swizzled padded layout that keeps both
// the row reads of A and the transposing reads of B free of bank conflicts.
// ---------------------------------------------------------------------------
namespace dkv {
constexpr int NW = 8;
constexpr int NB = 4;                                          // chunk buffers
constexpr int QSL = 28, OSL = 20;                              // 16-byte slots per swizzled row
constexpr int QPX = QSL * 8, OPX = OSL * 8;                    // pitches (elements)
constexpr int QBLK = bwd::QC * QSL / 64;                       // 1 KB blocks per Q chunk (14)
constexpr int OBLK = bwd::QC * OSL / 64;                       // ... per dO chunk (10)
// copy slots of a chunk, all issued by the four B waves (slot k by wave
// k % 4): [0, QBLK) Q blocks, [QBLK, QBLK+OBLK) dO blocks, then LSE/D, then
// the two mask-word tiles
constexpr int K_LD = QBLK + OBLK, K_W = K_LD + 1, NCOPY = K_W + 2;  // 27
constexpr int NSLOT = (NCOPY + 3) / 4;                              // per B wave, at most (7)
// P and dS tiles: [32 queries][32 keys], 64-byte rows of eight 4-key groups
// (8 bytes each); group g of query q sits at group g ^ ((q >> 2) & 7). A
// writes 8-byte groups of 32 queries at one group index, B reads them back
// transposed (4 queries x 8 groups per 32 lanes): both land on 32 distinct
// 8-byte bank pairs. (Unswizzled 80-byte rows gave two-way conflicts.)
constexpr int TP = 32;  // pitch (elements)
__device__ __forceinline__ int pds_swz(int q) { return (q >> 2) & 7; }
static_assert(bwd::QC * QSL % 64 == 0 && bwd::QC * OSL % 64 == 0, "chunks must be whole 1 KB blocks");
static_assert(NCOPY % 4 == 3, "B waves 0-2 issue NSLOT copies per chunk, wave 3 one fewer");
static_assert(bwd::QC == 32, "one copy instruction moves a chunk's LSE and D, one a mask tile");
}  // namespace dkv

// HANDOFF: also store dS^T for the fragment-reading dQ kernel (the workspace
// holds them); without it dQ is recomputed by attn_bwd_dq_recompute_kernel.
template <bool HANDOFF>
__global__ __launch_bounds__(dkv::NW * 64) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ ws, const uint64_t* __restrict__ bits,
    const uint8_t* __restrict__ cls, int B, int S, int Sk, int ratio, int H, float scale, float scale_log2,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, u32x4* __restrict__ dsf) {
  using namespace bwd;
  using dkv::NW;
  using dkv::NB;
  __shared__ __attribute__((aligned(1024))) unsigned char smQ[NB][dkv::QBLK * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char smO[NB][dkv::OBLK * 1024];
  // P and dS of each A wave as [32 queries][32 keys] tiles (64-byte rows, 4-key
  // groups swizzled), which B reads transposed as MFMA B operands
  __shared__ __attribute__((aligned(16))) uint16_t smP[2][4][32 * dkv::TP];
  __shared__ __attribute__((aligned(16))) uint16_t smT[2][4][32 * dkv::TP];
  // per chunk: LSE in base-2 units of its 32 queries, then D
  __shared__ __attribute__((aligned(16))) float smLD[NB][2 * QC];
  // per chunk: 32-bit halves of the mask words of the workgroup's two key
  // tiles: [buf][tile][half][query]
  __shared__ __attribute__((aligned(16))) uint32_t smW[NB][2][2][QC];
  // tile classes of the workgroup's two key tiles for every 128-query tile
  __shared__ uint8_t scls[2][kMaxS / 128];
  // the workgroup's non-empty chunks in order: chunk index | tile0 flag << 14 | tile1 flag << 15
  __shared__ uint16_t clist[kMaxS / QC];
  __shared__ int s_nlist;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so per-wave data is scalar
  const int half = lane >> 5, col = lane & 31;
  const bool roleA = wid < 4;
  const int kw = wid & 3;
  const int W = (Sk + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int nkb = (Sk + 127) / 128;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);  // a (b, h)'s key blocks share an XCD
  const int kblk = L % nkb;
  const int bh = L / nkb;
  const int b = bh / H, h = bh % H;
  const int kb0 = kblk * 128;
  const int s0 = kb0 + kw * 32;   // this wave pair's first key
  const int sk = s0 + col;        // this lane's key
  const bool kvalid = sk < Sk;
  const int kt_lo = kb0 / 64;     // workgroup's first key tile
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;
  const uint16_t* qbase = q + (size_t)b * S * rs_qk + (size_t)h * DQK;
  const uint16_t* obase = dout + (size_t)b * S * rs_v + (size_t)h * DV;
  const float* drow = ws + ((size_t)b * H + h) * S;                       // D
  const float* lrow = ws + (size_t)B * H * S + ((size_t)b * H + h) * S;   // LSE * log2(e)
  const uint32_t* wbase = (const uint32_t*)bits + (size_t)b * S * W * 2;

  const int nchunks = (S + QC - 1) / QC;
  for (int i = tid; i < 2 * NQ; i += blockDim.x) {
    const int which = i / NQ, qt = i % NQ, kt = kt_lo + which;
    scls[which][qt] = kt < NK ? cls[((size_t)b * NQ + qt) * NK + kt] : 0;
  }
  __syncthreads();  // class column staged
  if (wid == 0) {   // compact the non-empty chunks from the diagonal on
    int cnt = 0;
    // from the chunk of the first query that sees the workgroup's first key
    for (int base = (ratio * kb0 + ratio - 1) / QC; base < nchunks; base += 64) {
      const int qc = base + lane;
      int fl = 0;
      if (qc < nchunks) fl = (scls[0][qc * QC / 128] != 0) | ((scls[1][qc * QC / 128] != 0) << 1);
      const uint64_t m = __ballot(fl != 0);
      if (fl) clist[cnt + lanes_below(m)] = (uint16_t)(qc | (fl << 14));
      cnt += __popcll(m);
    }
    if (lane == 0) s_nlist = cnt;
  }
  __syncthreads();
  const int nlist = s_nlist;
  auto entry = [&](int j) __attribute__((always_inline)) -> int { return j < nlist ? (int)clist[j] : -1; };
  // this wave pair's keys take part in the chunk: its key tile is non-empty
  // there and the chunk reaches the pair's first key (causal)
  auto active = [&](int e) __attribute__((always_inline)) {
    return ((e >> (14 + (kw >> 1))) & 1) != 0 && ratio * s0 + ratio - 1 <= (e & 0x3FFF) * QC + QC - 1;
  };

  // source offsets (elements from the chunk's first row) of this lane's Q / dO
  // slots: swizzled padded rows, pad slots copy the row's last chunk
  auto slot_src = [&](int kslot, int& row) __attribute__((always_inline)) -> uint32_t {
    if (kslot < dkv::QBLK) {
      const int slot = kslot * 64 + lane, pc = slot % dkv::QSL;
      row = slot / dkv::QSL;
      const int c = pc < DQK / 8 ? swz_chunk(row, pc) : DQK / 8 - 1;
      return (uint32_t)(row * rs_qk + c * 8);
    }
    const int slot = (kslot - dkv::QBLK) * 64 + lane, pc = slot % dkv::OSL;
    row = slot / dkv::OSL;
    const int c = pc < DV / 8 ? swz_chunk(row, pc) : DV / 8 - 1;
    return (uint32_t)(row * rs_v + c * 8);
  };
  // B wave kw issues copy slots kw, kw+4, ...: NSLOT, or NSLOT-1 for kw == 3
  uint32_t soff[dkv::NSLOT];
#pragma unroll
  for (int i = 0; i < dkv::NSLOT; ++i) {
    int row;
    const int kslot = kw + 4 * i;
    soff[i] = kslot < dkv::K_LD ? slot_src(kslot, row) : 0u;
  }
  // chunk qc's copies into buffer bi (B waves)
  auto issue = [&](int qc, int bi) __attribute__((always_inline)) {
    const int q0 = qc * QC;
    const bool ragged = q0 + QC > S;  // rows past S copy row S-1
    const uint16_t* qsrc = uniform_ptr(qbase + (size_t)q0 * rs_qk);
    const uint16_t* osrc = uniform_ptr(obase + (size_t)q0 * rs_v);
#pragma unroll
    for (int i = 0; i < dkv::NSLOT; ++i) {
      const int kslot = kw + 4 * i;
      if (kslot < dkv::QBLK) {
        uint32_t off = soff[i];
        if (ragged) {
          int row;
          off = slot_src(kslot, row);
          off -= (uint32_t)((row - min(row, S - 1 - q0)) * rs_qk);
        }
        g2lds16_async_off(qsrc, 2 * off, smQ[bi] + kslot * 1024);
      } else if (kslot < dkv::K_LD) {
        uint32_t off = soff[i];
        if (ragged) {
          int row;
          off = slot_src(kslot, row);
          off -= (uint32_t)((row - min(row, S - 1 - q0)) * rs_v);
        }
        g2lds16_async_off(osrc, 2 * off, smO[bi] + (kslot - dkv::QBLK) * 1024);
      } else if (kslot == dkv::K_LD) {
        const int t = min(q0 + col, S - 1);
        g2lds4_async(half ? drow + t : lrow + t, smLD[bi]);
      } else if (kslot < dkv::NCOPY) {
        const int which = kslot - dkv::K_W;
        const int t = min(q0 + col, S - 1), kt = min(kt_lo + which, NK - 1);
        g2lds4_async(wbase + ((size_t)t * W + kt) * 2 + half, smW[bi][which]);
      }
    }
  };
  // The wave that copies a mask tile clears, once the copy has landed, the
  // rows of a ragged last chunk that lie past S (they hold row S-1's words).
  auto fix_ragged = [&](int qc, int bi) __attribute__((always_inline)) {
    const int q0 = qc * QC;
    if (q0 + QC <= S) return;
#pragma unroll
    for (int i = 0; i < dkv::NSLOT; ++i) {
      const int kslot = kw + 4 * i;
      if (kslot >= dkv::K_W && kslot < dkv::NCOPY && q0 + col >= S) smW[bi][kslot - dkv::K_W][half][col] = 0u;
    }
  };

  int e0 = entry(0), e1 = entry(1), e2 = entry(2);  // current, next, and the one after
  if (!roleA) {
    if (e0 >= 0) issue(e0 & 0x3FFF, 0);
    if (e1 >= 0) issue(e1 & 0x3FFF, 1);
  }
  // B: chunk e0 (issued two chunks back) complete, then published; e1's copies
  // may still be in flight
  auto publish_b = [&](int it) __attribute__((always_inline)) {
    if (e1 >= 0) {
      if (kw == 3)
        wait_vmem_n<dkv::NSLOT - 1>();
      else
        wait_vmem_n<dkv::NSLOT>();
    } else {
      wait_vmem();
    }
    fix_ragged(e0 & 0x3FFF, it % NB);
    lds_barrier();
  };

  if (roleA) {
    __builtin_amdgcn_s_setprio(1);
    // K/V fragments of this lane's key
    u32x4 kf[DQK / 16], vf[DV / 16];
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (kvalid) z = *(const u32x4*)(k + ((size_t)b * Sk + sk) * rs_qk + (size_t)h * DQK + ks * 16 + 8 * half);
      kf[ks] = z;
    }
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (kvalid) z = *(const u32x4*)(v + ((size_t)b * Sk + sk) * rs_v + (size_t)h * DV + ks * 16 + 8 * half);
      vf[ks] = z;
    }
    wait_vmem();  // once: the loop's waits then only concern chunk copies
    // byte offsets of this lane's b128 fragment rows in the swizzled Q / dO
    // chunks, for even and odd k steps (k step ks adds 64 * (ks / 2) bytes)
    const int u = (col >> 2) & 3;
    uint32_t qa[2], oa[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      qa[par] = (uint32_t)(col * dkv::QPX * 2 + 16 * ((2 * par + half) ^ u));
      oa[par] = (uint32_t)(col * dkv::OPX * 2 + 16 * ((2 * par + half) ^ u));
    }
    const int wsel = (kw >> 1), hsel = (s0 >> 5) & 1;  // the pair's key tile and word half
    // element offset of this lane's 4-key group 4*p2 + half (+ 2: ^ 8) of row
    // col in the P / dS tiles: p2 adds ^ 16
    const int pds_base = col * dkv::TP + 4 * (half ^ dkv::pds_swz(col));
    // a chunk's dS^T fragments are stored right after the next barrier, while
    // the wave waits for its first LDS reads, not at the end of the chunk,
    // where the wave is on the way to the barrier
    u32x4 pend[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    u32x4* pfr = dsf;
    bool have = false;
    for (int it = 0; e0 >= 0; ++it) {
      lds_barrier();  // chunk e0 visible (B waited for its copies); B is done with P/dS buffer it&1
      if (HANDOFF && have) {  // streamed: read once, by the dQ kernel
        __builtin_nontemporal_store(pend[0], pfr);
        __builtin_nontemporal_store(pend[1], pfr + 64);
        have = false;
      }
      const int e3 = entry(it + 3);
      if (active(e0)) {
        const int bi = it % NB, qc = e0 & 0x3FFF;
        const char* sQ = (const char*)smQ[bi];
        const char* sO = (const char*)smO[bi];
        f32x16 sacc, dpacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
        // transposed scores: S^T = K Q^T and dP^T = V dO^T, so lane (half, col)
        // holds query col and keys 8i + 4*half + r (i, r = 0..3) of the pair
        // the two accumulator chains alternate, and each operand read is issued
        // four MFMAs ahead of its use (a read one MFMA ahead waits on the LDS)
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks) {
          sacc = mfma32(kf[ks], *(const u32x4*)(sQ + qa[ks & 1] + 64 * (ks >> 1)), sacc);
          if (ks < DV / 16) dpacc = mfma32(vf[ks], *(const u32x4*)(sO + oa[ks & 1] + 64 * (ks >> 1)), dpacc);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // the last 4 MFMAs
        // the lane's query: base-2 LSE, D and the pair's 32-bit half of its mask
        // word, shifted so that key 8i + 4*half + r sits at bit 8i + r. FULL
        // tiles have every in-range bit set.
        const float Lq = smLD[bi][col], Dq = smLD[bi][QC + col];
        const uint32_t Wq = smW[bi][wsel][hsel][col] >> (4 * half);
        u32x4* fr = dsf + (((size_t)bh * dsf_base(nchunks, ratio, NK) + dsf_base(qc, ratio, NK) + kt_lo + (kw >> 1)) * 4 +
                           2 * (kw & 1)) * 64 + lane;
        // P and dS. On a chunk of a FULL tile every pair is kept and the mask
        // select is skipped; not on a ragged last chunk, whose rows past S (kept
        // out of the tile class) rely on their cleared mask words.
        auto softmax = [&](auto FULLC) __attribute__((always_inline)) {
          constexpr bool FULL = decltype(FULLC)::value;
#pragma unroll
          for (int p2 = 0; p2 < 2; ++p2) {
            float p[8], ds[8];
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) {
              const int r = 8 * p2 + c8;
              const float e = fast_exp2(fmaf(sacc[r], scale_log2, -Lq));
              float pr = e;
              if constexpr (!FULL) {
                // keep ? P : 0 as a bit select on an all-ones / all-zeros field
                const int keep = __builtin_amdgcn_sbfe((int)Wq, 8 * (r >> 2) + (r & 3), 1);
                pr = __int_as_float(keep & __float_as_int(e));
              }
              p[c8] = pr;
              ds[c8] = pr * (dpacc[r] - Dq);
            }
            // keys 16*p2 + 4*half + 0..3 and 16*p2 + 8 + 4*half + 0..3 of query
            // col: a row segment of the [query][key] P and dS tiles, and, for dS,
            // exactly the dQ kernel's B-operand fragment for this 16-key step
            // (4-key groups 4*p2 + half and 4*p2 + half + 2 of the row, swizzled)
            const u32x4 pp = pack8(p), dsp = pack8(ds);
            const int o0 = pds_base ^ (16 * p2), o1 = o0 ^ 8;
            *(u32x2*)(smP[it & 1][kw] + o0) = u32x2{pp[0], pp[1]};
            *(u32x2*)(smP[it & 1][kw] + o1) = u32x2{pp[2], pp[3]};
            *(u32x2*)(smT[it & 1][kw] + o0) = u32x2{dsp[0], dsp[1]};
            *(u32x2*)(smT[it & 1][kw] + o1) = u32x2{dsp[2], dsp[3]};
            pend[p2] = dsp;
            pfr = fr;
            have = true;
          }
        };
        if (__builtin_amdgcn_readfirstlane((int)scls[wsel][qc >> 2]) == 2 && qc * QC + QC <= S)
          softmax(std::integral_constant<bool, true>{});
        else
          softmax(std::integral_constant<bool, false>{});
      }
      e0 = e1;
      e1 = e2;
      e2 = e3;
    }
    if (HANDOFF && have) {
      __builtin_nontemporal_store(pend[0], pfr);
      __builtin_nontemporal_store(pend[1], pfr + 64);
    }
    lds_barrier();  // matches B's final barrier
  } else {
    // B wave kw owns the 64 keys of A waves 2*kh and 2*kh+1 (kh = kw / 2) and
    // half of their ten 32-row blocks of dK^T and dV^T: role 0 dK^T rows
    // 0..159, role 1 dK^T rows 160..191 and all of dV^T. Each transposed Q^T /
    // dO^T fragment read from LDS then feeds two MFMAs (one per key block).
    const int kh = kw >> 1;
    const int sb = kb0 + 64 * kh;  // first key of the 64
    // byte offsets of this lane's transposing reads in the swizzled Q / dO
    // chunks: rows r0 + j/4 and r0 + 8 + j/4 (r0 = 16*p2 + 4*half), 4-column
    // group j%4 of the lane's 16-column half; column block n adds 64*n bytes
    const int j16 = lane & 15, g = (lane >> 4) & 1;
    uint32_t qt[2][2], ot[2][2];
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int row = 16 * p2 + 4 * half + 8 * kk + (j16 >> 2);
        const int chunk = (2 * g + ((j16 & 3) >> 1)) ^ ((row >> 2) & 3);
        qt[p2][kk] = (uint32_t)(row * dkv::QPX * 2 + 16 * chunk + 8 * (j16 & 1));
        ot[p2][kk] = (uint32_t)(row * dkv::OPX * 2 + 16 * chunk + 8 * (j16 & 1));
      }
    // one code path per role: a runtime role test inside the loop made the
    // compiler keep both roles' operands live
    auto run = [&](auto R) __attribute__((always_inline)) {
      constexpr int role = decltype(R)::value;
      f32x16 acc[2][5];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 5; ++i)
#pragma unroll
          for (int x = 0; x < 16; ++x) acc[j][i][x] = 0.f;
      auto tr = [&](const char* base, uint32_t oa_, uint32_t ob_) __attribute__((always_inline)) -> u32x4 {
        const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base + oa_));
        const v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base + ob_));
        const u32x2 ux = __builtin_bit_cast(u32x2, x), uy = __builtin_bit_cast(u32x2, y);
        return u32x4{ux[0], ux[1], uy[0], uy[1]};
      };
      // B operand from a P / dS tile: lane (half, col) gets key col of the
      // tile's queries r0 + {0..3} and r0 + 8 + {0..3} (r0 a multiple of 4).
      // Transposing read: source lane j of each 16-lane group g16 points at
      // the 4-key group 4*g16 + j%4 of query r + j/4.
      auto pds_frag = [&](const uint16_t* X, int r0) __attribute__((always_inline)) -> u32x4 {
        const int j = lane & 15, g = 4 * ((lane >> 4) & 1) + (j & 3);
        const int ra = r0 + (j >> 2), rb = r0 + 8 + (j >> 2);
        const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_ptr)(X + ra * dkv::TP + 4 * (g ^ dkv::pds_swz(ra))));
        const v4i16 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_ptr)(X + rb * dkv::TP + 4 * (g ^ dkv::pds_swz(rb))));
        const u32x2 ua = __builtin_bit_cast(u32x2, a), uc = __builtin_bit_cast(u32x2, c);
        return u32x4{ua[0], ua[1], uc[0], uc[1]};
      };
      // dK^T[d, s] += Q^T[d, q] dS[q, s] and dV^T[e, s] += dO^T[e, q] P[q, s]
      // for the chunk of iteration `it`; the query order inside each 16-query
      // step matches the A waves' accumulator rows. When only the first key
      // block took part in the chunk (the diagonal), the second block's P and dS
      // operands are zero.
      auto update = [&](int it, bool both) __attribute__((always_inline)) {
        const char* sQ = (const char*)smQ[it % NB];
        const char* sO = (const char*)smO[it % NB];
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          const int r0 = 16 * p2 + 4 * half;
          // lane (half, col): key col of the block, queries r0 + {0..3, 8..11}
          const u32x4 d0 = pds_frag(smT[it & 1][2 * kh], r0);
          u32x4 d1 = pds_frag(smT[it & 1][2 * kh + 1], r0);
          if (!both) d1 = z;
          if constexpr (role == 0) {
#pragma unroll
            for (int d2 = 0; d2 < 5; ++d2) {
              const u32x4 a = tr(sQ + 64 * d2, qt[p2][0], qt[p2][1]);
              acc[0][d2] = mfma32(a, d0, acc[0][d2]);
              acc[1][d2] = mfma32(a, d1, acc[1][d2]);
            }
          } else {
            const u32x4 p0 = pds_frag(smP[it & 1][2 * kh], r0);
            u32x4 p1 = pds_frag(smP[it & 1][2 * kh + 1], r0);
            if (!both) p1 = z;
            const u32x4 a = tr(sQ + 64 * 5, qt[p2][0], qt[p2][1]);
            acc[0][0] = mfma32(a, d0, acc[0][0]);
            acc[1][0] = mfma32(a, d1, acc[1][0]);
#pragma unroll
            for (int eb = 0; eb < DV / 32; ++eb) {
              const u32x4 o = tr(sO + 64 * eb, ot[p2][0], ot[p2][1]);
              acc[0][1 + eb] = mfma32(o, p0, acc[0][1 + eb]);
              acc[1][1 + eb] = mfma32(o, p1, acc[1][1 + eb]);
            }
          }
        }
      };
      // the A waves of key block j took part in chunk e: their key tile is
      // non-empty there and the chunk reaches the block's first key
      auto act = [&](int e, int j) __attribute__((always_inline)) {
        return ((e >> (14 + kh)) & 1) != 0 && ratio * (sb + 32 * j) + ratio - 1 <= (e & 0x3FFF) * QC + QC - 1;
      };
      bool prev = false, prev2 = false;
      int it = 0;
      for (; e0 >= 0; ++it) {
        publish_b(it);
        if (e2 >= 0) issue(e2 & 0x3FFF, (it + 2) % NB);
        const int e3 = entry(it + 3);
        if (prev) update(it - 1, prev2);  // the chunk A finished before this barrier
        prev = act(e0, 0);
        prev2 = act(e0, 1);
        e0 = e1;
        e1 = e2;
        e2 = e3;
      }
      lds_barrier();  // A's P and dS of the last chunk are visible
      if (prev) update(it - 1, prev2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int s = sb + 32 * j + col;
        if (s >= Sk) continue;
        uint16_t* dkrow = dk + ((size_t)b * Sk + s) * rs_qk + (size_t)h * DQK;
        uint16_t* dvrow = dv + ((size_t)b * Sk + s) * rs_v + (size_t)h * DV;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          // role 0: dK^T block i; role 1: dK^T block 5 (i == 0), dV^T block i-1
          const bool isk = role == 0 || i == 0;
          const float sc = isk ? scale : 1.f;
          uint16_t* row = isk ? dkrow + 32 * (role == 0 ? i : 5) : dvrow + 32 * (i - 1);
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const int d = 8 * gg + 4 * half;
            *(u32x2*)(row + d) = u32x2{pack_bf2(acc[j][i][4 * gg] * sc, acc[j][i][4 * gg + 1] * sc),
                                       pack_bf2(acc[j][i][4 * gg + 2] * sc, acc[j][i][4 * gg + 3] * sc)};
          }
        }
      }
    };
    if (kw & 1)
      run(std::integral_constant<int, 1>{});
    else
      run(std::integral_constant<int, 0>{});
  }
}

// ---------------------------------------------------------------------------
// dQ, query-major, from the dS^T fragments the key-major kernel stored:
// dQ^T[d, q] = scale * sum_s K^T[d, s] dS^T[s, q]. Workgroup = (b, h, 256
// queries), 8 waves (two per SIMD) of one 32-query chunk each. It walks the
// non-empty 64-key tiles up to the diagonal. K tiles are double buffered in
// natural layout and read transposed; each wave's 4 KB of fragments per tile
// go to a private three-slot LDS ring, two tiles ahead (they stream from
// HBM). Every copy is a direct global->LDS copy issued through the untracked
// asm path, and each wave issues exactly four fragment copies per tile
// (harmless ones where it has nothing to take), so one counted wait covers
// both. A wave takes a tile only where the key-major kernel wrote it: its own
// 128-query tile is non-empty there, and only the 32-key halves that start at
// or before its last query (causal).
// ---------------------------------------------------------------------------
namespace dqk {
constexpr int NW = 8, QW = 32 * NW;
// 16-byte slots per padded K row: at 28 slots (448 B) the 4 rows x 4 slots of
// a transposing read fall on 16 distinct bank groups (at 25 slots, two-way
// conflicts). Pad slots copy the row's last chunk.
constexpr int KSL = bwd::DQK / 8 + 4;
constexpr int KBLK = bwd::TK * KSL / 64;
constexpr int KI = (KBLK + NW - 1) / NW;
constexpr int NF = 3;  // fragment ring slots
static_assert(KSL * 8 == bwd::QP, "pitch");
}  // namespace dqk

__global__ __launch_bounds__(dqk::NW * 64) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ k, const u32x4* __restrict__ dsf, const uint8_t* __restrict__ cls, int B,
    int S, int Sk, int ratio, int H, float scale, uint16_t* __restrict__ dq) {
  using namespace bwd;
  using dqk::NW;
  using dqk::QW;
  __shared__ __attribute__((aligned(1024))) uint16_t smK[2][TK * QP];
  __shared__ __attribute__((aligned(1024))) u32x4 smF[dqk::NF][NW][4][64];
  __shared__ uint8_t scls[2][kMaxTiles];  // tile classes of the workgroup's two 128-query tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so per-wave data is scalar
  const int half = lane >> 5, col = lane & 31;
  const int NQ = (S + 127) / 128, NK = (Sk + 63) / 64;
  const int NQW = (S + QW - 1) / QW;
  const int nchunks = (S + QC - 1) / QC;
  // the query blocks of a (b, h) on one XCD (they share K), costliest first
  int bh, qw;
  grouped_order(xcd_remap((int)blockIdx.x, (int)gridDim.x), NQW, B * H, bh, qw);
  const int b = bh / H, h = bh % H;
  const int qc = qw * NW + wid;  // this wave's chunk
  const bool wvalid = qc < nchunks;
  const int tq = qc * QC + col;
  const int qt_w = min(NQ - 1, qc * QC / 128);
  const int qt0 = qw * QW / 128, qt1 = min(NQ - 1, qt0 + 1);
  const size_t rs_qk = (size_t)H * DQK;
  const uint16_t* kbase = uniform_ptr(k + (size_t)b * Sk * rs_qk + (size_t)h * DQK);
  // this (b, h)'s fragment tiles, and this chunk's: key tile kt at + 256 * kt (u32x4 units)
  const u32x4* fbh = uniform_ptr(dsf + (size_t)bh * dsf_base(nchunks, ratio, NK) * 256);
  const u32x4* fch = uniform_ptr(fbh + dsf_base(wvalid ? qc : 0, ratio, NK) * 256);
  const int kl_q = (qc * QC + QC) / ratio - 1;  // last key this chunk's last query sees

  f32x16 dqacc[DQK / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dqacc[i][j] = 0.f;

  // last key tile any of the workgroup's queries sees (-1: none)
  const int kl_last = (min(S - 1, qw * QW + QW - 1) + 1) / ratio - 1;
  const int kt_last = kl_last < 0 ? -1 : kl_last / TK;
  stage_bytes(scls[0], cls + ((size_t)b * NQ + qt0) * NK, kt_last + 1);
  stage_bytes(scls[1], cls + ((size_t)b * NQ + qt1) * NK, kt_last + 1);
  const uint8_t* cls0 = scls[0];
  const uint8_t* cls1 = scls[1];
  const uint8_t* clsw = scls[qt_w - qt0];
  auto next_tile = [&](int kt) {
    int n = kt + 1;
    while (n <= kt_last && cls0[n] == 0 && cls1[n] == 0) ++n;
    return n;
  };
  // this wave's 1 KB blocks of a K tile: byte offsets within the tile's rows
  uint32_t koff[dqk::KI];
  int krow[dqk::KI];
#pragma unroll
  for (int i = 0; i < dqk::KI; ++i) {
    const int slot = (wid + i * NW) * 64 + lane;
    krow[i] = slot / dqk::KSL;
    koff[i] = (uint32_t)((krow[i] * rs_qk + min(slot % dqk::KSL, DQK / 8 - 1) * 8) * 2);
  }
  auto issue_k = [&](int kt, int buf) {
    const uint16_t* tb = kbase + (size_t)kt * TK * rs_qk;
    const int lim = Sk - 1 - kt * TK;  // last in-range row of the tile
#pragma unroll
    for (int i = 0; i < dqk::KI; ++i)
      if (wid + i * NW < dqk::KBLK) {
        const int dr = krow[i] - min(krow[i], lim);  // rows past S copy row S-1
        g2lds16_async_off(tb, koff[i] - (uint32_t)(dr * rs_qk * 2), (char*)smK[buf] + (wid + i * NW) * 1024);
      }
  };
  // 32-key halves of tile kt this wave takes: 0, 1 or 2 (causal at 32 keys)
  auto halves = [&](int kt) -> int {
    if (kt > kt_last || !wvalid || clsw[kt] == 0) return 0;
    return (64 * kt <= kl_q) + (64 * kt + 32 <= kl_q);
  };
  // the four fragment blocks of tile kt into ring slot f; k steps the wave
  // does not take copy this (b, h)'s first block instead
  auto issue_f = [&](int kt, int nh, int f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4* src = (j < 2 * nh) ? fch + 256 * kt + 64 * j : fbh;
      g2lds16_async_off_nt(src, (uint32_t)lane * 16u, &smF[f][wid][j][0]);
    }
  };

  __syncthreads();  // class rows staged
  int kt = next_tile(-1);
  int kn = next_tile(kt);
  int nh = halves(kt), nh1 = halves(kn);
  if (kt <= kt_last) issue_k(kt, 0);
  issue_f(kt, nh, 0);
  issue_f(kn, nh1, 1);
  int buf = 0, fs = 0;
  while (kt <= kt_last) {
    const int kn2 = next_tile(kn);
    const int nh2 = halves(kn2);
    wait_vmem_n<4>();  // K tile kt and its fragments are in; tile kn's fragments may still fly
    __syncthreads();   // tile kt visible in `buf`; every wave is done with the other buffer
    if (kn <= kt_last) issue_k(kn, buf ^ 1);
    issue_f(kn2, nh2, fs == 0 ? 2 : fs - 1);
    const uint16_t* sK = smK[buf];
    // dQ^T[d, q] += K^T[d, s] dS^T[s, q]; the fragment of k step (kb, p2)
    // holds keys kb*32 + 16*p2 + 4*half + {0..3, 8..11}
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (kb < nh) {
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          const int r0 = kb * 32 + 16 * p2 + 4 * half;
          const u32x4 db = smF[fs][wid][2 * kb + p2][lane];
          u32x4 ka[DQK / 32];
#pragma unroll
          for (int i = 0; i < DQK / 32; ++i) ka[i] = lds_tr_frag(sK, QP, r0, r0 + 8, i * 32);
#pragma unroll
          for (int i = 0; i < DQK / 32; ++i) dqacc[i] = mfma32(ka[i], db, dqacc[i]);
        }
      }
    nh = nh1;
    nh1 = nh2;
    buf ^= 1;
    fs = fs == 2 ? 0 : fs + 1;
    kt = kn;
    kn = kn2;
  }
  wait_vmem();  // no copy outlives the workgroup
  if (wvalid && tq < S) {
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
// dQ, query-major, recomputing dS (no handoff): for shapes whose dS tiles would
// not fit the workspace. Workgroup = (b, h, 256 queries), 8 waves (two per
// SIMD) of 32 queries. Q and dO of the lane's query stay in VGPRs; K and V
// tiles are double buffered in natural layout. Per 32-key half of a tile it
// forms S^T = K Q^T and dP^T = V dO^T, then P = exp2(S^T scale log2e - LSE2)
// on the kept pairs and dS = P (dP - D), and accumulates dQ^T += K^T dS^T.
// Every operation and its order match the key-major kernel's A role and the
// fragment-reading dQ kernel, so the result is the same as with the handoff
// (halves that kernel skips contribute exact zeros here).
// ---------------------------------------------------------------------------
namespace dqr {
constexpr int NW = 8, QW = 32 * NW;
constexpr int KSL = bwd::DQK / 8 + 1, VSL = bwd::DV / 8 + 1;  // 16-byte slots per padded row
constexpr int KP = KSL * 8, VP = VSL * 8;                     // pitches (elements)
constexpr int KBLK = bwd::TK * KSL / 64, VBLK = bwd::TK * VSL / 64;  // 1 KB blocks per tile
constexpr int KI = (KBLK + NW - 1) / NW, VI = (VBLK + NW - 1) / NW;  // blocks per wave
static_assert(bwd::TK * KSL % 64 == 0 && bwd::TK * VSL % 64 == 0, "tiles must be whole 1 KB blocks");
}  // namespace dqr

__global__ __launch_bounds__(dqr::NW * 64) void attn_bwd_dq_recompute_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ ws, const uint64_t* __restrict__ bits,
    const uint8_t* __restrict__ cls, int B, int S, int Sk, int ratio, int H, float scale, float scale_log2,
    uint16_t* __restrict__ dq) {
  using namespace bwd;
  using dqr::NW;
  using dqr::QW;
  __shared__ __attribute__((aligned(1024))) uint16_t smK[2][TK * dqr::KP];
  __shared__ __attribute__((aligned(1024))) uint16_t smV[2][TK * dqr::VP];
  __shared__ uint8_t scls[2][kMaxTiles];  // tile classes of the workgroup's two 128-query tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so per-wave data is scalar
  const int half = lane >> 5, col = lane & 31;
  const int W = (Sk + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int NQW = (S + QW - 1) / QW;
  int bh, qw;
  grouped_order(xcd_remap((int)blockIdx.x, (int)gridDim.x), NQW, B * H, bh, qw);
  const int b = bh / H, h = bh % H;
  const int tq = qw * QW + wid * 32 + col;  // this lane's query
  const bool qvalid = tq < S;
  const int qt_w = min(NQ - 1, (qw * QW + wid * 32) / 128);
  const int qt0 = qw * QW / 128, qt1 = min(NQ - 1, qt0 + 1);
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;
  const uint16_t* kbase = k + (size_t)b * Sk * rs_qk + (size_t)h * DQK;
  const uint16_t* vbase = v + (size_t)b * Sk * rs_v + (size_t)h * DV;

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
  // D and the base-2 LSE of the lane's query, from the prologue's workspace
  const size_t qi = ((size_t)b * H + h) * S + (qvalid ? tq : 0);
  const float Dq = qvalid ? ws[qi] : 0.f;
  const float Lq = qvalid ? ws[(size_t)B * H * S + qi] : 0.f;

  f32x16 dqacc[DQK / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dqacc[i][j] = 0.f;

  // last key tile any of the workgroup's queries sees (-1: none); key s is
  // visible to query t when ratio * s + ratio - 1 <= t
  const int kl_last = (min(S - 1, qw * QW + QW - 1) + 1) / ratio - 1;
  const int kt_last = kl_last < 0 ? -1 : kl_last / TK;
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
  // this wave's 1 KB blocks of a tile; pad slots copy a harmless chunk and rows
  // past the last key copy row Sk-1
  auto issue = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < dqr::KI; ++i) {
      const int j = wid + i * NW;
      if (j < dqr::KBLK) {
        const int slot = j * 64 + lane, row = slot / dqr::KSL, c = min(slot % dqr::KSL, dqr::KSL - 2);
        const int s = min(kt * TK + row, Sk - 1);
        g2lds16(kbase + (size_t)s * rs_qk + c * 8, (char*)smK[buf] + j * 1024);
      }
    }
#pragma unroll
    for (int i = 0; i < dqr::VI; ++i) {
      const int j = wid + i * NW;
      if (j < dqr::VBLK) {
        const int slot = j * 64 + lane, row = slot / dqr::VSL, c = min(slot % dqr::VSL, dqr::VSL - 2);
        const int s = min(kt * TK + row, Sk - 1);
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
    const int kn = next_tile(kt);
    wait_vmem();
    __syncthreads();  // tile kt visible in `buf`; every wave is done with the other buffer
    const uint64_t mw_n = kn <= kt_last ? word(kn) : 0ull;
    if (kn <= kt_last) issue(kn, buf ^ 1);
    if (__ballot(mw != 0ull)) {
      const uint16_t* sK = smK[buf];
      const uint16_t* sV = smV[buf];
      // this lane's keys are kb*32 + 8i + 4*half + r: the word pre-shifted by 4*half
      const uint64_t mwh = mw >> (4 * half);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t Wq = (uint32_t)(mwh >> (32 * kb));
        f32x16 sacc, dpacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks)
          sacc = mfma32(*(const u32x4*)(sK + (kb * 32 + col) * dqr::KP + ks * 16 + 8 * half), qf[ks], sacc);
#pragma unroll
        for (int ks = 0; ks < DV / 16; ++ks)
          dpacc = mfma32(*(const u32x4*)(sV + (kb * 32 + col) * dqr::VP + ks * 16 + 8 * half), of[ks], dpacc);
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          float ds[8];
#pragma unroll
          for (int c8 = 0; c8 < 8; ++c8) {
            const int r = 8 * p2 + c8;
            const int keep = __builtin_amdgcn_sbfe((int)Wq, 8 * (r >> 2) + (r & 3), 1);
            const float pr = __int_as_float(keep & __float_as_int(fast_exp2(fmaf(sacc[r], scale_log2, -Lq))));
            ds[c8] = pr * (dpacc[r] - Dq);
          }
          const u32x4 db = pack8(ds);
          const int r0 = kb * 32 + 16 * p2 + 4 * half;
#pragma unroll
          for (int i = 0; i < DQK / 32; ++i)
            dqacc[i] = mfma32(lds_tr_frag(sK, dqr::KP, r0, r0 + 8, i * 32), db, dqacc[i]);
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

hipError_t launch_attn_bwd_dq_recompute(const void* q, const void* k, const void* v, const void* dout,
                                        const float* ws, const uint64_t* bits, const uint8_t* cls, int B, int S,
                                        int Sk, int ratio, int H, float scale, void* dq, hipStream_t st) {
  const size_t nq = (size_t)((S + dqr::QW - 1) / dqr::QW) * B * H;
  hipLaunchKernelGGL(attn_bwd_dq_recompute_kernel, dim3((unsigned)nq), dim3(dqr::NW * 64), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, ws, bits,
                     cls, B, S, Sk, ratio, H, scale, scale * 1.4426950408889634f, (uint16_t*)dq);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dq_mfma(const void* k, const void* dsf, const uint8_t* cls, int B, int S, int Sk,
                                   int ratio, int H, float scale, void* dq, hipStream_t st) {
  const size_t nq = (size_t)((S + dqk::QW - 1) / dqk::QW) * B * H;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)nq), dim3(dqk::NW * 64), 0, st, (const uint16_t*)k,
                     (const u32x4*)dsf, cls, B, S, Sk, ratio, H, scale, (uint16_t*)dq);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv_mfma(const void* q, const void* k, const void* v, const void* dout,
                                     const float* ws, const uint64_t* bits, const uint8_t* cls, int B, int S,
                                     int Sk, int ratio, int H, float scale, void* dk, void* dv, void* dsf,
                                     hipStream_t st) {
  const size_t nkv = (size_t)((Sk + 127) / 128) * B * H;
  if (dsf)
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<true>, dim3((unsigned)nkv), dim3(dkv::NW * 64), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, ws, bits,
                       cls, B, S, Sk, ratio, H, scale, scale * 1.4426950408889634f, (uint16_t*)dk, (uint16_t*)dv,
                       (u32x4*)dsf);
  else
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<false>, dim3((unsigned)nkv), dim3(dkv::NW * 64), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, ws, bits,
                       cls, B, S, Sk, ratio, H, scale, scale * 1.4426950408889634f, (uint16_t*)dk, (uint16_t*)dv,
                       nullptr);
  return hipGetLastError();
}

}  // namespace dsa
