// Lightning-indexer scores (gfx950).
//
// I[b,t,s] = sum_j w[b,t,j] * max(0, q_idx[b,t,j,:] . k_idx[b,s,:]) for s in
// valid(t) (causal with the diagonal, same segment). Source: "DeepSeek3.2:
// Onboard sparse attention", Background (the indexer's parametric query-key
// product) and "What this PR does", item 2 (64 index heads x 128).
// Keys may be compressed blocks ("Add Flash Attention Support to Deepseek v4",
// Description; "Implement QK attention head chunking for CSA [Deepseek v4]",
// Description): Sk keys, key s standing for tokens ratio*s .. ratio*s +
// ratio - 1 and visible to query t once its block is complete, s <=
// (t + 1) / ratio - 1. ratio 1 and Sk = S is the token-level indexer.
//
// MFMA kernel: per query t, the product of its index heads with a tile of 32
// keys is a [Hi x 32] GEMM with K = Di. Heads go on the MFMA row dimension and
// keys on the column dimension. Each lane then owns one key column and 16
// head rows per 32-head block, so the ReLU and the w-weighted sum over heads
// are in-lane float32 FMAs, with one exchange between the two lane halves.
// q_idx[t] (Hi x Di bf16, 16 KB at 64 x 128) stays in VGPRs as MFMA A
// fragments for the whole key loop. A 128-key k_idx tile is copied straight
// into padded LDS (global_load_lds) once per workgroup (4 waves = 4
// consecutive queries) and double buffered. The tile is four 32-key column
// blocks, software-pipelined: the MFMAs of one block run while the previous
// block's ReLU and weighted sums are formed, across the tile barrier too.
// Lane l stores key 128*kt + l from blocks 0/1 and 128*kt + 64 + l from
// blocks 2/3. With segment IDs the walk starts at the tile of the rows'
// first same-segment key (packed documents skip the keys of earlier ones).
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

template <int HB, int KS, typename OutT>
__global__ __launch_bounds__(256) void index_scores_mfma_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    const uint16_t* __restrict__ w, const int32_t* __restrict__ seg, int B, int S, int Sk, int ratio,
    int row0, int nrows, OutT* __restrict__ scores, int64_t ld) {
  constexpr int Hi = HB * 32, Di = KS * 16;
  constexpr int TILE = 128;                  // keys per iteration: four 32-key MFMA column blocks
  constexpr int SL = Di / 8 + 1;             // 16-byte slots per padded LDS key row
  constexpr int ROWE = SL * 8;               // padded row pitch in elements (conflict-free b128 reads)
  constexpr int NBLK = (TILE * SL + 63) / 64;  // 1 KB blocks per tile
  constexpr int BI = (NBLK + 3) / 4;           // blocks per wave
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2][NBLK * 1024];
  __shared__ int32_t lseg[2][TILE];            // segment IDs of the tile's keys (when given)
  __shared__ uint32_t red[4];
  static_assert((Di * 2 & (Di * 2 - 1)) == 0, "key rows are a power-of-two number of bytes");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int nrb = (nrows + 3) / 4;
  // Row blocks longest first, the batch index fastest. Blocks are dealt to
  // the 8 XCDs round-robin in dispatch order, so every XCD gets an equal share
  // of long and short rows (a contiguous split per XCD leaves one XCD with all
  // of a batch's longest rows), and the row blocks that run together on an
  // XCD stream the same k_idx tiles, once, through its L2.
  const int L = (int)blockIdx.x;
  const int b = L % B;
  const int rb = nrb - 1 - L / B;
  const int r = rb * 4 + wid;
  const bool active = r < nrows;
  const int t = row0 + r;
  const int t_last = row0 + min(nrows - 1, rb * 4 + 3);
  const int kl_last = (t_last + 1) / ratio - 1;  // last key any of the rows sees
  if (kl_last < 0) return;                       // the whole workgroup: no visible key
  const int nkt = kl_last / TILE + 1;
  const int tk = (t + 1) / ratio - 1;            // this row's last visible key
  const uint16_t* kb_base = uniform_ptr(k_idx + (size_t)b * Sk * Di);

  u32x4 afrag[HB][KS];
  float wreg[HB][16];
  int seg_t = 0;
  if (active) {
    const uint16_t* qrow = q_idx + ((size_t)b * S + t) * Hi * Di;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        afrag[hb][ks] = *(const u32x4*)(qrow + (size_t)(hb * 32 + col) * Di + ks * 16 + 8 * half);
    const uint16_t* wrow = w + ((size_t)b * S + t) * Hi;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) wreg[hb][rr] = bf2f(wrow[hb * 32 + acc_row(rr, half)]);
    if (seg) seg_t = seg[(size_t)b * S + t];
  } else {
    // a row past the range runs the workgroup's MFMAs on zeros and stores nothing
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) afrag[hb][ks] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) wreg[hb][rr] = 0.f;
    }
  }

  // this wave's 1 KB blocks of the padded [TILE rows][SL slots] tile; slots
  // past a row's data or the tile copy a harmless chunk. Waves 1 and 2 also
  // copy the tile's segment IDs. Copies go through the untracked asm path;
  // each wave waits for its own before the barrier that publishes the tile. A
  // tile inside the sequence is copied from a scalar base plus fixed lane
  // offsets; the last, partial one clamps its rows to S - 1.
  uint32_t coff[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int slot = (wid + i * 4) * 64 + lane;
    const bool in = slot < TILE * SL;
    const int row = in ? slot / SL : 0, c = in ? min(slot % SL, SL - 2) : 0;
    coff[i] = (uint32_t)((row * Di + c * 8) * 2);
  }
  auto issue = [&](int kt, int buf) {
    if ((kt + 1) * TILE <= Sk) {
      const uint16_t* tb = kb_base + (size_t)kt * TILE * Di;
#pragma unroll
      for (int i = 0; i < BI; ++i)
        if (wid + i * 4 < NBLK) g2lds16_async_off(tb, coff[i], lds[buf] + (wid + i * 4) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < BI; ++i)
        if (wid + i * 4 < NBLK) {
          const int row = (int)(coff[i] / (Di * 2));
          const int s = min(kt * TILE + row, Sk - 1);
          const uint32_t c_bytes = coff[i] % (Di * 2);
          g2lds16_async((const char*)(kb_base + (size_t)s * Di) + c_bytes, lds[buf] + (wid + i * 4) * 1024);
        }
    }
    if (seg && (wid == 1 || wid == 2)) {
      const int h = wid - 1;
      g2lds4_async(seg + (size_t)b * S + min(kt * TILE + 64 * h + lane, S - 1), lseg[buf] + 64 * h);
    }
  };
  // [Hi x 32] scores of the 32-key column block sb of the tile in buffer buf
  auto mfma_block = [&](int buf, int sb, f32x16 (&acc)[HB]) {
    const uint16_t* sk = (const uint16_t*)lds[buf] + (sb * 32 + col) * ROWE + 8 * half;
    u32x4 bq[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bq[ks] = *(const u32x4*)(sk + ks * 16);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[hb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32(afrag[hb][ks], bq[ks], acc[hb]);
  };
  // w-weighted ReLU sum over the heads for key col; both lane halves end
  // with the total
  auto head_sum = [&](const f32x16 (&acc)[HB]) -> float {
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        part[rr & 3] = fmaf(wreg[hb][rr], fmaxf(acc[hb][rr], 0.f), part[rr & 3]);
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    return half_sum(tot);
  };

  // Software pipeline over 32-key blocks: the MFMAs of one block run while
  // the previous block's sums are formed, across the tile barrier. Lane l
  // stores keys 128*kt + l (half 0 from block 0, half 1 from block 1) and
  // 128*kt + 64 + l (blocks 2 and 3). The second store comes after the
  // barrier and the first half a tile before the next one, so the wait for
  // the next tile's copies does not wait for a store issued just before it.
  OutT* out_row = scores + ((size_t)b * nrows + r) * ld;
  f32x16 accA[HB], accB[HB];
  // With segment IDs, valid(t) starts at t's segment's first position: the
  // loop starts at the tile of the first position whose ID is one of the
  // workgroup's rows' IDs (the smallest of their first positions), found by a
  // forward scan of 1024 positions per step. Rows past the range use the
  // first row's ID.
  int kt0 = 0;
  if (seg) {
    const int32_t* segb = seg + (size_t)b * S;
    int ids[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ids[i] = segb[row0 + min(rb * 4 + i, nrows - 1)];
    uint32_t first = 0xffffffffu;
    for (int base = 0; base <= t_last && first == 0xffffffffu; base += 1024) {
      uint32_t m = 0xffffffffu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = base + 256 * j + tid;
        if (p <= t_last) {
          const int sp = segb[p];
          if (sp == ids[0] || sp == ids[1] || sp == ids[2] || sp == ids[3]) m = min(m, (uint32_t)p);
        }
      }
      m = wave_umin(m);
      if (lane == 0) red[wid] = m;
      __syncthreads();
      first = min(min(red[0], red[1]), min(red[2], red[3]));
      __syncthreads();
    }
    // found (every row's own position matches); the same in every lane, made
    // provably uniform so that tile bases stay in scalar registers
    kt0 = __builtin_amdgcn_readfirstlane((int)(first / TILE));
  }
  wait_vmem();  // this wave's query fragments and weights are in
  issue(kt0, 0);
  wait_vmem();
  lds_barrier();
  if (kt0 + 1 < nkt) issue(kt0 + 1, 1);
  mfma_block(0, 0, accA);
  for (int kt = kt0; kt < nkt; ++kt) {
    const int buf = (kt - kt0) & 1;
    const int s_lo = kt * TILE + lane, s_hi = s_lo + 64;
    bool ok_lo = active && s_lo <= tk, ok_hi = active && s_hi <= tk;
    if (seg) {
      ok_lo = ok_lo && lseg[buf][lane] == seg_t;
      ok_hi = ok_hi && lseg[buf][64 + lane] == seg_t;
    }
    mfma_block(buf, 1, accB);
    const float t0 = head_sum(accA);
    mfma_block(buf, 2, accA);
    const float t1 = head_sum(accB);
    if (ok_lo) Elem<OutT>::store(out_row + s_lo, half ? t1 : t0);
    mfma_block(buf, 3, accB);
    const float t2 = head_sum(accA);
    float t3;
    if (kt + 1 < nkt) {
      wait_vmem();
      lds_barrier();  // tile kt+1 visible; every wave is done with tile kt
      if (kt + 2 < nkt) issue(kt + 2, buf);
      mfma_block(buf ^ 1, 0, accA);
      t3 = head_sum(accB);
    } else {
      t3 = head_sum(accB);
    }
    if (ok_hi) Elem<OutT>::store(out_row + s_hi, half ? t3 : t2);
  }
}

// Plain kernel for any (Hi, Di) and fp32 or bf16 inputs: one thread per key s,
// the query's Hi x Di index vectors staged in LDS as float32.
template <typename InT, typename OutT>
__global__ __launch_bounds__(256) void index_scores_plain_kernel(
    const InT* __restrict__ q_idx, const InT* __restrict__ k_idx, const InT* __restrict__ w,
    const int32_t* __restrict__ seg, int S, int Sk, int ratio, int Hi, int Di, int row0, int nrows,
    OutT* __restrict__ scores, int64_t ld) {
  extern __shared__ float smem[];  // Hi*Di query values, then Hi weights
  const int nkb = (Sk + 255) / 256;
  const int r = blockIdx.x / nkb, kb = blockIdx.x % nkb, b = blockIdx.y;
  const int t = row0 + r;
  const int tk = (t + 1) / ratio - 1;  // last visible key
  const int s = kb * 256 + threadIdx.x;
  if (kb * 256 > tk) return;  // whole block in the future (uniform)
  float* qs = smem;
  float* ws = smem + Hi * Di;
  const InT* qrow = q_idx + ((size_t)b * S + t) * Hi * Di;
  for (int i = threadIdx.x; i < Hi * Di; i += 256) qs[i] = Elem<InT>::load(qrow + i);
  for (int i = threadIdx.x; i < Hi; i += 256) ws[i] = Elem<InT>::load(w + ((size_t)b * S + t) * Hi + i);
  __syncthreads();
  if (s > tk) return;
  if (seg && seg[(size_t)b * S + s] != seg[(size_t)b * S + t]) return;
  const InT* krow = k_idx + ((size_t)b * Sk + s) * Di;
  float part = 0.f;
  for (int j = 0; j < Hi; ++j) {
    float dot = 0.f;
    for (int d = 0; d < Di; ++d) dot = fmaf(qs[j * Di + d], Elem<InT>::load(krow + d), dot);
    part = fmaf(ws[j], fmaxf(dot, 0.f), part);
  }
  Elem<OutT>::store(scores + ((size_t)b * nrows + r) * ld + s, part);
}

template <int HB, int KS>
static hipError_t launch_mfma_t(const void* q_idx, const void* k_idx, const void* w,
                                const int32_t* seg, int B, int S, int Sk, int ratio, int row0, int nrows,
                                void* scores, bool out_bf16, int64_t ld, hipStream_t st) {
  const int nrb = (nrows + 3) / 4;
  dim3 grid((unsigned)(nrb * B)), block(256);
  if (out_bf16)
    hipLaunchKernelGGL((index_scores_mfma_kernel<HB, KS, uint16_t>), grid, block, 0, st,
                       (const uint16_t*)q_idx, (const uint16_t*)k_idx, (const uint16_t*)w, seg, B,
                       S, Sk, ratio, row0, nrows, (uint16_t*)scores, ld);
  else
    hipLaunchKernelGGL((index_scores_mfma_kernel<HB, KS, float>), grid, block, 0, st,
                       (const uint16_t*)q_idx, (const uint16_t*)k_idx, (const uint16_t*)w, seg, B,
                       S, Sk, ratio, row0, nrows, (float*)scores, ld);
  return hipGetLastError();
}

hipError_t launch_index_scores_mfma(const void* q_idx, const void* k_idx, const void* w,
                                    const int32_t* seg, int B, int S, int Sk, int ratio, int Hi, int Di,
                                    int row0, int nrows, void* scores, bool out_bf16, int64_t ld,
                                    hipStream_t st) {
  if (Hi == 64 && Di == 128)
    return launch_mfma_t<2, 8>(q_idx, k_idx, w, seg, B, S, Sk, ratio, row0, nrows, scores, out_bf16, ld, st);
  if (Hi == 32 && Di == 128)
    return launch_mfma_t<1, 8>(q_idx, k_idx, w, seg, B, S, Sk, ratio, row0, nrows, scores, out_bf16, ld, st);
  if (Hi == 64 && Di == 64)
    return launch_mfma_t<2, 4>(q_idx, k_idx, w, seg, B, S, Sk, ratio, row0, nrows, scores, out_bf16, ld, st);
  if (Hi == 32 && Di == 64)
    return launch_mfma_t<1, 4>(q_idx, k_idx, w, seg, B, S, Sk, ratio, row0, nrows, scores, out_bf16, ld, st);
  return hipErrorInvalidValue;
}

hipError_t launch_index_scores_plain(const void* q_idx, const void* k_idx, const void* w,
                                     const int32_t* seg, int B, int S, int Sk, int ratio, int Hi, int Di,
                                     bool in_bf16, int row0, int nrows, void* scores,
                                     bool out_bf16, int64_t ld, hipStream_t st) {
  dim3 grid((unsigned)(((Sk + 255) / 256) * nrows), (unsigned)B), block(256);
  const size_t shm = ((size_t)Hi * Di + Hi) * sizeof(float);  // the caller bounds it to 64 KB
#define DSA_IDX_PLAIN(IT, OT)                                                               \
  hipLaunchKernelGGL((index_scores_plain_kernel<IT, OT>), grid, block, shm, st, (const IT*)q_idx, \
                     (const IT*)k_idx, (const IT*)w, seg, S, Sk, ratio, Hi, Di, row0, nrows, (OT*)scores, ld)
  if (in_bf16) {
    if (out_bf16) DSA_IDX_PLAIN(uint16_t, uint16_t); else DSA_IDX_PLAIN(uint16_t, float);
  } else {
    if (out_bf16) DSA_IDX_PLAIN(float, uint16_t); else DSA_IDX_PLAIN(float, float);
  }
#undef DSA_IDX_PLAIN
  return hipGetLastError();
}

}  // namespace dsa
