// Lightning-indexer scores from fp8 (E4M3) inputs, and the row quantizer that
// produces them (gfx950).
//
// Source: "DeepSeek3.2: Onboard sparse attention", What this PR does, item 4
// (the original indexer runs on quantized fp8 inputs) and item 2 (64 index
// heads x 128); Background (the indexer's query-key product). The page names
// no format. Here: OCP E4M3 codes with one float32 scale per row, scale =
// amax / 448, codes = round-to-nearest-even(x / scale); per (token, index
// head) rows for q_idx, per token rows for k_idx.
//
// With q = q8 * sq and k = k8 * sk (sq, sk >= 0),
//   I[t,s] = sum_j w[t,j] max(0, q[t,j,:] . k[s,:])
//          = sk[s] * sum_j (w[t,j] sq[t,j]) max(0, q8[t,j,:] . k8[s,:]),
// so the MFMAs run on the raw codes (v_mfma_f32_32x32x64_f8f6f4, twice the
// bf16 rate), the query scales fold into the head weights and the key scale
// multiplies the head sum. The tiling is the bf16 indexer's: heads on the
// MFMA rows and keys on the columns, so ReLU and the weighted head sum are
// in-lane; q8[t] stays in VGPRs; 128-key tiles of k8 (and their scales, and
// segment IDs when given) are copied global->LDS and double buffered; four
// 32-key column blocks per tile are software-pipelined. Within a 64-wide k
// step a lane holds 32 consecutive codes of its row (A) or column (B); any
// assignment of k to lanes works as long as both operands use the same one.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));

// fp8 x fp8 -> fp32 32x32x64 MFMA, both operands E4M3, no block scaling
__device__ __forceinline__ f32x16 mfma32_fp8(v8i a, v8i b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Row quantizer: one wave per row of D = 64 * E elements; lane l holds the E
// consecutive elements from E * l. amax is a wave reduction of |x| bit
// patterns (monotone for non-negative floats). The divisions are IEEE
// float32 (correctly rounded), the conversion rounds to nearest even.
// ---------------------------------------------------------------------------
template <typename InT, int E>
__global__ __launch_bounds__(256) void quant_fp8_rows_kernel(const InT* __restrict__ x, int64_t nrows,
                                                             uint8_t* __restrict__ codes,
                                                             float* __restrict__ scale) {
  constexpr int D = 64 * E;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;  // the whole wave leaves together
  const InT* xr = x + row * D + E * lane;
  float v[E];
  uint32_t am = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] = Elem<InT>::load(xr + e);
    am = max(am, __float_as_uint(v[e]) & 0x7fffffffu);
  }
  const float amax = __uint_as_float(wave_umax(am));
  const float sc = amax / 448.0f;
  const float div = sc > 0.f ? sc : 1.0f;
  float y[E < 2 ? 2 : E];
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = sc > 0.f ? fminf(fmaxf(v[e] / div, -448.0f), 448.0f) : 0.f;
  if constexpr (E == 1) y[1] = 0.f;
  uint8_t* cr = codes + row * D + E * lane;
  if constexpr (E == 1) {
    *cr = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false) & 0xff);
  } else if constexpr (E == 2) {
    *(uint16_t*)cr = (uint16_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false) & 0xffff);
  } else {
    uint32_t wd[E / 4];
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i], y[4 * i + 1], 0, false);  // bytes 0, 1
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i + 2], y[4 * i + 3], pk, true);  // bytes 2, 3
      wd[i] = (uint32_t)pk;
    }
    if constexpr (E == 4)
      *(uint32_t*)cr = wd[0];
    else
      *(u32x2*)cr = u32x2{wd[0], wd[1]};
  }
  if (lane == 0) scale[row] = sc;
}

// ---------------------------------------------------------------------------
// fp8 indexer, one query per wave, 4 queries per workgroup.
// ---------------------------------------------------------------------------
template <int HB, int KS, typename OutT>
__global__ __launch_bounds__(256) void index_scores_fp8_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, const uint16_t* __restrict__ w, const int32_t* __restrict__ seg, int B,
    int S, int row0, int nrows, OutT* __restrict__ scores, int64_t ld) {
  constexpr int Hi = HB * 32, Di = KS * 64;
  constexpr int TILE = 128;                    // keys per iteration: four 32-key MFMA column blocks
  constexpr int SL = Di / 16 + 1;              // 16-byte slots per padded LDS key row
  constexpr int ROWB = SL * 16;                // padded row pitch in bytes (conflict-free b128 reads)
  constexpr int NBLK = (TILE * SL + 63) / 64;  // 1 KB blocks per tile
  constexpr int BI = (NBLK + 3) / 4;           // blocks per wave
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2][NBLK * 1024];
  __shared__ int32_t lseg[2][TILE];            // segment IDs of the tile's keys (when given)
  __shared__ float lks[2][TILE];               // key scales of the tile's keys

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int nrb = (nrows + 3) / 4;
  // row blocks longest first, the batch index fastest (as in the bf16 indexer)
  const int L = (int)blockIdx.x;
  const int b = L % B;
  const int rb = nrb - 1 - L / B;
  const int r = rb * 4 + wid;
  const bool active = r < nrows;
  const int t = row0 + r;
  const int t_last = row0 + min(nrows - 1, rb * 4 + 3);
  const int nkt = t_last / TILE + 1;
  const uint8_t* kb_base = uniform_ptr(k8 + (size_t)b * S * Di);

  v8i afrag[HB][KS];
  float wreg[HB][16];
  int seg_t = 0;
  if (active) {
    const uint8_t* qrow = q8 + ((size_t)b * S + t) * Hi * Di;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const uint8_t* p = qrow + (size_t)(hb * 32 + col) * Di + k * 64 + 32 * half;
        const u32x4 lo = *(const u32x4*)p, hi = *(const u32x4*)(p + 16);
        afrag[hb][k] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                           (int)hi[3]};
      }
    const uint16_t* wrow = w + ((size_t)b * S + t) * Hi;
    const float* qsrow = qs + ((size_t)b * S + t) * Hi;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int j = hb * 32 + acc_row(rr, half);
        wreg[hb][rr] = bf2f(wrow[j]) * qsrow[j];
      }
    if (seg) seg_t = seg[(size_t)b * S + t];
  } else {
    // a row past the range runs the workgroup's MFMAs on zeros and stores nothing
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int k = 0; k < KS; ++k) afrag[hb][k] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) wreg[hb][rr] = 0.f;
    }
  }

  // this wave's 1 KB blocks of the padded [TILE rows][SL slots] tile; slots
  // past a row's data or the tile copy a harmless chunk. Waves 0 and 3 copy
  // the tile's key scales, waves 1 and 2 its segment IDs. Every copy goes
  // through the untracked asm path; each wave waits for all of its own
  // before the barrier that publishes the tile.
  uint32_t coff[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int slot = (wid + i * 4) * 64 + lane;
    const bool in = slot < TILE * SL;
    const int row = in ? slot / SL : 0, c = in ? min(slot % SL, SL - 2) : 0;
    coff[i] = (uint32_t)(row * Di + c * 16);
  }
  auto issue = [&](int kt, int buf) {
    if ((kt + 1) * TILE <= S) {
      const uint8_t* tb = kb_base + (size_t)kt * TILE * Di;
#pragma unroll
      for (int i = 0; i < BI; ++i)
        if (wid + i * 4 < NBLK) g2lds16_async_off(tb, coff[i], lds[buf] + (wid + i * 4) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < BI; ++i)
        if (wid + i * 4 < NBLK) {
          const int row = (int)(coff[i] / Di);
          const int s = min(kt * TILE + row, S - 1);
          g2lds16_async(kb_base + (size_t)s * Di + coff[i] % Di, lds[buf] + (wid + i * 4) * 1024);
        }
    }
    if (wid == 0 || wid == 3) {
      const int h = wid == 3;
      g2lds4_async(ks + (size_t)b * S + min(kt * TILE + 64 * h + lane, S - 1), lks[buf] + 64 * h);
    } else if (seg) {
      const int h = wid - 1;
      g2lds4_async(seg + (size_t)b * S + min(kt * TILE + 64 * h + lane, S - 1), lseg[buf] + 64 * h);
    }
  };
  // [Hi x 32] code products of the 32-key column block sb of the tile in buffer buf
  auto mfma_block = [&](int buf, int sb, f32x16 (&acc)[HB]) {
    const unsigned char* sk = lds[buf] + (sb * 32 + col) * ROWB + 32 * half;
    v8i bq[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const u32x4 lo = *(const u32x4*)(sk + k * 64), hi = *(const u32x4*)(sk + k * 64 + 16);
      bq[k] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[hb][i] = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32_fp8(afrag[hb][k], bq[k], acc[hb]);
  };
  // (w * q scale)-weighted ReLU sum over the heads for key col; both lane
  // halves end with the total
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

  // Software pipeline over 32-key blocks, as in the bf16 indexer: lane l
  // stores key 128*kt + l (half 0 from block 0, half 1 from block 1) and
  // 128*kt + 64 + l (blocks 2 and 3), each scaled by its key scale.
  OutT* out_row = scores + ((size_t)b * nrows + r) * ld;
  f32x16 accA[HB], accB[HB];
  wait_vmem();  // this wave's query fragments and weights are in
  issue(0, 0);
  wait_vmem();
  lds_barrier();
  if (nkt > 1) issue(1, 1);
  mfma_block(0, 0, accA);
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const int s_lo = kt * TILE + lane, s_hi = s_lo + 64;
    bool ok_lo = active && s_lo <= t, ok_hi = active && s_hi <= t;
    if (seg) {
      ok_lo = ok_lo && lseg[buf][lane] == seg_t;
      ok_hi = ok_hi && lseg[buf][64 + lane] == seg_t;
    }
    const float sc_lo = lks[buf][lane], sc_hi = lks[buf][64 + lane];
    mfma_block(buf, 1, accB);
    const float t0 = head_sum(accA);
    mfma_block(buf, 2, accA);
    const float t1 = head_sum(accB);
    if (ok_lo) Elem<OutT>::store(out_row + s_lo, sc_lo * (half ? t1 : t0));
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
    if (ok_hi) Elem<OutT>::store(out_row + s_hi, sc_hi * (half ? t3 : t2));
  }
}

template <int HB, int KS>
static hipError_t launch_fp8_t(const void* q8, const float* qs, const void* k8, const float* ks, const void* w,
                               const int32_t* seg, int B, int S, int row0, int nrows, void* scores,
                               bool out_bf16, int64_t ld, hipStream_t st) {
  const int nrb = (nrows + 3) / 4;
  dim3 grid((unsigned)(nrb * B)), block(256);
  if (out_bf16)
    hipLaunchKernelGGL((index_scores_fp8_kernel<HB, KS, uint16_t>), grid, block, 0, st, (const uint8_t*)q8, qs,
                       (const uint8_t*)k8, ks, (const uint16_t*)w, seg, B, S, row0, nrows, (uint16_t*)scores, ld);
  else
    hipLaunchKernelGGL((index_scores_fp8_kernel<HB, KS, float>), grid, block, 0, st, (const uint8_t*)q8, qs,
                       (const uint8_t*)k8, ks, (const uint16_t*)w, seg, B, S, row0, nrows, (float*)scores, ld);
  return hipGetLastError();
}

hipError_t launch_index_scores_fp8(const void* q8, const float* qs, const void* k8, const float* ks,
                                   const void* w, const int32_t* seg, int B, int S, int Hi, int Di, int row0,
                                   int nrows, void* scores, bool out_bf16, int64_t ld, hipStream_t st) {
  if (Hi == 64 && Di == 128)
    return launch_fp8_t<2, 2>(q8, qs, k8, ks, w, seg, B, S, row0, nrows, scores, out_bf16, ld, st);
  if (Hi == 32 && Di == 128)
    return launch_fp8_t<1, 2>(q8, qs, k8, ks, w, seg, B, S, row0, nrows, scores, out_bf16, ld, st);
  if (Hi == 64 && Di == 64)
    return launch_fp8_t<2, 1>(q8, qs, k8, ks, w, seg, B, S, row0, nrows, scores, out_bf16, ld, st);
  if (Hi == 32 && Di == 64)
    return launch_fp8_t<1, 1>(q8, qs, k8, ks, w, seg, B, S, row0, nrows, scores, out_bf16, ld, st);
  return hipErrorInvalidValue;
}

hipError_t launch_quant_fp8_rows(const void* x, bool in_bf16, int64_t nrows, int D, uint8_t* codes,
                                 float* scale, hipStream_t st) {
  const dim3 grid((unsigned)((nrows + 3) / 4)), block(256);
#define DSA_QUANT(T, E)                                                                                   \
  hipLaunchKernelGGL((quant_fp8_rows_kernel<T, E>), grid, block, 0, st, (const T*)x, nrows, codes, scale)
  switch ((in_bf16 ? 16 : 0) | (D / 64)) {
    case 16 | 1: DSA_QUANT(uint16_t, 1); break;
    case 16 | 2: DSA_QUANT(uint16_t, 2); break;
    case 16 | 4: DSA_QUANT(uint16_t, 4); break;
    case 16 | 8: DSA_QUANT(uint16_t, 8); break;
    case 1: DSA_QUANT(float, 1); break;
    case 2: DSA_QUANT(float, 2); break;
    case 4: DSA_QUANT(float, 4); break;
    case 8: DSA_QUANT(float, 8); break;
    default: return hipErrorInvalidValue;
  }
#undef DSA_QUANT
  return hipGetLastError();
}

}  // namespace dsa
