// The indexer's KL auxiliary loss and its gradient (gfx950).
//
// Sources: "Support Ring Attention with DeepSeek DSA Sparse Indexer",
// sections "Isolated Flax NNX Auxiliary Loss" and "Loss Harvesting &
// Objective Injection" (an indexer loss joins the objective and trains the
// indexer's query/key projections); "Implement QK attention head chunking for
// CSA [Deepseek v4]", review of calculate_csa_indexer_loss (the teacher is a
// float32 softmax of the attention scores, zeroed on invalid tokens, summed
// over heads, from inputs that carry no gradient). With kept(t) the row's kept
// keys (the selection mask's row):
//   teacher p_t(s) = (1/H) sum_h P_h(t,s), P_h the attention probability of
//                    head h over kept(t) (each P_h sums to 1, so this is the
//                    heads' sum normalised);
//   student q_t(s) = softmax over kept(t) of I[t,s];
//   loss = (1/N) sum_t KL(p_t || q_t) over the N rows with a kept key;
//   dloss/dI[t,s] = (q_t(s) - p_t(s)) / N on kept pairs, and through
//   I = sum_j w_j ReLU(u_j), u_j = q_idx[t,j] . k_idx[s] (ReLU'(0) = 0):
//     dw[t,j] = sum_s g ReLU(u_j), dq_idx[t,j] = sum_s g w_j [u_j > 0] k_idx[s],
//     dk_idx[s] = sum_t sum_j g w_j [u_j > 0] q_idx[t,j].
//
// Kernels, in call order:
//   indexer_teacher_kernel   query-major like the attention forward, with the
//       key axis split into chunks of 4 tiles across workgroups: for each head
//       it walks the chunk's non-empty 64-key tiles, forms S^T = K Q^T with
//       MFMA, adds exp2(S^T scale log2e - LSE_h) into per-tile register
//       accumulators, and after the last head writes the mean at each kept
//       key's rank (the popcount of the row's mask bits before it), so the
//       teacher row lines up with the ascending index list.
//   indexer_kl_count_kernel  N (rows whose index list is not empty).
//   indexer_kl_kernel        one wave per row: the student softmax over the
//       kept scores, KL, and g = (q - p)/N written densely over [0, t] of the
//       gradient row (0 at keys that are not kept).
//   indexer_kl_finalize_kernel  the loss: one workgroup sums the rows' KL in
//       a fixed order (deterministic).
//   indexer_bwd_dq_kernel    (runs after dk) query-major, per query and 32-head block:
//       U^T = K Q^T (keys on MFMA rows, heads on columns, the lane's q_idx
//       fragments are the B operand), G^T = g w [U > 0], and dq^T += K^T G^T
//       with G^T going straight from the accumulator into the B operand (key
//       order permuted inside each 16-key step, as the attention forward does
//       with P); dw is an in-lane sum of g ReLU(U).
//   indexer_bwd_dk_kernel    key-major, per 32-key block and 32-head block, with
//       each key block's queries split into segments across workgroups:
//       U = Q_t K^T (heads on rows, keys on columns, the lane's k_idx
//       fragments are the B operand), G = g w [U > 0], dk^T += Q_t^T G, with
//       q_idx[t] staged in LDS two queries per stage. The float32 partials of the head
//       blocks and segments (staged in dq_idx's memory before dq is written)
//       are added in a fixed order by indexer_bwd_dk_combine_kernel.
// No atomics anywhere, so every result is deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

// ---------------------------------------------------------------------------
// Teacher
// ---------------------------------------------------------------------------
namespace itc {
constexpr int TK = 64, NW = 8, QW = 32 * NW;
constexpr int CH = 4;   // key tiles per workgroup: the key axis is split so the grid fills the chip
constexpr int NBK = 3;  // K tile buffers: copies run two (head, tile) steps ahead
}  // namespace itc

// Workgroup = (b, 256-query block, chunk of CH key tiles), 8 waves of 32
// queries. Heads are the outer loop and the chunk's non-empty tiles the inner
// one, so a wave loads its queries' fragments of a head once (after the
// head's last tile, for the next head) and keeps the per-tile head sums of
// exp2(S scale log2e - LSE_h) in registers across heads. K tiles of (head,
// tile) go through three LDS buffers, issued two steps ahead; every wave
// issues the same number of copies per tile (dummies where it has none), so a
// counted wait inside a head leaves the next tile's copies in flight. After
// the last head, each lane writes the mean at each kept key's rank (the
// popcount of its row's mask bits before it), so the teacher row lines up
// with the ascending index list.
template <int DQK>
__global__ __launch_bounds__(itc::NW * 64) void indexer_teacher_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ lse,
    const uint64_t* __restrict__ bits, const uint8_t* __restrict__ cls, int B, int S, int H, int K,
    float scale_log2, float inv_h, float* __restrict__ teacher) {
  using itc::CH;
  using itc::NBK;
  using itc::NW;
  using itc::QW;
  using itc::TK;
  constexpr int KS = DQK / 16;
  constexpr int KSL = DQK / 8 + 1;      // 16-byte slots per padded LDS key row (one pad slot)
  constexpr int KP = KSL * 8;           // pitch (elements)
  constexpr int KBLK = TK * KSL / 64;   // 1 KB blocks per tile
  constexpr int KI = (KBLK + NW - 1) / NW;  // copies per wave and tile (some of them dummies)
  static_assert(TK * KSL % 64 == 0, "tiles are whole 1 KB blocks");
  __shared__ __attribute__((aligned(1024))) uint16_t smK[NBK][TK * KP];
  __shared__ __attribute__((aligned(1024))) unsigned char smX[1024];  // target of the dummy copies, never read
  __shared__ uint8_t scls[2][kMaxTiles];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int W = (S + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int NQW = (S + QW - 1) / QW;
  const int NCH = (NK + CH - 1) / CH;
  // batch fastest, then chunk, query blocks from the last (longest rows) on
  const int b = (int)blockIdx.x % B;
  const int c = ((int)blockIdx.x / B) % NCH;
  const int qw = NQW - 1 - (int)blockIdx.x / (B * NCH);
  const int kt_end = min(S - 1, qw * QW + QW - 1) / TK;  // the block's last key tile (diagonal)
  const int c_last = kt_end / CH;
  if (c > c_last) return;  // whole workgroup: the chunk lies past the block's diagonal
  const int kt_lo = c * CH;
  const int kt_last = min(kt_end, kt_lo + CH - 1);
  const int tq = qw * QW + wid * 32 + col;
  const bool qvalid = tq < S;
  const int qt_w = min(NQ - 1, (qw * QW + wid * 32) / 128);
  const int qt0 = qw * QW / 128, qt1 = min(NQ - 1, qt0 + 1);
  const size_t rs = (size_t)H * DQK;  // token stride of q and k
  const uint16_t* kb_base = k + (size_t)b * S * rs;
  const uint16_t* q_row = q + ((size_t)b * S + (qvalid ? tq : 0)) * rs;
  const float* lse_b = lse + (size_t)b * H * S + (qvalid ? tq : 0);

  uint32_t koff[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int slot = (min(wid + i * NW, KBLK - 1)) * 64 + lane;
    koff[i] = (uint32_t)(((slot / KSL) * rs + min(slot % KSL, KSL - 2) * 8) * 2);
  }
  // K tile kt of head h into buffer buf (rows past S copy row S-1), through
  // the untracked copy path: exactly KI copies per wave
  auto issue = [&](int kt, int h, int buf) {
    const char* tb = uniform_ptr((const char*)(kb_base + (size_t)kt * TK * rs + (size_t)h * DQK));
    const int lim = S - 1 - kt * TK;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int blk = wid + i * NW;
      char* dst = blk < KBLK ? (char*)smK[buf] + blk * 1024 : (char*)smX;
      if (lim >= TK - 1) {
        g2lds16_async_off(tb, koff[i], dst);
      } else {
        const int row = ((min(blk, KBLK - 1)) * 64 + lane) / KSL;
        const int dr = row - min(row, lim);
        g2lds16_async(tb + koff[i] - (size_t)dr * rs * 2, dst);
      }
    }
  };
  // q fragments and the natural-log LSE of head h
  auto load_q = [&](int h, u32x4 (&f)[KS], float& L) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (qvalid) z = *(const u32x4*)(q_row + (size_t)h * DQK + ks * 16 + 8 * half);
      f[ks] = z;
    }
    L = qvalid ? lse_b[(size_t)h * S] : 0.f;
  };

  stage_bytes(scls[0], cls + ((size_t)b * NQ + qt0) * NK, kt_last + 1);
  stage_bytes(scls[1], cls + ((size_t)b * NQ + qt1) * NK, kt_last + 1);
  const uint64_t* bits_q = bits + ((size_t)b * S + (qvalid ? tq : 0)) * W;
  float* trow = teacher + ((size_t)b * S + (qvalid ? tq : 0)) * K;
  __syncthreads();  // class rows staged
  // the chunk's tiles that are non-empty for the workgroup: bit j for tile
  // kt_lo + j (uniform); tile_n(n) is the n-th of them
  int tmask = 0;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int kt = kt_lo + j;
    if (kt <= kt_last && (scls[0][kt] != 0 || scls[1][kt] != 0)) tmask |= 1 << j;
  }
  tmask = __builtin_amdgcn_readfirstlane(tmask);
  const int nt = __popc(tmask);
  auto tile_n = [&](int n) {
    int m = tmask, kt = kt_lo;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i == n) kt = kt_lo + __builtin_ctz(m | (1 << CH));
      m &= m - 1;
    }
    return kt;
  };
  const uint8_t* clsw = scls[qt_w - qt0];

  float acc[CH][2][16];
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][kb][r] = 0.f;

  if (nt > 0) {
    // step s = h * nt + j handles tile tl[j] of head h, from buffer s % NBK
    const int nsteps = H * nt;
    auto step_tile = [&](int s_) { return tile_n(s_ % nt); };
    auto step_head = [&](int s_) { return s_ / nt; };
    issue(step_tile(0), 0, 0);
    if (nsteps > 1) issue(step_tile(1), step_head(1), 1);
    u32x4 qf[KS];
    float Lh;
    load_q(0, qf, Lh);
    int s = 0;
    for (int h = 0; h < H; ++h) {
      const float Lc = Lh * 1.4426950408889634f;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        if (j < nt) {  // wave-uniform
          // this step's K tile (issued two steps back) and, at a head's first
          // tile, the head's q fragments; the next step's copies may still fly
          if (j == 0 || s + 1 >= nsteps)
            wait_vmem();
          else
            wait_vmem_n<KI>();
          lds_barrier();  // tile visible; every wave is done with the buffer step s+2 goes to
          if (s + 2 < nsteps) issue(step_tile(s + 2), step_head(s + 2), (s + 2) % NBK);
          const int kt = tile_n(j);
          if (clsw[kt] != 0) {
            const uint16_t* sK = smK[s % NBK];
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
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[j][kb][r] += fast_exp2(fmaf(sacc[kb][r], scale_log2, -Lc));
          }
          ++s;
        }
      }
      // the next head's fragments (waited for at its first tile)
      if (h + 1 < H) load_q(h + 1, qf, Lh);
    }
  }

  // kept keys of this row before the chunk, then the chunk's tiles in order:
  // the kept keys' mean at their ranks. Lane (half, col) holds keys
  // 32*kb + 8*(r/4) + 4*half + r%4 of a tile.
  int base = 0;
  if (qvalid)
    for (int w0 = 0; w0 < kt_lo; ++w0) base += __popcll(bits_q[w0]);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    if (j < nt) {
      const int kt = tile_n(j);
      const int cw = clsw[kt];
      const uint64_t wd = (!qvalid || cw == 0) ? 0ull : (cw == 2 ? ~0ull : bits_q[kt]);
      if (wd) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int pos = 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
            const int rank = base + __popcll(wd & ((1ull << pos) - 1ull));
            // a row keeps at most K keys when the mask came with K-wide lists; the check
            // keeps a narrower teacher buffer in bounds all the same
            if (((wd >> pos) & 1ull) && rank < K) trow[rank] = acc[j][kb][r] * inv_h;
          }
        base += __popcll(wd);
      }
    }
  }
  // the chunk with the diagonal has seen every kept key of its rows
  if (qvalid && c == c_last)
    for (int i = base; i < K; ++i) trow[i] = 0.f;
}

hipError_t launch_indexer_teacher(const void* q, const void* k, const float* lse, const uint64_t* bits,
                                  const uint8_t* cls, int B, int S, int H, int Dqk, int K, float scale,
                                  float* teacher, hipStream_t st) {
  const int nqw = (S + itc::QW - 1) / itc::QW;
  const int nch = ((S + itc::TK - 1) / itc::TK + itc::CH - 1) / itc::CH;
  const dim3 grid((unsigned)((size_t)nqw * nch * B)), block(itc::NW * 64);
  const float sl2 = scale * 1.4426950408889634f, ih = 1.f / (float)H;
#define DSA_TEACHER(D)                                                                                      \
  hipLaunchKernelGGL(indexer_teacher_kernel<D>, grid, block, 0, st, (const uint16_t*)q, (const uint16_t*)k, \
                     lse, bits, cls, B, S, H, K, sl2, ih, teacher)
  if (Dqk == 192)
    DSA_TEACHER(192);
  else if (Dqk == 128)
    DSA_TEACHER(128);
  else if (Dqk == 64)
    DSA_TEACHER(64);
  else
    return hipErrorInvalidValue;
#undef DSA_TEACHER
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Student softmax, KL and the gradient w.r.t. the scores
// ---------------------------------------------------------------------------
// N = rows with a non-empty index list, stored as float in loss2[1]
__global__ __launch_bounds__(1024) void indexer_kl_count_kernel(const int32_t* __restrict__ idx, int64_t nrows,
                                                                int K, float* __restrict__ loss2) {
  __shared__ uint32_t part[16];
  // 16 rows per thread and round trip: the loads of a batch are issued together
  uint32_t c = 0;
  for (int64_t i0 = 0; i0 < nrows; i0 += 16 * 1024) {
    int32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t i = i0 + (int64_t)u * 1024 + threadIdx.x;
      v[u] = i < nrows ? idx[i * K] : -1;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) c += v[u] >= 0 ? 1u : 0u;
  }
  c = wave_sum(c);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t n = 0;
    for (int i = 0; i < 16; ++i) n += part[i];
    loss2[1] = (float)n;
  }
}

// One wave per row. The index list holds the row's kept keys ascending, then
// -1 (as dsa_topk writes it); teacher entry j belongs to idx entry j.
template <typename ST>
__global__ __launch_bounds__(256) void indexer_kl_kernel(const ST* __restrict__ scores, int64_t ld,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ teacher,
                                                         const uint64_t* __restrict__ bits, int B, int S, int K,
                                                         const float* __restrict__ loss2, float* __restrict__ row_kl,
                                                         float* __restrict__ dscores, int64_t ld_ds) {
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (size_t)B * S) return;  // the whole wave leaves together
  const int t = (int)(row % S);
  const int W = (S + 63) / 64;
  const int32_t* irow = idx + row * K;
  const float* prow = teacher + row * K;
  const ST* srow = scores + row * ld;
  float* grow = dscores + row * ld_ds;
  const float N = loss2[1];
  const float invN = N > 0.f ? 1.f / N : 0.f;
  // The index list goes in batches of 64*U entries, U per lane: the U index
  // loads of a batch are issued together, then the U score gathers, so a
  // batch costs two memory round trips instead of two per entry.
  constexpr int U = 16;
  // pass 1: running max and sum of exp over the kept scores, per lane, then
  // combined over the wave
  float m = -INFINITY, z = 0.f;
  for (int j0 = 0; j0 < K; j0 += 64 * U) {
    int sj[U];
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 64 * u + lane;
      sj[u] = j < K ? irow[j] : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = (sj[u] >= 0 && sj[u] <= t) ? Elem<ST>::load(srow + sj[u]) : -INFINITY;
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) bm = fmaxf(bm, v[u]);
    const float mn = fmaxf(m, bm);
    if (mn != -INFINITY) {
      float add = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) add += expf(v[u] - mn);  // exp(-inf) = 0 for entries not kept
      z = z * expf(m - mn) + add;                          // m = -inf: z is still 0
      m = mn;
    }
  }
  const float M = wave_max(m);
  float kl = 0.f;
  if (M != -INFINITY) {
    const float logz = logf(wave_sumf(m == -INFINITY ? 0.f : z * expf(m - M)));
    // pass 2: KL terms and the gradient at the kept keys
    for (int j0 = 0; j0 < K; j0 += 64 * U) {
      int sj[U];
      float pj[U], v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + 64 * u + lane;
        sj[u] = j < K ? irow[j] : -1;
        pj[u] = j < K ? prow[j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = (sj[u] >= 0 && sj[u] <= t) ? Elem<ST>::load(srow + sj[u]) : 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (sj[u] < 0 || sj[u] > t) continue;  // kept keys lie in [0, t]
        const float logq = v[u] - M - logz;
        const float p = pj[u];
        if (p > 0.f) kl += p * (logf(p) - logq);
        grow[sj[u]] = (expf(logq) - p) * invN;
      }
    }
  }
  // zeros over [0, t] at the keys that are not kept: 64 mask words per load,
  // lane w holding word w0 + w
  const uint64_t* brow = bits + row * W;
  const int nwd = t / 64 + 1;
  for (int w0 = 0; w0 < nwd; w0 += 64) {
    const uint64_t bw = w0 + lane < nwd ? brow[w0 + lane] : 0ull;
    const int nw = min(64, nwd - w0);
    for (int w = 0; w < nw; ++w) {
      const uint64_t word = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bw >> 32), w) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bw, w);
      const int s = 64 * (w0 + w) + lane;
      if (s <= t && !((word >> lane) & 1ull)) grow[s] = 0.f;
    }
  }
  kl = wave_sumf(kl);
  if (lane == 0) row_kl[row] = kl;
}

// loss2[0] = sum of row_kl / N, summed in a fixed order
__global__ __launch_bounds__(1024) void indexer_kl_finalize_kernel(const float* __restrict__ row_kl, int64_t nrows,
                                                                   float* __restrict__ loss2) {
  __shared__ float part[1024];
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < nrows; i += 1024) s += row_kl[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float N = loss2[1];
    loss2[0] = N > 0.f ? part[0] / N : 0.f;
  }
}

hipError_t launch_indexer_kl(const void* scores, bool score_bf16, int64_t ld, const int32_t* idx,
                             const float* teacher, const uint64_t* bits, int B, int S, int K, float* row_kl,
                             float* loss2, float* dscores, int64_t ld_ds, hipStream_t st) {
  const int64_t nrows = (int64_t)B * S;
  hipLaunchKernelGGL(indexer_kl_count_kernel, dim3(1), dim3(1024), 0, st, idx, nrows, K, loss2);
  const dim3 grid((unsigned)((nrows + 3) / 4)), block(256);
  if (score_bf16)
    hipLaunchKernelGGL(indexer_kl_kernel<uint16_t>, grid, block, 0, st, (const uint16_t*)scores, ld, idx, teacher,
                       bits, B, S, K, loss2, row_kl, dscores, ld_ds);
  else
    hipLaunchKernelGGL(indexer_kl_kernel<float>, grid, block, 0, st, (const float*)scores, ld, idx, teacher, bits,
                       B, S, K, loss2, row_kl, dscores, ld_ds);
  hipLaunchKernelGGL(indexer_kl_finalize_kernel, dim3(1), dim3(1024), 0, st, row_kl, nrows, loss2);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Indexer backward (64 index heads of dim 128, bf16)
// ---------------------------------------------------------------------------
namespace ibw {
constexpr int HI = 64, DI = 128, HB = HI / 32, KS = DI / 16;
constexpr int SL = 20, PX = SL * 8;  // swizzled rows: 16 data + 4 pad slots (320 B)
constexpr int TK = 64;               // keys per tile (dq kernel)
constexpr int QPW = 8 / HB;          // queries per dq workgroup (8 waves = queries x head blocks)
constexpr int KB = 128;              // keys per dk workgroup (4 key blocks x 2 head blocks)
constexpr int NBUF = 3;              // dk stage buffers (copies two queries ahead)
}  // namespace ibw

// dq_idx and dw. Workgroup = (b, QPW consecutive queries); wave w takes query
// t0 + w / HB and heads 32 * (w % HB) .. +31.
__global__ __launch_bounds__(512) void indexer_bwd_dq_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const uint16_t* __restrict__ w,
    const float* __restrict__ dscores, int64_t ld, const uint8_t* __restrict__ cls, int B, int S,
    uint16_t* __restrict__ dq_idx, uint16_t* __restrict__ dw) {
  using namespace ibw;
  constexpr int NBLK = TK * SL / 64;          // 1 KB blocks per k_idx tile (20)
  constexpr int BI = (NBLK + 7) / 8;          // per wave (3): waves 4-7 copy two blocks and a gradient row
  static_assert(NBLK == 20 && QPW == 4, "copy slots: waves 0-3 take 3 blocks, waves 4-7 2 blocks + 1 row");
  __shared__ __attribute__((aligned(1024))) uint16_t smK[3][TK * PX];
  __shared__ __attribute__((aligned(16))) float smG[3][QPW][TK];  // the tile's gradient entries per query
  __shared__ uint8_t scls[kMaxTiles];                             // the query tile's class row

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int NQB = (S + QPW - 1) / QPW;
  const int b = (int)blockIdx.x % B;
  const int qb = NQB - 1 - (int)blockIdx.x / B;     // costliest first
  const int t0 = qb * QPW;
  const int t = t0 + wid / HB, hb = wid % HB;
  const bool qvalid = t < S;
  const int t_last = min(S - 1, t0 + QPW - 1);
  const int NQ = (S + 127) / 128, NK = (S + 63) / 64;
  const uint16_t* kbase = k_idx + (size_t)b * S * DI;

  // B operand of U^T = K Q^T: lane (half, col) holds q_idx[t, 32*hb + col, 16*ks + 8*half + 0..7]
  u32x4 qf[KS];
  float wl = 0.f;
  {
    const uint16_t* qr = q_idx + (((size_t)b * S + (qvalid ? t : 0)) * HI + hb * 32 + col) * DI;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (qvalid) z = *(const u32x4*)(qr + ks * 16 + 8 * half);
      qf[ks] = z;
    }
    if (qvalid) wl = bf2f(w[((size_t)b * S + t) * HI + hb * 32 + col]);
  }
  wait_vmem();  // once: q_idx fragments and the weight are in before the tile loop
  // swizzled copy of a 64-key tile: chunk c of row r at slot swz_chunk(r, c);
  // pad slots copy the row's last chunk; rows past S copy row S-1. Waves 4-7
  // also copy query (w - 4)'s gradient entries of the tile (keys past S copy
  // key S-1's; entries past the query are never used). Every copy goes through
  // the untracked path and every wave issues exactly three per tile, so a
  // counted wait finds one tile complete while the next is in flight.
  auto issue = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int blk = wid + i * 8;
      if (blk < NBLK) {
        const int slot = blk * 64 + lane, r = slot / SL, sl = slot % SL;
        // slot sl of row r holds chunk sl ^ ((r >> 2) & 3) (swz_chunk is an involution); pad slots the last chunk
        const int c = sl < DI / 8 ? swz_chunk(r, sl) : DI / 8 - 1;
        const int s = min(kt * TK + r, S - 1);
        g2lds16_async(kbase + (size_t)s * DI + c * 8, (char*)smK[buf] + blk * 1024);
      } else {
        const int qq = wid - 4, tt = min(t0 + qq, S - 1), s = min(kt * TK + lane, S - 1);
        g2lds4_async(dscores + ((size_t)b * S + tt) * ld + s, smG[buf][qq]);
      }
    }
  };

  f32x16 dqacc[DI / 32];
#pragma unroll
  for (int i = 0; i < DI / 32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dqacc[i][j] = 0.f;
  float dwacc = 0.f;

  const int kt_last = t_last / TK;
  // the QPW queries share one 128-query tile: its class row, staged in LDS
  stage_bytes(scls, cls + ((size_t)b * NQ + t0 / 128) * NK, kt_last + 1);
  __syncthreads();
  auto next_tile = [&](int kt) {
    int n = kt + 1;
    while (n <= kt_last && scls[n] == 0) ++n;
    return n;
  };
  // three tile buffers, copies two tiles ahead
  int kt = next_tile(-1);
  int kn = next_tile(kt);
  if (kt <= kt_last) issue(kt, 0);
  if (kn <= kt_last) issue(kn, 1);
  int buf = 0;
  while (kt <= kt_last) {
    const int kn2 = next_tile(kn);
    if (kn <= kt_last)
      wait_vmem_n<BI>();  // tile kt's copies are in; tile kn's (the last BI) may still fly
    else
      wait_vmem();
    lds_barrier();  // tile kt visible; every wave is done with the buffer tile kn2 goes to
    if (kn2 <= kt_last) issue(kn2, buf == 0 ? 2 : buf - 1);
    const uint16_t* sK = smK[buf];
    const float* gq = smG[buf][wid / HB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int s0 = kt * TK + kb * 32;
      if (!qvalid || s0 > t) continue;  // wave-uniform: the block lies past this query
      f32x16 u;
#pragma unroll
      for (int i = 0; i < 16; ++i) u[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) u = mfma32(lds_frag_x(sK, PX, kb * 32 + col, 2 * ks + half), qf[ks], u);
      // lane (half, col): keys s0 + 8*i + 4*half + j (r = 4i + j); only [0, t] of the row is written
      float g[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 gv = *(const f32x4*)(gq + kb * 32 + 8 * i + 4 * half);
#pragma unroll
        for (int j = 0; j < 4; ++j) g[4 * i + j] = gv[j];
      }
      if (s0 + 31 > t) {  // wave-uniform: only the diagonal block has keys past the query
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (s0 + 8 * (r >> 2) + 4 * half + (r & 3) > t) g[r] = 0.f;
      }
      float G[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dwacc = fmaf(g[r], fmaxf(u[r], 0.f), dwacc);
        G[r] = u[r] > 0.f ? g[r] * wl : 0.f;
      }
      // dq^T[d, head] += K^T[d, key] G^T[key, head], keys permuted inside each 16-key step
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        const u32x4 gb = pack8(G + 8 * p2);
        const int r0 = kb * 32 + 16 * p2 + 4 * half;
#pragma unroll
        for (int db = 0; db < DI / 32; ++db) dqacc[db] = mfma32(lds_tr_frag_x(sK, PX, r0, r0 + 8, db * 32), gb, dqacc[db]);
      }
    }
    buf = buf == 2 ? 0 : buf + 1;
    kt = kn;
    kn = kn2;
  }
  dwacc = half_sum(dwacc);
  if (qvalid) {
    uint16_t* dqr = dq_idx + (((size_t)b * S + t) * HI + hb * 32 + col) * DI;
#pragma unroll
    for (int db = 0; db < DI / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * half;
        *(u32x2*)(dqr + d) = u32x2{pack_bf2(dqacc[db][4 * g4], dqacc[db][4 * g4 + 1]),
                                   pack_bf2(dqacc[db][4 * g4 + 2], dqacc[db][4 * g4 + 3])};
      }
    if (half == 0) dw[((size_t)b * S + t) * HI + hb * 32 + col] = f2bf(dwacc);
  }
}

// dk_idx, partial sums. Workgroup = (b, 128 keys, query segment qs): the
// queries are split into absolute segments [qs*qseg, (qs+1)*qseg) across
// workgroups, so no workgroup walks a whole causal column alone, and the
// workgroups of one (b, qs) -- every key block that segment reaches -- are
// adjacent in the XCD-remapped block order: they run together on one XCD and
// read the same q_idx rows, mostly from its L2. 8 waves: wave w takes keys
// 32*(w%4) .. and heads 32*(w/4) ..; per query, q_idx[t] (64 x 128, swizzled),
// w[t] and the gradient row's 128 entries are staged in LDS, three queries
// deep. Query tiles that are EMPTY for both of the workgroup's key tiles are
// skipped. Each wave writes its float32 partial dk (its keys, its 32 heads, its
// segment) to `part`; indexer_bwd_dk_combine_kernel adds them in a fixed order.
__global__ __launch_bounds__(512) void indexer_bwd_dk_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const uint16_t* __restrict__ w,
    const float* __restrict__ dscores, int64_t ld, const uint8_t* __restrict__ cls, int B, int S, int qseg,
    float* __restrict__ part) {
  using namespace ibw;
  constexpr int QBLK = HI * SL / 64;   // 1 KB blocks of a staged q_idx[t] (20)
  // copies per wave per query: 20 q blocks over 8 waves (3, 3, 3, 3, 2, 2, 2, 2), then
  // waves 4-5 the gradient entries (2 x 64 floats), wave 6 the weights, wave 7 a filler
  constexpr int NCP = 3;
  // NBUF stages of two queries each (one barrier per pair)
  __shared__ __attribute__((aligned(1024))) uint16_t smQ[NBUF][2][HI * PX];
  __shared__ __attribute__((aligned(16))) float smG[NBUF][2][KB];
  __shared__ __attribute__((aligned(16))) uint16_t smW[NBUF][2][128];  // 64 weights (+ filler room)
  __shared__ uint16_t qlist[kMaxS / 128];
  __shared__ int s_nq;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int kbk = wid & 3, hb = wid >> 2;
  const int NSEG = (S + qseg - 1) / qseg, nkb = (S + KB - 1) / KB;
  const int Lb = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int kblk = Lb % nkb;
  const int qs = (Lb / nkb) % NSEG;
  const int b = Lb / (nkb * NSEG);
  const int k0 = kblk * KB;
  // this workgroup's queries: [q_lo, (qs+1)*qseg) ∩ [0, S); both ends multiples of 128 or S
  const int q_lo = max(k0, qs * qseg);
  if (q_lo >= min(S, (qs + 1) * qseg)) return;        // whole workgroup: no query of the segment reaches the keys
  const int seg = qs - k0 / qseg;                      // the partial's index among key block k0's segments
  const int sk = k0 + kbk * 32 + col;                  // this lane's key
  const bool kvalid = sk < S;
  const int NQ = (S + 127) / 128, NK = (S + 63) / 64;
  const int kt0 = k0 / 64, kt1 = min(NK - 1, kt0 + 1);

  // B operand of U = Q_t K^T: lane (half, col) holds k_idx[sk, 16*ks + 8*half + 0..7]
  u32x4 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (kvalid) z = *(const u32x4*)(k_idx + ((size_t)b * S + sk) * DI + ks * 16 + 8 * half);
    kf[ks] = z;
  }
  // once: the loop's counted waits then only concern the staging copies (which
  // the compiler does not track), and it adds no wait of its own for kf
  wait_vmem();
  // the segment's query tiles that are non-empty for one of the two key tiles
  const int qt_hi = min(NQ, (qs + 1) * qseg / 128);
  if (wid == 0) {
    int cnt = 0;
    for (int base = q_lo / 128; base < qt_hi; base += 64) {
      const int qt = base + lane;
      bool ne = false;
      if (qt < qt_hi) {
        const uint8_t* c = cls + ((size_t)b * NQ + qt) * NK;
        ne = c[kt0] != 0 || c[kt1] != 0;
      }
      const uint64_t m = __ballot(ne);
      if (ne) qlist[cnt + lanes_below(m)] = (uint16_t)qt;
      cnt += __popcll(m);
    }
    if (lane == 0) s_nq = cnt;
  }
  __syncthreads();
  const int nq = s_nq;
  // the queries, in order: every query of the listed 128-query tiles (k0 is a
  // multiple of 128, so the first listed tile starts at or after the keys);
  // the query after tt, moving to the next listed tile at a tile end or at S
  auto advance = [&](int& qi, int tt) __attribute__((always_inline)) -> int {
    const int n = tt + 1;
    if ((n & 127) != 0 && n < S) return n;
    ++qi;
    return qi < nq ? 128 * (int)qlist[qi] : -1;
  };
  // this wave's copy slots, fixed per wave: q blocks, then g / w / filler.
  // Each slot's per-lane byte offset is fixed, so it is formed once; per
  // query only the scalar row bases change.
  uint32_t coff[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int blk = wid + 8 * i;
    if (blk < QBLK) {
      const int slot = blk * 64 + lane, r = slot / SL, sl = slot % SL;
      // slot sl of row r holds chunk sl ^ ((r >> 2) & 3) (swz_chunk is an involution); pad slots the last chunk
      const int c = sl < DI / 8 ? swz_chunk(r, sl) : DI / 8 - 1;
      coff[i] = (uint32_t)((r * DI + c * 8) * 2);
    } else if (blk == QBLK + 0 || blk == QBLK + 1) {
      coff[i] = (uint32_t)min(k0 + 64 * (blk - QBLK) + lane, S - 1) * 4u;
    } else if (blk == QBLK + 2) {
      coff[i] = (uint32_t)(2 * (lane & 31)) * 2u;  // 64 bf16 weights: lanes 32-63 repeat lanes 0-31
    } else {
      coff[i] = (uint32_t)min(k0 + lane, S - 1) * 4u;  // filler: the same data as the first gradient slot
    }
  }
  auto issue = [&](int tt, int bi, int k) __attribute__((always_inline)) {
    const size_t row = (size_t)b * S + tt;
    const uint16_t* qs = uniform_ptr(q_idx + row * HI * DI);
    const float* gs = uniform_ptr(dscores + row * ld);
    const uint16_t* ws = uniform_ptr(w + row * HI);
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int blk = wid + 8 * i;
      if (blk < QBLK)
        g2lds16_async_off(qs, coff[i], (char*)smQ[bi][k] + blk * 1024);
      else if (blk == QBLK + 0 || blk == QBLK + 1)
        g2lds4_async_off(gs, coff[i], smG[bi][k] + 64 * (blk - QBLK));
      else if (blk == QBLK + 2)
        g2lds4_async_off(ws, coff[i], smW[bi][k]);
      else
        g2lds4_async_off(gs, coff[i], smG[bi][k]);
    }
  };
  static_assert(QBLK + 3 <= 8 * NCP, "copy slots");

  f32x16 dkacc[DI / 32];
#pragma unroll
  for (int i = 0; i < DI / 32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dkacc[i][j] = 0.f;

  // the queries in pairs, in order; a stage holds a pair, copies run two pairs
  // ahead. A pair with one query copies it twice, so that every wave issues
  // exactly 2 * NCP copies per stage.
  int qiC = 0;
  auto next_q = [&](int tt) __attribute__((always_inline)) -> int { return tt >= 0 ? advance(qiC, tt) : -1; };
  auto issue2 = [&](int t0, int t1, int bi) __attribute__((always_inline)) {
    issue(t0, bi, 0);
    issue(t1 >= 0 ? t1 : t0, bi, 1);
  };
  // one query of the stage in buffer bi, slot k
  auto compute = [&](int tq, int bi, int k) __attribute__((always_inline)) {
    const uint16_t* sQ = smQ[bi][k];
    // U[head, key] = q_idx[t, head] . k_idx[key]: heads on rows (this wave's
    // 32-head block), keys on columns
    if (k0 + kbk * 32 <= tq) {  // wave-uniform: some of the wave's keys are at or before the query
      f32x16 u;
#pragma unroll
      for (int i = 0; i < 16; ++i) u[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) u = mfma32(lds_frag_x(sQ, PX, hb * 32 + col, 2 * ks + half), kf[ks], u);
      const float g = sk <= tq ? smG[bi][k][kbk * 32 + col] : 0.f;
      // accumulator rows 4i .. 4i+3 are heads hb*32 + 8i + 4*half + 0..3: one 8-byte read each
      float G[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x2 wv = *(const u32x2*)(smW[bi][k] + hb * 32 + 8 * i + 4 * half);
        const float wr[4] = {__uint_as_float(wv[0] << 16), __uint_as_float(wv[0] & 0xffff0000u),
                             __uint_as_float(wv[1] << 16), __uint_as_float(wv[1] & 0xffff0000u)};
#pragma unroll
        for (int j = 0; j < 4; ++j) G[4 * i + j] = u[4 * i + j] > 0.f ? g * wr[j] : 0.f;
      }
      // dk^T[d, key] += q_idx[t]^T[d, head] G[head, key], heads permuted inside each 16-head step
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        const u32x4 gb = pack8(G + 8 * p2);
        const int r0 = hb * 32 + 16 * p2 + 4 * half;
#pragma unroll
        for (int db = 0; db < DI / 32; ++db) dkacc[db] = mfma32(lds_tr_frag_x(sQ, PX, r0, r0 + 8, db * 32), gb, dkacc[db]);
      }
    }
  };
  int a0 = nq > 0 ? 128 * (int)qlist[0] : -1;
  int a1 = next_q(a0);
  int b0 = next_q(a1), b1 = next_q(b0);
  int c0 = next_q(b1), c1 = next_q(c0);
  if (a0 >= 0) issue2(a0, a1, 0);
  if (b0 >= 0) issue2(b0, b1, 1);
  int bi = 0;
  while (a0 >= 0) {
    if (b0 >= 0)
      wait_vmem_n<2 * NCP>();  // pair a's copies done; pair b's may still fly
    else
      wait_vmem();
    lds_barrier();
    if (c0 >= 0) issue2(c0, c1, (bi + 2) % NBUF);
    compute(a0, bi, 0);
    if (a1 >= 0) compute(a1, bi, 1);
    bi = (bi + 1) % NBUF;
    a0 = b0;
    a1 = b1;
    b0 = c0;
    b1 = c1;
    c0 = next_q(c1);
    c1 = next_q(c0);
  }
  wait_vmem();
  // partial [(seg * 2 + hb)][b][key][d] (float32), zeros where nothing was added
  if (kvalid) {
    float* pr = part + (((size_t)(seg * 2 + hb) * B + b) * S + sk) * DI;
#pragma unroll
    for (int db = 0; db < DI / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(f32x4*)(pr + db * 32 + 8 * g4 + 4 * half) =
            f32x4{dkacc[db][4 * g4], dkacc[db][4 * g4 + 1], dkacc[db][4 * g4 + 2], dkacc[db][4 * g4 + 3]};
  }
}

// dk_idx[b, s, :] = the sum of the partials of key s's segments and head
// blocks, in a fixed order; one thread per 4 dims
__global__ __launch_bounds__(256) void indexer_bwd_dk_combine_kernel(const float* __restrict__ part, int B, int S,
                                                                     int qseg, uint16_t* __restrict__ dk_idx) {
  using namespace ibw;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)B * S * (DI / 4)) return;
  const int d4 = (int)(i % (DI / 4));
  const size_t bs = i / (DI / 4);
  const int s = (int)(bs % S), b = (int)(bs / S);
  const int k0 = s / KB * KB;
  const int nseg = (S + qseg - 1) / qseg - k0 / qseg;  // segments that reach key s's block
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < 2 * nseg; ++j) {
    const f32x4 v = *(const f32x4*)(part + (((size_t)j * B + b) * S + s) * DI + 4 * d4);
    acc += v;
  }
  *(u32x2*)(dk_idx + bs * DI + 4 * d4) = u32x2{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3])};
}

hipError_t launch_indexer_bwd(const void* q_idx, const void* k_idx, const void* w, const float* dscores, int64_t ld,
                              const uint8_t* cls, int B, int S, void* dq_idx, void* dk_idx, void* dw,
                              hipStream_t st) {
  using namespace ibw;
  // dk first: its float32 partials (2 head blocks x nseg query segments, 1 KB
  // per key each) are staged in dq_idx's memory (16 KB per query), which the
  // dq kernel then overwrites; nseg <= 16 keeps them inside it
  const int qseg = max(512, ((S + 15) / 16 + 127) / 128 * 128);
  const int nseg = (S + qseg - 1) / qseg;
  const int nkb = (S + KB - 1) / KB;
  float* part = (float*)dq_idx;
  hipLaunchKernelGGL(indexer_bwd_dk_kernel, dim3((unsigned)((size_t)nkb * nseg * B)), dim3(512), 0, st,
                     (const uint16_t*)q_idx, (const uint16_t*)k_idx, (const uint16_t*)w, dscores, ld, cls, B, S, qseg,
                     part);
  const size_t nthr = (size_t)B * S * (DI / 4);
  hipLaunchKernelGGL(indexer_bwd_dk_combine_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, st, part, B,
                     S, qseg, (uint16_t*)dk_idx);
  const int nqb = (S + QPW - 1) / QPW;
  hipLaunchKernelGGL(indexer_bwd_dq_kernel, dim3((unsigned)(nqb * B)), dim3(512), 0, st, (const uint16_t*)q_idx,
                     (const uint16_t*)k_idx, (const uint16_t*)w, dscores, ld, cls, B, S, (uint16_t*)dq_idx,
                     (uint16_t*)dw);
  return hipGetLastError();
}

}  // namespace dsa
