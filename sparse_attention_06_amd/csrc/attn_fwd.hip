// Block-sparse flash-attention forward over the DSA selection mask (gfx950).
//
// Source: "Support Ring Attention with DeepSeek DSA Sparse Indexer", Forward
// Flow (one [batch, S, S] index mask for all heads, combined with causal; on
// kept entries the logit is the scaled query-key product, others drop out);
// "Integrate DeepSeek Sparse Attention with Tokamax Flash Attention",
// Description (flash attention driven by a dynamic 3-D index mask).
//
// Keys may be compressed blocks ("Add Flash Attention Support to Deepseek v4",
// Description): Sk keys, key s visible to query t when s <= (t + 1) / ratio -
// 1; the mask rows are then ceil(Sk / 64) words. ratio 1 and Sk = S is DSA.
//
// MFMA kernel (bf16, Dqk = 192, Dv = 128). A workgroup is one (b, h, 256-query
// block) with 8 waves of 32 queries each, two waves per SIMD. It walks the
// 64-key tiles that are non-empty for either of its two 128-query tiles; the
// list of them is compacted into LDS once at start, so the walk costs one LDS
// read per tile, issued a tile ahead. PARTIAL tiles read one u64 selection
// word per query (loaded unconditionally a tile ahead, the tile class applied
// where the word is used, so no branch ever joins on a pending load).
//   S^T = K Q^T: keys on MFMA rows, queries on columns, so each lane owns one
//   query and 16 logits of each 32-key block. Max and sum are in-lane, with
//   one exchange between lane halves. Q stays in VGPRs.
//   O^T += V^T P^T: probabilities go straight from the S^T accumulator into
//   the B operand, with the key order inside each 16-key step permuted to
//   match; V^T comes through the transposing LDS read with the same order.
// Each wave software-pipelines its 32-key blocks: while the MFMAs of block
// i+1's scores run, the VALU forms block i's probabilities; while block i's
// PV MFMAs run, block i+1 is masked and its max taken. Hard scheduling fences
// hold that interleave (six groups of two score MFMAs, four of two PV MFMAs).
// The online-softmax reference max is updated per block, lazily: O and l are
// rescaled only when a block max passes it by more than 2^8.
// K tiles are double buffered and V tiles triple buffered, both copied two
// tiles ahead by direct global->LDS copies spread over the score groups of the
// step after the tile barrier; one barrier per tile. Tiles are unpadded
// (384-byte K rows, 256-byte V rows) with XOR-swizzled 16-byte chunks (K:
// chunk ^ ((row >> 1) & 7); V: chunk ^ 4 * (row & 3)) that keep the K row
// reads and the V transposing reads free of bank conflicts, so a tile is a
// whole number of 1 KB copy blocks per wave (3 K + 2 V). exp2 is the hardware
// v_exp_f32 with the scale folded in (scale * log2 e).
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

namespace fwd {
constexpr int DQK = 192, DV = 128, TK = 64;
constexpr int NW = 8;                // waves per workgroup: two per SIMD
constexpr int QW = 32 * NW;          // queries per workgroup (two 128-query tiles)
constexpr int KS = DQK / 16;         // k steps of S^T
constexpr int KCH = DQK / 8, VCH = DV / 8;  // 16-byte chunks per K row (24) and V row (16), unpadded
constexpr int KBLK = TK * KCH / 64, VBLK = TK * VCH / 64;  // 1 KB blocks per tile: 24, 16
constexpr int KC = KBLK / NW, VC = VBLK / NW;  // copies per wave: 3 K, 2 V
constexpr int NC = KC + VC;
constexpr int KBUF = 2, VBUF = 3;    // K tiles double, V tiles triple buffered
static_assert(KBLK % NW == 0 && VBLK % NW == 0, "copies split evenly over the waves");
// swizzles: physical 16-byte chunk of logical chunk c in row r
__device__ __forceinline__ constexpr int kswz(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ constexpr int vswz(int r, int c) { return c ^ (4 * (r & 3)); }
}  // namespace fwd

__global__ __launch_bounds__(fwd::NW * 64) void attn_fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint64_t* __restrict__ bits, const uint8_t* __restrict__ cls, int B, int S, int Sk, int ratio, int H,
    float scale_log2, uint16_t* __restrict__ o, float* __restrict__ lse) {
  using namespace fwd;
  __shared__ __attribute__((aligned(1024))) uint16_t smK[KBUF][KBLK * 512];
  __shared__ __attribute__((aligned(1024))) uint16_t smV[VBUF][VBLK * 512];
  __shared__ uint8_t scls[2][kMaxTiles];
  __shared__ uint32_t tlist[kMaxTiles + 2];  // non-empty tiles: kt | class0 << 16 | class1 << 24
  __shared__ int s_ntl;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int W = (Sk + 63) / 64, NQ = (S + 127) / 128, NK = W;
  const int NQW = (S + QW - 1) / QW;
  int bh, qw;
  grouped_order(xcd_remap((int)blockIdx.x, (int)gridDim.x), NQW, B * H, bh, qw);
  const int b = bh / H, h = bh % H;
  const int tq = qw * QW + wid * 32 + col;
  const bool qvalid = tq < S;
  const int qt_w = min(NQ - 1, (qw * QW + wid * 32) / 128);
  const int qt0 = qw * QW / 128, qt1 = min(NQ - 1, qt0 + 1);
  const size_t rs_qk = (size_t)H * DQK, rs_v = (size_t)H * DV;
  const uint16_t* kbase = k + (size_t)b * Sk * rs_qk + (size_t)h * DQK;
  const uint16_t* vbase = v + (size_t)b * Sk * rs_v + (size_t)h * DV;

  // copy c < KC moves K block wid + 8c, copy KC + c' V block wid + 8c'. Lane l
  // fills LDS slot 64*blk + l, i.e. row slot / chunks-per-row at physical chunk
  // slot % chunks-per-row, from the logical chunk the swizzle puts there.
  auto copy_row = [&](int c) -> int {
    const int blk = wid + NW * (c < KC ? c : c - KC);
    return c < KC ? (blk * 64 + lane) / KCH : (blk * 64 + lane) / VCH;
  };
  auto copy_off = [&](int c, int row) -> uint32_t {
    const int blk = wid + NW * (c < KC ? c : c - KC);
    if (c < KC) {
      const int pc = (blk * 64 + lane) % KCH;
      return (uint32_t)((row * rs_qk + kswz(row, pc) * 8) * 2);
    }
    const int pc = (blk * 64 + lane) % VCH;
    return (uint32_t)((row * rs_v + vswz(row, pc) * 8) * 2);
  };
  uint32_t coff[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) coff[c] = copy_off(c, copy_row(c));
  // copy c of the tile whose K/V rows start at ksrc / vsrc; lim is the tile's
  // last in-range row. On a ragged last tile, rows past it copy from row lim
  // (finite data under keys that every mask drops)
  auto copy = [&](int c, const uint16_t* ksrc, const uint16_t* vsrc, int lim, uint16_t* kdst, uint16_t* vdst)
      __attribute__((always_inline)) {
    uint32_t off = coff[c];
    if (lim < TK - 1) {  // wave-uniform, rare: recomputed here, never hoisted into live registers
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int blk = wid + NW * (c < KC ? c : c - KC);
      const int slot = blk * 64 + ln;
      const int row = c < KC ? slot / KCH : slot / VCH;
      const int r = min(row, lim);
      off = c < KC ? (uint32_t)((r * rs_qk + kswz(row, slot % KCH) * 8) * 2)
                   : (uint32_t)((r * rs_v + vswz(row, slot % VCH) * 8) * 2);
    }
    if (c < KC)
      g2lds16_async_off(ksrc, off, (char*)kdst + (wid + NW * c) * 1024);
    else
      g2lds16_async_off(vsrc, off, (char*)vdst + (wid + NW * (c - KC)) * 1024);
  };

  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qvalid) z = *(const u32x4*)(q + ((size_t)b * S + tq) * rs_qk + (size_t)h * DQK + ks * 16 + 8 * half);
    qf[ks] = z;
  }

  float m = -INFINITY, l = 0.f, neg_m = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[eb][i] = 0.f;

  // last key tile any of the workgroup's queries sees (-1: none)
  const int kl_last = (min(S - 1, qw * QW + QW - 1) + 1) / ratio - 1;
  const int kt_last = kl_last < 0 ? -1 : kl_last / TK;
  stage_bytes(scls[0], cls + ((size_t)b * NQ + qt0) * NK, kt_last + 1);
  stage_bytes(scls[1], cls + ((size_t)b * NQ + qt1) * NK, kt_last + 1);
  const uint8_t* cls0 = scls[0];
  const uint8_t* cls1 = scls[1];
  const uint64_t* bits_q = bits + ((size_t)b * S + (qvalid ? tq : 0)) * W;
  // this lane's selection word of a tile is loaded unconditionally (clamped
  // index) and its class applied where it is used, so no branch joins on a
  // pending load: sel 0 = no key kept, 1 = all kept (FULL), 2 = the loaded word
  const int qsh = 16 + 8 * (qt_w - qt0);
  auto word_raw = [&](int kt) -> uint64_t { return bits_q[min(kt, kt_last)]; };
  auto word_sel = [&](uint32_t ent) -> int {
    const int c = (int)((ent >> qsh) & 0xff);
    return !qvalid || (int)(ent & 0xffff) > kt_last || c == 0 ? 0 : c == 2 ? 1 : 2;
  };
  auto word_of = [&](uint64_t raw, int sel) -> uint64_t { return sel == 2 ? raw : sel == 1 ? ~0ull : 0ull; };
  auto issue_tile = [&](int kt, uint16_t* kdst, uint16_t* vdst) __attribute__((always_inline)) {
    const uint16_t* ks = uniform_ptr(kbase + (size_t)kt * TK * rs_qk);
    const uint16_t* vs = uniform_ptr(vbase + (size_t)kt * TK * rs_v);
    const int lim = Sk - 1 - kt * TK;
#pragma unroll
    for (int c = 0; c < NC; ++c) copy(c, ks, vs, lim, kdst, vdst);
  };

  // logits r0..r0+3 of a 32-key block masked (keep ? x : -inf), with the running max
  auto mask_max = [&](f32x16& s, uint64_t mw, int kb, int r0, float (&tm)[4]) __attribute__((always_inline)) {
    const uint32_t w = (uint32_t)((mw >> (4 * half)) >> (32 * kb));
#pragma unroll
    for (int r = r0; r < r0 + 4; ++r) {
      const int keep = __builtin_amdgcn_sbfe((int)w, 8 * (r >> 2) + (r & 3), 1);
      const float x = __int_as_float((keep & __float_as_int(s[r])) | (~keep & (int)0xff800000u));
      s[r] = x;
      tm[r & 3] = fmaxf(tm[r & 3], x);
    }
  };
  // lazy max: O and l are rescaled only when a block max passes the reference max by more than 2^8
  auto bump = [&](float tmax) __attribute__((always_inline)) {
    const bool bq = tmax > m + 8.f;
    if (__ballot(bq)) {
      const float m_new = bq ? tmax : m;
      const float alpha = bq ? fast_exp2(m - m_new) : 1.f;
      l *= alpha;
#pragma unroll
      for (int eb = 0; eb < 4; ++eb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[eb][i] *= alpha;
      m = m_new;
    }
    neg_m = m == -INFINITY ? 0.f : -m;
  };
  // LDS fragment reads: a per-lane base (one per k step mod 4 for K, one per
  // 32-dim block for V, the swizzle folded in) plus a constant offset
  const int g_k = (col >> 1) & 7;
  int kb4[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) kb4[bb] = col * DQK + 8 * ((2 * bb + half) ^ g_k);
  const int jj = lane & 15, rr = jj >> 2;
  int vb4[4];
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
    vb4[eb] = (4 * half + rr) * DV + 8 * (4 * (eb ^ rr) + 2 * ((lane >> 4) & 1) + ((jj & 3) >> 1)) + 4 * (jj & 1);
  // S^T A fragment: keys kb*32 + col, dims 16ks + 8*half ..
  auto kread = [&](const uint16_t* sK, int ks, int kb) __attribute__((always_inline)) -> u32x4 {
    return *(const u32x4*)(sK + kb4[ks & 3] + kb * 32 * DQK + 64 * (ks >> 2));
  };
  // V^T fragment for keys kb*32 + 16*p2 + {4h..4h+3, 8+4h..8+4h+3} (h the lane half), dims eb*32..
  auto vread = [&](const uint16_t* sV, int kb, int p2, int eb) __attribute__((always_inline)) -> u32x4 {
    const uint16_t* base = sV + vb4[eb] + (kb * 32 + 16 * p2) * DV;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)base);
    const v4i16 bb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base + 8 * DV));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, bb);
    return u32x4{ua[0], ua[1], ub[0], ub[1]};
  };

  u32x4 pf[2];
  float ls[4];
  // probabilities of 8 logits (p2 half, c8 in [c0, c0+4)) of a block
  auto soft4 = [&](const f32x16& sc, int p2, int c0, float (&pv8)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int c8 = c0; c8 < c0 + 4; ++c8) {
      pv8[c8] = fast_exp2(fmaf(sc[8 * p2 + c8], scale_log2, neg_m));
      ls[c8 & 3] += pv8[c8];
    }
  };
  auto pack = [&](int p2, const float (&pv8)[8]) __attribute__((always_inline)) {
    pf[p2] = u32x4{pack_bf2(pv8[0], pv8[1]), pack_bf2(pv8[2], pv8[3]), pack_bf2(pv8[4], pv8[5]),
                   pack_bf2(pv8[6], pv8[7])};
  };

  f32x16 S0, S1;
  u32x4 ka[2], vf[2];
  float pvA[8], pvB[8];
  __syncthreads();  // class rows staged
  if (wid == 0) {   // compact the tiles that are non-empty for either query tile
    int cnt = 0;
    for (int base = 0; base <= kt_last; base += 64) {
      const int kt = base + lane;
      const int c0 = kt <= kt_last ? cls0[kt] : 0, c1 = kt <= kt_last ? cls1[kt] : 0;
      const bool ne = (c0 | c1) != 0;
      const uint64_t mb = __ballot(ne);
      if (ne) tlist[cnt + lanes_below(mb)] = (uint32_t)kt | ((uint32_t)c0 << 16) | ((uint32_t)c1 << 24);
      cnt += __popcll(mb);
    }
    if (lane < 2) tlist[cnt + lane] = (uint32_t)(kt_last + 1);  // two sentinels: past the last tile
    if (lane == 0) s_ntl = cnt;
  }
  __syncthreads();
  const int ntl = s_ntl;
  if (ntl == 0) {
    if (qvalid) {
      uint16_t* orow = o + ((size_t)b * S + tq) * rs_v + (size_t)h * DV;
#pragma unroll
      for (int eb = 0; eb < 4; ++eb)
#pragma unroll
        for (int g = 0; g < 4; ++g) *(u32x2*)(orow + eb * 32 + 8 * g + 4 * half) = u32x2{0u, 0u};
      if (half == 0) lse[((size_t)b * H + h) * S + tq] = -INFINITY;
    }
    return;
  }
  uint32_t e_c = tlist[0], e_n = tlist[1];
  int kc = (int)(e_c & 0xffff), kn = (int)(e_n & 0xffff);
  int jpos = 0;  // position of tile kc in the workgroup's tile list
  issue_tile(kc, smK[0], smV[0]);
  if (kn <= kt_last) issue_tile(kn, smK[1], smV[1]);
  uint64_t raw_c = word_raw(kc), raw_n = word_raw(kn);
  int sel_c = word_sel(e_c), sel_n = word_sel(e_n);
  wait_vmem();
  lds_barrier();
  const uint64_t mw_c0 = word_of(raw_c, sel_c);
  // block (0, 0): scores, mask, max
  {
#pragma unroll
    for (int i = 0; i < 16; ++i) S0[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) S0 = mfma32(kread(smK[0], ks, 0), qf[ks], S0);
    float tm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += 4) mask_max(S0, mw_c0, 0, r0, tm);
    bump(half_max(fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]))) * scale_log2);
  }

  // One pipeline step: probabilities of block Sc (in pvA/pvB, then pf) while
  // the scores of the next block (key half kbn of the K tile at sKn) go into
  // Sn; then O += V^T P^T of block Sc (key half kbc of the V tile at sVc)
  // while Sn is masked with word mwn and its max taken. `cp(g)` issues the
  // tile copies of score group g.
  auto step = [&](f32x16& Sc, f32x16& Sn, const uint16_t* sKn, int kbn, uint64_t mwn, const uint16_t* sVc,
                  int kbc, auto cp) __attribute__((always_inline)) {
    ls[0] = ls[1] = ls[2] = ls[3] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) Sn[i] = 0.f;
    ka[0] = kread(sKn, 0, kbn);
    ka[1] = kread(sKn, 1, kbn);
    __builtin_amdgcn_sched_barrier(0);
    // phase 1: 6 groups of 2 score MFMAs; probabilities in slices of 4
#pragma unroll
    for (int g = 0; g < 6; ++g) {
      cp(g);
      Sn = mfma32(ka[0], qf[2 * g], Sn);
      if (2 * g + 2 < KS) ka[0] = kread(sKn, 2 * g + 2, kbn);
      Sn = mfma32(ka[1], qf[2 * g + 1], Sn);
      if (2 * g + 3 < KS) ka[1] = kread(sKn, 2 * g + 3, kbn);
      if (g < 2) soft4(Sc, 0, 4 * (g & 1), pvA);
      else if (g < 4) soft4(Sc, 1, 4 * (g & 1), pvB);
      if (g == 1) pack(0, pvA);
      if (g == 3) pack(1, pvB);
      if (g == 5) {
        vf[0] = vread(sVc, kbc, 0, 0);
        vf[1] = vread(sVc, kbc, 0, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase 2: 4 groups of 2 PV MFMAs; masks and max of the next block
    float tm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int p2 = g >> 1, e0 = 2 * (g & 1);
      oacc[e0] = mfma32(vf[0], pf[p2], oacc[e0]);
      if (g + 1 < 4) vf[0] = vread(sVc, kbc, (g + 1) >> 1, 2 * ((g + 1) & 1));
      oacc[e0 + 1] = mfma32(vf[1], pf[p2], oacc[e0 + 1]);
      if (g + 1 < 4) vf[1] = vread(sVc, kbc, (g + 1) >> 1, 2 * ((g + 1) & 1) + 1);
      mask_max(Sn, mwn, kbn, 4 * g, tm);
      __builtin_amdgcn_sched_barrier(0);
    }
    l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    bump(half_max(fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]))) * scale_log2);
  };
  auto no_cp = [](int) {};

  for (;;) {
    const uint16_t* sKc = smK[jpos & 1];
    const uint16_t* sKn = smK[(jpos + 1) & 1];
    const uint16_t* sVc = smV[jpos % 3];
    const uint32_t e_nn = tlist[min(jpos + 2, ntl + 1)];  // read early; used after the barrier
    // step (j, 0): scores of key half 1 of tile j, probabilities and O of half 0
    step(S0, S1, sKc, 1, word_of(raw_c, sel_c), sVc, 0, no_cp);
    const bool has_n = kn <= kt_last;
    // every wave is done with K(j) and V(j-1); K(j+1) and V(j+1) have landed
    wait_vmem();
    lds_barrier();
    const int knn = (int)(__builtin_amdgcn_readfirstlane((int)e_nn) & 0xffff);
    const uint64_t raw_nn = word_raw(knn);
    const int sel_nn = word_sel(e_nn);
    // copies of tile j+2 (when there is none, of tile j again: valid memory,
    // into buffers that are not read again)
    const int kcp = knn <= kt_last ? knn : kc;
    const uint16_t* ks = uniform_ptr(kbase + (size_t)kcp * TK * rs_qk);
    const uint16_t* vs = uniform_ptr(vbase + (size_t)kcp * TK * rs_v);
    const int lim = Sk - 1 - kcp * TK;
    uint16_t* kd = smK[jpos & 1];
    uint16_t* vd = smV[(jpos + 2) % 3];
    auto cp = [&](int g) __attribute__((always_inline)) { if (g < NC) copy(g, ks, vs, lim, kd, vd); };
    // step (j, 1): scores of key half 0 of tile j+1 (after the last tile: of a
    // stale buffer, masked to nothing and dropped), probabilities and O of half 1 of tile j
    step(S1, S0, sKn, 0, word_of(raw_n, sel_n), sVc, 1, cp);
    if (!has_n) {
      wait_vmem();  // no copy may still be landing when the workgroup's LDS is released
      break;
    }
    raw_c = raw_n; sel_c = sel_n;
    raw_n = raw_nn; sel_n = sel_nn;
    kc = kn;
    kn = knn;
    ++jpos;
  }

  const float l_tot = half_sum(l);
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
      lse[((size_t)b * H + h) * S + tq] = l_tot > 0.f ? m * 0.69314718055994530942f + logf(l_tot) : -INFINITY;
  }
}

// Plain kernel for any head dims <= 256 and fp32 or bf16: one wave per
// (b, t, h), 64 keys (one mask word) per step. Lanes own keys for the logits
// and head-dim slots for the output.
template <typename T>
__global__ __launch_bounds__(256) void attn_fwd_plain_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const uint64_t* __restrict__ bits, int B, int S, int Sk, int ratio, int H, int Dqk, int Dv, float scale,
    T* __restrict__ o, float* __restrict__ lse) {
  __shared__ float qs[4][256];
  __shared__ float ps[4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + wid;  // (b, t, h) flattened
  if (row >= (size_t)B * S * H) return;             // whole wave leaves together
  const int h = (int)(row % H);
  const int t = (int)((row / H) % S);
  const int b = (int)(row / ((size_t)H * S));
  const int W = (Sk + 63) / 64;
  const int tk = (t + 1) / ratio - 1;  // last visible key
  const T* qrow = q + ((size_t)b * S + t) * H * Dqk + (size_t)h * Dqk;
  for (int d = lane; d < Dqk; d += 64) qs[wid][d] = Elem<T>::load(qrow + d);
  __builtin_amdgcn_wave_barrier();
  float m = -INFINITY, l = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const uint64_t* brow = bits + ((size_t)b * S + t) * W;
  for (int w = 0; w < (tk + 64) / 64; ++w) {
    const uint64_t word = brow[w];
    if (word == 0ull) continue;
    const int s = 64 * w + lane;
    float x = -INFINITY;
    if ((word >> lane) & 1ull) {
      const T* krow = k + ((size_t)b * Sk + s) * H * Dqk + (size_t)h * Dqk;
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
      const T* vrow = v + ((size_t)b * Sk + 64 * w + jj) * H * Dv + (size_t)h * Dv;
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
                                const uint8_t* cls, int B, int S, int Sk, int ratio, int H, float scale, void* o,
                                float* lse, hipStream_t st) {
  const size_t nblk = (size_t)((S + fwd::QW - 1) / fwd::QW) * B * H;
  hipLaunchKernelGGL(attn_fwd_mfma_kernel, dim3((unsigned)nblk), dim3(fwd::NW * 64), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, bits, cls, B, S, Sk, ratio, H,
                     scale * 1.4426950408889634f, (uint16_t*)o, lse);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_plain(const void* q, const void* k, const void* v, const uint64_t* bits,
                                 int B, int S, int Sk, int ratio, int H, int Dqk, int Dv, float scale, bool bf16,
                                 void* o, float* lse, hipStream_t st) {
  const size_t nblk = ((size_t)B * S * H + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL(attn_fwd_plain_kernel<uint16_t>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, bits, B, S, Sk, ratio, H,
                       Dqk, Dv, scale, (uint16_t*)o, lse);
  else
    hipLaunchKernelGGL(attn_fwd_plain_kernel<float>, dim3((unsigned)nblk), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, bits, B, S, Sk, ratio, H, Dqk, Dv,
                       scale, (float*)o, lse);
  return hipGetLastError();
}

}  // namespace dsa
