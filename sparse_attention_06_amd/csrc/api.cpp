// C ABI of the DSA hot path: host-side argument checks, then kernel launches.
// Every check runs before any HIP call, so the error paths can be exercised on
// a machine without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/dsa.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dsa_status ok() {
  g_err[0] = '\0';
  return DSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQ(cond, code, ...)                 \
  do {                                       \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define REQ_PTR(p)                                                                   \
  do {                                                                               \
    REQ((p) != nullptr, DSA_ERR_INVALID_ARG, "%s must not be NULL", #p);             \
    REQ(aligned16(p), DSA_ERR_INVALID_ARG, "%s must be 16-byte aligned", #p);        \
  } while (0)

dsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(dsa_dtype d) { return d == DSA_BF16 || d == DSA_FP32; }

uint64_t* bits_of(void* mask) { return (uint64_t*)mask; }
uint8_t* cls_of(void* mask, int B, int S, int Sk) { return (uint8_t*)mask + dsa::bits_bytes(B, S, Sk); }
uint8_t* cls_of(void* mask, int B, int S) { return cls_of(mask, B, S, S); }

}  // namespace

extern "C" {

size_t dsa_mask_bytes(int B, int S) {
  if (B < 1 || S < 1) return 0;
  return dsa::bits_bytes(B, S) + (size_t)B * dsa::n_qtiles(S) * dsa::n_ktiles(S);
}

static bool attn_mfma(int Dqk, int Dv, dsa_dtype dtype) {
  return dtype == DSA_BF16 && Dqk == 192 && Dv == 128;
}

// Workspace layout: D, then lse * log2(e) (float32 [B,H,S] each); with the dS
// handoff, the dS^T fragments after them, from a 256-byte boundary.
static size_t bwd_frag_offset(int B, int S, int H) {
  return (2 * (size_t)B * H * S * sizeof(float) + 255) / 256 * 256;
}
static size_t bwd_handoff_bytes(int B, int S, int H) {
  return (size_t)B * H * dsa::dsf_tile_base((S + 31) / 32) * 4096;
}
// The MFMA backward hands dS from the key-major to the query-major kernel when
// the workspace the caller passes has room for it; otherwise dQ recomputes dS.
static bool bwd_handoff(int B, int S, int H, int Dqk, int Dv, dsa_dtype dtype, size_t workspace_bytes) {
  return attn_mfma(Dqk, Dv, dtype) && workspace_bytes >= bwd_frag_offset(B, S, H) + bwd_handoff_bytes(B, S, H);
}

// the dS handoff over Sk compressed keys: every 32-query chunk holds all key tiles
static size_t csa_handoff_bytes(int B, int S, int Sk, int H, int ratio) {
  return (size_t)B * H * dsa::dsf_base((S + 31) / 32, ratio, dsa::n_ktiles(Sk)) * 4096;
}

size_t dsa_bwd_workspace_min_bytes(int B, int S, int H) {
  if (B < 1 || S < 1 || H < 1) return 0;
  return bwd_frag_offset(B, S, H);
}

size_t dsa_bwd_workspace_bytes(int B, int S, int H, int Dqk, int Dv, dsa_dtype dtype) {
  if (B < 1 || S < 1 || H < 1) return 0;
  if (attn_mfma(Dqk, Dv, dtype) && bwd_handoff_bytes(B, S, H) <= (size_t)DSA_BWD_HANDOFF_MAX_BYTES)
    return bwd_frag_offset(B, S, H) + bwd_handoff_bytes(B, S, H);
  return bwd_frag_offset(B, S, H);
}

size_t dsa_csa_bwd_workspace_bytes(int B, int S, int Sk, int ratio, int H, int Dqk, int Dv, dsa_dtype dtype) {
  if (B < 1 || S < 1 || Sk < 1 || ratio < 1 || H < 1) return 0;
  const size_t hb = csa_handoff_bytes(B, S, Sk, H, ratio);
  if (attn_mfma(Dqk, Dv, dtype) && hb <= (size_t)DSA_BWD_HANDOFF_MAX_BYTES) return bwd_frag_offset(B, S, H) + hb;
  return bwd_frag_offset(B, S, H);
}

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

const char* dsa_last_error(void) { return g_err; }

int dsa_version(void) { return 100; }  // 0.1.0

// the indexer over Sk keys of ratio tokens each (ratio 1, Sk = S: token level)
static dsa_status index_scores_impl(const void* q_idx, const void* k_idx, const void* w, const int32_t* seg, int B,
                                    int S, int Sk, int ratio, int Hi, int Di, dsa_dtype in_dtype, int row0,
                                    int nrows, void* scores, dsa_dtype score_dtype, int64_t ld, void* stream,
                                    const char* name) {
  REQ(dtype_ok(in_dtype) && dtype_ok(score_dtype), DSA_ERR_INVALID_ARG, "unknown dtype");
  const bool in_bf16 = in_dtype == DSA_BF16, out_bf16 = score_dtype == DSA_BF16;
  REQ(!in_bf16 || Di % 8 == 0, DSA_ERR_UNSUPPORTED, "bf16 index dim must be a multiple of 8");
  hipStream_t st = (hipStream_t)stream;
  if (in_bf16 && (Hi == 32 || Hi == 64) && (Di == 64 || Di == 128))
    return hip_status(dsa::launch_index_scores_mfma(q_idx, k_idx, w, seg, B, S, Sk, ratio, Hi, Di, row0, nrows,
                                                    scores, out_bf16, ld, st),
                      name);
  // the plain kernel stages the query's Hi x Di values and Hi weights as
  // float32 in 64 KB of LDS; the product is formed in 64 bits
  REQ(((int64_t)Hi * Di + Hi) * 4 <= 65536, DSA_ERR_UNSUPPORTED,
      "Hi*Di=%lld too large for the plain indexer kernel", (long long)Hi * Di);
  return hip_status(dsa::launch_index_scores_plain(q_idx, k_idx, w, seg, B, S, Sk, ratio, Hi, Di, in_bf16, row0,
                                                   nrows, scores, out_bf16, ld, st),
                    name);
}

dsa_status dsa_index_scores(const void* q_idx, const void* k_idx, const void* w,
                            const int32_t* seg, int B, int S, int Hi, int Di,
                            dsa_dtype in_dtype, int row0, int nrows, void* scores,
                            dsa_dtype score_dtype, int64_t ld, void* stream) {
  REQ_PTR(q_idx);
  REQ_PTR(k_idx);
  REQ_PTR(w);
  REQ_PTR(scores);
  REQ(seg == nullptr || aligned16(seg), DSA_ERR_INVALID_ARG, "seg must be 16-byte aligned");
  REQ(B >= 1 && S >= 1 && Hi >= 1 && Di >= 1, DSA_ERR_INVALID_ARG,
      "sizes must be >= 1 (B=%d S=%d Hi=%d Di=%d)", B, S, Hi, Di);
  REQ(S <= dsa::kMaxS, DSA_ERR_UNSUPPORTED, "S=%d exceeds %d", S, dsa::kMaxS);
  REQ(row0 >= 0 && nrows >= 1 && (int64_t)row0 + nrows <= S, DSA_ERR_INVALID_ARG,
      "rows [%d, %d) outside [0, %d)", row0, row0 + nrows, S);
  REQ(ld >= S, DSA_ERR_INVALID_ARG, "ld=%lld < S=%d", (long long)ld, S);
  return index_scores_impl(q_idx, k_idx, w, seg, B, S, S, 1, Hi, Di, in_dtype, row0, nrows, scores, score_dtype,
                           ld, stream, "dsa_index_scores");
}

dsa_status dsa_quant_fp8_rows(const void* x, dsa_dtype x_dtype, int64_t nrows, int D, uint8_t* codes,
                              float* scale, void* stream) {
  REQ_PTR(x);
  REQ_PTR(codes);
  REQ_PTR(scale);
  REQ(dtype_ok(x_dtype), DSA_ERR_INVALID_ARG, "unknown dtype");
  REQ(aligned16(x) && aligned16(codes) && ((uintptr_t)scale & 3) == 0, DSA_ERR_INVALID_ARG,
      "x and codes must be 16-byte aligned, scale 4-byte aligned");
  REQ(nrows >= 1, DSA_ERR_INVALID_ARG, "nrows=%lld must be >= 1", (long long)nrows);
  REQ(D == 64 || D == 128 || D == 256 || D == 512, DSA_ERR_UNSUPPORTED, "D=%d not in {64, 128, 256, 512}", D);
  // one wave per row, 256-thread blocks: the grid's thread count must stay below 2^32
  REQ(nrows <= ((int64_t)1 << 26), DSA_ERR_UNSUPPORTED, "nrows=%lld exceeds 2^26", (long long)nrows);
  return hip_status(dsa::launch_quant_fp8_rows(x, x_dtype == DSA_BF16, nrows, D, codes, scale,
                                               (hipStream_t)stream),
                    "dsa_quant_fp8_rows");
}

dsa_status dsa_index_scores_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                                const float* k_scale, const void* w, const int32_t* seg, int B, int S,
                                int Hi, int Di, int row0, int nrows, void* scores, dsa_dtype score_dtype,
                                int64_t ld, void* stream) {
  REQ_PTR(q8);
  REQ_PTR(q_scale);
  REQ_PTR(k8);
  REQ_PTR(k_scale);
  REQ_PTR(w);
  REQ_PTR(scores);
  REQ(aligned16(q8) && aligned16(k8), DSA_ERR_INVALID_ARG, "q8 and k8 must be 16-byte aligned");
  REQ(seg == nullptr || aligned16(seg), DSA_ERR_INVALID_ARG, "seg must be 16-byte aligned");
  REQ(B >= 1 && S >= 1 && Hi >= 1 && Di >= 1, DSA_ERR_INVALID_ARG,
      "sizes must be >= 1 (B=%d S=%d Hi=%d Di=%d)", B, S, Hi, Di);
  REQ(S <= dsa::kMaxS, DSA_ERR_UNSUPPORTED, "S=%d exceeds %d", S, dsa::kMaxS);
  REQ((Hi == 32 || Hi == 64) && (Di == 64 || Di == 128), DSA_ERR_UNSUPPORTED,
      "fp8 indexer needs Hi in {32, 64} and Di in {64, 128} (Hi=%d Di=%d)", Hi, Di);
  REQ(row0 >= 0 && nrows >= 1 && (int64_t)row0 + nrows <= S, DSA_ERR_INVALID_ARG,
      "rows [%d, %d) outside [0, %d)", row0, row0 + nrows, S);
  REQ(ld >= S, DSA_ERR_INVALID_ARG, "ld=%lld < S=%d", (long long)ld, S);
  REQ(dtype_ok(score_dtype), DSA_ERR_INVALID_ARG, "unknown score dtype");
  return hip_status(dsa::launch_index_scores_fp8(q8, q_scale, k8, k_scale, w, seg, B, S, Hi, Di, row0, nrows,
                                                 scores, score_dtype == DSA_BF16, ld, (hipStream_t)stream),
                    "dsa_index_scores_fp8");
}

dsa_status dsa_indexer_rope(const void* x, int B, int S, int nh, int D, int rope_dim, const float* cos_t,
                            const float* sin_t, int P, const int32_t* pos, void* out, void* stream) {
  REQ_PTR(x);
  REQ_PTR(cos_t);
  REQ_PTR(sin_t);
  REQ_PTR(out);
  REQ(aligned16(x) && aligned16(out) && aligned16(cos_t) && aligned16(sin_t), DSA_ERR_INVALID_ARG,
      "x, out and the tables must be 16-byte aligned");
  REQ(pos == nullptr || aligned16(pos), DSA_ERR_INVALID_ARG, "pos must be 16-byte aligned");
  REQ(B >= 1 && S >= 1 && nh >= 1 && D >= 1 && P >= 1, DSA_ERR_INVALID_ARG,
      "sizes must be >= 1 (B=%d S=%d nh=%d D=%d P=%d)", B, S, nh, D, P);
  REQ(D % 8 == 0 && rope_dim % 16 == 0 && rope_dim >= 16 && rope_dim <= D, DSA_ERR_UNSUPPORTED,
      "need D %% 8 == 0 and rope_dim %% 16 == 0 in [16, D] (D=%d rope_dim=%d)", D, rope_dim);
  REQ(pos != nullptr || P >= S, DSA_ERR_INVALID_ARG, "without positions the tables need P >= S (P=%d S=%d)", P, S);
  REQ((int64_t)B * S * nh * (D / 8) < ((int64_t)1 << 32) - 256, DSA_ERR_UNSUPPORTED, "too many vectors");
  return hip_status(dsa::launch_rope_rows(x, B, S, nh, D, rope_dim, P, cos_t, sin_t, pos, out,
                                          (hipStream_t)stream),
                    "dsa_indexer_rope");
}

static dsa_status topk_impl(const void* scores, dsa_dtype score_dtype, int64_t ld, const int32_t* seg, int B, int S,
                            int Sk, int ratio, int K, int row0, int nrows, int32_t* idx, void* mask, void* stream,
                            const char* name) {
  REQ(row0 % DSA_TILE_Q == 0 && ((row0 + nrows) % DSA_TILE_Q == 0 || row0 + nrows == S),
      DSA_ERR_INVALID_ARG, "row slab [%d, %d) must start and end on a %d-row query tile (or at S)",
      row0, row0 + nrows, DSA_TILE_Q);
  REQ(dtype_ok(score_dtype), DSA_ERR_INVALID_ARG, "unknown score dtype");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = dsa::launch_topk(scores, score_dtype == DSA_BF16, ld, seg, B, S, Sk, ratio, K, row0, nrows, idx,
                                  bits_of(mask), st);
  if (e != hipSuccess) return hip_status(e, name);
  const int qt0 = row0 / DSA_TILE_Q, qt1 = (row0 + nrows + DSA_TILE_Q - 1) / DSA_TILE_Q;
  return hip_status(dsa::launch_tile_classes(bits_of(mask), B, S, Sk, qt0, qt1, cls_of(mask, B, S, Sk), st), name);
}

dsa_status dsa_topk(const void* scores, dsa_dtype score_dtype, int64_t ld, const int32_t* seg,
                    int B, int S, int K, int row0, int nrows, int32_t* idx, void* mask,
                    void* stream) {
  REQ_PTR(scores);
  REQ_PTR(idx);
  REQ_PTR(mask);
  REQ(seg == nullptr || aligned16(seg), DSA_ERR_INVALID_ARG, "seg must be 16-byte aligned");
  REQ(B >= 1 && S >= 1 && K >= 1, DSA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d S=%d K=%d)", B, S, K);
  REQ(S <= dsa::kMaxS, DSA_ERR_UNSUPPORTED, "S=%d exceeds %d", S, dsa::kMaxS);
  REQ(row0 >= 0 && nrows >= 1 && (int64_t)row0 + nrows <= S, DSA_ERR_INVALID_ARG,
      "rows [%d, %d) outside [0, %d)", row0, row0 + nrows, S);
  REQ(ld >= S, DSA_ERR_INVALID_ARG, "ld=%lld < S=%d", (long long)ld, S);
  return topk_impl(scores, score_dtype, ld, seg, B, S, S, 1, K, row0, nrows, idx, mask, stream, "dsa_topk");
}

static dsa_status build_mask_impl(const int32_t* idx, const int32_t* seg, int B, int S, int Sk, int ratio, int K,
                                  void* mask, void* stream, const char* name) {
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = dsa::launch_build_bits(idx, seg, B, S, Sk, ratio, K, bits_of(mask), st);
  if (e != hipSuccess) return hip_status(e, name);
  return hip_status(dsa::launch_tile_classes(bits_of(mask), B, S, Sk, 0, dsa::n_qtiles(S), cls_of(mask, B, S, Sk),
                                             st),
                    name);
}

dsa_status dsa_build_mask(const int32_t* idx, const int32_t* seg, int B, int S, int K, void* mask,
                          void* stream) {
  REQ_PTR(idx);
  REQ_PTR(mask);
  REQ(seg == nullptr || aligned16(seg), DSA_ERR_INVALID_ARG, "seg must be 16-byte aligned");
  REQ(B >= 1 && S >= 1 && K >= 1, DSA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d S=%d K=%d)", B, S, K);
  REQ(S <= dsa::kMaxS, DSA_ERR_UNSUPPORTED, "S=%d exceeds %d", S, dsa::kMaxS);
  return build_mask_impl(idx, seg, B, S, S, 1, K, mask, stream, "dsa_build_mask");
}

static dsa_status check_attn(int B, int S, int H, int Dqk, int Dv, float scale, dsa_dtype dtype) {
  REQ(B >= 1 && S >= 1 && H >= 1 && Dqk >= 1 && Dv >= 1, DSA_ERR_INVALID_ARG,
      "sizes must be >= 1 (B=%d S=%d H=%d Dqk=%d Dv=%d)", B, S, H, Dqk, Dv);
  REQ(S <= dsa::kMaxS, DSA_ERR_UNSUPPORTED, "S=%d exceeds %d", S, dsa::kMaxS);
  REQ(dtype_ok(dtype), DSA_ERR_INVALID_ARG, "unknown dtype");
  REQ(scale == scale && scale > 0.f, DSA_ERR_INVALID_ARG, "softmax_scale must be > 0");
  REQ(Dqk <= 256 && Dv <= 256, DSA_ERR_UNSUPPORTED, "head dims above 256 (Dqk=%d Dv=%d)", Dqk, Dv);
  REQ(dtype != DSA_BF16 || (Dqk % 8 == 0 && Dv % 8 == 0), DSA_ERR_UNSUPPORTED,
      "bf16 head dims must be multiples of 8");
  return DSA_OK;
}

static dsa_status attn_fwd_impl(const void* q, const void* k, const void* v, const void* mask, int B, int S, int Sk,
                                int ratio, int H, int Dqk, int Dv, float softmax_scale, dsa_dtype dtype, void* o,
                                float* lse, void* stream, const char* name) {
  hipStream_t st = (hipStream_t)stream;
  void* m = const_cast<void*>(mask);
  if (attn_mfma(Dqk, Dv, dtype))
    return hip_status(dsa::launch_attn_fwd_mfma(q, k, v, bits_of(m), cls_of(m, B, S, Sk), B, S, Sk, ratio, H,
                                                softmax_scale, o, lse, st),
                      name);
  return hip_status(dsa::launch_attn_fwd_plain(q, k, v, bits_of(m), B, S, Sk, ratio, H, Dqk, Dv, softmax_scale,
                                               dtype == DSA_BF16, o, lse, st),
                    name);
}

dsa_status dsa_sparse_attn_fwd(const void* q, const void* k, const void* v, const void* mask,
                               int B, int S, int H, int Dqk, int Dv, float softmax_scale,
                               dsa_dtype dtype, void* o, float* lse, void* stream) {
  REQ_PTR(q);
  REQ_PTR(k);
  REQ_PTR(v);
  REQ_PTR(mask);
  REQ_PTR(o);
  REQ_PTR(lse);
  dsa_status s = check_attn(B, S, H, Dqk, Dv, softmax_scale, dtype);
  if (s != DSA_OK) return s;
  return attn_fwd_impl(q, k, v, mask, B, S, S, 1, H, Dqk, Dv, softmax_scale, dtype, o, lse, stream,
                       "dsa_sparse_attn_fwd");
}

// ---------------------------------------------------------------- compressed sparse attention
static dsa_status check_csa(int B, int S, int Sk, int ratio) {
  REQ(B >= 1 && S >= 1, DSA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d S=%d)", B, S);
  REQ(S <= dsa::kMaxS, DSA_ERR_UNSUPPORTED, "S=%d exceeds %d", S, dsa::kMaxS);
  REQ(ratio >= 1, DSA_ERR_INVALID_ARG, "ratio=%d must be >= 1", ratio);
  REQ(Sk >= 1 && Sk == S / ratio, DSA_ERR_INVALID_ARG, "Sk=%d must be S / ratio = %d (and >= 1)", Sk, S / ratio);
  return DSA_OK;
}

size_t dsa_csa_mask_bytes(int B, int S, int Sk) {
  if (B < 1 || S < 1 || Sk < 1) return 0;
  return dsa::bits_bytes(B, S, Sk) + (size_t)B * dsa::n_qtiles(S) * dsa::n_ktiles(Sk);
}

dsa_status dsa_csa_index_scores(const void* q_idx, const void* k_idx, const void* w, int B, int S, int Sk, int ratio,
                                int Hi, int Di, dsa_dtype in_dtype, int row0, int nrows, void* scores,
                                dsa_dtype score_dtype, int64_t ld, void* stream) {
  REQ_PTR(q_idx);
  REQ_PTR(k_idx);
  REQ_PTR(w);
  REQ_PTR(scores);
  dsa_status s = check_csa(B, S, Sk, ratio);
  if (s != DSA_OK) return s;
  REQ(Hi >= 1 && Di >= 1, DSA_ERR_INVALID_ARG, "sizes must be >= 1 (Hi=%d Di=%d)", Hi, Di);
  REQ(row0 >= 0 && nrows >= 1 && (int64_t)row0 + nrows <= S, DSA_ERR_INVALID_ARG,
      "rows [%d, %d) outside [0, %d)", row0, row0 + nrows, S);
  REQ(ld >= Sk, DSA_ERR_INVALID_ARG, "ld=%lld < Sk=%d", (long long)ld, Sk);
  return index_scores_impl(q_idx, k_idx, w, nullptr, B, S, Sk, ratio, Hi, Di, in_dtype, row0, nrows, scores,
                           score_dtype, ld, stream, "dsa_csa_index_scores");
}

dsa_status dsa_csa_topk(const void* scores, dsa_dtype score_dtype, int64_t ld, int B, int S, int Sk, int ratio, int K,
                        int row0, int nrows, int32_t* idx, void* mask, void* stream) {
  REQ_PTR(scores);
  REQ_PTR(idx);
  REQ_PTR(mask);
  dsa_status s = check_csa(B, S, Sk, ratio);
  if (s != DSA_OK) return s;
  REQ(K >= 1, DSA_ERR_INVALID_ARG, "K=%d must be >= 1", K);
  REQ(row0 >= 0 && nrows >= 1 && (int64_t)row0 + nrows <= S, DSA_ERR_INVALID_ARG,
      "rows [%d, %d) outside [0, %d)", row0, row0 + nrows, S);
  REQ(ld >= Sk, DSA_ERR_INVALID_ARG, "ld=%lld < Sk=%d", (long long)ld, Sk);
  return topk_impl(scores, score_dtype, ld, nullptr, B, S, Sk, ratio, K, row0, nrows, idx, mask, stream,
                   "dsa_csa_topk");
}

dsa_status dsa_csa_build_mask(const int32_t* idx, int B, int S, int Sk, int ratio, int K, void* mask, void* stream) {
  REQ_PTR(idx);
  REQ_PTR(mask);
  dsa_status s = check_csa(B, S, Sk, ratio);
  if (s != DSA_OK) return s;
  REQ(K >= 1, DSA_ERR_INVALID_ARG, "K=%d must be >= 1", K);
  return build_mask_impl(idx, nullptr, B, S, Sk, ratio, K, mask, stream, "dsa_csa_build_mask");
}

dsa_status dsa_csa_sparse_attn_fwd(const void* q, const void* k, const void* v, const void* mask, int B, int S,
                                   int Sk, int ratio, int H, int Dqk, int Dv, float softmax_scale, dsa_dtype dtype,
                                   void* o, float* lse, void* stream) {
  REQ_PTR(q);
  REQ_PTR(k);
  REQ_PTR(v);
  REQ_PTR(mask);
  REQ_PTR(o);
  REQ_PTR(lse);
  dsa_status s = check_csa(B, S, Sk, ratio);
  if (s != DSA_OK) return s;
  s = check_attn(B, S, H, Dqk, Dv, softmax_scale, dtype);
  if (s != DSA_OK) return s;
  return attn_fwd_impl(q, k, v, mask, B, S, Sk, ratio, H, Dqk, Dv, softmax_scale, dtype, o, lse, stream,
                       "dsa_csa_sparse_attn_fwd");
}

static dsa_status check_bwd_common(const void* q, const void* k, const void* v, const void* dout,
                                   const float* lse, const void* mask, int B, int S, int H, int Dqk,
                                   int Dv, float scale, dsa_dtype dtype, const void* workspace,
                                   size_t workspace_bytes) {
  REQ_PTR(q);
  REQ_PTR(k);
  REQ_PTR(v);
  REQ_PTR(dout);
  REQ_PTR(lse);
  REQ_PTR(mask);
  REQ_PTR(workspace);
  dsa_status s = check_attn(B, S, H, Dqk, Dv, scale, dtype);
  if (s != DSA_OK) return s;
  const size_t need = dsa_bwd_workspace_min_bytes(B, S, H);
  REQ(workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, need);
  return DSA_OK;
}

dsa_status dsa_sparse_attn_bwd_prep(const void* o, const void* dout, const float* lse, int B, int S, int H,
                                    int Dqk, int Dv, dsa_dtype dtype, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  REQ_PTR(o);
  REQ_PTR(dout);
  REQ_PTR(lse);
  REQ_PTR(workspace);
  dsa_status s = check_attn(B, S, H, Dqk, Dv, 1.f, dtype);
  if (s != DSA_OK) return s;
  const size_t need = dsa_bwd_workspace_min_bytes(B, S, H);
  REQ(workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, need);
  return hip_status(dsa::launch_attn_bwd_prep(o, dout, lse, B, S, H, Dv, dtype == DSA_BF16, (float*)workspace,
                                              (hipStream_t)stream),
                    "dsa_sparse_attn_bwd_prep");
}

dsa_status dsa_sparse_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                                    const float* lse, const void* mask, int B, int S, int H, int Dqk,
                                    int Dv, float softmax_scale, dsa_dtype dtype, void* dk, void* dv,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status s = check_bwd_common(q, k, v, dout, lse, mask, B, S, H, Dqk, Dv, softmax_scale, dtype,
                                  workspace, workspace_bytes);
  if (s != DSA_OK) return s;
  REQ_PTR(dk);
  REQ_PTR(dv);
  hipStream_t st = (hipStream_t)stream;
  void* m = const_cast<void*>(mask);
  const float* ws = (const float*)workspace;
  if (attn_mfma(Dqk, Dv, dtype)) {
    void* dsf = bwd_handoff(B, S, H, Dqk, Dv, dtype, workspace_bytes)
                    ? (void*)((char*)workspace + bwd_frag_offset(B, S, H)) : nullptr;
    return hip_status(dsa::launch_attn_bwd_dkdv_mfma(q, k, v, dout, ws, bits_of(m), cls_of(m, B, S), B, S, S, 1, H,
                                                     softmax_scale, dk, dv, dsf, st),
                      "dsa_sparse_attn_bwd_dkdv");
  }
  return hip_status(dsa::launch_attn_bwd_dkdv_plain(q, k, v, dout, lse, ws, bits_of(m), B, S, S, 1, H, Dqk, Dv,
                                                    softmax_scale, dtype == DSA_BF16, dk, dv, st),
                    "dsa_sparse_attn_bwd_dkdv");
}

dsa_status dsa_sparse_attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                                  const float* lse, const void* mask, int B, int S, int H, int Dqk,
                                  int Dv, float softmax_scale, dsa_dtype dtype, void* dq,
                                  const void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status s = check_bwd_common(q, k, v, dout, lse, mask, B, S, H, Dqk, Dv, softmax_scale, dtype,
                                  workspace, workspace_bytes);
  if (s != DSA_OK) return s;
  REQ_PTR(dq);
  hipStream_t st = (hipStream_t)stream;
  void* m = const_cast<void*>(mask);
  const float* ws = (const float*)workspace;
  if (bwd_handoff(B, S, H, Dqk, Dv, dtype, workspace_bytes))
    return hip_status(dsa::launch_attn_bwd_dq_mfma(k, (const char*)workspace + bwd_frag_offset(B, S, H),
                                                   cls_of(m, B, S), B, S, S, 1, H, softmax_scale, dq, st),
                      "dsa_sparse_attn_bwd_dq");
  if (attn_mfma(Dqk, Dv, dtype))
    return hip_status(dsa::launch_attn_bwd_dq_recompute(q, k, v, dout, ws, bits_of(m), cls_of(m, B, S), B, S, S,
                                                        1, H, softmax_scale, dq, st),
                      "dsa_sparse_attn_bwd_dq");
  return hip_status(dsa::launch_attn_bwd_dq_plain(q, k, v, dout, lse, ws, bits_of(m), B, S, S, 1, H, Dqk, Dv,
                                                  softmax_scale, dtype == DSA_BF16, dq, st),
                    "dsa_sparse_attn_bwd_dq");
}

dsa_status dsa_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, const void* mask, int B, int S,
                               int H, int Dqk, int Dv, float softmax_scale, dsa_dtype dtype,
                               void* dq, void* dk, void* dv, void* workspace,
                               size_t workspace_bytes, void* stream) {
  dsa_status s = check_bwd_common(q, k, v, dout, lse, mask, B, S, H, Dqk, Dv, softmax_scale, dtype,
                                  workspace, workspace_bytes);
  if (s != DSA_OK) return s;
  REQ_PTR(o);
  REQ_PTR(dq);
  REQ_PTR(dk);
  REQ_PTR(dv);
  s = dsa_sparse_attn_bwd_prep(o, dout, lse, B, S, H, Dqk, Dv, dtype, workspace, workspace_bytes, stream);
  if (s != DSA_OK) return s;
  s = dsa_sparse_attn_bwd_dkdv(q, k, v, dout, lse, mask, B, S, H, Dqk, Dv, softmax_scale, dtype, dk, dv,
                               workspace, workspace_bytes, stream);
  if (s != DSA_OK) return s;
  return dsa_sparse_attn_bwd_dq(q, k, v, dout, lse, mask, B, S, H, Dqk, Dv, softmax_scale, dtype, dq,
                                workspace, workspace_bytes, stream);
}


// compressed keys: the prologue, then the key-major and query-major kernels
// over the Sk entries (MFMA for bf16 192/128, with the dS handoff when the
// workspace holds it; plain otherwise)
dsa_status dsa_csa_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const float* lse, const void* mask, int B, int S, int Sk, int ratio, int H,
                                   int Dqk, int Dv, float softmax_scale, dsa_dtype dtype, void* dq, void* dk,
                                   void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  REQ_PTR(q);
  REQ_PTR(k);
  REQ_PTR(v);
  REQ_PTR(o);
  REQ_PTR(dout);
  REQ_PTR(lse);
  REQ_PTR(mask);
  REQ_PTR(dq);
  REQ_PTR(dk);
  REQ_PTR(dv);
  REQ_PTR(workspace);
  dsa_status s = check_csa(B, S, Sk, ratio);
  if (s != DSA_OK) return s;
  s = check_attn(B, S, H, Dqk, Dv, softmax_scale, dtype);
  if (s != DSA_OK) return s;
  const size_t need = dsa_bwd_workspace_min_bytes(B, S, H);
  REQ(workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  const bool bf16 = dtype == DSA_BF16;
  void* m = const_cast<void*>(mask);
  const uint64_t* bits = bits_of(m);
  float* ws = (float*)workspace;
  hipError_t e = dsa::launch_attn_bwd_prep(o, dout, lse, B, S, H, Dv, bf16, ws, st);
  if (attn_mfma(Dqk, Dv, dtype)) {
    // the MFMA key-major kernel, handing dS to the MFMA dQ kernel when the
    // workspace holds it (else the MFMA dQ kernel that recomputes dS)
    const bool handoff = workspace_bytes >= bwd_frag_offset(B, S, H) + csa_handoff_bytes(B, S, Sk, H, ratio);
    void* dsf = handoff ? (void*)((char*)workspace + bwd_frag_offset(B, S, H)) : nullptr;
    if (e == hipSuccess)
      e = dsa::launch_attn_bwd_dkdv_mfma(q, k, v, dout, ws, bits, cls_of(m, B, S, Sk), B, S, Sk, ratio, H,
                                         softmax_scale, dk, dv, dsf, st);
    if (e == hipSuccess)
      e = handoff ? dsa::launch_attn_bwd_dq_mfma(k, dsf, cls_of(m, B, S, Sk), B, S, Sk, ratio, H, softmax_scale, dq, st)
                  : dsa::launch_attn_bwd_dq_recompute(q, k, v, dout, ws, bits, cls_of(m, B, S, Sk), B, S, Sk, ratio,
                                                      H, softmax_scale, dq, st);
    return hip_status(e, "dsa_csa_sparse_attn_bwd");
  }
  if (e == hipSuccess)
    e = dsa::launch_attn_bwd_dkdv_plain(q, k, v, dout, lse, ws, bits, B, S, Sk, ratio, H, Dqk, Dv, softmax_scale,
                                        bf16, dk, dv, st);
  if (e == hipSuccess)
    e = dsa::launch_attn_bwd_dq_plain(q, k, v, dout, lse, ws, bits, B, S, Sk, ratio, H, Dqk, Dv, softmax_scale, bf16,
                                      dq, st);
  return hip_status(e, "dsa_csa_sparse_attn_bwd");
}

// ---------------------------------------------------------------------------
// Indexer KL auxiliary loss
// ---------------------------------------------------------------------------
dsa_status dsa_indexer_teacher(const void* q, const void* k, const float* lse, const void* mask, int B, int S, int H,
                               int Dqk, int K, float softmax_scale, dsa_dtype dtype, float* teacher, void* stream) {
  REQ_PTR(q);
  REQ_PTR(k);
  REQ_PTR(lse);
  REQ_PTR(mask);
  REQ_PTR(teacher);
  REQ(B >= 1 && S >= 1 && H >= 1 && K >= 1, DSA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d S=%d H=%d K=%d)", B, S,
      H, K);
  REQ(S <= dsa::kMaxS, DSA_ERR_UNSUPPORTED, "S=%d exceeds %d", S, dsa::kMaxS);
  REQ(dtype_ok(dtype), DSA_ERR_INVALID_ARG, "unknown dtype");
  REQ(softmax_scale == softmax_scale && softmax_scale > 0.f, DSA_ERR_INVALID_ARG, "softmax_scale must be > 0");
  REQ(dtype == DSA_BF16 && (Dqk == 64 || Dqk == 128 || Dqk == 192), DSA_ERR_UNSUPPORTED,
      "the teacher takes bf16 q, k with Dqk in {64, 128, 192} (Dqk=%d)", Dqk);
  void* m = const_cast<void*>(mask);
  return hip_status(dsa::launch_indexer_teacher(q, k, lse, bits_of(m), cls_of(m, B, S), B, S, H, Dqk, K,
                                                softmax_scale, teacher, (hipStream_t)stream),
                    "dsa_indexer_teacher");
}

dsa_status dsa_indexer_kl(const void* scores, dsa_dtype score_dtype, int64_t ld, const int32_t* idx,
                          const float* teacher, const void* mask, int B, int S, int K, float* row_kl, float* loss,
                          float* dscores, int64_t ld_ds, void* stream) {
  REQ_PTR(scores);
  REQ_PTR(idx);
  REQ_PTR(teacher);
  REQ_PTR(mask);
  REQ_PTR(row_kl);
  REQ_PTR(dscores);
  REQ(loss != nullptr && ((uintptr_t)loss & 7) == 0, DSA_ERR_INVALID_ARG, "loss must be a non-NULL, 8-byte aligned float[2]");
  REQ(B >= 1 && S >= 1 && K >= 1, DSA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d S=%d K=%d)", B, S, K);
  REQ(S <= dsa::kMaxS, DSA_ERR_UNSUPPORTED, "S=%d exceeds %d", S, dsa::kMaxS);
  REQ(ld >= S && ld_ds >= S, DSA_ERR_INVALID_ARG, "ld=%lld and ld_ds=%lld must be >= S=%d", (long long)ld,
      (long long)ld_ds, S);
  REQ(dtype_ok(score_dtype), DSA_ERR_INVALID_ARG, "unknown score dtype");
  return hip_status(dsa::launch_indexer_kl(scores, score_dtype == DSA_BF16, ld, idx, teacher,
                                           bits_of(const_cast<void*>(mask)), B, S, K, row_kl, loss, dscores, ld_ds,
                                           (hipStream_t)stream),
                    "dsa_indexer_kl");
}

dsa_status dsa_indexer_bwd(const void* q_idx, const void* k_idx, const void* w, const float* dscores, int64_t ld,
                           const void* mask, int B, int S, int Hi, int Di, dsa_dtype dtype, void* dq_idx,
                           void* dk_idx, void* dw, void* stream) {
  REQ_PTR(q_idx);
  REQ_PTR(k_idx);
  REQ_PTR(w);
  REQ_PTR(dscores);
  REQ_PTR(mask);
  REQ_PTR(dq_idx);
  REQ_PTR(dk_idx);
  REQ_PTR(dw);
  REQ(B >= 1 && S >= 1 && Hi >= 1 && Di >= 1, DSA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d S=%d Hi=%d Di=%d)", B,
      S, Hi, Di);
  REQ(S <= dsa::kMaxS, DSA_ERR_UNSUPPORTED, "S=%d exceeds %d", S, dsa::kMaxS);
  REQ(ld >= S, DSA_ERR_INVALID_ARG, "ld=%lld must be >= S=%d", (long long)ld, S);
  REQ(dtype_ok(dtype), DSA_ERR_INVALID_ARG, "unknown dtype");
  REQ(dtype == DSA_BF16 && Hi == 64 && Di == 128, DSA_ERR_UNSUPPORTED,
      "the indexer backward takes bf16 inputs with 64 index heads of dim 128 (Hi=%d Di=%d)", Hi, Di);
  return hip_status(dsa::launch_indexer_bwd(q_idx, k_idx, w, dscores, ld, cls_of(const_cast<void*>(mask), B, S), B, S,
                                            dq_idx, dk_idx, dw, (hipStream_t)stream),
                    "dsa_indexer_bwd");
}

// ---------------------------------------------------------------------------
// Allocation-free backward: the workspace is a file-scope device array, one
// copy per GPU, whose address is looked up once per device and kept.
// ---------------------------------------------------------------------------
}  // extern "C"

static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device. In host code the array's
// name is only a stand-in, so kernels and copies get this address instead.
dsa_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  REQ(dev >= 0 && dev < kMaxDevices, DSA_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    REQ(p != nullptr, DSA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}
}  // namespace

extern "C" {

dsa_status dsa_sparse_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                       const void* dout, const float* lse, const void* mask, int B, int S,
                                       int H, int Dqk, int Dv, float softmax_scale, dsa_dtype dtype,
                                       void* dq, void* dk, void* dv, void* stream) {
  // every argument check comes before the first HIP call
  REQ_PTR(q);
  REQ_PTR(k);
  REQ_PTR(v);
  REQ_PTR(o);
  REQ_PTR(dout);
  REQ_PTR(lse);
  REQ_PTR(mask);
  REQ_PTR(dq);
  REQ_PTR(dk);
  REQ_PTR(dv);
  dsa_status s = check_attn(B, S, H, Dqk, Dv, softmax_scale, dtype);
  if (s != DSA_OK) return s;
  const size_t need = dsa_bwd_workspace_min_bytes(B, S, H);
  REQ(need <= (size_t)DSA_NOALLOC_SCRATCH_BYTES, DSA_ERR_UNSUPPORTED,
      "B*H*S = %lld needs %zu bytes of scratch; the allocation-free backward holds %llu "
      "(B*H*S <= %llu); use dsa_sparse_attn_bwd with a workspace",
      (long long)B * H * S, need, (unsigned long long)DSA_NOALLOC_SCRATCH_BYTES,
      (unsigned long long)(DSA_NOALLOC_SCRATCH_BYTES / 8));
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != DSA_OK) return s;
  // the minimum workspace: D and the base-2 LSE, both overwritten in full by
  // the prologue, and the recompute route for dQ (no dS tiles)
  return dsa_sparse_attn_bwd(q, k, v, o, dout, lse, mask, B, S, H, Dqk, Dv, softmax_scale, dtype, dq, dk, dv, ws,
                             need, stream);
}

}  // extern "C"
