// Internal launchers of the DSA kernels. The public ABI (dsa.h) validates its
// arguments on the host and then calls these; each returns the launch's
// hipError_t (hipSuccess when nothing had to be launched).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Largest sequence length the library accepts. A build-mask row (S/64 words)
// must fit one workgroup's 64 KB of dynamic LDS with room to spare, and the
// attention kernels stage a workgroup's tile-class rows (S/64 bytes each) in
// LDS.
constexpr int kMaxS = 1 << 18;

// Key axis: Sk keys, key s visible to query t when s <= (t + 1) / ratio - 1
// (compressed blocks of `ratio` tokens); ratio 1 and Sk = S is token-level DSA.
// Masks built over it have ceil(Sk / 64) words per row and ceil(Sk / 64) key
// tiles.
// scores: in_bf16 selects bf16 vs fp32 inputs, out_bf16 the score storage.
hipError_t launch_index_scores_mfma(const void* q_idx, const void* k_idx, const void* w,
                                    const int32_t* seg, int B, int S, int Sk, int ratio, int Hi, int Di,
                                    int row0, int nrows, void* scores, bool out_bf16, int64_t ld,
                                    hipStream_t st);
hipError_t launch_index_scores_plain(const void* q_idx, const void* k_idx, const void* w,
                                     const int32_t* seg, int B, int S, int Sk, int ratio, int Hi, int Di,
                                     bool in_bf16, int row0, int nrows, void* scores,
                                     bool out_bf16, int64_t ld, hipStream_t st);

hipError_t launch_index_scores_fp8(const void* q8, const float* qs, const void* k8, const float* ks,
                                   const void* w, const int32_t* seg, int B, int S, int Hi, int Di, int row0,
                                   int nrows, void* scores, bool out_bf16, int64_t ld, hipStream_t st);
hipError_t launch_quant_fp8_rows(const void* x, bool in_bf16, int64_t nrows, int D, uint8_t* codes,
                                 float* scale, hipStream_t st);
hipError_t launch_rope_rows(const void* x, int B, int S, int nh, int D, int rope_dim, int P, const float* cos_t,
                            const float* sin_t, const int32_t* pos, void* out, hipStream_t st);
hipError_t launch_topk(const void* scores, bool score_bf16, int64_t ld, const int32_t* seg, int B, int S, int Sk,
                       int ratio, int K, int row0, int nrows, int32_t* idx, uint64_t* bits, hipStream_t st);
hipError_t launch_build_bits(const int32_t* idx, const int32_t* seg, int B, int S, int Sk, int ratio, int K,
                             uint64_t* bits, hipStream_t st);
hipError_t launch_tile_classes(const uint64_t* bits, int B, int S, int Sk, int qt0, int qt1, uint8_t* cls,
                               hipStream_t st);

hipError_t launch_attn_fwd_mfma(const void* q, const void* k, const void* v, const uint64_t* bits,
                                const uint8_t* cls, int B, int S, int Sk, int ratio, int H, float scale, void* o,
                                float* lse, hipStream_t st);
hipError_t launch_attn_fwd_plain(const void* q, const void* k, const void* v, const uint64_t* bits,
                                 int B, int S, int Sk, int ratio, int H, int Dqk, int Dv, float scale, bool bf16,
                                 void* o, float* lse, hipStream_t st);

// backward prologue: D = rowsum(dout * o) and lse * log2(e), two float32
// [B,H,S] arrays at the start of the workspace
hipError_t launch_attn_bwd_prep(const void* o, const void* dout, const float* lse, int B, int S, int H, int Dv,
                                bool bf16, float* ws, hipStream_t st);
// backward, key-major: reads D and the base-2 LSE from ws, writes dk and dv
// and the dS^T fragments (dsf) for the dQ kernel
hipError_t launch_attn_bwd_dkdv_mfma(const void* q, const void* k, const void* v, const void* dout,
                                     const float* ws, const uint64_t* bits, const uint8_t* cls, int B, int S,
                                     int Sk, int ratio, int H, float scale, void* dk, void* dv, void* dsf,
                                     hipStream_t st);
hipError_t launch_attn_bwd_dkdv_plain(const void* q, const void* k, const void* v, const void* dout,
                                      const float* lse, const float* D, const uint64_t* bits, int B,
                                      int S, int Sk, int ratio, int H, int Dqk, int Dv, float scale, bool bf16,
                                      void* dk, void* dv, hipStream_t st);
// backward, query-major: dq from the dS^T fragments of the key-major kernel
// (which then gets a non-null dsf), or with dS recomputed from q, k, v, dout
// and the workspace's D and base-2 LSE (key-major kernel given dsf = nullptr)
hipError_t launch_attn_bwd_dq_recompute(const void* q, const void* k, const void* v, const void* dout,
                                        const float* ws, const uint64_t* bits, const uint8_t* cls, int B, int S,
                                        int Sk, int ratio, int H, float scale, void* dq, hipStream_t st);
hipError_t launch_attn_bwd_dq_mfma(const void* k, const void* dsf, const uint8_t* cls, int B, int S, int Sk,
                                   int ratio, int H, float scale, void* dq, hipStream_t st);
hipError_t launch_attn_bwd_dq_plain(const void* q, const void* k, const void* v,
                                    const void* dout, const float* lse, const float* D, const uint64_t* bits,
                                    int B, int S, int Sk, int ratio, int H, int Dqk, int Dv, float scale,
                                    bool bf16, void* dq, hipStream_t st);

// indexer KL auxiliary loss: teacher [B,S,K] (bf16 q, k with Dqk in {64, 128,
// 192}); student softmax, KL per row, loss2 = {loss, N} and the dense score
// gradient over [0, t] of each row; the indexer backward (64 x 128 bf16)
hipError_t launch_indexer_teacher(const void* q, const void* k, const float* lse, const uint64_t* bits,
                                  const uint8_t* cls, int B, int S, int H, int Dqk, int K, float scale,
                                  float* teacher, hipStream_t st);
hipError_t launch_indexer_kl(const void* scores, bool score_bf16, int64_t ld, const int32_t* idx,
                             const float* teacher, const uint64_t* bits, int B, int S, int K, float* row_kl,
                             float* loss2, float* dscores, int64_t ld_ds, hipStream_t st);
hipError_t launch_indexer_bwd(const void* q_idx, const void* k_idx, const void* w, const float* dscores, int64_t ld,
                              const uint8_t* cls, int B, int S, void* dq_idx, void* dk_idx, void* dw,
                              hipStream_t st);

// dS^T fragments that the key-major backward kernel leaves for the dQ kernel:
// per (b, h), 32-query chunk qc holds key tiles 0 .. qc/2 (the causal ones),
// each as four 1 KB MFMA B-operand blocks (one per 16-key step). This is the
// first tile of chunk qc; dsf_tile_base(number of chunks) is the count per (b, h).
__host__ __device__ inline size_t dsf_tile_base(int qc) {
  const size_t m = (size_t)(qc >> 1);
  return (qc & 1) ? (m + 1) * (m + 1) : m * (m + 1);
}
// The same for any key axis: token keys (ratio 1) use the causal layout above;
// compressed keys give every chunk all nkt key tiles of its (b, h).
__host__ __device__ inline size_t dsf_base(int qc, int ratio, int nkt) {
  return ratio == 1 ? dsf_tile_base(qc) : (size_t)qc * nkt;
}

// layout helpers shared by the host side
inline int mask_words(int S) { return (S + 63) / 64; }
inline int n_qtiles(int S) { return (S + 127) / 128; }
inline int n_ktiles(int S) { return (S + 63) / 64; }
inline size_t bits_bytes(int B, int S, int Sk) { return (size_t)B * S * mask_words(Sk) * 8; }
inline size_t bits_bytes(int B, int S) { return bits_bytes(B, S, S); }

}  // namespace dsa
