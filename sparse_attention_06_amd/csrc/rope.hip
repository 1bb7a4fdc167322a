// Partial RoPE of the indexer inputs, concatenated layout (gfx950).
//
// Source: "DeepSeek3.2: Onboard sparse attention", What this PR does, item 1,
// Indexer: the indexer applies partial RoPE to q and k with the same YaRN
// frequencies as MLA, in the concatenated rather than the interleaved layout.
// Here the frequencies arrive as cos/sin tables indexed by position; the first
// rope_dim dims of every vector rotate, dim i paired with i + rope_dim/2:
//   y_i     = x_i c_i - x_{i+h} s_i,   y_{i+h} = x_{i+h} c_i + x_i s_i,
// each product and each sum rounded to float32 (no fused multiply-add), the
// result rounded to bf16. The other dims are copied.
//
// One thread per work item of a vector: item j < h/8 rotates the 8-element
// chunk at 8j together with its partner chunk h dims later; when the output is
// a separate buffer, the remaining items copy the chunks past the rotated part
// (in place there is nothing to copy). 16-byte loads and stores; HBM-bound.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

// x and out may be the same buffer: every element is read and written by one thread only
__global__ __launch_bounds__(256) void rope_rows_kernel(const uint16_t* x, int64_t nvec, int nh,
                                                        int S, int D, int h, int P, const float* __restrict__ ct,
                                                        const float* __restrict__ st,
                                                        const int32_t* __restrict__ pos,
                                                        uint16_t* out) {
  const int nrot = h / 8;                             // rotating items per vector
  const int ipv = nrot + (x != out ? (D - 2 * h) / 8 : 0);  // items per vector
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= nvec * ipv) return;
  const int64_t v = gid / ipv;
  const int j = (int)(gid % ipv);
  const int64_t tok = v / nh;  // b * S + t
  const uint16_t* xv = x + v * D;
  uint16_t* ov = out + v * D;
  if (j >= nrot) {  // past the rotated part: copy
    const int c = 2 * h + 8 * (j - nrot);
    *(u32x4*)(ov + c) = *(const u32x4*)(xv + c);
    return;
  }
  const int c0 = 8 * j;
  // positions outside the tables are clamped to them (an out-of-range
  // position gives a wrong rotation, never an out-of-bounds read)
  const int p = min(max(pos ? pos[tok] : (int)(tok % S), 0), P - 1);
  const u32x4 ra = *(const u32x4*)(xv + c0), rb = *(const u32x4*)(xv + c0 + h);
  const float* cp = ct + (size_t)p * h + c0;
  const float* sp = st + (size_t)p * h + c0;
  float ya[8], yb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // each product and sum is rounded on its own: no contraction into v_fma
#pragma clang fp contract(off)
    const uint32_t wa = ra[e >> 1], wb = rb[e >> 1];
    const float a = bf2f((uint16_t)((e & 1) ? (wa >> 16) : (wa & 0xffff)));
    const float b = bf2f((uint16_t)((e & 1) ? (wb >> 16) : (wb & 0xffff)));
    const float c = cp[e], s = sp[e];
    ya[e] = a * c - b * s;
    yb[e] = b * c + a * s;
  }
  *(u32x4*)(ov + c0) = u32x4{pack_bf2(ya[0], ya[1]), pack_bf2(ya[2], ya[3]), pack_bf2(ya[4], ya[5]),
                             pack_bf2(ya[6], ya[7])};
  *(u32x4*)(ov + c0 + h) = u32x4{pack_bf2(yb[0], yb[1]), pack_bf2(yb[2], yb[3]), pack_bf2(yb[4], yb[5]),
                                 pack_bf2(yb[6], yb[7])};
}

hipError_t launch_rope_rows(const void* x, int B, int S, int nh, int D, int rope_dim, int P, const float* cos_t,
                            const float* sin_t, const int32_t* pos, void* out, hipStream_t st) {
  const int64_t nvec = (int64_t)B * S * nh;
  const int64_t nthr = nvec * (rope_dim / 16 + (x != out ? (D - rope_dim) / 8 : 0));
  const dim3 grid((unsigned)((nthr + 255) / 256)), block(256);
  hipLaunchKernelGGL(rope_rows_kernel, grid, block, 0, st, (const uint16_t*)x, nvec, nh, S, D, rope_dim / 2, P,
                     cos_t, sin_t, pos, (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace dsa
