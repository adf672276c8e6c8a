// Block-sparse attention forward in fp32 throughout (reference-precision path).
//
// Same operation as the bf16 kernel (ScalingAttention, section 4.3.2).  The kept
// key blocks are visited exactly as the CRM forward iterator of Appendix E,
// Algorithm 2 walks them: per mask word, report base + count-trailing-zeros and
// clear the lowest set bit until the word is empty.  Each kept block is processed
// as four 16-key sub-tiles with an online softmax; math is plain fp32 VALU.
#include <cmath>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int NT = 256;
constexpr int SUB = 16;

template <int D>
__global__ __launch_bounds__(NT) void attn_fwd_f32_kernel(const float* __restrict__ Q,
                                                          const float* __restrict__ K,
                                                          const float* __restrict__ V,
                                                          const uint64_t* __restrict__ mask,
                                                          int N, int nb, int W, float scale,
                                                          float* __restrict__ O) {
  constexpr int DQ = D / 4;   // output columns per thread
  __shared__ float qs[64][D + 1];
  __shared__ float ks[SUB][D + 1];
  __shared__ float vs[SUB][D + 1];
  __shared__ float ss[64][SUB + 1];

  const int tid = threadIdx.x;
  const int r = tid >> 2;        // query row within the block
  const int qd = tid & 3;        // which quarter of the columns / sub-tile keys
  const int h = blockIdx.x / nb;
  const int u = blockIdx.x - h * nb;
  const size_t head_off = (size_t)h * N * D;
  const uint64_t* mrow = mask + ((size_t)h * nb + u) * W;

  for (int i = tid; i < 64 * D; i += NT) {
    const int row = i / D, col = i % D;
    const int g = 64 * u + row;
    qs[row][col] = g < N ? Q[head_off + (size_t)g * D + col] : 0.f;
  }

  float acc[DQ];
#pragma unroll
  for (int j = 0; j < DQ; ++j) acc[j] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int tail = nb & 63;

  for (int w = 0; w < W; ++w) {
    uint64_t word = mrow[w];
    if (w == W - 1 && tail) word &= (1ull << tail) - 1ull;
    const int base = 64 * w;
    while (word) {
      const int vb = base + __ffsll((unsigned long long)word) - 1;
      word &= word - 1ull;
      for (int s0 = 0; s0 < 64; s0 += SUB) {
        const int key0 = 64 * vb + s0;
        if (key0 >= N) break;
        __syncthreads();
        for (int i = tid; i < SUB * D; i += NT) {
          const int kr = i / D, col = i % D;
          const int g = key0 + kr;
          ks[kr][col] = g < N ? K[head_off + (size_t)g * D + col] : 0.f;
          vs[kr][col] = g < N ? V[head_off + (size_t)g * D + col] : 0.f;
        }
        __syncthreads();
        for (int jj = 0; jj < SUB / 4; ++jj) {
          const int j = qd * (SUB / 4) + jj;
          float dot = 0.f;
          for (int c2 = 0; c2 < D; ++c2) dot = fmaf(qs[r][c2], ks[j][c2], dot);
          ss[r][j] = (key0 + j < N) ? dot * scale : -INFINITY;
        }
        __syncthreads();
        float mt = ss[r][0];
        for (int j = 1; j < SUB; ++j) mt = fmaxf(mt, ss[r][j]);
        const float mn = fmaxf(m, mt);
        const float alpha = expf(m - mn);
        float ps = 0.f;
#pragma unroll
        for (int c2 = 0; c2 < DQ; ++c2) acc[c2] *= alpha;
        for (int j = 0; j < SUB; ++j) {
          const float p = expf(ss[r][j] - mn);
          ps += p;
#pragma unroll
          for (int c2 = 0; c2 < DQ; ++c2) acc[c2] = fmaf(p, vs[j][qd * DQ + c2], acc[c2]);
        }
        l = l * alpha + ps;
        m = mn;
      }
    }
  }
  const int g = 64 * u + r;
  if (g < N) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    float* orow = O + head_off + (size_t)g * D + qd * DQ;
#pragma unroll
    for (int c2 = 0; c2 < DQ; ++c2) orow[c2] = acc[c2] * inv;
  }
}

}  // namespace
}  // namespace bsa

extern "C" int sparse_attn_fwd_f32(const float* q, const float* k, const float* v,
                                   const uint64_t* mask_bits, int n_heads, int seq_len,
                                   int head_dim, int block_q, int block_k, float scale, float* out,
                                   hipStream_t stream) {
  using namespace bsa;
  int rc = check_attn_args(q, k, v, mask_bits, out, n_heads, seq_len, head_dim, block_q, block_k,
                           scale, 16);
  if (rc) return rc;
  const int nb = n_blocks(seq_len, 64);
  const int W = n_words(nb);
  const dim3 grid((unsigned)(n_heads * nb)), block(NT);
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, block, 0, stream, q, k, v, mask_bits,
                       seq_len, nb, W, scale, out);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, block, 0, stream, q, k, v, mask_bits,
                       seq_len, nb, W, scale, out);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
