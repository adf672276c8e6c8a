// Mean-pooled block proxy scores (SCOPE abstract: block-level proxy scores feed
// the mask predictor; the pooling is the block aggregation of ScalingAttention
// Eq. 1 applied to Q and K):
//   qbar_u = mean of the real tokens of block u (fp32), same for kbar_v,
//   S[h][u][v] = scale * <qbar_u, kbar_v>  (fp32).
//
// Two kernels.  The pooling pass reads Q and K once, 16 bytes per lane with rows
// coalesced, and is bound by HBM bandwidth.  The score pass is a small fp32
// product per head (nb x d times d x nb) on fp32 MFMA, tiled 64x64 through LDS.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int NT = 256;

// grid (nb, n_heads, 2): z selects Q (0) or K (1).  Threads split a block's rows
// into row groups; each thread sums 8 consecutive dims over its rows in fp32.
template <int D>
__global__ __launch_bounds__(NT) void pool_kernel(const unsigned short* __restrict__ q,
                                                  const unsigned short* __restrict__ k, int N,
                                                  int nb, float* __restrict__ means) {
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int GROUPS = NT / CPR;      // row groups
  __shared__ float part[GROUPS][D + 1];
  const int u = blockIdx.x, h = blockIdx.y, which = blockIdx.z;
  const unsigned short* x = (which ? k : q) + (size_t)h * N * D;
  const int tid = threadIdx.x;
  const int ch = tid % CPR, rg = tid / CPR;
  const int row0 = 64 * u;
  const int rows = min(64, N - row0);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = rg; r < rows; r += GROUPS) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)(row0 + r) * D + 8 * ch);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += __uint_as_float(w[j] << 16);
      acc[2 * j + 1] += __uint_as_float(w[j] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[rg][8 * ch + j] = acc[j];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int g2 = 0; g2 < GROUPS; ++g2) s += part[g2][tid];
    means[(((size_t)which * gridDim.y + h) * nb + u) * D + tid] = s / (float)rows;
  }
}

// grid (ceil(nb/64), ceil(nb/64), n_heads): one 64x64 output tile per workgroup,
// each wave a 32x32 quarter on v_mfma_f32_32x32x2_f32 (fp32 products, fp32
// accumulation).  The tile's qbar and kbar rows are staged in LDS with a row
// stride of D + 1 floats.  Operand layout (32x32xK MFMA): lane l holds
// A[l % 32][l / 32] and B[l / 32][l % 32]; result register i of lane l is
// element (8 (i / 4) + 4 (l / 32) + i % 4, l % 32).
template <int D>
__global__ __launch_bounds__(NT) void score_kernel(const float* __restrict__ qbar,
                                                   const float* __restrict__ kbar, int nb,
                                                   float scale, float* __restrict__ S) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  constexpr int LD = D + 1;
  __shared__ float qa[64 * LD];   // [row][dim]
  __shared__ float kb[64 * LD];
  const int h = blockIdx.z;
  const int u0 = 64 * blockIdx.y, v0 = 64 * blockIdx.x;
  const int tid = threadIdx.x;
  const float* qh = qbar + (size_t)h * nb * D;
  const float* kh = kbar + (size_t)h * nb * D;
  for (int i = tid; i < 64 * D / 4; i += NT) {
    const int r = i / (D / 4), c4 = i % (D / 4);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (u0 + r < nb) a = *reinterpret_cast<const float4*>(qh + (size_t)(u0 + r) * D + 4 * c4);
    if (v0 + r < nb) b = *reinterpret_cast<const float4*>(kh + (size_t)(v0 + r) * D + 4 * c4);
    float* qd = qa + r * LD + 4 * c4;
    float* kd = kb + r * LD + 4 * c4;
    qd[0] = a.x; qd[1] = a.y; qd[2] = a.z; qd[3] = a.w;
    kd[0] = b.x; kd[1] = b.y; kd[2] = b.z; kd[3] = b.w;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;        // this wave's 32x32 quarter
  const int l32 = lane & 31, kg = lane >> 5;
  const float* arow = qa + (32 * wm + l32) * LD + kg;
  const float* brow = kb + (32 * wn + l32) * LD + kg;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll 16
  for (int k = 0; k < D; k += 2) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(arow[k], brow[k], acc, 0, 0, 0);
  float* Sh = S + (size_t)h * nb * nb;
  const int vv = v0 + 32 * wn + l32;
  if (vv < nb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int uu = u0 + 32 * wm + 8 * (i >> 2) + 4 * kg + (i & 3);
      if (uu < nb) Sh[(size_t)uu * nb + vv] = scale * acc[i];
    }
  }
}

}  // namespace
}  // namespace bsa

extern "C" int block_scores_meanpool(const void* q, const void* k, int n_heads, int seq_len,
                                     int head_dim, int block, float scale, float* scores,
                                     hipStream_t stream) {
  using namespace bsa;
  if (!q || !k || !scores) return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scores, 4))
    return fail(BSA_ERR_INVALID_ARG, "misaligned pointer argument");
  if (n_heads < 1 || seq_len < 1) return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (block != 64) return fail(BSA_ERR_UNSUPPORTED, "only 64-token blocks are implemented");
  if (head_dim != 64 && head_dim != 128)
    return fail(BSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (!std::isfinite(scale)) return fail(BSA_ERR_INVALID_ARG, "scale must be finite");
  const int nb = n_blocks(seq_len, 64);
  if (n_heads > 65535 || nb > 65535)
    return fail(BSA_ERR_INVALID_ARG, "problem too large");
  const size_t mean_bytes = (size_t)2 * n_heads * nb * head_dim * sizeof(float);
  float* means = static_cast<float*>(scratch(mean_bytes, stream));
  if (!means) return BSA_ERR_HIP;
  const float* qbar = means;
  const float* kbar = means + (size_t)n_heads * nb * head_dim;
  const auto* qq = static_cast<const unsigned short*>(q);
  const auto* kk = static_cast<const unsigned short*>(k);
  const dim3 pgrid(nb, n_heads, 2), sgrid((nb + 63) / 64, (nb + 63) / 64, n_heads);
  if (head_dim == 128) {
    hipLaunchKernelGGL(pool_kernel<128>, pgrid, dim3(NT), 0, stream, qq, kk, seq_len, nb, means);
    BSA_CHECK_HIP(hipGetLastError());
    hipLaunchKernelGGL(score_kernel<128>, sgrid, dim3(NT), 0, stream, qbar, kbar, nb, scale, scores);
  } else {
    hipLaunchKernelGGL(pool_kernel<64>, pgrid, dim3(NT), 0, stream, qq, kk, seq_len, nb, means);
    BSA_CHECK_HIP(hipGetLastError());
    hipLaunchKernelGGL(score_kernel<64>, sgrid, dim3(NT), 0, stream, qbar, kbar, nb, scale, scores);
  }
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
