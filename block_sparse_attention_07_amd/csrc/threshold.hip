// Mask instantiation from a threshold map: M = I(T <= p*_h), packed.
//
// ScalingAttention, section 4.1.2 (Eq. 2 and the comparison after it) and
// Appendix A, Algorithm 1 (static block mask generation): a head's threshold
// map records, per block, the smallest sparsity level at which the block is
// active, and the mask for the head's level p* is an element-wise comparison.
//
// One wave builds one 64-bit mask word: lane i compares T[h][u][64 w + i] with
// p*_h (a coalesced 256-byte read per word) and a ballot assembles the word.
// The comparison is float32 and inclusive; NaN compares false.
#include <algorithm>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int NT = 256;

// A wave owns runs of WPW consecutive mask words: lane j tests key 64 w + j of
// each word, the WPW loads are issued before the WPW ballots, and lane k then
// stores word k of the run.
constexpr int WPW = 8;

__global__ __launch_bounds__(NT) void threshold_kernel(const float* __restrict__ T,
                                                       const float* __restrict__ p_head, int nq,
                                                       int nk, int W, long long words,
                                                       uint64_t* __restrict__ mask) {
  const int lane = threadIdx.x & 63;
  const long long runs = (words + WPW - 1) / WPW;
  const long long stride = (long long)gridDim.x * (NT / 64);
  for (long long run = (long long)blockIdx.x * (NT / 64) + (threadIdx.x >> 6); run < runs; run += stride) {
    const long long w0 = run * WPW;
    long long row = w0 / W;
    int w = (int)(w0 - row * W);
    int h = (int)(row / nq);
    int u = (int)(row - (long long)h * nq);
    float ph = p_head[h];
    bool keep[WPW];
#pragma unroll
    for (int k = 0; k < WPW; ++k) {
      const int v = 64 * w + lane;
      keep[k] = false;
      if (w0 + k < words && v < nk) keep[k] = T[(size_t)row * nk + v] <= ph;
      if (++w == W) {
        w = 0;
        ++row;
        if (++u == nq && w0 + k + 1 < words) {
          u = 0;
          ph = p_head[++h];
        }
      }
    }
    uint64_t mine = 0;
#pragma unroll
    for (int k = 0; k < WPW; ++k) {
      const uint64_t bits = __ballot(keep[k]);
      if (lane == k) mine = bits;
    }
    if (lane < WPW && w0 + lane < words) mask[w0 + lane] = mine;
  }
}

}  // namespace
}  // namespace bsa

extern "C" int mask_from_threshold_map(const float* thresholds, const float* p_head, int n_heads,
                                       int n_q_blocks, int n_k_blocks, uint64_t* mask_bits,
                                       hipStream_t stream) {
  using namespace bsa;
  if (!thresholds || !p_head || !mask_bits) return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(thresholds, 4) || !aligned(p_head, 4) || !aligned(mask_bits, 8))
    return fail(BSA_ERR_INVALID_ARG, "misaligned pointer argument");
  if (n_heads < 1 || n_q_blocks < 1 || n_k_blocks < 1)
    return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  const long long rows = (long long)n_heads * n_q_blocks;
  if (rows > 0x7fffffffLL) return fail(BSA_ERR_INVALID_ARG, "problem too large");
  const int W = n_words(n_k_blocks);
  const long long words = rows * W;
  const long long waves_per_block = NT / 64;
  const long long runs = (words + WPW - 1) / WPW;
  const long long blocks = std::min<long long>((runs + waves_per_block - 1) / waves_per_block, 1 << 16);
  hipLaunchKernelGGL(threshold_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, thresholds, p_head,
                     n_q_blocks, n_k_blocks, W, words, mask_bits);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
