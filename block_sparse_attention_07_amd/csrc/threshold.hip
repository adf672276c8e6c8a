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

__global__ __launch_bounds__(NT) void threshold_kernel(const float* __restrict__ T,
                                                       const float* __restrict__ p_head, int nq,
                                                       int nk, int W, long long words,
                                                       uint64_t* __restrict__ mask) {
  const int lane = threadIdx.x & 63;
  const long long stride = (long long)gridDim.x * (NT / 64);
  for (long long wid = (long long)blockIdx.x * (NT / 64) + (threadIdx.x >> 6); wid < words; wid += stride) {
    const long long row = wid / W;
    const int w = (int)(wid - row * W);
    const int h = (int)(row / nq);
    const int v = 64 * w + lane;
    bool keep = false;
    if (v < nk) keep = T[(size_t)row * nk + v] <= p_head[h];
    const uint64_t bits = __ballot(keep);
    if (lane == 0) mask[wid] = bits;
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
  const long long blocks = std::min<long long>((words + waves_per_block - 1) / waves_per_block, 1 << 16);
  hipLaunchKernelGGL(threshold_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, thresholds, p_head,
                     n_q_blocks, n_k_blocks, W, words, mask_bits);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
