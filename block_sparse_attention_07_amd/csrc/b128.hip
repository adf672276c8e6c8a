// ScalingAttention's own mask granularity: 128 x 128-token blocks, rows packed in 32-bit
// words.
//
// ScalingAttention, section 4.3.2: the CRM row mask is an aligned uint32 array,
// one bit per KV block of 128 tokens, so one word covers 32 blocks; Appendix E,
// Algorithm 2 walks it with a base that advances 32 per word.
//
// Such a mask is the same mask over 64-token blocks with every bit doubled in
// both directions: 64-block (u, v) is kept iff 128-block (u/2, v/2) is.  Word w
// of a 32-bit row covers 128-blocks 32w..32w+31, i.e. 64-blocks 64w..64w+63,
// which is word w of the 64-bit row, so the expansion is word for word: spread
// the 32 bits to the even positions and copy each to the odd one above it; 64-row
// u reads 128-row u/2.  The two 64-rows of every 128-row are then identical, the
// planner pairs them, and the 128-query workgroups fetch each K/V tile once for
// both, which is the K/V feed per flop of a 128 x 128 tile.
#include <algorithm>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int NT = 256;

// Bit b of x moves to bit 2b (interleave with zeros by the usual shift-and-mask
// ladder: halves, bytes, nibbles, pairs, single bits).
__device__ __forceinline__ uint64_t spread_even(uint32_t x32) {
  uint64_t x = x32;
  x = (x | (x << 16)) & 0x0000FFFF0000FFFFull;
  x = (x | (x << 8)) & 0x00FF00FF00FF00FFull;
  x = (x | (x << 4)) & 0x0F0F0F0F0F0F0F0Full;
  x = (x | (x << 2)) & 0x3333333333333333ull;
  x = (x | (x << 1)) & 0x5555555555555555ull;
  return x;
}

__global__ __launch_bounds__(NT) void expand_b128_kernel(const uint32_t* __restrict__ in, int nb64,
                                                         int nb128, int W, uint64_t lastmask,
                                                         long long words,
                                                         uint64_t* __restrict__ out) {
  const long long stride = (long long)gridDim.x * NT;
  for (long long i = (long long)blockIdx.x * NT + threadIdx.x; i < words; i += stride) {
    const long long row = i / W;
    const int w = (int)(i - row * W);
    const int h = (int)(row / nb64);
    const int u = (int)(row - (long long)h * nb64);
    const uint64_t e = spread_even(in[((size_t)h * nb128 + (u >> 1)) * W + w]);
    uint64_t y = e | (e << 1);
    if (w == W - 1) y &= lastmask;
    out[i] = y;
  }
}

}  // namespace

int launch_expand_b128(const uint32_t* mask_words, int n_heads, int seq_len, uint64_t* mask_bits,
                       hipStream_t stream) {
  const int nb64 = n_blocks(seq_len, 64);
  const int nb128 = n_blocks(seq_len, 128);
  const int W = n_words(nb64);
  const int tail = nb64 - 64 * (W - 1);
  const uint64_t lastmask = tail == 64 ? ~0ull : ((1ull << tail) - 1);
  const long long words = (long long)n_heads * nb64 * W;
  const long long blocks = std::min<long long>((words + NT - 1) / NT, 1 << 16);
  hipLaunchKernelGGL(expand_b128_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, mask_words, nb64,
                     nb128, W, lastmask, words, mask_bits);
  BSA_CHECK_HIP(hipGetLastError());
  return BSA_OK;
}

}  // namespace bsa

extern "C" int mask_b128_to_b64(const uint32_t* mask_words, int n_heads, int seq_len,
                                uint64_t* mask_bits, hipStream_t stream) {
  using namespace bsa;
  if (!mask_words || !mask_bits) return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(mask_words, 4) || !aligned(mask_bits, 8))
    return fail(BSA_ERR_INVALID_ARG, "misaligned pointer argument");
  if (n_heads < 1 || seq_len < 1)
    return fail(BSA_ERR_INVALID_ARG, "n_heads (%d) and seq_len (%d) must be >= 1", n_heads, seq_len);
  if ((long long)n_heads * n_blocks(seq_len, 64) > 0x7fffffffLL)
    return fail(BSA_ERR_INVALID_ARG, "problem too large");
  int rc = launch_expand_b128(mask_words, n_heads, seq_len, mask_bits, stream);
  return rc ? rc : ok();
}

extern "C" int sparse_attn_fwd_b128(const void* q, const void* k, const void* v,
                                    const uint32_t* mask_words, int n_heads, int seq_len,
                                    int head_dim, float scale, void* out, hipStream_t stream) {
  using namespace bsa;
  int rc = check_attn_args(q, k, v, mask_words, out, n_heads, seq_len, head_dim, 64, 64, scale, 16, 4);
  if (rc) return rc;
  const int nb = n_blocks(seq_len, 64);
  const size_t rows = (size_t)n_heads * nb;
  const size_t off_tiles = (rows * 4 + 255) & ~size_t(255);
  const size_t off_order = (off_tiles + (size_t)n_heads * 8 + 255) & ~size_t(255);
  const size_t off_mask = (off_order + rows * 4 + 255) & ~size_t(255);
  const size_t off_vt = (off_mask + rows * n_words(nb) * 8 + 255) & ~size_t(255);
  ScratchLease lease(off_vt + vt_bytes(n_heads, seq_len, head_dim));
  char* ws = static_cast<char*>(lease.get());
  if (!ws) return BSA_ERR_HIP;
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  int64_t* tiles = reinterpret_cast<int64_t*>(ws + off_tiles);
  int32_t* order = reinterpret_cast<int32_t*>(ws + off_order);
  uint64_t* mask = reinterpret_cast<uint64_t*>(ws + off_mask);
  rc = launch_expand_b128(mask_words, n_heads, seq_len, mask, stream);
  if (rc) return rc;
  rc = launch_plan(mask, n_heads, seq_len, counts, tiles, order, stream);
  if (rc) return rc;
  return launch_attn_bf16(q, k, v, mask, order, n_heads, seq_len, head_dim, scale, out, ws + off_vt,
                          stream);
}
