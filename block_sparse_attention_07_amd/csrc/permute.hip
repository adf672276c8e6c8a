// Token gather / scatter along a permutation (Hilbert-ordered attention: DFSAttn
// abstract for the reordering, SCOPE abstract for attending over the original
// keys/values and mapping outputs back).  16 bytes per thread, rows of one
// head contiguous, so both the reads and the writes of a row are coalesced.
#include "bsa_internal.h"

namespace bsa {
namespace {

__global__ void permute_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ perm,
                               int n_heads, int N, int cpr, int inverse, uint4* __restrict__ y) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long per_head = (long long)N * cpr;
  if (idx >= per_head * n_heads) return;
  const int h = (int)(idx / per_head);
  const long long rem = idx - h * per_head;
  const int i = (int)(rem / cpr);
  const int ch = (int)(rem - (long long)i * cpr);
  const int j = perm[i];
  if (j < 0 || j >= N) return;
  const long long base = h * per_head;
  if (inverse)
    y[base + (long long)j * cpr + ch] = x[base + (long long)i * cpr + ch];
  else
    y[base + (long long)i * cpr + ch] = x[base + (long long)j * cpr + ch];
}

}  // namespace
}  // namespace bsa

extern "C" int permute_tokens(const void* x, const int32_t* perm, int n_heads, int seq_len,
                              int head_dim, int elem_bytes, int inverse, void* y,
                              hipStream_t stream) {
  using namespace bsa;
  if (!x || !perm || !y) return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (x == y) return fail(BSA_ERR_INVALID_ARG, "x and y must not alias");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(perm, 4))
    return fail(BSA_ERR_INVALID_ARG, "misaligned pointer argument");
  if (n_heads < 1 || seq_len < 1 || head_dim < 1) return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (elem_bytes != 2 && elem_bytes != 4) return fail(BSA_ERR_UNSUPPORTED, "elem_bytes must be 2 or 4");
  if ((head_dim * elem_bytes) % 16) return fail(BSA_ERR_UNSUPPORTED, "row bytes must be a multiple of 16");
  const int cpr = head_dim * elem_bytes / 16;
  const long long total = (long long)n_heads * seq_len * cpr;
  if (total > (1LL << 40)) return fail(BSA_ERR_INVALID_ARG, "problem too large");
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint4*>(x), perm, n_heads, seq_len, cpr, inverse ? 1 : 0,
                     static_cast<uint4*>(y));
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
