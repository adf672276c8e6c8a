// Host-only 3D Hilbert token order (DFSAttn abstract names Hilbert-curve token
// reordering; the construction is J. Skilling, "Programming the Hilbert curve",
// AIP Conf. Proc. 707, 2004).
//
// Each token's (t, y, x) is converted to Skilling's "transposed" Hilbert form:
// walking the bit levels from the top, axis 0's low bits are inverted or
// exchanged with axis i's depending on axis i's bit at that level; a Gray-code
// pass across axes and a final correction mask follow.  The curve index is the
// bits of the transposed coordinates interleaved from the top level down, axis
// 0 first.  Tokens are then sorted by index (indices are distinct).
#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

#include "bsa_internal.h"

namespace bsa {
namespace {

uint64_t hilbert_index3(uint32_t a0, uint32_t a1, uint32_t a2, int bits) {
  uint32_t x[3] = {a0, a1, a2};
  for (uint32_t q = 1u << (bits - 1); q > 1; q >>= 1) {
    const uint32_t low = q - 1;
    for (int i = 0; i < 3; ++i) {
      if (x[i] & q) {
        x[0] ^= low;
      } else {
        const uint32_t t = (x[0] ^ x[i]) & low;
        x[0] ^= t;
        x[i] ^= t;
      }
    }
  }
  x[1] ^= x[0];
  x[2] ^= x[1];
  uint32_t fix = 0;
  for (uint32_t q = 1u << (bits - 1); q > 1; q >>= 1)
    if (x[2] & q) fix ^= q - 1;
  for (int i = 0; i < 3; ++i) x[i] ^= fix;
  uint64_t idx = 0;
  for (int b = bits - 1; b >= 0; --b)
    for (int i = 0; i < 3; ++i) idx = (idx << 1) | ((x[i] >> b) & 1u);
  return idx;
}

}  // namespace
}  // namespace bsa

extern "C" int hilbert3d_order(int T, int H, int W, int32_t* perm_host) {
  using namespace bsa;
  if (!perm_host) return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (T < 1 || H < 1 || W < 1) return fail(BSA_ERR_INVALID_ARG, "grid sizes must be >= 1");
  const long long n = (long long)T * H * W;
  if (n >= (1LL << 31)) return fail(BSA_ERR_INVALID_ARG, "grid too large");
  int m = std::max(T, std::max(H, W)) - 1;
  int bits = 1;
  while ((1 << bits) <= m) ++bits;
  if (bits > 21) return fail(BSA_ERR_INVALID_ARG, "grid side too large");
  std::vector<std::pair<uint64_t, int32_t>> keyed((size_t)n);
  size_t id = 0;
  for (int t = 0; t < T; ++t)
    for (int y = 0; y < H; ++y)
      for (int x = 0; x < W; ++x, ++id)
        keyed[id] = {hilbert_index3((uint32_t)t, (uint32_t)y, (uint32_t)x, bits), (int32_t)id};
  std::sort(keyed.begin(), keyed.end());
  for (size_t i = 0; i < keyed.size(); ++i) perm_host[i] = keyed[i].second;
  return ok();
}
