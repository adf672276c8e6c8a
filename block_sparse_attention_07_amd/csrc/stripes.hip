// PSA stripe tuples -> packed row masks (PSA page, Figure 3, Appendix Tables 7-9).
//
// The kept test factorises into a temporal test on the frame distance and a
// spatial test on the spatial-block distance.  When frames hold whole blocks
// (and at most 64 of them), a row's mask is its spatial pattern repeated over
// the frames its temporal test keeps: one wave per row builds the pattern with a
// ballot and each lane assembles whole words from the frames a word overlaps.
// Otherwise one thread per output word places its query block and each of the
// word's 64 key blocks in (frame, spatial block) coordinates and applies both
// tests.  Integer arithmetic only, either way.
#include "bsa_internal.h"

namespace bsa {
namespace {

struct Coords {
  int per;            // blocks per frame when frames hold whole blocks, else 0
  int frame_tokens;
};

__device__ __forceinline__ void place(int b, const Coords& cd, int& t, int& s) {
  if (cd.per) {
    t = b / cd.per;
    s = b - t * cd.per;
  } else {
    const long long first = (long long)b * 64;
    t = (int)(first / cd.frame_tokens);
    s = (int)((first - (long long)t * cd.frame_tokens) / 64);
  }
}

// Band of `width` distances centred on `offset`, repeating with period
// width + gap when gap > 0.  Non-positive widths or negative gaps keep nothing.
__device__ __forceinline__ bool in_stripe(int dist, int width, int offset, int gap) {
  if (width < 1 || gap < 0) return false;
  const int x = dist - offset + width / 2;
  if (gap == 0) return x >= 0 && x < width;
  const int period = width + gap;
  int r = x % period;
  if (r < 0) r += period;
  return r < width;
}

__global__ void stripes_kernel(const int32_t* __restrict__ params, long long total, int nb, int W,
                               Coords cd, uint64_t* __restrict__ mask) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int w = (int)(idx % W);
  const long long row = idx / W;
  const int u = (int)(row % nb);
  const int h = (int)(row / nb);
  const int32_t* p = params + 7 * h;
  const int full = p[0], tw = p[1], to = p[2], ts = p[3], sw = p[4], so = p[5], ss = p[6];
  int tu, su;
  place(u, cd, tu, su);
  uint64_t word = 0;
  const int v0 = 64 * w;
  const int vend = min(v0 + 64, nb);
  for (int v = v0; v < vend; ++v) {
    bool keep = full != 0;
    if (!keep) {
      int tv, sv;
      place(v, cd, tv, sv);
      keep = in_stripe(tv - tu, tw, to, ts) && in_stripe(sv - su, sw, so, ss);
    }
    if (keep) word |= 1ull << (v - v0);
  }
  mask[idx] = word;
}

// Frames of `per` whole blocks, per <= 64; one wave per row (h, u), 4 rows per
// workgroup.
__global__ __launch_bounds__(256) void stripes_aligned_kernel(const int32_t* __restrict__ params, int n_rows,
                                                              int nb, int W, int per,
                                                              uint64_t* __restrict__ mask) {
  const int row = (int)((blockIdx.x * 256u + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;                 // uniform per wave
  const int h = row / nb, u = row - h * nb;
  const int32_t* p = params + 7 * h;
  const int full = p[0], tw = p[1], to = p[2], ts = p[3], sw = p[4], so = p[5], ss = p[6];
  uint64_t* out = mask + (size_t)row * W;
  const int tail = nb & 63;
  const uint64_t lastmask = tail ? ((1ull << tail) - 1ull) : ~0ull;
  if (full) {
    for (int w = lane; w < W; w += 64) out[w] = w == W - 1 ? lastmask : ~0ull;
    return;
  }
  const int tu = u / per, su = u - tu * per;
  // bit sv: spatial block sv of a frame passes the spatial test; bit tv (for the
  // first 64 frames): frame tv passes the temporal test
  const uint64_t sp = __ballot(lane < per && in_stripe(lane - su, sw, so, ss));
  const uint64_t tp = __ballot(in_stripe(lane - tu, tw, to, ts));
  for (int w = lane; w < W; w += 64) {
    const int v0 = 64 * w;
    const int vend = min(v0 + 64, nb);
    uint64_t word = 0;
    for (int tv = v0 / per; tv * per < vend; ++tv) {
      if (tv < 64 ? !((tp >> tv) & 1ull) : !in_stripe(tv - tu, tw, to, ts)) continue;
      const int lo = max(v0, tv * per), hi = min(vend, (tv + 1) * per);
      const int n = hi - lo;                  // 1 .. 64 blocks of frame tv in this word
      const uint64_t seg = n == 64 ? ~0ull : ((1ull << n) - 1ull);
      word |= ((sp >> (lo - tv * per)) & seg) << (lo - v0);
    }
    out[w] = word;
  }
}

}  // namespace
}  // namespace bsa

extern "C" int mask_from_stripes(const int32_t* params, int n_heads, int n_frames, int frame_tokens,
                                 int seq_len, int block, uint64_t* mask_bits, hipStream_t stream) {
  using namespace bsa;
  if (!params || !mask_bits) return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(params, 4) || !aligned(mask_bits, 8))
    return fail(BSA_ERR_INVALID_ARG, "misaligned pointer argument");
  if (n_heads < 1 || n_frames < 1 || frame_tokens < 1 || seq_len < 1)
    return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  if ((long long)n_frames * frame_tokens != seq_len)
    return fail(BSA_ERR_INVALID_ARG, "n_frames * frame_tokens (%lld) != seq_len (%d)",
                (long long)n_frames * frame_tokens, seq_len);
  if (block != 64) return fail(BSA_ERR_UNSUPPORTED, "only 64-token blocks are implemented");
  const int nb = n_blocks(seq_len, 64);
  const int W = n_words(nb);
  const long long total = (long long)n_heads * nb * W;
  if (total > (1LL << 40)) return fail(BSA_ERR_INVALID_ARG, "problem too large");
  Coords cd{frame_tokens % 64 == 0 ? frame_tokens / 64 : 0, frame_tokens};
  if (cd.per >= 1 && cd.per <= 64) {
    const int n_rows = n_heads * nb;
    hipLaunchKernelGGL(stripes_aligned_kernel, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, stream, params,
                       n_rows, nb, W, cd.per, mask_bits);
    BSA_CHECK_HIP(hipGetLastError());
    return ok();
  }
  const long long grid = (total + 255) / 256;
  hipLaunchKernelGGL(stripes_kernel, dim3((unsigned)grid), dim3(256), 0, stream, params, total, nb, W,
                     cd, mask_bits);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
