// Tile scheduler: per-row kept-block counts, per-head totals and a work order.
//
// The packed row mask (ScalingAttention, section 4.3.2) already tells how many
// kept tiles each (head, query block) row will run; a popcount pass turns that
// into a schedule, and adjacent rows with identical masks are paired so that
// one workgroup serves both.  Heads run in decreasing total work so the heaviest heads are
// dispatched first and the lightest fill the tail.  Within a head, rows run in
// decreasing kept-block count: the workgroups resident at the same time then
// hold rows of nearly equal length, start together, walk their ascending tile
// lists at the same pace and finish together, so tiles one of them fetches are
// still in the XCD's L2 when the others ask for them.
#include "bsa_internal.h"

namespace bsa {
namespace {

__global__ void fill_i64_kernel(int64_t* __restrict__ p, int n, int64_t value) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

// One wave per row: lane w reads word w (coalesced), popcounts it, and the wave
// sums the counts.  Each workgroup adds its rows' counts to the head totals
// with one atomic per head it touches (rows of a workgroup are consecutive).
constexpr int RC_THREADS = 256;
constexpr int RC_ROWS_PER_WAVE = 4;
constexpr int RC_ROWS = RC_THREADS / 64 * RC_ROWS_PER_WAVE;   // rows per workgroup

__global__ __launch_bounds__(RC_THREADS) void row_counts_kernel(const uint64_t* __restrict__ mask,
                                                                int n_rows, int nb, int W,
                                                                uint64_t lastmask,
                                                                int32_t* __restrict__ counts,
                                                                int64_t* __restrict__ head_tiles) {
  __shared__ int wave_sum[RC_ROWS];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * RC_ROWS;
  for (int k = 0; k < RC_ROWS_PER_WAVE; ++k) {
    const int slot = wave * RC_ROWS_PER_WAVE + k;
    const int row = row0 + slot;
    int c = 0;
    if (row < n_rows) {
      const uint64_t* m = mask + (size_t)row * W;
      for (int w = lane; w < W; w += 64) c += __popcll(w == W - 1 ? (m[w] & lastmask) : m[w]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if (lane == 0) {
      wave_sum[slot] = c;
      if (row < n_rows) counts[row] = c;
    }
  }
  __syncthreads();
  // rows row0 .. row0 + RC_ROWS - 1 belong to heads h_first .. h_last
  if (threadIdx.x < RC_ROWS) {
    const int row = row0 + (int)threadIdx.x;
    if (row < n_rows) {
      const int h = row / nb;
      // the first row of each head within this workgroup sums that head's rows
      if (threadIdx.x == 0 || (row - 1) / nb != h) {
        int64_t sum = 0;
        for (int j = threadIdx.x; j < RC_ROWS && row0 + j < n_rows && (row0 + j) / nb == h; ++j) sum += wave_sum[j];
        atomicAdd(reinterpret_cast<unsigned long long*>(head_tiles + h), (unsigned long long)sum);
      }
    }
  }
}

// One workgroup per head: rank the head among all heads (more work first, ties
// by head index), then lay out the head's segment of nb work slots.  Adjacent
// query blocks (u, u+1), u even, whose mask rows are identical become one pair
// entry (2 H nb ... : value H nb + h nb + u), processed by 128-query workgroups;
// the other rows are single entries (h nb + u); the slots freed by pairs hold -1.
// Within the segment: pairs, then singles, each in decreasing kept-block count
// (ties by query block), then the -1 slots.
constexpr int SORT_MAX_NB = 8192;   // rows per head ranked in LDS; longer heads keep u order, no pairs
constexpr int HO_THREADS = 1024;

__global__ __launch_bounds__(HO_THREADS) void head_order_kernel(const int64_t* __restrict__ head_tiles,
                                                                const int32_t* __restrict__ counts,
                                                                const uint64_t* __restrict__ mask,
                                                                int n_heads, int nb, int W,
                                                                uint64_t lastmask,
                                                                int32_t* __restrict__ order) {
  __shared__ int partial[HO_THREADS / 64];
  __shared__ uint32_t srt[SORT_MAX_NB];
  __shared__ unsigned char pair[SORT_MAX_NB / 2];
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int64_t mine = head_tiles[h];
  int before = 0;
  for (int j = tid; j < n_heads; j += HO_THREADS) {
    const int64_t t = head_tiles[j];
    before += (t > mine) || (t == mine && j < h);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) before += __shfl_xor(before, off);
  if ((tid & 63) == 0) partial[tid >> 6] = before;
  const bool sort_rows = nb <= SORT_MAX_NB;
  if (sort_rows) {
    for (int i = tid; i < nb / 2; i += HO_THREADS) {
      const uint64_t* r0 = mask + ((size_t)h * nb + 2 * i) * W;
      const uint64_t* r1 = r0 + W;
      bool eq = true;
      for (int w = 0; w < W && eq; ++w) {
        const uint64_t m = (w == W - 1) ? lastmask : ~0ull;
        eq = ((r0[w] ^ r1[w]) & m) == 0;
      }
      pair[i] = eq;
    }
  }
  __syncthreads();
  int rank = 0;
#pragma unroll
  for (int i = 0; i < HO_THREADS / 64; ++i) rank += partial[i];
  int32_t* dst = order + (size_t)rank * nb;
  const int total = n_heads * nb;
  if (!sort_rows) {
    for (int u = tid; u < nb; u += HO_THREADS) dst[u] = h * nb + u;
    return;
  }
  // Sort key: class (0 pair lead, 1 single, 2 pair follower), then count
  // descending, then u ascending -- one unique 30-bit value per row, sorted
  // ascending by a bitonic network over the next power of two (padding sorts
  // last).
  int P = 1;
  while (P < nb) P <<= 1;
  for (int u = tid; u < P; u += HO_THREADS) {
    uint32_t v = 0xFFFFFFFFu;
    if (u < nb) {
      const bool paired = (u >> 1) < nb / 2 && pair[u >> 1];
      const uint32_t cls = paired ? ((u & 1) ? 2u : 0u) : 1u;
      const uint32_t key = (cls << 15) + (16383u - (uint32_t)counts[(size_t)h * nb + u]);
      v = (key << 13) | (uint32_t)u;
    }
    srt[u] = v;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += HO_THREADS) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t a = srt[i], b = srt[l];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            srt[i] = b;
            srt[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < nb; r += HO_THREADS) {
    const uint32_t v = srt[r];
    const int u = (int)(v & 8191u);
    const uint32_t cls = v >> 28;
    dst[r] = cls == 0 ? total + h * nb + u : (cls == 1 ? h * nb + u : -1);
  }
}

}  // namespace

int launch_plan(const uint64_t* mask, int n_heads, int seq_len, int32_t* counts, int64_t* head_tiles,
                int32_t* order, hipStream_t stream) {
  const int nb = n_blocks(seq_len, 64);
  const int W = n_words(nb);
  const int rows = n_heads * nb;
  const int tail = nb & 63;
  const uint64_t lastmask = tail ? ((1ull << tail) - 1ull) : ~0ull;
  hipLaunchKernelGGL(fill_i64_kernel, dim3((n_heads + 255) / 256), dim3(256), 0, stream, head_tiles,
                     n_heads, (int64_t)0);
  BSA_CHECK_HIP(hipGetLastError());
  hipLaunchKernelGGL(row_counts_kernel, dim3((rows + RC_ROWS - 1) / RC_ROWS), dim3(RC_THREADS), 0, stream,
                     mask, rows, nb, W, lastmask, counts, head_tiles);
  BSA_CHECK_HIP(hipGetLastError());
  hipLaunchKernelGGL(head_order_kernel, dim3(n_heads), dim3(HO_THREADS), 0, stream, head_tiles, counts,
                     mask, n_heads, nb, W, lastmask, order);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}

}  // namespace bsa

extern "C" int sparse_attn_plan(const uint64_t* mask_bits, int n_heads, int seq_len, int block,
                                int32_t* row_counts, int64_t* head_tiles, int32_t* work_order,
                                hipStream_t stream) {
  using namespace bsa;
  if (!mask_bits || !row_counts || !head_tiles || !work_order)
    return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(mask_bits, 8) || !aligned(head_tiles, 8) || !aligned(row_counts, 4) ||
      !aligned(work_order, 4))
    return fail(BSA_ERR_INVALID_ARG, "misaligned pointer argument");
  if (n_heads < 1 || seq_len < 1) return fail(BSA_ERR_INVALID_ARG, "n_heads and seq_len must be >= 1");
  if (block != 64) return fail(BSA_ERR_UNSUPPORTED, "only 64-token blocks are implemented");
  if ((long long)n_heads * n_blocks(seq_len, 64) > 0x7fffffffLL)
    return fail(BSA_ERR_INVALID_ARG, "problem too large");
  return launch_plan(mask_bits, n_heads, seq_len, row_counts, head_tiles, work_order, stream);
}
