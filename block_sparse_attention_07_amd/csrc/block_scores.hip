// Mean-pooled block proxy scores (SCOPE abstract: block-level proxy scores feed
// the mask predictor; the pooling is the block aggregation of ScalingAttention
// Eq. 1 applied to Q and K):
//   qbar_u = mean of the real tokens of block u (fp32), same for kbar_v,
//   S[h][u][v] = scale * <qbar_u, kbar_v>  (fp32).
//
// The pooling pass reads Q and K once, 16 bytes per lane with rows
// coalesced, and is bound by HBM bandwidth; it stores each fp32 mean m as three
// bf16 numbers, m1 = bf16(m), m2 = bf16(m - m1), m3 = bf16(m - m1 - m2), whose sum
// is m exactly (8 + 8 + 8 significant bits; every subtraction is exact).  The
// score pass forms the product per head (nb x d times d x nb) on bf16 MFMA from
// the six partial products a_i b_j with i + j <= 4, smallest first, with fp32
// accumulation; the three dropped ones are below 3 * 2^-24 of
// sum_c |qbar_c kbar_c|, as small as fp32 rounding of the product itself.  (fp32
// MFMA takes 2.7 times the cycles for the same product.)  The score pass runs
// as strips of 32 (or 16) whole rows through LDS when they fit there, so every
// strip of S is written as one contiguous run; larger nb use 128 x 128 tiles.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int NT = 256;
typedef unsigned short u16;

__device__ __forceinline__ u16 bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (u16)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);   // finite inputs only
}

// grid (nb, n_heads, 2): z selects Q (0) or K (1).  Threads split a block's rows
// into row groups; each thread sums 8 consecutive dims over its rows in fp32.
// Output: split[z][part 0..2][h][u][d] bf16.
template <int D>
__global__ __launch_bounds__(NT) void pool_kernel(const u16* __restrict__ q, const u16* __restrict__ k,
                                                  int N, int nb, u16* __restrict__ split) {
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int GROUPS = NT / CPR;      // row groups
  constexpr int PER = 64 / GROUPS;      // rows per thread in a full block
  __shared__ float part[GROUPS][D + 1];
  const int u = blockIdx.x, h = blockIdx.y, which = blockIdx.z;
  const u16* x = (which ? k : q) + (size_t)h * N * D;
  const int tid = threadIdx.x;
  const int ch = tid % CPR, rg = tid / CPR;
  const int row0 = 64 * u;
  const int rows = min(64, N - row0);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += __uint_as_float(w[j] << 16);
      acc[2 * j + 1] += __uint_as_float(w[j] & 0xffff0000u);
    }
  };
  if (rows == 64) {
    uint4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
      v[i] = *reinterpret_cast<const uint4*>(x + (size_t)(row0 + rg + GROUPS * i) * D + 8 * ch);
#pragma unroll
    for (int i = 0; i < PER; ++i) add(v[i]);
  } else {
    for (int r = rg; r < rows; r += GROUPS)
      add(*reinterpret_cast<const uint4*>(x + (size_t)(row0 + r) * D + 8 * ch));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[rg][8 * ch + j] = acc[j];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int g2 = 0; g2 < GROUPS; ++g2) s += part[g2][tid];
    const float m = s / (float)rows;
    const u16 p1 = bf16_rne(m);
    const float r1 = m - __uint_as_float((uint32_t)p1 << 16);
    const u16 p2 = bf16_rne(r1);
    const u16 p3 = bf16_rne(r1 - __uint_as_float((uint32_t)p2 << 16));
    const size_t plane = (size_t)gridDim.y * nb * D;
    u16* dst = split + (size_t)which * 3 * plane + ((size_t)h * nb + u) * D + tid;
    dst[0] = p1;
    dst[plane] = p2;
    dst[2 * plane] = p3;
  }
}

// One 128x128 output tile per workgroup, each wave a 64x64 quarter made of 2 x 2 blocks of 32x32 on
// v_mfma_f32_32x32x16_bf16.  Operands come straight from global memory (L2)
// into registers: lane l holds row l % 32 of a block, dims 16 ks + 8 (l / 32)
// .. +7 for k-step ks, which is the A layout (rows = u) and the B layout
// (columns = v) alike.  Rows past nb read row nb - 1 and are not stored.
// Result register i of lane l is element (8 (i / 4) + 4 (l / 32) + i % 4, l % 32)
// of a 32x32 block.
// Tiles: a panel is 128 rows u of one head; its nvb = ceil(nb / 128) tiles
// cover all columns.  Rows of S are nb floats apart, so cache lines straddle
// tile and row ends; workgroup i runs on XCD i mod 8 (workgroups are handed to
// the XCDs in turn), and every tile of a panel is given to the same XCD, so
// both halves of a straddling line meet in one L2 before they are written back.
template <int D>
__global__ __launch_bounds__(NT) void score_kernel(const u16* __restrict__ split, int n_heads, int nb,
                                                   int nvb, float scale, float* __restrict__ S) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  constexpr int NKS = D / 16;
  const int k8 = blockIdx.x >> 3;
  const int panel = 8 * (k8 / nvb) + (blockIdx.x & 7);
  const int vb = k8 % nvb;
  const int nub = nvb;                                  // panels per head (square S)
  if (panel >= n_heads * nub) return;
  const int h = panel / nub;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int u0 = 128 * (panel - h * nub) + 64 * (wave >> 1);
  const int v0 = 128 * vb + 64 * (wave & 1);
  const size_t plane = (size_t)n_heads * nb * D;
  const u16* qs = split + (size_t)h * nb * D;
  const u16* ks_ = split + 3 * plane + (size_t)h * nb * D;
  int ra[2], rb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    ra[j] = min(u0 + 32 * j + l32, nb - 1) * D + 8 * g;
    rb[j] = min(v0 + 32 * j + l32, nb - 1) * D + 8 * g;
  }
  auto ld = [&](const u16* base, int off) { return *reinterpret_cast<const bf16x8*>(base + off); };
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  // The operands of k-step ks + 1 are loaded while the MFMAs of k-step ks run.
  bf16x8 av[2][3][2], bv[2][3][2];
  auto load = [&](int ks, int buf) {
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        av[buf][t][j] = ld(qs + t * plane, ra[j] + 16 * ks);
        bv[buf][t][j] = ld(ks_ + t * plane, rb[j] + 16 * ks);
      }
  };
  // (i, j) with i + j <= 4 (parts numbered from 1), smallest terms first
  constexpr int PI[6] = {2, 0, 1, 1, 0, 0};
  constexpr int PJ[6] = {0, 2, 1, 0, 1, 0};
  load(0, 0);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < NKS) load(ks + 1, cur ^ 1);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int t = 0; t < 6; ++t)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cur][PI[t]][a], bv[cur][PJ[t]][b], acc[a][b],
                                                              0, 0, 0);
  }
  float* Sh = S + (size_t)h * nb * nb;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int vv = v0 + 32 * b + l32;
    if (vv >= nb) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int uu = u0 + 32 * a + 8 * (i >> 2) + 4 * g + (i & 3);
        if (uu < nb) Sh[(size_t)uu * nb + vv] = scale * acc[a][b][i];
      }
  }
}

// Strip form of the score pass: one workgroup of 8 waves per R consecutive
// rows u of one head computes all nb columns into LDS, laid out exactly as
// the rows sit in S, and then writes the strip as one contiguous run (R rows
// of nb floats), so no cache line of S is written in parts by different
// workgroups.  Products on v_mfma_f32_16x16x32_bf16: lane l holds A[l % 16]
// [8 (l / 16) .. +7] (rows u) and B[8 (l / 16) .. +7][l % 16] (columns v); result
// register i of lane l is C[4 (l / 16) + i][l % 16].  Wave w takes the 16-column
// tiles w, w + 8, ...; the k-bar parts stream from L2 once per strip.  Workgroup i
// runs on XCD i mod 8, and all strips of head h go to XCD h mod 8, so a head's
// k-bar parts (0.9 MB at d = 128, nb = 1182) stay in that XCD's L2.
constexpr int ST = 512;
template <int D, int R>
__global__ __launch_bounds__(ST) void score_strip_kernel(const u16* __restrict__ split, int n_heads, int nb,
                                                         int n_strips, float scale, float* __restrict__ S) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int NKS = D / 32;
  constexpr int RT = R / 16;
  extern __shared__ float strip[];            // [R][nb]
  const int k8 = blockIdx.x >> 3;
  const int h = 8 * (k8 / n_strips) + (blockIdx.x & 7);
  if (h >= n_heads) return;
  const int u0 = R * (k8 % n_strips);
  const int rows = min(R, nb - u0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const size_t plane = (size_t)n_heads * nb * D;
  const u16* qs = split + (size_t)h * nb * D;
  const u16* ks_ = split + 3 * plane + (size_t)h * nb * D;
  auto ld = [&](const u16* base, size_t off) { return *reinterpret_cast<const bf16x8*>(base + off); };
  bf16x8 av[RT][NKS][3];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const size_t ro = (size_t)min(u0 + 16 * rt + l16, nb - 1) * D + 8 * g4;
#pragma unroll
    for (int k = 0; k < NKS; ++k)
#pragma unroll
      for (int t = 0; t < 3; ++t) av[rt][k][t] = ld(qs + t * plane, ro + 32 * k);
  }
  // (i, j) with i + j <= 4 (parts numbered from 1), smallest terms first
  constexpr int PI[6] = {2, 0, 1, 1, 0, 0};
  constexpr int PJ[6] = {0, 2, 1, 0, 1, 0};
  const int n_ct = (nb + 15) / 16;
  // The k-bar parts of the next column tile are loaded while the current one
  // is multiplied; the row tiles' accumulators alternate inside each product so
  // that consecutive MFMAs are independent.
  bf16x8 bv[2][NKS][3];
  auto load_b = [&](int ct, int buf) {
    const size_t co = (size_t)min(16 * ct + l16, nb - 1) * D + 8 * g4;
#pragma unroll
    for (int k = 0; k < NKS; ++k)
#pragma unroll
      for (int t = 0; t < 3; ++t) bv[buf][k][t] = ld(ks_ + t * plane, co + 32 * k);
  };
  auto tile = [&](int ct, int buf) {
    f32x4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NKS; ++k)
#pragma unroll
      for (int t = 0; t < 6; ++t)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[rt][k][PI[t]], bv[buf][k][PJ[t]], acc[rt], 0, 0, 0);
    const int v = 16 * ct + l16;
    if (v < nb) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * g4 + i;
          if (r < rows) strip[r * nb + v] = scale * acc[rt][i];
        }
    }
  };
  constexpr int WS = ST / 64;                 // waves per workgroup
  int ct = wave;
  if (ct < n_ct) load_b(ct, 0);
  for (; ct < n_ct; ct += 2 * WS) {
    if (ct + WS < n_ct) load_b(ct + WS, 1);
    tile(ct, 0);
    if (ct + WS >= n_ct) break;
    if (ct + 2 * WS < n_ct) load_b(ct + 2 * WS, 0);
    tile(ct + WS, 1);
  }
  __syncthreads();
  float* dst = S + ((size_t)h * nb + u0) * nb;
  const int n = rows * nb;
  for (int i = threadIdx.x; i < n; i += ST) dst[i] = strip[i];
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
  // pooled means as three bf16 parts: [Q, K][part][n_heads][nb][head_dim]
  const size_t split_bytes = (size_t)6 * n_heads * nb * head_dim * sizeof(unsigned short);
  ScratchLease lease(split_bytes);
  auto* split = static_cast<unsigned short*>(lease.get());
  if (!split) return BSA_ERR_HIP;
  const auto* qq = static_cast<const unsigned short*>(q);
  const auto* kk = static_cast<const unsigned short*>(k);
  const int nvb = (nb + 127) / 128;
  if ((long long)8 * nvb * ((n_heads * (long long)nvb + 7) / 8) > 0x7fffffffLL)
    return fail(BSA_ERR_INVALID_ARG, "problem too large");
  // strips of R rows when R rows of scores fit in a workgroup's LDS, else 128x128 tiles
  int dev = 0, lds_max = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    lds_max = 0;
  const size_t lds = (size_t)lds_max;
  const int strip_rows = (size_t)32 * nb * 4 <= lds ? 32 : ((size_t)16 * nb * 4 <= lds ? 16 : 0);
  const dim3 pgrid(nb, n_heads, 2), sgrid(8 * nvb * ((n_heads * nvb + 7) / 8));
  if (head_dim == 128) {
    hipLaunchKernelGGL(pool_kernel<128>, pgrid, dim3(NT), 0, stream, qq, kk, seq_len, nb, split);
    BSA_CHECK_HIP(hipGetLastError());
    if (strip_rows == 32)
      hipLaunchKernelGGL((score_strip_kernel<128, 32>), dim3(8u * (unsigned)((nb + 31) / 32) * (unsigned)((n_heads + 7) / 8)),
                         dim3(ST), (size_t)32 * nb * 4, stream, split, n_heads, nb, (nb + 31) / 32, scale, scores);
    else if (strip_rows == 16)
      hipLaunchKernelGGL((score_strip_kernel<128, 16>), dim3(8u * (unsigned)((nb + 15) / 16) * (unsigned)((n_heads + 7) / 8)),
                         dim3(ST), (size_t)16 * nb * 4, stream, split, n_heads, nb, (nb + 15) / 16, scale, scores);
    else
      hipLaunchKernelGGL(score_kernel<128>, sgrid, dim3(NT), 0, stream, split, n_heads, nb, nvb, scale, scores);
  } else {
    hipLaunchKernelGGL(pool_kernel<64>, pgrid, dim3(NT), 0, stream, qq, kk, seq_len, nb, split);
    BSA_CHECK_HIP(hipGetLastError());
    if (strip_rows == 32)
      hipLaunchKernelGGL((score_strip_kernel<64, 32>), dim3(8u * (unsigned)((nb + 31) / 32) * (unsigned)((n_heads + 7) / 8)),
                         dim3(ST), (size_t)32 * nb * 4, stream, split, n_heads, nb, (nb + 31) / 32, scale, scores);
    else if (strip_rows == 16)
      hipLaunchKernelGGL((score_strip_kernel<64, 16>), dim3(8u * (unsigned)((nb + 15) / 16) * (unsigned)((n_heads + 7) / 8)),
                         dim3(ST), (size_t)16 * nb * 4, stream, split, n_heads, nb, (nb + 15) / 16, scale, scores);
    else
      hipLaunchKernelGGL(score_kernel<64>, sgrid, dim3(NT), 0, stream, split, n_heads, nb, nvb, scale, scores);
  }
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
