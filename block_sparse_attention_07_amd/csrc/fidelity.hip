// Hellinger distance / Fidelity Score between dense and sparse attention rows.
//
// ScalingAttention section 4.2.1 (Eqs. 3 and 4) and section 4.2.3 (rows drawn
// by block-wise stratified sampling).  For a sampled query row, P is the dense
// softmax over every key and P~ the softmax over the keys its mask row keeps.
// P~ is P restricted to the kept keys and renormalised, so with rho the dense
// mass on kept keys
//
//     H(P, P~)^2 = 1 - sum_j sqrt(p_j p~_j) = 1 - sqrt(rho),
//     H = sqrt((1 - rho) / (1 + sqrt(rho))),
//
// and only two partition sums per row are needed: Z_keep over kept keys and
// Z_drop over dropped keys, both relative to the row's running maximum; the
// second form has no cancellation when H is small.  A row that keeps nothing
// gets H = 1.
//
// Pass 1: one workgroup per (1024-key chunk, head, group of 16 sampled rows)
// computes the logits of its rows against its keys on v_mfma_f32_16x16x32_bf16
// (the 16 sampled rows are the A operand, held in registers; each 16-key tile
// of K is the B operand, loaded straight from memory; exact bf16 products,
// fp32 accumulation) and reduces (max, Z_keep, Z_drop) per row.  Pass 2: one workgroup per head merges the chunks,
// writes each row's H and the head's Fidelity Score 1 - mean H.
#include <algorithm>
#include <cmath>

#include "bsa_internal.h"

namespace bsa {
namespace {

typedef unsigned short u16;
constexpr int NT = 256;
constexpr int RG = 16;          // sampled rows per workgroup
constexpr int CHUNK = 1024;     // keys per workgroup (16 blocks of 64)

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Merge two (max, Z_keep, Z_drop) triples in the exp2 domain.
__device__ __forceinline__ void merge(float& m, float& zk, float& zd, float m2, float zk2, float zd2) {
  const float mn = fmaxf(m, m2);
  const float f1 = m == -INFINITY ? 0.f : exp2f(m - mn);
  const float f2 = m2 == -INFINITY ? 0.f : exp2f(m2 - mn);
  zk = zk * f1 + zk2 * f2;
  zd = zd * f1 + zd2 * f2;
  m = mn;
}

// Operand layouts of v_mfma_f32_16x16x32_bf16: lane l holds A[l % 16][8 (l / 16) ..
// +7] and B[8 (l / 16) .. +7][l % 16]; result register i of lane l is C[4 (l / 16) + i]
// [l % 16].  Wave w walks keys 256 w .. 256 w + 255 of the chunk in 16-key tiles;
// each lane keeps (max, Z_keep, Z_drop) for its four rows over its key column,
// starting from a large finite max so keys past the sequence end (logit -inf)
// contribute exactly nothing.
template <int D>
__global__ __launch_bounds__(NT) void fidelity_partial_kernel(const u16* __restrict__ Q,
                                                              const u16* __restrict__ K,
                                                              const uint64_t* __restrict__ mask,
                                                              const int32_t* __restrict__ rows, int N,
                                                              int nb, int W, int n_rows, float c,
                                                              int n_chunks, float* __restrict__ part) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int NKS = D / 32;
  __shared__ uint32_t keepbits[RG];
  __shared__ float red[NT / 64][RG][3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int chunk = blockIdx.x, h = blockIdx.y, r0 = blockIdx.z * RG;
  const int nr = min(RG, n_rows - r0);
  const int32_t* hrows = rows + (size_t)h * n_rows + r0;

  bf16x8 qa[NKS];
  {
    const int tok = l16 < nr ? hrows[l16] : -1;
    const bool ok = tok >= 0 && tok < N;
    const u16* qr = Q + ((size_t)h * N + (ok ? tok : 0)) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 x = *reinterpret_cast<const uint4*>(qr + 32 * ks);
      if (!ok) x = make_uint4(0, 0, 0, 0);
      qa[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  if (tid < RG) {
    uint32_t bits = 0;
    if (tid < nr) {
      const int tok = hrows[tid];
      if (tok >= 0 && tok < N) {
        const uint64_t* mrow = mask + ((size_t)h * nb + tok / 64) * W;
        for (int b = 0; b < CHUNK / 64; ++b) {
          const int blk = chunk * (CHUNK / 64) + b;
          if (blk < nb && ((mrow[blk >> 6] >> (blk & 63)) & 1ull)) bits |= 1u << b;
        }
      }
    }
    keepbits[tid] = bits;
  }
  __syncthreads();

  float m[4], zk[4], zd[4];
  uint32_t kb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -1.0e30f;
    zk[i] = 0.f;
    zd[i] = 0.f;
    kb[i] = keepbits[4 * g4 + i];
  }
  const int kbeg = chunk * CHUNK + wave * (CHUNK / 4);
  const int kend = min(N, kbeg + CHUNK / 4);
  for (int t0 = kbeg; t0 < kend; t0 += 16) {
    const int key = t0 + l16;
    const bool kin = key < N;
    const u16* kr = K + ((size_t)h * N + (kin ? key : N - 1)) * D + 8 * g4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 kv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kr + 32 * ks));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kv, acc, 0, 0, 0);
    }
    const uint32_t b = (uint32_t)((t0 - chunk * CHUNK) >> 6);    // 64-key block within the chunk
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sv = kin ? acc[i] * c : -INFINITY;
      const float mn = fmaxf(m[i], sv);
      const float f = exp2f(m[i] - mn);
      const float e = exp2f(sv - mn);
      const bool kept = (kb[i] >> b) & 1u;
      zk[i] = zk[i] * f + (kept ? e : 0.f);
      zd[i] = zd[i] * f + (kept ? 0.f : e);
      m[i] = mn;
    }
  }
  // Reduce over the 16 lanes that share each row, then over the waves.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      const float m2 = __shfl_xor(m[i], off), k2 = __shfl_xor(zk[i], off), d2 = __shfl_xor(zd[i], off);
      merge(m[i], zk[i], zd[i], m2, k2, d2);
    }
    if (l16 == 0) {
      red[wave][4 * g4 + i][0] = m[i];
      red[wave][4 * g4 + i][1] = zk[i];
      red[wave][4 * g4 + i][2] = zd[i];
    }
  }
  __syncthreads();
  if (tid < nr) {
    float mm = red[0][tid][0], kk = red[0][tid][1], dd = red[0][tid][2];
    for (int wv = 1; wv < NT / 64; ++wv) merge(mm, kk, dd, red[wv][tid][0], red[wv][tid][1], red[wv][tid][2]);
    float* o = part + (((size_t)h * n_rows + r0 + tid) * n_chunks + chunk) * 3;
    o[0] = mm;
    o[1] = kk;
    o[2] = dd;
  }
}

__global__ __launch_bounds__(NT) void fidelity_combine_kernel(const float* __restrict__ part,
                                                              const int32_t* __restrict__ rows, int N,
                                                              int n_rows, int n_chunks,
                                                              float* __restrict__ row_h,
                                                              float* __restrict__ head_f) {
  __shared__ float sums[NT];
  const int h = blockIdx.x, tid = threadIdx.x;
  float acc = 0.f;
  for (int r = tid; r < n_rows; r += NT) {
    const int tok = rows[(size_t)h * n_rows + r];
    float H = NAN;
    if (tok >= 0 && tok < N) {
      const float* p = part + ((size_t)h * n_rows + r) * n_chunks * 3;
      float m = -INFINITY, zk = 0.f, zd = 0.f;
      for (int ch = 0; ch < n_chunks; ++ch) merge(m, zk, zd, p[3 * ch], p[3 * ch + 1], p[3 * ch + 2]);
      if (zk > 0.f) {
        const float tot = zk + zd;
        H = sqrtf((zd / tot) / (1.f + sqrtf(zk / tot)));
      } else {
        H = 1.f;
      }
    }
    row_h[(size_t)h * n_rows + r] = H;
    acc += H;
  }
  sums[tid] = acc;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (tid < s) sums[tid] += sums[tid + s];
    __syncthreads();
  }
  if (tid == 0 && head_f) head_f[h] = 1.f - sums[0] / (float)n_rows;
}

}  // namespace
}  // namespace bsa

extern "C" int attn_fidelity(const void* q, const void* k, const uint64_t* mask_bits,
                             const int32_t* rows, int n_heads, int seq_len, int head_dim, int block,
                             int n_rows, float scale, float* row_hellinger, float* head_fidelity,
                             hipStream_t stream) {
  using namespace bsa;
  if (!q || !k || !mask_bits || !rows || !row_hellinger)
    return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(mask_bits, 8) || !aligned(rows, 4) ||
      !aligned(row_hellinger, 4) || (head_fidelity && !aligned(head_fidelity, 4)))
    return fail(BSA_ERR_INVALID_ARG, "misaligned pointer argument");
  if (n_heads < 1 || seq_len < 1 || n_rows < 1) return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(BSA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (block != 64) return fail(BSA_ERR_UNSUPPORTED, "only 64-token blocks are implemented");
  if (head_dim != 64 && head_dim != 128) return fail(BSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (n_heads > 65535 || (n_rows + RG - 1) / RG > 65535)
    return fail(BSA_ERR_UNSUPPORTED, "at most 65535 heads and 65535 * 16 rows per call");
  const int nb = n_blocks(seq_len, 64);
  const int W = n_words(nb);
  const int n_chunks = (seq_len + CHUNK - 1) / CHUNK;
  ScratchLease lease((size_t)n_heads * n_rows * n_chunks * 3 * sizeof(float));
  float* part = static_cast<float*>(lease.get());
  if (!part) return BSA_ERR_HIP;
  const float c = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)n_chunks, (unsigned)n_heads, (unsigned)((n_rows + RG - 1) / RG));
  const u16* Q = static_cast<const u16*>(q);
  const u16* K = static_cast<const u16*>(k);
  if (head_dim == 128)
    hipLaunchKernelGGL(fidelity_partial_kernel<128>, grid, dim3(NT), 0, stream, Q, K, mask_bits, rows,
                       seq_len, nb, W, n_rows, c, n_chunks, part);
  else
    hipLaunchKernelGGL(fidelity_partial_kernel<64>, grid, dim3(NT), 0, stream, Q, K, mask_bits, rows,
                       seq_len, nb, W, n_rows, c, n_chunks, part);
  BSA_CHECK_HIP(hipGetLastError());
  hipLaunchKernelGGL(fidelity_combine_kernel, dim3((unsigned)n_heads), dim3(NT), 0, stream, part, rows,
                     seq_len, n_rows, n_chunks, row_hellinger, head_fidelity);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
