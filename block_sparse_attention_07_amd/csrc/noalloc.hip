// sparse_attn_fwd_noalloc: the bf16 attention for callers that cannot allocate
// device memory (code under stream capture, tight serving loops).  Its scratch
// memory -- the work plan and the transposed V -- lives in one fixed array in
// the library's code object, so a call allocates, frees and synchronises
// nothing.  The heads go through in chunks whose plan and transposed V fit the
// array; each chunk runs the same planner and kernels as sparse_attn_fwd on
// its slice of q, k, v, mask and out, in stream order, so the output is the
// same bit for bit.
#include <mutex>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr size_t kScratchBytes = size_t(256) << 20;
constexpr int kMaxDevices = 64;

// The array itself.  In host code this name stands for the host-side shadow of
// the symbol, not a device address: device code receives the address that
// hipGetSymbolAddress returns for the current device (scratch_ptr below).
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per device.
void* scratch_ptr() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(BSA_ERR_UNSUPPORTED, "device ordinal %d exceeds %d", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      hip_fail(e, "hipGetSymbolAddress (fixed scratch array)");
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace
}  // namespace bsa

extern "C" int sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                       const uint64_t* mask_bits, int n_heads, int seq_len,
                                       int head_dim, int block_q, int block_k, float scale,
                                       void* out, hipStream_t stream) {
  using namespace bsa;
  int rc = check_attn_args(q, k, v, mask_bits, out, n_heads, seq_len, head_dim, block_q, block_k,
                           scale, 16);
  if (rc) return rc;
  // heads per chunk: as many as fit, a multiple of 4 when at least 4 fit (the
  // single-row launches split the XCDs into 4 groups of heads), all when all fit
  int per = 0;
  while (per < n_heads && attn_workspace_bytes(per + 1, seq_len, head_dim) <= kScratchBytes) ++per;
  if (per == 0)
    return fail(BSA_ERR_UNSUPPORTED,
                "one head at seq_len %d, head_dim %d needs %zu bytes of scratch; the fixed array "
                "holds %zu",
                seq_len, head_dim, attn_workspace_bytes(1, seq_len, head_dim), kScratchBytes);
  if (per < n_heads && per >= 4) per -= per % 4;
  char* ws = static_cast<char*>(scratch_ptr());
  if (!ws) return BSA_ERR_HIP;
  const int nb = n_blocks(seq_len, 64);
  const size_t head_elems = (size_t)seq_len * head_dim;
  const size_t head_words = (size_t)nb * n_words(nb);
  for (int h0 = 0; h0 < n_heads; h0 += per) {
    const int c = n_heads - h0 < per ? n_heads - h0 : per;
    const size_t off = (size_t)h0 * head_elems * 2;
    rc = attn_bf16_with_workspace(static_cast<const char*>(q) + off, static_cast<const char*>(k) + off,
                                  static_cast<const char*>(v) + off, mask_bits + (size_t)h0 * head_words, c,
                                  seq_len, head_dim, scale, static_cast<char*>(out) + off, ws, stream);
    if (rc) return rc;
  }
  return ok();
}
