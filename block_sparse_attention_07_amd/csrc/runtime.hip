// Host runtime: error reporting, argument validation, the per-device scratch
// buffer and the small query entry points.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "bsa_internal.h"

namespace bsa {

namespace {
thread_local char g_msg[512] = "";

constexpr int kMaxDevices = 64;
struct Scratch {
  std::mutex mu;          // held by a lease from acquisition until its entry point returns
  void* ptr = nullptr;
  size_t bytes = 0;
};
Scratch g_scratch[kMaxDevices];
}  // namespace

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_msg[0] = '\0';
  return BSA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(BSA_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

// The device's buffer is only ever replaced by a thread that holds its lock, and
// every entry point that uses the buffer holds the lock until all of its launches
// are enqueued.  So when a larger buffer is needed, every launch that can touch
// the old one is already on some stream, and one device-wide synchronisation
// covers them all before the old buffer is freed.
ScratchLease::ScratchLease(size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_fail(e, "hipGetDevice");
    return;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(BSA_ERR_UNSUPPORTED, "device ordinal %d exceeds %d", dev, kMaxDevices);
    return;
  }
  Scratch& s = g_scratch[dev];
  s.mu.lock();
  dev_ = dev;
  if (s.bytes >= bytes && s.ptr) {
    ptr_ = s.ptr;
    return;
  }
  if (s.ptr) {
    e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      hip_fail(e, "hipDeviceSynchronize (scratch growth)");
      return;
    }
    (void)hipFree(s.ptr);
    s.ptr = nullptr;
    s.bytes = 0;
  }
  size_t want = bytes < (size_t(1) << 20) ? (size_t(1) << 20) : bytes;
  want = (want + 4095) & ~size_t(4095);
  void* p = nullptr;
  e = hipMalloc(&p, want);
  if (e != hipSuccess) {
    hip_fail(e, "hipMalloc (scratch)");
    return;
  }
  s.ptr = p;
  s.bytes = want;
  ptr_ = p;
}

ScratchLease::~ScratchLease() {
  if (dev_ >= 0) g_scratch[dev_].mu.unlock();
}

int check_attn_args(const void* q, const void* k, const void* v, const void* mask, const void* out,
                    int n_heads, int seq_len, int head_dim, int block_q, int block_k, float scale,
                    size_t elem_align, size_t mask_align) {
  if (!q || !k || !v || !mask || !out) return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(q, elem_align) || !aligned(k, elem_align) || !aligned(v, elem_align) ||
      !aligned(out, elem_align))
    return fail(BSA_ERR_INVALID_ARG, "q, k, v and out must be %zu-byte aligned", elem_align);
  if (!aligned(mask, mask_align))
    return fail(BSA_ERR_INVALID_ARG, "the mask must be %zu-byte aligned", mask_align);
  if (n_heads < 1 || seq_len < 1)
    return fail(BSA_ERR_INVALID_ARG, "n_heads (%d) and seq_len (%d) must be >= 1", n_heads, seq_len);
  if (block_q != 64 || block_k != 64)
    return fail(BSA_ERR_UNSUPPORTED, "only 64x64 blocks are implemented (got %dx%d)", block_q, block_k);
  if (head_dim != 64 && head_dim != 128)
    return fail(BSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(BSA_ERR_INVALID_ARG, "scale must be finite and > 0");
  const long long nb = n_blocks(seq_len, 64);
  if ((long long)n_heads * nb > 0x7fffffffLL ||
      (long long)n_heads * seq_len * (long long)head_dim > (1LL << 40))
    return fail(BSA_ERR_INVALID_ARG, "problem too large");
  return BSA_OK;
}

}  // namespace bsa

extern "C" const char* bsa_last_error(void) { return bsa::g_msg; }

extern "C" int bsa_mask_words(int seq_len, int block) {
  if (seq_len < 1 || block < 1) return -1;
  return bsa::n_words(bsa::n_blocks(seq_len, block));
}
