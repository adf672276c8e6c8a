// Internal helpers shared by the library's translation units: error state,
// argument checks, per-device scratch memory and small device utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/bsattn.h"

namespace bsa {

// Record a message for bsa_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the thread's message; returns BSA_OK.
int ok();
// Map a HIP status to BSA_ERR_HIP with the call site named.
int hip_fail(hipError_t e, const char* what);

// Per-device scratch buffer owned by the library, grown on demand.  A lease
// holds the current device's scratch lock from construction to destruction, so
// an entry point keeps its lease until every launch that uses the buffer is
// enqueued; another thread can then never free the buffer under it.  get() is
// nullptr (with the error recorded) when the buffer could not be provided.
class ScratchLease {
 public:
  explicit ScratchLease(size_t bytes);
  ~ScratchLease();
  ScratchLease(const ScratchLease&) = delete;
  ScratchLease& operator=(const ScratchLease&) = delete;
  void* get() const { return ptr_; }

 private:
  int dev_ = -1;
  void* ptr_ = nullptr;
};

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int n_blocks(int seq_len, int block) { return (seq_len + block - 1) / block; }
inline int n_words(int nb) { return (nb + 63) / 64; }

// Checks shared by the attention entry points.
int check_attn_args(const void* q, const void* k, const void* v, const void* mask, const void* out,
                    int n_heads, int seq_len, int head_dim, int block_q, int block_k, float scale,
                    size_t elem_align, size_t mask_align = 8);
// Expand 32-bit rows over 128-token blocks into 64-bit rows over 64-token blocks
// (b128.hip).
int launch_expand_b128(const uint32_t* mask_words, int n_heads, int seq_len, uint64_t* mask_bits,
                       hipStream_t stream);

// Launch the row-count / head-order planner (defined in plan.hip).
int launch_plan(const uint64_t* mask, int n_heads, int seq_len, int32_t* counts, int64_t* head_tiles,
                int32_t* order, hipStream_t stream);

// Bytes of the transposed-V workspace the bf16 attention path needs.
size_t vt_bytes(int n_heads, int seq_len, int head_dim);
// Bytes of the workspace of the unplanned bf16 attention (plan + transposed V,
// 256-byte aligned parts), and that attention run on a given workspace
// (attn_bf16.hip).
size_t attn_workspace_bytes(int n_heads, int seq_len, int head_dim);
int attn_bf16_with_workspace(const void* q, const void* k, const void* v, const uint64_t* mask_bits,
                             int n_heads, int seq_len, int head_dim, float scale, void* out, char* ws,
                             hipStream_t stream);
// Launch the bf16 attention path (V transpose into `vt`, then the attention
// kernel) with an optional work order (attn_bf16.hip).
int launch_attn_bf16(const void* q, const void* k, const void* v, const uint64_t* mask,
                     const int32_t* order, int n_heads, int seq_len, int head_dim, float scale,
                     void* out, void* vt, hipStream_t stream);

}  // namespace bsa

#define BSA_CHECK_HIP(call)                                  \
  do {                                                       \
    hipError_t _e = (call);                                  \
    if (_e != hipSuccess) return ::bsa::hip_fail(_e, #call); \
  } while (0)
