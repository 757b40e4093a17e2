// Host-side status handling shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "csa2.h"
#include "csa2_measure.h"

namespace csa2 {

// Record a message as the calling thread's last error and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// CSA2_OK, or CSA2_ERR_HIP with the runtime's message recorded.
int hip_status(hipError_t e, const char* what);

// Status of the most recent launch on this thread.
inline int launch_status(const char* what) { return hip_status(hipGetLastError(), what); }

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace sizes (bytes) of the ops that need one.
size_t index_full_ws_bytes(int B, long long total_len, int P, int k);
size_t index_full_block_ws_bytes(int B, int T, int shared, long long total_len, int k);
size_t sparse_attn_ws_bytes(int B, int Hq, int D, int k, int window);
int sparse_attn_splits(int B, int Hq, int k, int window);

}  // namespace csa2
