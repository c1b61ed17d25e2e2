// Host-side helpers shared by the C-ABI translation units of libnvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nvq.h"

namespace nvq {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

// Bump allocator over a caller workspace.  The status word always lives in
// the first 256 bytes.
struct WsCarve {
  char* base;
  size_t off = kAlign;  // [0, 256): status word
  explicit WsCarve(void* ws) : base(static_cast<char*>(ws)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
  uint32_t* status() const { return reinterpret_cast<uint32_t*>(base); }
};

inline int hip_status(hipError_t e) { return e == hipSuccess ? NVQ_OK : NVQ_EHIP; }
inline int last_launch() { return hip_status(hipGetLastError()); }

// Number of compute units of the current device (cached per process).
int device_cu_count();

// Clears the workspace status word with a one-thread kernel (no memset node,
// so the call is safe inside captured graphs).
int clear_status(uint32_t* status, hipStream_t s);

}  // namespace nvq
