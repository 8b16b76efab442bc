// Device helpers shared by the prefill kernels of libmamba_scan: raw buffer
// loads and stores with a wave-uniform descriptor.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_device.h"

namespace mscan {

// Raw buffer access: a wave-uniform descriptor (base, size in bytes) in SGPRs,
// a per-lane byte offset in a VGPR and a wave-uniform byte offset in an SGPR.
// Reads at or past `bytes` return 0 and writes there are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
  const int32_t n = static_cast<int32_t>(bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}
template <int IO>
__device__ __forceinline__ typename Io<IO>::T buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (IO == 0) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
  } else {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  }
}
__device__ __forceinline__ int32_t buf_load_i32(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
template <int IO>
__device__ __forceinline__ void buf_store(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (IO == 0) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16(Io<1>::from_float(v), r, voff, soff, 0);
  }
}

}  // namespace mscan
