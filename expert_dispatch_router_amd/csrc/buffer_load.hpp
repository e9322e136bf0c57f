// buffer_load.hpp -- raw buffer loads of gfx950 (device code only).
#pragma once

#include "moe_internal.hpp"

namespace moe {

// gfx9 raw-buffer descriptor word 3 (32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

// 128-bit raw buffer load; offsets past the resource's byte range read 0.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

}  // namespace moe
