// Wave-wide (64-lane) inclusive scans on gfx950 with DPP, no LDS round trips:
// row shifts by 1, 2, 4 and 8 within each row of 16 lanes, then lane 15 of a row
// into the next row, then lane 31 into rows 2 and 3.  Lanes with no source read 0.
// Internal to libuniprefill.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace up {

template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp_in(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWMASK, 0xf, true);
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp_in64(uint64_t v) {
  const uint32_t lo = dpp_in<CTRL, ROWMASK>((uint32_t)v);
  const uint32_t hi = dpp_in<CTRL, ROWMASK>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) {
  v += dpp_in<0x111, 0xf>(v);
  v += dpp_in<0x112, 0xf>(v);
  v += dpp_in<0x114, 0xf>(v);
  v += dpp_in<0x118, 0xf>(v);
  v += dpp_in<0x142, 0xa>(v);
  v += dpp_in<0x143, 0xc>(v);
  return v;
}

__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v) {
  v += dpp_in64<0x111, 0xf>(v);
  v += dpp_in64<0x112, 0xf>(v);
  v += dpp_in64<0x114, 0xf>(v);
  v += dpp_in64<0x118, 0xf>(v);
  v += dpp_in64<0x142, 0xa>(v);
  v += dpp_in64<0x143, 0xc>(v);
  return v;
}

// Float inclusive scan in the same fixed pattern: lane 63 ends with the wave's sum,
// always associated the same way (bitwise reproducible).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_in_f32(float v) {
  return __uint_as_float(dpp_in<CTRL, ROWMASK>(__float_as_uint(v)));
}
__device__ __forceinline__ float wave_scan_f32(float v) {
  v += dpp_in_f32<0x111, 0xf>(v);
  v += dpp_in_f32<0x112, 0xf>(v);
  v += dpp_in_f32<0x114, 0xf>(v);
  v += dpp_in_f32<0x118, 0xf>(v);
  v += dpp_in_f32<0x142, 0xa>(v);
  v += dpp_in_f32<0x143, 0xc>(v);
  return v;
}

// Value of lane 63 (the wave total after an inclusive scan).
__device__ __forceinline__ uint64_t lane63_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace up
