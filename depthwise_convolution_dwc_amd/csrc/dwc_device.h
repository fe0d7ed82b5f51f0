// dwc_device.h -- device-side helpers shared by the libdwc kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dwc_geom.h"

namespace dwc {

// Operand storage types.  bf16 is kept as its raw 16 bits, fp8 as its code.
template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_F16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_E4M3> { static constexpr int bytes = 1; };
template <> struct Elem<DT_E5M2> { static constexpr int bytes = 1; };

// An fp8 code (the low byte of c) as float: the hardware conversion, which
// reads the OCP e4m3 / e5m2 encodings on gfx950.  Exact.
template <int DT>
__device__ __forceinline__ float fp8_to_f32(uint32_t c) {
  if constexpr (DT == DT_E4M3) return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
  else return __builtin_amdgcn_cvt_f32_bf8((int)c, 0);
}

// Buffer resource over [base, base + bytes).  A raw buffer load whose
// per-lane offset is >= bytes returns 0, which is how every kernel reads the
// implicit zero padding without branches.  The range check covers the
// VGPR offset only, so every offset below goes in the VGPR operand.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Cache-policy operand of a buffer store that marks it non-temporal.  The
// vector kernels write each output once, in whole lines per wave, and
// nothing reads it back in the same launch, so their stores stream past
// the caches and leave them to the operands (measured on MI355X with every
// op rotating over >= 1 GiB: the stride-2 7x7 forward 34.8 -> 32.0 us, the
// 7x7 sweeps within 1%).  The packed kernels, whose workgroups write parts
// of a line that the L2 has to merge, use plain stores.
constexpr int kStoreNT = 2;

// Non-temporal store of one value at a per-lane address.
template <typename T>
__device__ __forceinline__ void store_nt(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}

// floor(p / d) from m = div_magic(d), for p, d < 2^16.
__device__ __forceinline__ int fast_div(int p, uint64_t m) {
  return (int)(((uint64_t)(uint32_t)p * m) >> 32);
}

// An offset that is always outside any resource built above.
constexpr uint32_t kOOB = 0x80000000u;

// The hardware hands workgroup b to XCD (b mod 8) on the MI355X's 8 XCDs.
// Give each XCD one contiguous range of logical tile ids so that tiles
// which read the same input rows share that XCD's L2.  The map is a
// permutation of [0, nblocks) whatever the device's XCD count, so another
// count changes only which tiles share an L2, never a result.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int x = bid % kXcd, k = bid / kXcd;
  const int q = nblocks / kXcd, r = nblocks % kXcd;
  return x * q + (x < r ? x : r) + k;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace dwc
