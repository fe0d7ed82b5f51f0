// inst_mfma_batch.hip -- instantiations and launcher of the packed-MFMA
// forward-type kernel with the batch in the matrix rows (bf16 / fp16).
#include "dwc_launch.h"
#include "dwc_mfma_batch.h"
#include "dwc_mfma_batch16.h"

namespace dwc {
namespace {

// Dynamic LDS above the default 64 KiB must be allowed per kernel once; the
// planner keeps every launch within one CU's LDS.
template <typename K>
hipError_t allow_lds(K kernel) {
  static const hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      kLdsPerCu);
  return e;
}

template <int DT, int CB, bool FLIP>
hipError_t go(const MfmaBatchArgs& a, hipStream_t s) {
  auto kernel = fwd_mfma_batch<DT, CB, FLIP>;
  if (a.lds_bytes > 65536) {
    const hipError_t e = allow_lds(kernel);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, dim3(a.num_blocks), dim3(64 * CB), a.lds_bytes, s, a);
  return hipGetLastError();
}

template <int DT, bool FLIP>
hipError_t by_cb(const MfmaBatchArgs& a, hipStream_t s) {
  if (a.cb == kBatchCb) return go<DT, kBatchCb, FLIP>(a, s);
  return hipErrorInvalidValue;
}

template <int DT, int NG, bool FLIP>
hipError_t go16(const MfmaBatchArgs& a, hipStream_t s) {
  auto kernel = fwd_mfma_batch16<DT, NG, FLIP>;
  if (a.lds_bytes > 65536) {
    const hipError_t e = allow_lds(kernel);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, dim3(a.num_blocks), dim3(512), a.lds_bytes, s, a);
  return hipGetLastError();
}

template <int DT, bool FLIP>
hipError_t by_ng(int ng, const MfmaBatchArgs& a, hipStream_t s) {
  if (ng == 1) return go16<DT, 1, FLIP>(a, s);
  if (ng == 2) return go16<DT, 2, FLIP>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_mfma_batch16(int dt, int ng, bool flip, const MfmaBatchArgs& a,
                                   hipStream_t s) {
  if (dt == DT_BF16) return flip ? by_ng<DT_BF16, true>(ng, a, s) : by_ng<DT_BF16, false>(ng, a, s);
  if (dt == DT_F16) return flip ? by_ng<DT_F16, true>(ng, a, s) : by_ng<DT_F16, false>(ng, a, s);
  if (dt == DT_E4M3) return flip ? by_ng<DT_E4M3, true>(ng, a, s) : by_ng<DT_E4M3, false>(ng, a, s);
  if (dt == DT_E5M2) return flip ? by_ng<DT_E5M2, true>(ng, a, s) : by_ng<DT_E5M2, false>(ng, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_mfma_batch(int dt, bool flip, const MfmaBatchArgs& a, hipStream_t s) {
  if (dt == DT_BF16) return flip ? by_cb<DT_BF16, true>(a, s) : by_cb<DT_BF16, false>(a, s);
  if (dt == DT_F16) return flip ? by_cb<DT_F16, true>(a, s) : by_cb<DT_F16, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace dwc
