// inst_mfma_h4.hip -- instantiations and launcher of the 16-bit forward-type
// kernel on the 4x4x4 matrix instructions (fwd_mfma_h4n).
#include "dwc_launch.h"
#include "dwc_mfma_h4.h"

namespace dwc {
namespace {

template <int DT, int FWI, int T, bool FLIP>
hipError_t go(const MfmaF32Args& a, hipStream_t s) {
  auto kernel = fwd_mfma_h4n<DT, FWI, T, FLIP>;
  if (a.lds_bytes > 65536) {
    // dynamic LDS above the default 64 KiB is allowed once per kernel
    static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                                    kLdsPerCu);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, dim3(a.num_blocks), dim3(64 * a.nw), a.lds_bytes, s, a);
  return hipGetLastError();
}

template <int DT, int FWI, bool FLIP>
hipError_t by_t(int t, const MfmaF32Args& a, hipStream_t s) {
#define DWC_CASE(TT) \
  if (t == TT) return go<DT, FWI, TT, FLIP>(a, s);
  DWC_H4M_T_LIST(DWC_CASE)
#undef DWC_CASE
  return hipErrorInvalidValue;
}

template <int DT, bool FLIP>
hipError_t by_fw(int fwi, int t, const MfmaF32Args& a, hipStream_t s) {
#define DWC_CASE(F) \
  if (fwi == F) return by_t<DT, F, FLIP>(t, a, s);
  DWC_H4M_FW_LIST(DWC_CASE)
#undef DWC_CASE
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t by_flip(int fwi, int t, bool flip, const MfmaF32Args& a, hipStream_t s) {
  return flip ? by_fw<DT, true>(fwi, t, a, s) : by_fw<DT, false>(fwi, t, a, s);
}

}  // namespace

hipError_t launch_fwd_mfma_h4(int dt, int fwi, int t, bool flip, const MfmaF32Args& a,
                              hipStream_t s) {
  if (dt == DT_BF16) return by_flip<DT_BF16>(fwi, t, flip, a, s);
  if (dt == DT_F16) return by_flip<DT_F16>(fwi, t, flip, a, s);
  return hipErrorInvalidValue;
}

}  // namespace dwc
