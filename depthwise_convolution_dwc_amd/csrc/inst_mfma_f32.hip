// inst_mfma_f32.hip -- instantiations and launcher of the fp32 matrix-core
// forward-type kernel (fwd_mfma_f32).
#include "dwc_launch.h"
#include "dwc_mfma_f32.h"

namespace dwc {
namespace {

template <int DT, int FWI, int T, bool FLIP, bool IMG>
hipError_t go(const MfmaF32Args& a, hipStream_t s) {
  void (*kernel)(MfmaF32Args);
  if constexpr (IMG) kernel = fwd_mfma_f32n<FWI, T, FLIP>;  // fp32 operands only
  else kernel = fwd_mfma_f32<DT, FWI, T, FLIP>;
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
hipError_t by_t(int t, bool img, const MfmaF32Args& a, hipStream_t s) {
  if (img) {  // 2 or 4 tiles: the accumulator ring takes the registers of more
    if constexpr (DT == DT_F32) {
      if (t == 2) return go<DT, FWI, 2, FLIP, true>(a, s);
      if (t == 4) return go<DT, FWI, 4, FLIP, true>(a, s);
    }
    return hipErrorInvalidValue;
  }
#define DWC_CASE(TT) \
  if (t == TT) return go<DT, FWI, TT, FLIP, false>(a, s);
  DWC_F32M_T_LIST(DWC_CASE)
#undef DWC_CASE
  return hipErrorInvalidValue;
}

template <int DT, bool FLIP>
hipError_t by_fw(int fwi, int t, bool img, const MfmaF32Args& a, hipStream_t s) {
#define DWC_CASE(F) \
  if (fwi == F) return by_t<DT, F, FLIP>(t, img, a, s);
  DWC_F32M_FW_LIST(DWC_CASE)
#undef DWC_CASE
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t by_flip(int fwi, int t, bool img, bool flip, const MfmaF32Args& a, hipStream_t s) {
  return flip ? by_fw<DT, true>(fwi, t, img, a, s) : by_fw<DT, false>(fwi, t, img, a, s);
}

template <int DT, int TW, int NB>
hipError_t go_w(const WgradF32Args& a, hipStream_t s) {
  auto kernel = wgrad_mfma_f32<DT, TW, NB>;
  hipLaunchKernelGGL(kernel, dim3(a.num_blocks), dim3(64 * a.nw), a.lds_bytes, s, a);
  return hipGetLastError();
}

template <int DT, int TW>
hipError_t by_nb(int nb, const WgradF32Args& a, hipStream_t s) {
#define DWC_CASE(B) \
  if (nb == B) return go_w<DT, TW, B>(a, s);
  DWC_WF32_NB_LIST(DWC_CASE)
#undef DWC_CASE
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t by_tw(int tw, int nb, const WgradF32Args& a, hipStream_t s) {
#define DWC_CASE(W) \
  if (tw == W) return by_nb<DT, W>(nb, a, s);
  DWC_WF32_TW_LIST(DWC_CASE)
#undef DWC_CASE
  return hipErrorInvalidValue;
}

}  // namespace

// dt: the operand type of x and dY (fp32, bf16 or fp16)
hipError_t launch_wgrad_mfma_f32(int dt, int tw, int nb, const WgradF32Args& a, hipStream_t s) {
  if (dt == DT_F32) return by_tw<DT_F32>(tw, nb, a, s);
  if (dt == DT_BF16) return by_tw<DT_BF16>(tw, nb, a, s);
  if (dt == DT_F16) return by_tw<DT_F16>(tw, nb, a, s);
  return hipErrorInvalidValue;
}

// dt: the operand type of the input and filter (the images kernel: fp32)
hipError_t launch_fwd_mfma_f32(int dt, int fwi, int t, bool img, bool flip,
                               const MfmaF32Args& a, hipStream_t s) {
  if (dt == DT_F32) return by_flip<DT_F32>(fwi, t, img, flip, a, s);
  if (dt == DT_BF16) return by_flip<DT_BF16>(fwi, t, img, flip, a, s);
  if (dt == DT_F16) return by_flip<DT_F16>(fwi, t, img, flip, a, s);
  return hipErrorInvalidValue;
}

}  // namespace dwc
