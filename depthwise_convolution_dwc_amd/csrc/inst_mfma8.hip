// inst_mfma8.hip -- instantiations and launchers of the packed-MFMA
// kernels for fp8 operands (e4m3 / e5m2): forward-type and filter gradient.
#include "dwc_launch.h"
#include "dwc_mfma8.h"

namespace dwc {
namespace {

template <typename K>
hipError_t allow_lds(K kernel) {
  static const hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      kMfmaMaxLds);
  return e;
}

template <int DT, int NF, int TILES, bool FLIP>
hipError_t go(const MfmaArgs& a, hipStream_t s) {
  auto kernel = fwd_mfma8<DT, NF, TILES, FLIP>;
  if (a.lds_bytes > 65536) {
    const hipError_t e = allow_lds(kernel);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, dim3(a.num_blocks), dim3(64 * kMfmaWaves), a.lds_bytes, s, a);
  return hipGetLastError();
}

template <int DT, int NF, bool FLIP>
hipError_t by_tiles(int tiles, const MfmaArgs& a, hipStream_t s) {
  if (tiles == 1) return go<DT, NF, 1, FLIP>(a, s);
  if (tiles == 2) return go<DT, NF, 2, FLIP>(a, s);
  if (tiles == 4) return go<DT, NF, 4, FLIP>(a, s);
  return hipErrorInvalidValue;
}

template <int DT, bool FLIP>
hipError_t by_nf(int nf, int tiles, const MfmaArgs& a, hipStream_t s) {
  if (nf == 1) return by_tiles<DT, 1, FLIP>(tiles, a, s);
  if (nf == 2) return by_tiles<DT, 2, FLIP>(tiles, a, s);
  return hipErrorInvalidValue;
}

template <int DT, int NFM, int NFN, int NK, int PF>
hipError_t wg_go(const WgradMfmaArgs& a, hipStream_t s) {
  auto kernel = wgrad_mfma8<DT, NFM, NFN, NK, PF>;
  if (a.lds_bytes > 65536) {
    const hipError_t e = allow_lds(kernel);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, dim3(a.num_blocks), dim3(64 * kMfmaWaves), a.lds_bytes, s, a);
  return hipGetLastError();
}

template <int DT, int NFM, int NFN, int NK>
hipError_t wg_by_pf(int pf, const WgradMfmaArgs& a, hipStream_t s) {
  if (pf == 1) return wg_go<DT, NFM, NFN, NK, 1>(a, s);
  if (pf == 2) return wg_go<DT, NFM, NFN, NK, 2>(a, s);
  return hipErrorInvalidValue;
}

template <int DT, int NFM, int NFN>
hipError_t wg_by_nk(int nk, int pf, const WgradMfmaArgs& a, hipStream_t s) {
  if (nk == 1) return wg_by_pf<DT, NFM, NFN, 1>(pf, a, s);
  if (nk == 2) return wg_by_pf<DT, NFM, NFN, 2>(pf, a, s);
  return hipErrorInvalidValue;
}

template <int DT, int NFM>
hipError_t wg_by_nfn(int nfn, int nk, int pf, const WgradMfmaArgs& a, hipStream_t s) {
  if (nfn == 1) return wg_by_nk<DT, NFM, 1>(nk, pf, a, s);
  if (nfn == 2) return wg_by_nk<DT, NFM, 2>(nk, pf, a, s);
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t wg_by_nfm(int nfm, int nfn, int nk, int pf, const WgradMfmaArgs& a, hipStream_t s) {
  if (nfm == 1) return wg_by_nfn<DT, 1>(nfn, nk, pf, a, s);
  if (nfm == 2) return wg_by_nfn<DT, 2>(nfn, nk, pf, a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_wgrad_mfma8(int dt, int nfm, int nfn, int nk, int pf, const WgradMfmaArgs& a,
                              hipStream_t s) {
  if (dt == DT_E4M3) return wg_by_nfm<DT_E4M3>(nfm, nfn, nk, pf, a, s);
  if (dt == DT_E5M2) return wg_by_nfm<DT_E5M2>(nfm, nfn, nk, pf, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_mfma8(int dt, int nf, int tiles, bool flip, const MfmaArgs& a,
                            hipStream_t s) {
  if (dt == DT_E4M3) return flip ? by_nf<DT_E4M3, true>(nf, tiles, a, s)
                                 : by_nf<DT_E4M3, false>(nf, tiles, a, s);
  if (dt == DT_E5M2) return flip ? by_nf<DT_E5M2, true>(nf, tiles, a, s)
                                 : by_nf<DT_E5M2, false>(nf, tiles, a, s);
  return hipErrorInvalidValue;
}

}  // namespace dwc
