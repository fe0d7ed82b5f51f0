// inst_direct.hip -- instantiations of the direct kernels for one operand
// dtype.  Compiled once per dtype with -DDWC_INST_DT=<0..4>, and once more
// per dtype with -DDWC_INST_PAD=1 for the forward-type kernel on filters
// narrower than the instantiated width (launch_fwd_direct_pad_dt<D>, only
// that launcher).
#include "dwc_kernels.h"
#include "dwc_launch.h"

#ifndef DWC_INST_DT
#error "DWC_INST_DT must be defined"
#endif
#ifndef DWC_INST_PAD
#define DWC_INST_PAD 0
#endif

#define DWC_CAT2(a, b) a##b
#define DWC_CAT(a, b) DWC_CAT2(a, b)

namespace dwc {
namespace {

constexpr int kDt = DWC_INST_DT;
constexpr bool kPad = DWC_INST_PAD != 0;

// a.pro.scale set: the fused-prologue variant (forward, FW <= kPrologueMaxFw)
template <int S, int TMW, bool FLIP>
hipError_t fwd_by_fw(int fw, const FwdArgs& a, int blocks, hipStream_t s) {
  switch (fw) {
#define DWC_CASE(F)                                                                     \
  case F:                                                                               \
    if (a.pro.scale) {                                                                  \
      if constexpr (!FLIP && F <= kPrologueMaxFw) {                                     \
        hipLaunchKernelGGL((fwd_rows<kDt, F, S, TMW, FLIP, true, kPad>), dim3(blocks),  \
                           dim3(kBlockThreads), 0, s, a);                               \
        return hipGetLastError();                                                       \
      }                                                                                 \
      return hipErrorInvalidValue;                                                      \
    }                                                                                   \
    hipLaunchKernelGGL((fwd_rows<kDt, F, S, TMW, FLIP, false, kPad>), dim3(blocks),     \
                       dim3(kBlockThreads), 0, s, a);                                   \
    return hipGetLastError();
    DWC_DIRECT_FW_LIST(DWC_CASE)
#undef DWC_CASE
  }
  return hipErrorInvalidValue;
}

template <int S, bool FLIP>
hipError_t fwd_by_tmw(int fw, int tmw, const FwdArgs& a, int blocks, hipStream_t s) {
  switch (tmw) {
#define DWC_CASE(T) \
  case T:           \
    return fwd_by_fw<S, T, FLIP>(fw, a, blocks, s);
    DWC_FWD_TMW_LIST(DWC_CASE)
#undef DWC_CASE
  }
  return hipErrorInvalidValue;
}

#if !DWC_INST_PAD
template <int S, int TJ>
hipError_t wgrad_by_fw(int fw, const WgradArgs& a, int blocks, hipStream_t s) {
  switch (fw) {
#define DWC_CASE(F)                                                                     \
  case F:                                                                               \
    hipLaunchKernelGGL((wgrad_rows<kDt, F, S, TJ>), dim3(blocks), dim3(kBlockThreads),  \
                       0, s, a);                                                        \
    return hipGetLastError();
    DWC_DIRECT_FW_LIST(DWC_CASE)
#undef DWC_CASE
  }
  return hipErrorInvalidValue;
}

template <int S>
hipError_t wgrad_by_tj(int fw, int tj, const WgradArgs& a, int blocks, hipStream_t s) {
  switch (tj) {
#define DWC_CASE(T) \
  case T:           \
    return wgrad_by_fw<S, T>(fw, a, blocks, s);
    DWC_WGRAD_TJ_LIST(DWC_CASE)
#undef DWC_CASE
  }
  return hipErrorInvalidValue;
}

// Sweep strips: 7 columns for every filter size; 14 only up to 5x5, where
// the ring, filter and two prefetched strips still fit in registers.
template <int TMW, bool FLIP>
hipError_t fwd_sweep_by_f(int f, const SweepArgs& a, int blocks, hipStream_t s) {
  switch (f) {
#define DWC_CASE(F)                                                                       \
  case F:                                                                                 \
    if constexpr (TMW == 7 || F <= 5) {                                                   \
      if (a.pro.scale) {                                                                  \
        if constexpr (!FLIP) {                                                            \
          hipLaunchKernelGGL((fwd_sweep<kDt, F, TMW, FLIP, true>), dim3(blocks),          \
                             dim3(kBlockThreads), 0, s, a);                               \
          return hipGetLastError();                                                       \
        }                                                                                 \
        return hipErrorInvalidValue;                                                      \
      }                                                                                   \
      hipLaunchKernelGGL((fwd_sweep<kDt, F, TMW, FLIP>), dim3(blocks), dim3(kBlockThreads), \
                         0, s, a);                                                        \
      return hipGetLastError();                                                           \
    }                                                                                     \
    break;
    DWC_SWEEP_F_LIST(DWC_CASE)
#undef DWC_CASE
  }
  return hipErrorInvalidValue;
}

// a.hybrid: fp16 sub-unit accumulation (fp16 operands only)
template <int TJ>
hipError_t wgrad_sweep_by_f(int f, const SweepArgs& a, int blocks, hipStream_t s) {
  switch (f) {
#define DWC_CASE(F)                                                                       \
  case F:                                                                                 \
    if constexpr (TJ == 7 || F <= 5) {                                                    \
      if (a.hybrid) {                                                                     \
        if constexpr (kDt == DT_F16) {                                                    \
          hipLaunchKernelGGL((wgrad_sweep_hyb<F, TJ>), dim3(blocks), dim3(kBlockThreads), \
                             0, s, a);                                                    \
          return hipGetLastError();                                                       \
        }                                                                                 \
        return hipErrorInvalidValue;                                                      \
      }                                                                                   \
      hipLaunchKernelGGL((wgrad_sweep<kDt, F, TJ>), dim3(blocks), dim3(kBlockThreads), 0, \
                         s, a);                                                           \
      return hipGetLastError();                                                           \
    }                                                                                     \
    break;
    DWC_SWEEP_F_LIST(DWC_CASE)
#undef DWC_CASE
  }
  return hipErrorInvalidValue;
}

#endif  // !DWC_INST_PAD

}  // namespace

#if !DWC_INST_PAD
hipError_t DWC_CAT(launch_dgrad_phase_dt, DWC_INST_DT)(int km, const DgradPhaseArgs& a,
                                                       int blocks, hipStream_t s) {
  switch (km) {
#define DWC_CASE(K)                                                                        \
  case K:                                                                                  \
    hipLaunchKernelGGL((dgrad_phase<kDt, K, kPhaseTmw>), dim3(blocks), dim3(kBlockThreads), \
                       0, s, a);                                                           \
    return hipGetLastError();
    DWC_PHASE_KM_LIST(DWC_CASE)
#undef DWC_CASE
  }
  return hipErrorInvalidValue;
}

hipError_t DWC_CAT(launch_fwd_sweep_dt, DWC_INST_DT)(int f, int tmw, bool flip, const SweepArgs& a,
                                                     int blocks, hipStream_t st) {
  if (tmw == 7) return flip ? fwd_sweep_by_f<7, true>(f, a, blocks, st)
                            : fwd_sweep_by_f<7, false>(f, a, blocks, st);
  if (tmw == 14) return flip ? fwd_sweep_by_f<14, true>(f, a, blocks, st)
                             : fwd_sweep_by_f<14, false>(f, a, blocks, st);
  return hipErrorInvalidValue;
}

hipError_t DWC_CAT(launch_wgrad_sweep_dt, DWC_INST_DT)(int f, int tj, const SweepArgs& a,
                                                       int blocks, hipStream_t st) {
  if (tj == 7) return wgrad_sweep_by_f<7>(f, a, blocks, st);
  if (tj == 14) return wgrad_sweep_by_f<14>(f, a, blocks, st);
  return hipErrorInvalidValue;
}

#endif  // !DWC_INST_PAD

// fw: the instantiated width (a.FW itself, or with DWC_INST_PAD the width
// the narrower a.FW runs on); s: the stride of both spatial axes (1 or 2;
// the data gradient only 1).
#if DWC_INST_PAD
hipError_t DWC_CAT(launch_fwd_direct_pad_dt, DWC_INST_DT)(
#else
hipError_t DWC_CAT(launch_fwd_direct_dt, DWC_INST_DT)(
#endif
    int fw, int s, int tmw, bool flip, const FwdArgs& a, int blocks, hipStream_t st) {
  if (kPad ? a.FW >= fw : a.FW != fw) return hipErrorInvalidValue;
  if (s == 1) return flip ? fwd_by_tmw<1, true>(fw, tmw, a, blocks, st)
                          : fwd_by_tmw<1, false>(fw, tmw, a, blocks, st);
  if (s == 2 && !flip) return fwd_by_tmw<2, false>(fw, tmw, a, blocks, st);
  return hipErrorInvalidValue;
}

#if !DWC_INST_PAD
// fw: the instantiated width, a.FW or wider (taps past a.FW are not written)
hipError_t DWC_CAT(launch_wgrad_direct_dt, DWC_INST_DT)(int fw, int s, int tj,
                                                        const WgradArgs& a, int blocks,
                                                        hipStream_t st) {
  if (a.FW > fw) return hipErrorInvalidValue;
  if (s == 1) return wgrad_by_tj<1>(fw, tj, a, blocks, st);
  if (s == 2) return wgrad_by_tj<2>(fw, tj, a, blocks, st);
  return hipErrorInvalidValue;
}
#endif  // !DWC_INST_PAD

}  // namespace dwc
