// dwc_launch.h -- host-side launchers of the libdwc kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "dwc_geom.h"

namespace dwc {

// Forward-type direct kernel for operand dtype dt (one object per dtype).
hipError_t launch_fwd_direct_dt0(int fw, int s, int tmw, bool flip, const FwdArgs& a,
                                 int blocks, hipStream_t st);
hipError_t launch_fwd_direct_dt1(int fw, int s, int tmw, bool flip, const FwdArgs& a,
                                 int blocks, hipStream_t st);
hipError_t launch_fwd_direct_dt2(int fw, int s, int tmw, bool flip, const FwdArgs& a,
                                 int blocks, hipStream_t st);

// Filter-gradient direct kernel for operand dtype dt.
// Strided data gradient by output phase; km: padded sub-filter size (one of
// DWC_PHASE_KM_LIST).
hipError_t launch_dgrad_phase_dt0(int km, const DgradPhaseArgs& a, int blocks, hipStream_t s);
hipError_t launch_dgrad_phase_dt1(int km, const DgradPhaseArgs& a, int blocks, hipStream_t s);
hipError_t launch_dgrad_phase_dt2(int km, const DgradPhaseArgs& a, int blocks, hipStream_t s);

hipError_t launch_wgrad_direct_dt0(int fw, int s, int tj, const WgradArgs& a, int blocks,
                                   hipStream_t st);
hipError_t launch_wgrad_direct_dt1(int fw, int s, int tj, const WgradArgs& a, int blocks,
                                   hipStream_t st);
hipError_t launch_wgrad_direct_dt2(int fw, int s, int tj, const WgradArgs& a, int blocks,
                                   hipStream_t st);

// Sweep kernels (stride 1, square filters up to 9x9).
#define DWC_DECL_SWEEP(D)                                                                 \
  hipError_t launch_fwd_sweep_dt##D(int f, int tmw, bool flip, const SweepArgs& a,         \
                                    int blocks, hipStream_t st);                         \
  hipError_t launch_wgrad_sweep_dt##D(int f, int tj, const SweepArgs& a, int blocks,       \
                                      hipStream_t st);
DWC_DECL_SWEEP(0)
DWC_DECL_SWEEP(1)
DWC_DECL_SWEEP(2)
#undef DWC_DECL_SWEEP

// Packed-MFMA forward-type kernel (bf16 / fp16 operands, stride 1): nf
// 16-tap fragments per filter row, tiles of 16 combinations per channel.
hipError_t launch_fwd_mfma(int dt, int nf, int tiles, bool flip, const MfmaArgs& a,
                           hipStream_t s);

// Packed-MFMA filter gradient: nfm / nfn 16-tap fragments of the filter
// width / height, nk 32-column chunks of the input width, pf staging items
// per thread.  Writes channel-blocked slice partials (reduce with
// cb = kWgmCb).
hipError_t launch_wgrad_mfma(int dt, int nfm, int nfn, int nk, int pf, const WgradMfmaArgs& a,
                             hipStream_t s);

enum GenericKind { GEN_FWD = 0, GEN_FWD_FLIP = 1, GEN_DGRAD = 2, GEN_WGRAD = 3 };
hipError_t launch_generic(int kind, int dt, const GenericArgs& a, hipStream_t st);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st);

}  // namespace dwc
