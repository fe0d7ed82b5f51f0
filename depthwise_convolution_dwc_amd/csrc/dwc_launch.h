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
hipError_t launch_wgrad_direct_dt0(int fw, int s, int tj, const WgradArgs& a, int blocks,
                                   hipStream_t st);
hipError_t launch_wgrad_direct_dt1(int fw, int s, int tj, const WgradArgs& a, int blocks,
                                   hipStream_t st);
hipError_t launch_wgrad_direct_dt2(int fw, int s, int tj, const WgradArgs& a, int blocks,
                                   hipStream_t st);

enum GenericKind { GEN_FWD = 0, GEN_FWD_FLIP = 1, GEN_DGRAD = 2, GEN_WGRAD = 3 };
hipError_t launch_generic(int kind, int dt, const GenericArgs& a, hipStream_t st);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st);

}  // namespace dwc
