// dwc_launch.h -- host-side launchers of the libdwc kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "dwc_geom.h"

namespace dwc {

// Operand dtypes with their own instantiation of the direct kernels (one
// object per dtype, DWC_INST_DT): fp32, bf16, fp16, fp8 e4m3, fp8 e5m2.
#define DWC_DT_LIST(X) X(0) X(1) X(2) X(3) X(4)

// Per operand dtype D:
//  * forward-type direct kernel (fw: the instantiated width; s: stride; flip:
//    the stride-1 data gradient); the _pad_ form for a filter narrower than
//    fw;
//  * strided data gradient by output phase (km: padded sub-filter size, one
//    of DWC_PHASE_KM_LIST);
//  * filter-gradient direct kernel;
//  * sweep kernels (stride 1, square filters up to 9x9).
#define DWC_DECL_DT(D)                                                                    \
  hipError_t launch_fwd_direct_dt##D(int fw, int s, int tmw, bool flip, const FwdArgs& a, \
                                     int blocks, hipStream_t st);                         \
  hipError_t launch_fwd_direct_pad_dt##D(int fw, int s, int tmw, bool flip,               \
                                         const FwdArgs& a, int blocks, hipStream_t st);   \
  hipError_t launch_dgrad_phase_dt##D(int km, const DgradPhaseArgs& a, int blocks,        \
                                      hipStream_t s);                                     \
  hipError_t launch_wgrad_direct_dt##D(int fw, int s, int tj, const WgradArgs& a,         \
                                       int blocks, hipStream_t st);                       \
  hipError_t launch_fwd_sweep_dt##D(int f, int tmw, bool flip, const SweepArgs& a,        \
                                    int blocks, hipStream_t st);                          \
  hipError_t launch_wgrad_sweep_dt##D(int f, int tj, const SweepArgs& a, int blocks,      \
                                      hipStream_t st);
DWC_DT_LIST(DWC_DECL_DT)
#undef DWC_DECL_DT

// Packed-MFMA forward-type kernel (bf16 / fp16 operands, stride 1): nf
// 16-tap fragments per filter row, tiles of 16 combinations per channel.
hipError_t launch_fwd_mfma(int dt, int nf, int tiles, bool flip, const MfmaArgs& a,
                           hipStream_t s);

// Packed-MFMA forward-type kernel with the batch in the matrix rows (bf16 /
// fp16 operands, stride 1, widths up to 32).
hipError_t launch_fwd_mfma_batch(int dt, bool flip, const MfmaBatchArgs& a, hipStream_t s);
// ... with 16 images per instruction and two channels per wave (ng output
// column groups of 16); bf16 / fp16 and fp8 (e4m3 / e5m2) operands.
hipError_t launch_fwd_mfma_batch16(int dt, int ng, bool flip, const MfmaBatchArgs& a,
                                   hipStream_t s);

// fp32 matrix-core forward-type kernel (fp32 operands, stride 1, FW <= 31,
// C % 16 == 0): fwi the instantiated band width (DWC_F32M_FW_LIST), t the
// 4-column output tiles per wave (DWC_F32M_T_LIST; 2 or 4 with img), img
// 4 images instead of 4 output rows as the matrix rows (fwd_mfma_f32n).
// 16-bit forward-type kernel on the 4x4x4 matrix instructions, 4 images as
// the matrix rows (fwd_mfma_h4n).
hipError_t launch_fwd_mfma_h4(int dt, int fwi, int t, bool flip, const MfmaF32Args& a,
                              hipStream_t s);
hipError_t launch_fwd_mfma_f32(int dt, int fwi, int t, bool img, bool flip,
                               const MfmaF32Args& a, hipStream_t s);

// fp32 matrix-core filter gradient (fp32 operands, stride 1, FH and FW <=
// 32, C % 16 == 0): tw = ceil(FW / 4) column tiles, nb 4-column output
// groups per wave (DWC_WF32_NB_LIST).  Writes channel-blocked slice
// partials (reduce with cb = kWf32Cb).
hipError_t launch_wgrad_mfma_f32(int dt, int tw, int nb, const WgradF32Args& a, hipStream_t s);

// Packed fp8 MFMA forward-type kernel (e4m3 / e5m2 operands, stride 1,
// 16x16x128 MFMAs over four filter rows each): nf 16-tap fragments per
// filter row, tiles of 16 combinations per channel, 16 channels per
// workgroup.
hipError_t launch_fwd_mfma8(int dt, int nf, int tiles, bool flip, const MfmaArgs& a,
                            hipStream_t s);

// Packed-MFMA filter gradient: nfm / nfn 16-tap fragments of the filter
// width / height, nk 32-column chunks of the input width, pf staging items
// per thread.  Writes channel-blocked slice partials (reduce with
// cb = kWgmCb).
hipError_t launch_wgrad_mfma(int dt, int nfm, int nfn, int nk, int pf, const WgradMfmaArgs& a,
                             hipStream_t s);
// The same for fp8 operands (16x16x128 MFMAs over four output rows each).
hipError_t launch_wgrad_mfma8(int dt, int nfm, int nfn, int nk, int pf, const WgradMfmaArgs& a,
                              hipStream_t s);

enum GenericKind { GEN_FWD = 0, GEN_FWD_FLIP = 1, GEN_DGRAD = 2, GEN_WGRAD = 3 };
hipError_t launch_generic(int kind, int dt, const GenericArgs& a, hipStream_t st);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st);

}  // namespace dwc
