// dwc_plan.h -- host-side validation and launch planning (no HIP calls).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/dwc.h"
#include "dwc_geom.h"

namespace dwc {

enum PlanKind { PLAN_NONE = 0, PLAN_DIRECT = 1, PLAN_GENERIC = 2, PLAN_MFMA = 3, PLAN_PHASE = 4 };

struct Plan {
  int op = 0;
  int dt = 0;
  int kind = PLAN_NONE;
  bool sweep = false;  // direct plan runs the sweep kernels
  int64_t oh = 0, ow = 0;
  bool empty = false;  // n == 0

  // direct kernels: the instantiated filter width they run on (FW itself,
  // else the next wider one, whose taps past FW are skipped)
  int kfw = 0;
  // forward-type direct kernel (forward, stride-1 data gradient)
  int tmw = 0;
  bool flip = false;
  FwdArgs fa{};
  int blocks = 0;

  // filter-gradient direct kernel
  int tj = 0, tfh = 0;
  WgradArgs wa{};
  int z = 1;
  size_t ws_bytes = 0;  // 0: slice partials are written straight to dW

  // sweep kernels (stride 1, square filters up to 9x9)
  SweepArgs sa{};

  // packed-MFMA forward-type kernel
  int nf = 0, cb = 0, tiles = 0;
  MfmaArgs ma{};
  // ... with the batch in the matrix rows
  bool batch = false;
  int bimg = 0;  // images per instruction: 32 (fwd_mfma_batch) or 16 (fwd_mfma_batch16)
  int bng = 0;   // 16-column output groups of fwd_mfma_batch16 (1 or 2)
  MfmaBatchArgs mb{};
  // fp32 matrix-core forward-type kernel
  bool f32m = false;
  int f32m_fwi = 0, f32m_t = 0;  // instantiated band width, 4-column tiles per wave
  bool f32m_img = false;         // 4 images (not 4 output rows) as the matrix rows
  MfmaF32Args mf{};
  // 16-bit forward-type kernel on 4x4x4 matrix instructions (arguments in mf)
  bool h4m = false;
  int h4m_fwi = 0, h4m_t = 0;  // instantiated band width, 4-column tiles per wave
  // fp32 matrix-core filter gradient
  bool wf32 = false;
  int wf32_tw = 0, wf32_nb = 0;  // column tiles, 4-column output groups per wave
  WgradF32Args wf{};
  // packed-MFMA filter gradient
  int nfm = 0, nfn = 0, nk = 0, pf = 0;
  WgradMfmaArgs wm{};
  // strided data gradient by output phase
  int km = 0;
  DgradPhaseArgs pa{};

  // generic kernels
  int gen_kind = 0;
  GenericArgs ga{};
};

// Validates `p` for `op` and fills `pl`.  Returns a dwc_status; on error
// `err` holds the message.
int make_plan(const dwc_problem* p, int op, Plan* pl, std::string* err);

// Checks the tensor pointers of a call (null, alignment, overlap of the
// output with the inputs, workspace).  No GPU access.
int check_pointers(const dwc_problem* p, const Plan& pl, const void* in0, const void* in1,
                   const void* out, const void* ws, size_t ws_bytes, std::string* err);

// Checks the scale and shift vectors of a fused-prologue forward (null,
// alignment, overlap with the output).
int check_prologue(const dwc_problem* p, const Plan& pl, const void* out, const float* scale,
                   const float* shift, std::string* err);

std::string describe(const Plan& pl);

void set_last_error(const std::string& msg);

// Compute units of the device the calls run on, which the planner's fill
// targets scale with: read once per device by the HIP side of the library
// (through the hook it installs when the library loads); MI355X's 256 when
// no device is visible (planning on a host without a GPU).
int device_cus();
void set_device_cus_hook(int (*hook)());

}  // namespace dwc
