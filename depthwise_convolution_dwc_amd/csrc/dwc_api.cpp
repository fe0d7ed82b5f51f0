// dwc_api.cpp -- the compute entry points of libdwc (extern "C").
// Validation happens in dwc_plan.cpp before any HIP call; this file only
// launches the planned kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "dwc_launch.h"
#include "dwc_plan.h"

using namespace dwc;

namespace {

int hip_fail(hipError_t e, const char* what) {
  set_last_error(std::string(what) + ": " + hipGetErrorString(e));
  return DWC_ERR_HIP;
}

hipError_t launch_fwd_type(const Plan& pl, const void* in, const void* filt, float* out,
                           hipStream_t s) {
  if (pl.kind == PLAN_PHASE) {
    DgradPhaseArgs g = pl.pa;
    g.dy = in;
    g.filt = filt;
    g.dx = out;
    switch (pl.dt) {
#define DWC_CASE(D) \
  case D: return launch_dgrad_phase_dt##D(pl.km, g, pl.blocks, s);
      DWC_DT_LIST(DWC_CASE)
#undef DWC_CASE
    }
    return hipErrorInvalidValue;
  }
  if (pl.kind == PLAN_MFMA && pl.h4m) {
    MfmaF32Args m = pl.mf;
    m.in = in;
    m.filt = filt;
    m.out = out;
    return launch_fwd_mfma_h4(pl.dt, pl.h4m_fwi, pl.h4m_t, pl.flip, m, s);
  }
  if (pl.kind == PLAN_MFMA && pl.f32m) {
    MfmaF32Args m = pl.mf;
    m.in = in;
    m.filt = filt;
    m.out = out;
    return launch_fwd_mfma_f32(pl.dt, pl.f32m_fwi, pl.f32m_t, pl.f32m_img, pl.flip, m, s);
  }
  if (pl.kind == PLAN_MFMA && pl.batch) {
    MfmaBatchArgs m = pl.mb;
    m.in = in;
    m.filt = filt;
    m.out = out;
    if (pl.bimg == kB16Img) return launch_fwd_mfma_batch16(pl.dt, pl.bng, pl.flip, m, s);
    return launch_fwd_mfma_batch(pl.dt, pl.flip, m, s);
  }
  if (pl.kind == PLAN_MFMA) {
    MfmaArgs m = pl.ma;
    m.in = in;
    m.filt = filt;
    m.out = out;
    if (pl.dt == DT_E4M3 || pl.dt == DT_E5M2)
      return launch_fwd_mfma8(pl.dt, pl.nf, pl.tiles, pl.flip, m, s);
    return launch_fwd_mfma(pl.dt, pl.nf, pl.tiles, pl.flip, m, s);
  }
  if (pl.kind == PLAN_DIRECT) {
    FwdArgs a = pl.fa;
    a.in = in;
    a.filt = filt;
    a.out = out;
    if (pl.sweep) {
      SweepArgs w = pl.sa;
      w.in = in;
      w.in2 = filt;
      w.out = out;
      switch (pl.dt) {
#define DWC_CASE(D) \
  case D: return launch_fwd_sweep_dt##D(w.F, pl.tmw, pl.flip, w, pl.blocks, s);
        DWC_DT_LIST(DWC_CASE)
#undef DWC_CASE
      }
      return hipErrorInvalidValue;
    }
    switch (pl.dt) {
#define DWC_CASE(D) \
  case D:                                                                            \
    return pl.kfw == a.FW ? launch_fwd_direct_dt##D(pl.kfw, a.SW, pl.tmw, pl.flip, a, pl.blocks, s) \
                          : launch_fwd_direct_pad_dt##D(pl.kfw, a.SW, pl.tmw, pl.flip, a, pl.blocks, s);
      DWC_DT_LIST(DWC_CASE)
#undef DWC_CASE
    }
    return hipErrorInvalidValue;
  }
  GenericArgs g = pl.ga;
  g.a = in;
  g.b = filt;
  g.out = out;
  return launch_generic(pl.gen_kind, pl.dt, g, s);
}

bool aligned16(const void* a) { return ((uintptr_t)a & 15) == 0; }

int prepare(const dwc_problem* p, int op, Plan* pl, const void* in0, const void* in1,
            const void* out, const void* ws, size_t ws_bytes) {
  std::string err;
  int st = make_plan(p, op, pl, &err);
  // The packed-MFMA kernels move 16-byte vectors: with a tensor that is not
  // 16-byte aligned, AUTO takes the vector kernels and MFMA is an error.
  // (The filter-gradient kernel also stores 16-byte partials into the
  // workspace.)
  if (st == DWC_OK && pl->kind == PLAN_MFMA && !pl->empty &&
      !(aligned16(in0) && aligned16(in1) && aligned16(out) &&
        (op != DWC_OP_BWD_FILTER || aligned16(ws)))) {
    if (p->algo == DWC_ALGO_MFMA) {
      set_last_error("packed-MFMA kernels need 16-byte aligned tensors");
      return DWC_ERR_MISALIGNED;
    }
    dwc_problem d = *p;
    d.algo = DWC_ALGO_DIRECT;
    st = make_plan(&d, op, pl, &err);
    if (st == DWC_ERR_UNSUPPORTED) {
      d.algo = DWC_ALGO_GENERIC;
      st = make_plan(&d, op, pl, &err);
    }
  }
  if (st == DWC_OK) st = check_pointers(p, *pl, in0, in1, out, ws, ws_bytes, &err);
  if (st != DWC_OK) set_last_error(err);
  return st;
}

// Launches a validated filter-gradient plan: the slice kernel, then the
// deterministic reduction of the slice partials held in `workspace`.
int run_bwd_filter(const dwc_problem* p, const Plan& pl, const void* x, const void* dy,
                   void* dw, void* workspace, hipStream_t s) {
  const int64_t m = (int64_t)p->fh * p->fw * p->c;
  if (pl.empty) {  // empty batch: dW = 0 (a sum over no terms)
    const hipError_t e = launch_reduce(ReduceArgs{nullptr, (float*)dw, m, 0}, s);
    return e == hipSuccess ? DWC_OK : hip_fail(e, "dwc_bwd_filter zero fill");
  }
  // One slice writes dW directly; several write partials to the workspace.
  float* part = pl.ws_bytes > 0 ? (float*)workspace : (float*)dw;
  hipError_t e;
  if (pl.kind == PLAN_MFMA && pl.wf32) {
    WgradF32Args w = pl.wf;
    w.x = x;
    w.dy = dy;
    w.ws = (float*)workspace;
    e = launch_wgrad_mfma_f32(pl.dt, pl.wf32_tw, pl.wf32_nb, w, s);
    if (e != hipSuccess) return hip_fail(e, "dwc_bwd_filter launch");
    e = launch_reduce(
        ReduceArgs{(const float*)workspace, (float*)dw, m, pl.z, kWf32Cb, w.C, w.FH * w.FW}, s);
    return e == hipSuccess ? DWC_OK : hip_fail(e, "dwc_bwd_filter reduce");
  }
  if (pl.kind == PLAN_MFMA) {
    WgradMfmaArgs w = pl.wm;
    w.x = x;
    w.dy = dy;
    w.ws = (float*)workspace;
    e = (pl.dt == DT_E4M3 || pl.dt == DT_E5M2)
            ? launch_wgrad_mfma8(pl.dt, pl.nfm, pl.nfn, pl.nk, pl.pf, w, s)
            : launch_wgrad_mfma(pl.dt, pl.nfm, pl.nfn, pl.nk, pl.pf, w, s);
    if (e != hipSuccess) return hip_fail(e, "dwc_bwd_filter launch");
    e = launch_reduce(
        ReduceArgs{(const float*)workspace, (float*)dw, m, pl.z, kWgmCb, w.C, w.FH * w.FW}, s);
    return e == hipSuccess ? DWC_OK : hip_fail(e, "dwc_bwd_filter reduce");
  }
  if (pl.kind == PLAN_DIRECT) {
    WgradArgs a = pl.wa;
    a.x = x;
    a.dy = dy;
    a.ws = part;
    if (pl.sweep) {
      SweepArgs w = pl.sa;
      w.in = x;
      w.in2 = dy;
      w.out = part;
      switch (pl.dt) {
#define DWC_CASE(D) \
  case D: e = launch_wgrad_sweep_dt##D(w.F, pl.tj, w, pl.blocks, s); break;
        DWC_DT_LIST(DWC_CASE)
#undef DWC_CASE
        default: e = hipErrorInvalidValue; break;
      }
    } else {
      switch (pl.dt) {
#define DWC_CASE(D) \
  case D: e = launch_wgrad_direct_dt##D(pl.kfw, a.SW, pl.tj, a, pl.blocks, s); break;
        DWC_DT_LIST(DWC_CASE)
#undef DWC_CASE
        default: e = hipErrorInvalidValue; break;
      }
    }
  } else {
    GenericArgs g = pl.ga;
    g.a = x;
    g.b = dy;
    g.out = part;
    e = launch_generic(pl.gen_kind, pl.dt, g, s);
  }
  if (e != hipSuccess) return hip_fail(e, "dwc_bwd_filter launch");
  if (pl.ws_bytes > 0) {
    e = launch_reduce(ReduceArgs{(const float*)workspace, (float*)dw, m, pl.z}, s);
    if (e != hipSuccess) return hip_fail(e, "dwc_bwd_filter reduce");
  }
  return DWC_OK;
}

// Fixed scratch of dwc_bwd_filter_noalloc: the filter gradient's slice
// partials, for callers that cannot allocate device memory.  Each device
// holds its own copy for the life of the process; host code reaches it only
// through the address hipGetSymbolAddress returns on that device.
constexpr size_t kScratchBytes = DWC_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The scratch's device address on the current device, looked up once per
// device with that device current.
int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    set_last_error("device index beyond the scratch table");
    return DWC_ERR_UNSUPPORTED;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_fail(g_scratch_err[dev], "hipGetSymbolAddress");
  *out = g_scratch_ptr[dev];
  return DWC_OK;
}

// Compute units per device, read once per device (the planner's fill
// targets scale with them: a partitioned GPU shows fewer).
std::once_flag g_cus_once[kMaxDevices];
int g_cus[kMaxDevices];

int current_device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();  // no device: the planner's default
    return 0;
  }
  std::call_once(g_cus_once[dev], [dev] {
    int v = 0;
    g_cus[dev] = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) ==
                         hipSuccess
                     ? v
                     : 0;
  });
  return g_cus[dev];
}

struct InstallCusHook {
  InstallCusHook() { set_device_cus_hook(current_device_cus); }
} g_install_cus_hook;

}  // namespace

extern "C" {

int dwc_fwd(const dwc_problem* p, const void* x, const void* w, void* y, void* stream) {
  Plan pl;
  const int st = prepare(p, DWC_OP_FWD, &pl, x, w, y, nullptr, 0);
  if (st != DWC_OK || pl.empty) return st;
  const hipError_t e = launch_fwd_type(pl, x, w, (float*)y, (hipStream_t)stream);
  return e == hipSuccess ? DWC_OK : hip_fail(e, "dwc_fwd launch");
}

int dwc_fwd_fused(const dwc_problem* p, const void* x, const float* scale, const float* shift,
                  int act, const void* w, void* y, void* stream) {
  if (!p) {
    set_last_error("problem pointer is NULL");
    return DWC_ERR_BAD_PARAM;
  }
  if (act < DWC_ACT_NONE || act > DWC_ACT_SILU) {
    set_last_error("unknown activation (act must be a dwc_act)");
    return DWC_ERR_BAD_PARAM;
  }
  if (p->algo != DWC_ALGO_AUTO && p->algo != DWC_ALGO_DIRECT) {
    set_last_error("the fused prologue runs on the direct vector kernels "
                   "(algo DWC_ALGO_AUTO or DWC_ALGO_DIRECT)");
    return DWC_ERR_UNSUPPORTED;
  }
  dwc_problem d = *p;
  d.algo = DWC_ALGO_DIRECT;
  Plan pl;
  std::string err;
  int st = make_plan(&d, DWC_OP_FWD, &pl, &err);
  if (st == DWC_OK && (pl.kind != PLAN_DIRECT || p->fw > kPrologueMaxFw)) st = DWC_ERR_UNSUPPORTED;
  if (st == DWC_ERR_UNSUPPORTED)
    err = "the fused prologue needs a filter width up to 9 and stride 1 or 2 "
          "(the direct vector kernels)";
  if (st == DWC_OK) st = check_pointers(&d, pl, x, w, y, nullptr, 0, &err);
  if (st == DWC_OK) st = check_prologue(&d, pl, y, scale, shift, &err);
  if (st != DWC_OK) {
    set_last_error(err);
    return st;
  }
  if (pl.empty) return DWC_OK;
  const float inf = __builtin_inff();
  Prologue pro{scale, shift, -inf, inf, 0};
  if (act == DWC_ACT_RELU) pro.lo = 0.f;
  if (act == DWC_ACT_RELU6) {
    pro.lo = 0.f;
    pro.hi = 6.f;
  }
  if (act == DWC_ACT_SILU) pro.silu = 1;
  pl.fa.pro = pro;
  pl.sa.pro = pro;
  const hipError_t e = launch_fwd_type(pl, x, w, (float*)y, (hipStream_t)stream);
  return e == hipSuccess ? DWC_OK : hip_fail(e, "dwc_fwd_fused launch");
}

int dwc_bwd_data(const dwc_problem* p, const void* dy, const void* w, void* dx, void* stream) {
  Plan pl;
  const int st = prepare(p, DWC_OP_BWD_DATA, &pl, dy, w, dx, nullptr, 0);
  if (st != DWC_OK || pl.empty) return st;
  const hipError_t e = launch_fwd_type(pl, dy, w, (float*)dx, (hipStream_t)stream);
  return e == hipSuccess ? DWC_OK : hip_fail(e, "dwc_bwd_data launch");
}

int dwc_bwd_filter(const dwc_problem* p, const void* x, const void* dy, void* dw,
                   void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  const int st = prepare(p, DWC_OP_BWD_FILTER, &pl, x, dy, dw, workspace, workspace_bytes);
  if (st != DWC_OK) return st;
  return run_bwd_filter(p, pl, x, dy, dw, workspace, (hipStream_t)stream);
}

int dwc_bwd_filter_noalloc(const dwc_problem* p, const void* x, const void* dy, void* dw,
                           void* stream) {
  if (!p) {
    set_last_error("problem pointer is NULL");
    return DWC_ERR_BAD_PARAM;
  }
  void* ws = nullptr;
  int st = scratch_of_current_device(&ws);
  if (st != DWC_OK) return st;
  // The automatic split is kept when its partial sums fit the scratch (the
  // same kernels and summation order as dwc_bwd_filter); otherwise the
  // largest split whose partials fit is taken (the planners' workspace grows
  // with the requested split), then, under AUTO, the vector kernels, whose
  // single slice needs no workspace.  A split the caller asked for is kept
  // or rejected.
  dwc_problem d = *p;
  Plan pl;
  st = prepare(&d, DWC_OP_BWD_FILTER, &pl, x, dy, dw, ws, kScratchBytes);
  const size_t first_need = pl.ws_bytes;
  if (st == DWC_ERR_WORKSPACE && p->wgrad_split == 0) {
    for (int32_t algo : {p->algo, (int32_t)DWC_ALGO_VECTOR, (int32_t)DWC_ALGO_GENERIC}) {
      if (algo != p->algo && p->algo != DWC_ALGO_AUTO) break;
      d = *p;
      d.algo = algo;
      int64_t lo = 1, hi = std::max<int64_t>(1, std::min<int64_t>(p->n * p->h, 0x7fffffff));
      d.wgrad_split = 1;
      st = prepare(&d, DWC_OP_BWD_FILTER, &pl, x, dy, dw, ws, kScratchBytes);
      if (st != DWC_OK) continue;
      while (lo < hi) {  // largest split that still fits
        const int64_t mid = lo + (hi - lo + 1) / 2;
        dwc_problem t = d;
        t.wgrad_split = (int32_t)mid;
        Plan q;
        std::string err;
        if (make_plan(&t, DWC_OP_BWD_FILTER, &q, &err) == DWC_OK && q.ws_bytes <= kScratchBytes)
          lo = mid;
        else
          hi = mid - 1;
      }
      d.wgrad_split = (int32_t)lo;
      st = prepare(&d, DWC_OP_BWD_FILTER, &pl, x, dy, dw, ws, kScratchBytes);
      if (st == DWC_OK) break;
    }
  }
  if (st == DWC_ERR_WORKSPACE) {
    set_last_error("the filter gradient needs " + std::to_string(first_need) +
                   " bytes of partial sums; dwc_bwd_filter_noalloc's fixed scratch holds " +
                   std::to_string(kScratchBytes) +
                   " bytes (use dwc_bwd_filter with a caller-owned workspace)");
    return st;
  }
  if (st != DWC_OK) return st;
  return run_bwd_filter(&d, pl, x, dy, dw, ws, (hipStream_t)stream);
}

}  // extern "C"
