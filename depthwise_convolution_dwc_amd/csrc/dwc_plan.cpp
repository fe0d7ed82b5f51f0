// dwc_plan.cpp -- validation, kernel choice and grid sizes of libdwc.
// Host-only: nothing here touches the GPU, so every error path can be
// exercised on a machine without one.
#include "dwc_plan.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>

namespace dwc {

namespace {

thread_local std::string g_last_error;
int (*g_cus_hook)() = nullptr;

constexpr int64_t kI32Max = 0x7fffffff;

int elem_bytes(int dt) { return dt == DT_F32 ? 4 : dt == DT_BF16 || dt == DT_F16 ? 2 : 1; }

bool sweep_f(int f) {
#define DWC_IS(F) if (f == F) return true;
  DWC_SWEEP_F_LIST(DWC_IS)
#undef DWC_IS
  return false;
}

bool direct_fw(int fw) {
#define DWC_IS(F) if (fw == F) return true;
  DWC_DIRECT_FW_LIST(DWC_IS)
#undef DWC_IS
  return false;
}

// The instantiated direct width a filter fw wide runs on: the narrowest
// listed width >= fw (0: wider than every instantiation).
int direct_kfw(int fw) {
#define DWC_IS(F) if (fw >= 1 && fw <= F) return F;
  DWC_DIRECT_FW_LIST(DWC_IS)
#undef DWC_IS
  return 0;
}

const char* dt_name(int dt) {
  static const char* const names[] = {"f32", "bf16", "f16", "e4m3", "e5m2"};
  return names[dt];
}

int fail(std::string* err, int code, const std::string& msg) {
  if (err) *err = msg;
  return code;
}

// Strip width (output columns per lane) of a forward-type launch or of a
// filter-gradient unit: the instantiated width with the fewest idle columns
// in the last strip, ties to the wider strip.
int pick_strip(int64_t ow) {
  const int cand[] = {14, 7};
  int best = cand[0];
  int64_t best_waste = -1;
  for (int c : cand) {
    const int64_t waste = (ow + c - 1) / c * c - ow;
    if (best_waste < 0 || waste < best_waste) {
      best = c;
      best_waste = waste;
    }
  }
  return best;
}

// Strip-width override for A/B timing: DWC_FWD_STRIP / DWC_WGRAD_STRIP set
// to an instantiated width (7 or 14) replace the automatic choice.
int strip_override(const char* var, int fallback) {
  const char* v = getenv(var);
  if (!v) return fallback;
  const int w = atoi(v);
  return (w == 7 || w == 14) ? w : fallback;
}

// Chunks per image for a sweep launch: enough waves (~2048, two per SIMD)
// to fill the GPU, with chunks of at least F rows (each chunk re-reads F-1
// halo rows).  A launch that would still hold less than one wave per CU
// takes chunks down to one row: its time is one wave's dependent chain, not
// the halo traffic (N=1 14x14 C=32 7x7: 10.1 -> 5.2 us with 14 one-row
// chunks instead of 2 of 7 rows; with full batches shorter chunks than F
// rows were slower).
int64_t sweep_chunks(int64_t waves_per_chunk, int64_t out_h, int f) {
  const int64_t w = std::max<int64_t>(waves_per_chunk, 1);
  int64_t target = 8 * (int64_t)device_cus();  // two waves per SIMD
  if (const char* v = getenv("DWC_SWEEP_WAVES")) target = std::max(1, atoi(v));
  const int64_t cpi = std::max<int64_t>(1, (target + w - 1) / w);
  const int64_t whole = std::max<int64_t>(1, out_h / f);  // chunks of at least F rows
  if (w * whole < (int64_t)device_cus()) return std::min<int64_t>(cpi, std::max<int64_t>(1, out_h));
  return std::min<int64_t>(cpi, whole);
}

// Number of slices of the N*OH axis for the filter gradient (§5.1 splits
// the accumulation axis into Z sub-problems whose sums are merged).  Z is
// the largest value that (a) does not overfill the GPU (~1024 workgroups),
// (b) leaves every workgroup at least one unit per wave, and (c) keeps the
// partial sums it writes and reads back under ~15% of the kernel's own
// estimated time.
int pick_split(int64_t rows, int64_t per_slice_blocks, int64_t strips, int64_t m, double flops,
               double bytes) {
  const int64_t target = 4 * (int64_t)device_cus();  // ~4 workgroups per CU
  const int64_t fill = (target + per_slice_blocks - 1) / per_slice_blocks;
  const int64_t groups_per_wave_set = (4 + strips - 1) / strips;  // row groups for 4 units
  const int64_t by_units = std::max<int64_t>(1, rows / (kWgradRows * groups_per_wave_set));
  const double t_est = std::max(flops / 100e12, bytes / 5e12);
  const double cap = 0.15 * t_est * 5e12 / (8.0 * (double)m);
  int64_t z = std::min<int64_t>({fill, by_units, (int64_t)std::max(1.0, std::floor(cap))});
  z = std::max<int64_t>(1, std::min(z, rows));
  return (int)std::min<int64_t>(z, 65535);
}

// Packed-MFMA plan of a forward-type problem (the forward map, or the
// stride-1 data gradient as the forward map of dY): false if the kernel does
// not apply.  Tiles of 16 (row, 16-column group) combinations: gt groups x
// 16/gt rows; 1, 2 or 4 tiles per channel and workgroup -- as many as the
// image height asks for (each B operand is read once per tile set) while
// the staged input rows, the zero-padded filter-row fragments and
// (afterwards) the staged outputs fit the workgroup's LDS.  The input tile
// holds the real image rows a workgroup reads between two zero rows; its row
// pitch gets 8 extra elements (an odd number of 16-byte units per row)
// where LDS allows, so that lanes reading consecutive rows hit distinct
// banks.  16 channels per workgroup (two per wave) with one 16-tap
// fragment, 8 (one per wave) with two.
bool plan_mfma(const FwdArgs& f, int dt, bool flip, Plan* q) {
  constexpr int kZRowElems = 32;  // one 16-tap fragment and its 16 leading zeros
  if ((dt != DT_BF16 && dt != DT_F16) || f.SH != 1 || f.SW != 1 || f.FW > 32 || f.C % 8 != 0)
    return false;
  const int groups = (f.OW + 15) / 16;
  const int gt = groups <= 1 ? 1 : groups <= 2 ? 2 : groups <= 4 ? 4 : 0;
  if (gt == 0) return false;
  const int rt = 16 / gt;
  const int nf = (f.FW + 15) / 16;
  const int cb = nf == 1 ? 16 : 8;
  const int need = (f.OH + rt - 1) / rt;
  MfmaArgs m{};
  m.N = f.N; m.IH = f.IH; m.IW = f.IW; m.C = f.C; m.OH = f.OH; m.OW = f.OW;
  m.FH = f.FH; m.FW = f.FW; m.PH = f.PH; m.PW = f.PW;
  m.gt = gt;
  m.rt_log = gt == 1 ? 4 : gt == 2 ? 3 : 2;
  m.wt = 16 * (gt + nf);
  int tiles = need <= 1 ? 1 : need <= 2 ? 2 : 4;
  // DWC_MFMA_TILES (1, 2 or 4) caps the tiles per workgroup, for A/B timing
  if (const char* v = getenv("DWC_MFMA_TILES")) {
    const int t = atoi(v);
    if (t == 1 || t == 2 || t == 4) tiles = std::min(tiles, t);
  }
  const int64_t z_bytes = ((int64_t)cb * f.FH * nf + 2) * kZRowElems * 2;
  int64_t lds = 0;
  for (;; tiles /= 2) {
    m.rblk = tiles * rt;
    m.xr = std::min(f.IH, m.rblk + f.FH - 1) + 2;  // real rows between two zero rows
    const int64_t out_bytes = (int64_t)m.rblk * f.OW * (cb + 4) * 4;
    bool fit = false;
    for (int pad : {8, 0}) {
      m.wp = m.wt + pad;
      lds = std::max((int64_t)cb * m.xr * m.wp * 2 + z_bytes, out_bytes);
      if (lds <= kMfmaMaxLds) {
        fit = true;
        break;
      }
    }
    if (fit) break;
    if (tiles == 1) return false;
  }
  m.lds_bytes = (int)lds;
  m.e_items = (m.wt / 2) * (cb / 8);
  m.e2 = 1;
  m.e2_log = 0;
  while (m.e2 < m.e_items) {
    m.e2 *= 2;
    ++m.e2_log;
  }
  if (m.e2 > 64 * kMfmaWaves) return false;
  m.rch = (f.OH + m.rblk - 1) / m.rblk;
  m.cblk = (f.C + cb - 1) / cb;
  const int64_t blocks = (int64_t)f.N * m.cblk * m.rch;
  if (blocks > kI32Max) return false;
  m.num_blocks = (int)blocks;
  // the kernels split filter taps into (row, column) with fast_div
  if ((int64_t)f.FH * f.FW >= 65536) return false;
  m.fw_magic = div_magic((uint32_t)f.FW);
  q->kind = PLAN_MFMA;
  q->flip = flip;
  q->nf = nf;
  q->cb = cb;
  q->tiles = tiles;
  q->blocks = (int)blocks;
  q->ma = m;
  q->fa = f;
  return true;
}

// The 16-image form of the batch-packed plan (fwd_mfma_batch16): bf16 /
// fp16 or fp8 operands, C % 16 == 0 (16 channels of a pixel: two 16-byte
// loads, or one for fp8), a batch of at least 8 images,
// the band and four row slots within one CU's LDS.  As many output rows as
// the LDS holds are staged per round.
static bool plan_mfma_batch16(const FwdArgs& f, int dt, Plan* q) {
  if (f.C % kB16Cb != 0 || f.N < 8) return false;
  const bool b8 = dt == DT_E4M3 || dt == DT_E5M2;
  const int eb = b8 ? 1 : 2;
  if ((int64_t)kB16Img * f.IH * f.IW * f.C * eb > kI32Max ||
      (int64_t)kB16Img * f.OH * f.OW * f.C > kI32Max)
    return false;
  MfmaBatchArgs m{};
  m.N = f.N; m.IH = f.IH; m.IW = f.IW; m.C = f.C; m.OH = f.OH; m.OW = f.OW;
  m.FH = f.FH; m.FW = f.FW; m.PH = f.PH; m.PW = f.PW;
  m.cb = kB16Cb;
  m.rch = (f.OH + kB16Rows - 1) / kB16Rows;
  m.cblk = f.C / m.cb;
  m.ng = (f.N + kB16Img - 1) / kB16Img;
  m.nq = kB16Rows + f.FH - 1;
  const int64_t band = (int64_t)kB16Cb * (f.FH + 1) * 64 * eb;
  const int64_t ring = (int64_t)kB16Slots * kB16Cb * (b8 ? kB16ChPitch8 : kB16ChPitch);
  const int64_t orow = (int64_t)kB16Img * (f.OW * kB16Opitch + 4) * 4;  // one output row
  if (band + ring > kLdsPerCu || orow > kLdsPerCu) return false;
  // one workgroup per CU (registers), so the output staging may take the
  // whole LDS: as many rows per round as fit
  m.orows = (int)std::min<int64_t>(kB16Rows, kLdsPerCu / orow);
  const int64_t lds = std::max(band + ring, m.orows * orow);
  m.lds_bytes = (int)lds;
  m.ow_magic = div_magic((uint32_t)f.OW);
  const int64_t blocks = (int64_t)m.cblk * m.rch * m.ng;
  if (blocks > kI32Max) return false;
  m.num_blocks = (int)blocks;
  m.fw_magic = div_magic((uint32_t)f.FW);
  q->bimg = kB16Img;
  q->bng = f.OW > 16 ? 2 : 1;
  q->blocks = (int)blocks;
  q->mb = m;
  return true;
}

// Packed-MFMA plan with the batch in the matrix rows (bf16 / fp16, stride
// 1): false if the kernel does not apply.  Input and output widths up to 32
// (one 32-column output tile, two 16-column input chunks), 0 <= PW <= 31
// and FW <= 32 (the band rows' zeros).  The 16-image kernel where it
// applies (DWC_MFMA_BATCH_IMG=32 picks the 32-image one), else the 32-image
// kernel: C % 8 == 0 (16-byte channel octets) and a batch of at least 16
// images (the matrix rows are images: smaller batches leave most of each
// instruction idle).
bool plan_mfma_batch(const FwdArgs& f, int dt, bool flip, Plan* q) {
  const bool b8 = dt == DT_E4M3 || dt == DT_E5M2;
  if ((dt != DT_BF16 && dt != DT_F16 && !b8) || f.SH != 1 || f.SW != 1 ||
      f.IW > kBatchMaxCols || f.OW > kBatchMaxCols || f.PW < 0 || f.PW > 31 || f.FW > 32 ||
      f.PH < 0 || f.FH > 64)
    return false;
  // DWC_MFMA_BATCH: 0 never, 1 wherever it applies (for tests and A/B
  // timing); unset: from kBatchMinFh (fp8: kBatchMinFh8) filter rows on,
  // and for 16-bit operands from kBatchMinFhRound rows where the 16-image
  // kernel's workgroups make one round of at least 3/4 of the CUs
  const char* env = getenv("DWC_MFMA_BATCH");
  if (env && atoi(env) == 0) return false;
  const int min_fh = b8 ? kBatchMinFh8 : f.OW <= kBatchNarrowOw ? kBatchMinFhNarrow : kBatchMinFh;
  const bool by_height = env || f.FH >= min_fh;
  if (!by_height && (b8 || f.FH < kBatchMinFhRound)) return false;
  Plan t = *q;  // q changes only when a kernel applies
  t.kind = PLAN_MFMA;
  t.batch = true;
  t.flip = flip;
  t.fa = f;
  const char* img = getenv("DWC_MFMA_BATCH_IMG");
  if ((b8 || !(img && atoi(img) == kBatchImg)) && plan_mfma_batch16(f, dt, &t)) {
    const int64_t cus = device_cus();
    if (!by_height && !(4 * (int64_t)t.blocks >= 3 * cus && t.blocks <= cus)) return false;
    *q = t;
    return true;
  }
  if (!by_height) return false;
  // the 32-image kernel takes bf16 / fp16 operands only
  if (b8 || f.C % kBatchCb != 0 || f.N < 16) return false;
  // 32-bit offsets into one image group's input and output
  if ((int64_t)kBatchImg * f.IH * f.IW * f.C * 2 > kI32Max ||
      (int64_t)kBatchImg * f.OH * f.OW * f.C > kI32Max)
    return false;
  MfmaBatchArgs m{};
  m.N = f.N; m.IH = f.IH; m.IW = f.IW; m.C = f.C; m.OH = f.OH; m.OW = f.OW;
  m.FH = f.FH; m.FW = f.FW; m.PH = f.PH; m.PW = f.PW;
  m.cb = kBatchCb;
  m.rch = (f.OH + kBatchRows - 1) / kBatchRows;
  m.cblk = f.C / m.cb;
  m.ng = (f.N + kBatchImg - 1) / kBatchImg;
  m.nq = kBatchRows + f.FH - 1;
  const int64_t band = (int64_t)m.cb * (f.FH + 1) * 64 * 2;
  const int64_t ring = (int64_t)kBatchSlots * m.cb * 4 * kBatchHalfPitch;
  const int64_t outs = (int64_t)kBatchImg * f.OW * 12 * 4;  // one output row's staging
  const int64_t lds = std::max(band + ring, outs);
  if (lds > kLdsPerCu) return false;
  m.lds_bytes = (int)lds;
  m.two_rows = 2 * outs <= lds ? 1 : 0;
  m.ow_magic = div_magic((uint32_t)f.OW);
  const int64_t blocks = (int64_t)m.cblk * m.rch * m.ng;
  if (blocks > kI32Max) return false;
  m.num_blocks = (int)blocks;
  m.fw_magic = div_magic((uint32_t)f.FW);
  t.bimg = kBatchImg;
  t.blocks = (int)blocks;
  t.mb = m;
  *q = t;
  return true;
}

// Issued 4x4x1 instructions per filter row of one row group for T-tile
// waves (the column groups of plan_mfma_f32, the first and last skipping
// their padding columns when `same`).
static int64_t f32m_cost(int ow, int fwi, int t, bool same) {
  const int na = 4 * t + fwi - 1, pwc = (fwi - 1) / 2;
  const int cg = ow >= 4 * t ? (ow + 4 * t - 1) / (4 * t) : 1;
  int64_t n = 0;
  for (int g = 0; g < cg; ++g) {
    const int ow0 = ow >= 4 * t ? std::min(g * 4 * t, ow - 4 * t) : 0;
    const int l = same && ow0 == 0 ? pwc : 0;
    const int r = same && ow0 + 4 * t == ow ? pwc : 0;
    for (int m = 0; m < t; ++m)
      for (int k = 0; k < fwi + 3; ++k) n += (4 * m + k >= l && 4 * m + k < na - r) ? 1 : 0;
  }
  return n;
}

// 16-bit plan on the 4x4x4 matrix instructions (fwd_mfma_h4n): false if the
// kernel does not apply.  bf16/fp16 operands, stride 1, C % 16 == 0,
// FW <= 17, the band of every filter row and the waves' row buffers in one
// CU's LDS, 32-bit offsets within the batch.  DWC_MFMA_H4: 0 never, 1
// wherever it applies.  AUTO takes it for filters of kH4mMinF to kH4mMaxF
// rows and columns on outputs at most kH4mMaxOw wide while its waves fill
// the GPU (MI355X, bf16, N=64: width 14 C=512 9x9 / 13x13 19 / 24 us
// against 28 / 32 us; width 7 C=1024 14 / 17 us against 42 / 48 us; at
// widths 28 and 56, at 17x17 and with fewer waves the other kernels are
// as fast or faster: the 13x13 N=128 28x28 C=512 forward 143 against
// 113 us).  T: 7 tiles per wave where the output is at least 28 wide, else
// 4.
static bool plan_mfma_h4(const FwdArgs& f, int dt, bool flip, Plan* q) {
  if ((dt != DT_BF16 && dt != DT_F16) || f.SH != 1 || f.SW != 1 || f.C % kH4mCb != 0 ||
      f.FW < 1 || f.FW > 17 || f.FH < 1)
    return false;
  const int64_t waves = (int64_t)((f.N + 3) / 4) * ((f.OH + kH4mRows - 1) / kH4mRows) *
                        ((f.OW + 15) / 16) * (f.C / kH4mCb);
  const bool pick = f.FH >= kH4mMinF && f.FH <= kH4mMaxF && f.FW >= kH4mMinF &&
                    f.FW <= kH4mMaxF && f.OW <= kH4mMaxOw && waves >= kH4mFillWaves;
  const char* env = getenv("DWC_MFMA_H4");
  if (env ? atoi(env) == 0 : !pick) return false;
  if ((int64_t)f.N * f.IH * f.IW * f.C * 2 >= kI32Max || (int64_t)f.OH * f.OW * f.C * 4 >= kI32Max)
    return false;
  const int fwi = h4m_fwi(f.FW);
  const int S = (fwi + 6) / 4;
  const int64_t lds = (int64_t)f.FH * S * 64 * 8;  // one channel block's band
  const bool same = f.PW == (fwi - 1) / 2 && f.FW == fwi && f.IW == f.OW;
  int t = f.OW >= 28 ? 7 : 4;
  if (const char* v = getenv("DWC_MFMA_H4_T")) {
    const int tv = atoi(v);
    if (tv == 4 || tv == 7) t = tv;
  }
  MfmaF32Args m{};
  m.N = f.N; m.IH = f.IH; m.IW = f.IW; m.C = f.C; m.OH = f.OH; m.OW = f.OW;
  m.FH = f.FH; m.FW = f.FW; m.PH = f.PH; m.PW = f.PW;
  // a wave: 4 images x kH4mRows rows x 4t columns x kH4mCb channels; the
  // workgroup's waves share the band of their channel block
  m.cblk = f.C / kH4mCb;
  m.rg = (f.OH + kH4mRows - 1) / kH4mRows;
  m.cg = f.OW >= 4 * t ? (f.OW + 4 * t - 1) / (4 * t) : 1;
  const int64_t tiles = (int64_t)((f.N + 3) / 4) * m.rg * m.cg;
  if (tiles > kI32Max) return false;
  m.tiles = (int)tiles;
  m.nw = (int)std::min<int64_t>(kH4mMaxWaves, tiles);
  m.same = same ? 1 : 0;
  m.groups = (int)((tiles + m.nw - 1) / m.nw);
  // the band, then each wave's row buffer (4 images x NAP columns x 32 bytes)
  const int na = 4 * (t + S - 1), nap = na + ((2 - na % 8) + 8) % 8;
  const int64_t lds_all = lds + (int64_t)m.nw * 4 * nap * 32;
  if (lds_all > kLdsPerCu) return false;
  m.lds_bytes = (int)lds_all;
  const int64_t blocks = (int64_t)m.cblk * m.groups;
  if (blocks > kI32Max) return false;
  m.num_blocks = (int)blocks;
  q->kind = PLAN_MFMA;
  q->h4m = true;
  q->h4m_fwi = fwi;
  q->h4m_t = t;
  q->flip = flip;
  q->blocks = (int)blocks;
  q->mf = m;
  q->fa = f;
  return true;
}

// fp32 matrix-core plan (fwd_mfma_f32, fwd_mfma_f32n): false if the kernels
// do not apply.  fp32 operands, stride 1, C % 16 == 0, FW <= 31, FH <= 64
// (the band of every filter row in LDS), 32-bit offsets within one image
// (within the batch for the images kernel).  DWC_MFMA_F32: 0 never, 1
// wherever it applies.
static bool plan_mfma_f32(const FwdArgs& f, int dt, bool flip, bool forced, Plan* q) {
  // 16-bit operands (widened as they are loaded, rows kernel only) come here
  // only where no packed 16-bit kernel applies (outputs wider than 64, or
  // bands past their LDS budget)
  if ((dt != DT_F32 && dt != DT_BF16 && dt != DT_F16) || f.SH != 1 || f.SW != 1 ||
      f.C % kF32mCb != 0 || f.FW < 1 || f.FW > 31 || f.FH < 1 || f.FH > 64)
    return false;
  if ((int64_t)f.IH * f.IW * f.C * 4 >= kI32Max || (int64_t)f.OH * f.OW * f.C * 4 >= kI32Max)
    return false;
  const int fwi = f32m_fwi(f.FW);
  const bool same = f.PW == (fwi - 1) / 2 && f.FW == fwi && f.IW == f.OW;
  const int rg = (f.OH + kF32mRows - 1) / kF32mRows;
  auto groups = [&](int t) { return f.OW >= 4 * t ? (f.OW + 4 * t - 1) / (4 * t) : 1; };
  // Images as the matrix rows (fwd_mfma_f32n: no row moves between lanes,
  // each input row loaded as the wave reaches it): 4 tiles per wave above
  // width 8, else 2.  It wins on outputs at most 16 wide with large filters
  // while it has 8 waves per CU (MI355X, N=64 C=512 14x14: 63-78 against
  // 66-97 us from 21x21 on; width 7: 27 and 39 against 37 and 42 us at
  // 27x27 and 31x31), and loses at widths 28 and 56 (1.2-1.35x: its loads'
  // latency is exposed per row) and with fewer waves.
  const int img_t = f.OW > 8 ? 4 : 2;
  const bool img_fill = f.N >= 4 && (int64_t)((f.N + 3) / 4) * rg * groups(img_t) * (f.C / kF32mCb) >=
                                        kF32mFillWaves;
  const bool img_auto = f.OW <= 16 && img_fill && f.FW >= (f.OW > 8 ? 21 : 27);
  // AUTO, from kF32mMinFh filter rows and columns:
  // - outputs at least kF32mMinOw wide (MI355X, N=64 stages: 1.0-1.5x the
  //   vector kernels from 13x13 on at widths 56 and 28);
  // - the largest filters on the narrowest outputs (width 7: 1.07x at 27x27,
  //   1.18x at 31x31), and the images kernel's cases above;
  // - outputs at most 16 wide whose vector kernel (a wave per 64 channels,
  //   4 rows, the whole width) has fewer than 8 waves per CU: 3-4x faster
  //   (N=8 14x14 C=512 31x31: 21 against 79 us; N=16 C=256 21x21: 17
  //   against 50 us).
  // - filters of 10 to 12 columns (and at least 10 rows) at any width: the
  //   vector kernels run them on their 13-wide body (11x11: 1.0-1.3x at
  //   widths 56, 28, 14 and 7).
  const bool vec_few = f.OW <= 16 && (int64_t)f.N * ((f.C + 63) / 64) * rg < kF32mFillWaves;
  const bool pick = (f.FH >= kF32mMinFh && f.FW >= kF32mMinFh &&
                     (f.OW >= kF32mMinOw || (f.OW <= 8 && f.FW >= 27) || img_auto || vec_few)) ||
                    (f.FH >= kF32mMinFPad && f.FW >= kF32mMinFPad && f.FW < kF32mMinFh);
  // 16-bit operands: on request only.  The widened rows kernel needs 130
  // registers (3 waves per SIMD) and loses to the 16-bit vector kernels as
  // often as it wins (MI355X, bf16 N=32 112x112 C=64: 175 against 131 us
  // at 13x13, 400 against 450 us at 27x27; N=64 56x56 C=128 31x31: 538
  // against 578 us).
  const char* env = getenv("DWC_MFMA_F32");
  if (!forced && (env ? atoi(env) == 0 : (!pick || dt != DT_F32))) return false;
  // the images kernel addresses 4 images of X from one buffer resource
  const bool img_ok = dt == DT_F32 && f.N >= 4 && (int64_t)f.N * f.IH * f.IW * f.C * 4 < kI32Max;
  // DWC_MFMA_F32_IMG: 0 never, 1 for every batch of 4 or more
  const char* iv = getenv("DWC_MFMA_F32_IMG");
  const bool img = img_ok && (iv ? atoi(iv) != 0 : img_auto);
  // The rows kernel's tile width T (4-column tiles per wave) issues the
  // fewest instructions over the output width; ties go to the wider tile.
  int best_t = 0;
  int64_t best = 0;
  for (int t : {7, 4, 2}) {
    const int64_t c = f32m_cost(f.OW, fwi, t, same);
    if (best_t == 0 || c < best) {
      best = c;
      best_t = t;
    }
  }
  if (img) best_t = img_t;
  if (const char* v = getenv("DWC_MFMA_F32_T")) {
    const int t = atoi(v);
    if ((t == 7 && !img) || t == 4 || t == 2) best_t = t;
  }
  const int t = best_t;
  MfmaF32Args m{};
  m.N = f.N; m.IH = f.IH; m.IW = f.IW; m.C = f.C; m.OH = f.OH; m.OW = f.OW;
  m.FH = f.FH; m.FW = f.FW; m.PH = f.PH; m.PW = f.PW;
  m.cblk = f.C / kF32mCb;
  m.rg = rg;
  m.cg = groups(t);
  const int64_t tiles = (int64_t)(img ? (f.N + 3) / 4 : f.N) * m.rg * m.cg;
  if (tiles > kI32Max) return false;
  m.tiles = (int)tiles;
  m.nw = (int)std::min<int64_t>(kF32mMaxWaves, tiles);
  m.same = same ? 1 : 0;
  m.groups = (int)((tiles + m.nw - 1) / m.nw);
  const int64_t lds = (int64_t)f.FH * (fwi + 6) * kF32mCb * 4;
  if (lds > kLdsPerCu) return false;
  m.lds_bytes = (int)lds;
  const int64_t blocks = (int64_t)m.cblk * m.groups;
  if (blocks > kI32Max) return false;
  m.num_blocks = (int)blocks;
  m.fw_magic = div_magic((uint32_t)f.FW);
  q->kind = PLAN_MFMA;
  q->f32m = true;
  q->f32m_fwi = fwi;
  q->f32m_t = t;
  q->f32m_img = img;
  q->flip = flip;
  q->blocks = (int)blocks;
  q->mf = m;
  q->fa = f;
  return true;
}

// Packed fp8 MFMA plan of a forward-type problem (e4m3 / e5m2 operands):
// false if the kernel does not apply.  The tiling of plan_mfma, in bytes:
// kMfma8Cb channels per workgroup, each 16x16x128 MFMA covering four filter
// rows (the fragment rows are padded to a multiple of four), the staged
// input row pitch an odd number of 16-byte units where LDS allows.
bool plan_mfma8(const FwdArgs& f, int dt, bool flip, Plan* q) {
  if ((dt != DT_E4M3 && dt != DT_E5M2) || f.SH != 1 || f.SW != 1 || f.FW > 32 ||
      f.C % kMfma8Cb != 0)
    return false;
  const int groups = (f.OW + 15) / 16;
  const int gt = groups <= 1 ? 1 : groups <= 2 ? 2 : groups <= 4 ? 4 : 0;
  if (gt == 0) return false;
  const int rt = 16 / gt;
  const int nf = (f.FW + 15) / 16;
  const int cb = kMfma8Cb;
  const int fhp = 4 * ((f.FH + 3) / 4);
  const int need = (f.OH + rt - 1) / rt;
  MfmaArgs m{};
  m.N = f.N; m.IH = f.IH; m.IW = f.IW; m.C = f.C; m.OH = f.OH; m.OW = f.OW;
  m.FH = f.FH; m.FW = f.FW; m.PH = f.PH; m.PW = f.PW;
  m.gt = gt;
  m.rt_log = gt == 1 ? 4 : gt == 2 ? 3 : 2;
  m.wt = 16 * (gt + nf);
  int tiles = need <= 1 ? 1 : need <= 2 ? 2 : 4;
  if (const char* v = getenv("DWC_MFMA_TILES")) {
    const int t = atoi(v);
    if (t == 1 || t == 2 || t == 4) tiles = std::min(tiles, t);
  }
  const int64_t z_bytes = ((int64_t)cb * fhp * nf + kZ8Tail) * kZ8Row;
  int64_t lds = 0;
  for (;; tiles /= 2) {
    m.rblk = tiles * rt;
    m.xr = std::min(f.IH, m.rblk + f.FH - 1) + 2;  // real rows between two zero rows
    const int64_t out_bytes = (int64_t)m.rblk * f.OW * (cb + 4) * 4;
    bool fit = false;
    for (int pad : {(m.wt / 16) % 2 == 0 ? 16 : 0, 0}) {
      m.wp = m.wt + pad;
      lds = std::max((int64_t)cb * m.xr * m.wp + z_bytes, out_bytes);
      if (lds <= kMfmaMaxLds) {
        fit = true;
        break;
      }
    }
    if (fit) break;
    if (tiles == 1) return false;
  }
  m.lds_bytes = (int)lds;
  m.e_items = m.wt / 4;  // column quads of one staged row
  m.e2 = 1;
  m.e2_log = 0;
  while (m.e2 < m.e_items) {
    m.e2 *= 2;
    ++m.e2_log;
  }
  if (m.e2 > 64 * kMfmaWaves) return false;
  m.rch = (f.OH + m.rblk - 1) / m.rblk;
  m.cblk = f.C / cb;
  const int64_t blocks = (int64_t)f.N * m.cblk * m.rch;
  if (blocks > kI32Max) return false;
  m.num_blocks = (int)blocks;
  // the kernels split filter taps into (row, column) with fast_div
  if ((int64_t)f.FH * f.FW >= 65536) return false;
  m.fw_magic = div_magic((uint32_t)f.FW);
  q->kind = PLAN_MFMA;
  q->flip = flip;
  q->nf = nf;
  q->cb = cb;
  q->tiles = tiles;
  q->blocks = (int)blocks;
  q->ma = m;
  q->fa = f;
  return true;
}

// Slices of whole images for the packed filter gradients (Z * cblk
// workgroups, `resident` of them at once).  A requested split is taken as
// it is.  Otherwise, where the slice partials are cheap (at most kWgmPartFrac
// of the operands' bytes with at least one round of workgroups), about
// kWgmFill rounds of workgroups: more, shorter slices measured faster than
// one round of long ones (MI355X, N=128 28x28 C=512: bf16 13x13 118 -> 98
// us at 43 slices instead of 12, e4m3 13x13 96 -> 80 us at 32 instead of
// 8, fp16 31x31 166 -> 158 us at 16 instead of 12).  Where they are not
// (a slice's partial outweighs the images it saves), the count whose
// dispatch rounds times images per slice (plus one image's worth of fixed
// cost per round) is least, preferring fewer slices (e4m3 31x31: 8).
static int64_t wgm_slices(const dwc_problem* p, int64_t nn, int64_t cblk, int64_t resident,
                          int64_t eb) {
  if (p->wgrad_split > 0) return std::min<int64_t>(p->wgrad_split, nn);
  const double part = (double)p->fh * p->fw * cblk * kWgmCb * 4;  // bytes per slice
  const double ops = (double)nn * ((double)p->h * p->w * 2) * p->c * eb;  // X and dY, about
  const int64_t cap = (int64_t)(kWgmPartFrac * ops / part);
  const int64_t floor_z = (resident + cblk - 1) / cblk;
  if (cap >= floor_z) {
    const int64_t target = (int64_t)(kWgmFill * (double)resident / (double)cblk + 0.999);
    const int64_t z = std::min(std::min(std::max(target, floor_z), cap), nn);
    const int64_t ipb = (nn + z - 1) / z;
    return (nn + ipb - 1) / ipb;
  }
  int64_t z = 1, best = -1;
  for (int64_t zc = 1; zc <= std::min<int64_t>(nn, 8 * resident); ++zc) {
    const int64_t ipb = (nn + zc - 1) / zc, zr = (nn + ipb - 1) / ipb;
    if (zr != zc) continue;  // same split as a smaller count
    const int64_t rounds = (zr * cblk + resident - 1) / resident;
    const int64_t cost = rounds * (ipb + 1);
    if (best < 0 || cost < best) {
      best = cost;
      z = zr;
    }
  }
  return z;
}

// Packed-MFMA filter-gradient plan: false if the kernel does not apply.
// kWgmCb channels per workgroup (one per wave); the batch is cut into Z
// slices of whole images so that Z * cblk workgroups (about 1024, or the
// requested split) fill the GPU; the staged X rows (plus a zero row), the
// zero-padded dY rows and (afterwards) the slice partial fit the LDS.
bool plan_wgrad_mfma(const dwc_problem* p, int64_t oh, int64_t ow, Plan* q) {
  const int dt = p->in_dtype;
  if ((dt != DT_BF16 && dt != DT_F16) || p->stride_h != 1 || p->stride_w != 1 || p->fw > 32 ||
      p->fh > 32 || p->w > 64 || p->c % kWgmCb != 0)
    return false;
  WgradMfmaArgs w{};
  w.N = (int)p->n; w.IH = (int)p->h; w.IW = (int)p->w; w.C = (int)p->c;
  w.OH = (int)oh; w.OW = (int)ow;
  w.FH = p->fh; w.FW = p->fw; w.PH = p->pad_h; w.PW = p->pad_w;
  const int nfm = (p->fw + 15) / 16, nfn = (p->fh + 15) / 16, nk = (int)((p->w + 31) / 32);
  w.cblk = w.C / kWgmCb;
  w.xr = w.IH + 1;
  w.xp = 32 * nk + 8;  // an odd number of 16-byte units per row
  // the A band of lane (q, m) starts at element 8q - 16 fm - m + pw + dpad
  // of a staged dY row and reads up to 10 elements from the even one below
  w.dpad = std::max(0, 16 * (nfm - 1) + 15 - w.PW);
  w.dyp = (32 * nk + w.PW + w.dpad + 2 + 7) / 8 * 8;
  // staging items: pixel pairs of the image (X) and the staged dY pairs
  // holding at least one real column
  w.hx = (w.IW + 1) / 2;
  w.ix = w.IH * w.hx;
  w.e_lo = w.dpad / 2;
  w.hd = (w.dpad + w.OW - 1) / 2 - w.e_lo + 1;
  w.id = w.OH * w.hd;
  const int items = std::max(w.ix, w.id);
  const int pf = (items + 64 * kMfmaWaves - 1) / (64 * kMfmaWaves);
  if (pf > kWgmMaxPf) return false;
  const int64_t stage = (int64_t)kWgmCb * (w.xr * w.xp + w.OH * w.dyp) * 2;
  const int64_t part = (int64_t)p->fh * p->fw * kWgmCb * 4;
  const int64_t lds = std::max(stage, part);
  if (lds > kMfmaMaxLds) return false;
  w.lds_bytes = (int)lds;
  // Slices of whole images (wgm_slices).  Workgroups resident at once: the
  // CUs times what one CU holds (LDS; registers: waves per SIMD / 2 for
  // 8-wave groups).
  const int64_t per_cu = std::max<int64_t>(
      1, std::min<int64_t>(kLdsPerCu / lds, wgm_waves_per_eu(nfm, nfn, nk, pf) / 2));
  const int64_t resident = (int64_t)device_cus() * per_cu;
  const int64_t nn = std::max<int64_t>(p->n, 1);  // an empty batch only zero-fills dW
  const int64_t z = wgm_slices(p, nn, w.cblk, resident, elem_bytes(dt));
  w.ipb = (int)((nn + z - 1) / z);
  w.Z = (int)((nn + w.ipb - 1) / w.ipb);
  const int64_t blocks = (int64_t)w.Z * w.cblk;
  if (blocks > kI32Max) return false;
  w.num_blocks = (int)blocks;
  q->kind = PLAN_MFMA;
  q->nfm = nfm;
  q->nfn = nfn;
  q->nk = nk;
  q->pf = pf;
  q->cb = kWgmCb;
  q->z = w.Z;
  q->blocks = w.num_blocks;
  q->wm = w;
  return true;
}


// fp32 matrix-core filter-gradient plan (wgrad_mfma_f32): false if the
// kernel does not apply.  fp32 operands, stride 1, FH and FW <= 32, C % 16
// == 0, 32-bit offsets within one image.  AUTO takes it from kWf32MinF
// filter rows and columns (DWC_MFMA_F32: 0 never, 1 wherever it applies).
// The output width is cut into column groups of 4 NB columns (the smallest
// NB that covers it, else 14); the (image, input row) pairs into Z slices
// so that the workgroups fill the GPU once (or the requested split).
static bool plan_wgrad_mfma_f32(const dwc_problem* p, int64_t oh, int64_t ow, bool forced,
                                Plan* q) {
  // 16-bit operands (widened as they are loaded) come here only where the
  // packed 16-bit filter gradient does not apply (inputs wider than 64, or
  // staged rows past its LDS budget)
  const int dt = p->in_dtype;
  if ((dt != DT_F32 && dt != DT_BF16 && dt != DT_F16) || p->stride_h != 1 ||
      p->stride_w != 1 || p->fw > 32 || p->fh > 32 || p->c % kWf32Cb != 0)
    return false;
  // AUTO: where the 4x4 tiles cover the filter with little waste (at least
  // 85% of the computed taps are real ones; 64% for filters at most 16
  // wide) and the filter has at least kWf32MinF rows and columns; on
  // outputs at most 8 wide only the largest filters (MI355X, N=64 stages:
  // 1.2-1.3x the vector kernels at 27x27 and 31x31 on 56, 28 and 14 wide
  // outputs, 0.7-0.9x at 17x17 and 21x21, whose tiles are 72-77% real taps;
  // 1.00-1.06x at 13x13 (66%); at width 7, 1.10x at 31x31, 0.91x at 27x27;
  // 11x11 (76%, on a 13-wide vector body): 1.2-1.6x at widths 56 to 7).
  const int64_t tiles = (int64_t)((p->fh + 3) / 4) * ((p->fw + 3) / 4);
  const int fill = p->fw <= 16 ? 64 : 85;
  const bool pick = p->fh >= kWf32MinF && p->fw >= kWf32MinF &&
                    (int64_t)p->fh * p->fw * 100 >= tiles * 16 * fill &&
                    (ow > 8 || p->fw >= 29 || p->fw <= 16);
  const char* env = getenv("DWC_MFMA_F32");
  if (!forced && (env ? atoi(env) == 0 : !pick)) return false;
  if (p->h * p->w * p->c * 4 >= kI32Max || oh * ow * p->c * 4 >= kI32Max) return false;
  WgradF32Args w{};
  w.N = (int)p->n; w.IH = (int)p->h; w.IW = (int)p->w; w.C = (int)p->c;
  w.OH = (int)oh; w.OW = (int)ow;
  w.FH = p->fh; w.FW = p->fw; w.PH = p->pad_h; w.PW = p->pad_w;
  const int tw = (p->fw + 3) / 4;
  int nb = 14;
  for (int c : {2, 4, 7, 14})
    if (4 * c >= ow) {
      nb = c;
      break;
    }
  w.cblk = w.C / kWf32Cb;
  w.cg = (int)((ow + 4 * nb - 1) / (4 * nb));
  const int xp = 4 * nb + 4 * tw;  // staged pixels per X row
  const int items = xp * (kWf32Cb / 4);
  w.nw = std::max((p->fh + 3) / 4, (items + 64 * kWf32StageItems - 1) / (64 * kWf32StageItems));
  if (w.nw > kWf32MaxWaves) return false;
  w.lds_bytes = 2 * xp * kWf32Cb * 4;
  const int64_t npairs = p->n * p->h;
  const int64_t nn = std::max<int64_t>(npairs, 1);  // an empty batch only zero-fills dW
  int64_t z;
  if (p->wgrad_split > 0) {
    z = std::min<int64_t>(p->wgrad_split, nn);
  } else {
    // one dispatch round: 16 waves per CU (four per SIMD, the registers of
    // the widest tiles)
    const int64_t resident = (int64_t)device_cus() * std::max(1, 16 / w.nw);
    z = std::max<int64_t>(1, std::min<int64_t>(nn, resident / ((int64_t)w.cblk * w.cg)));
  }
  const int64_t rps = (nn + z - 1) / z;
  w.rps = (int)rps;
  w.Z = (int)((nn + rps - 1) / rps);
  const int64_t blocks = (int64_t)w.cblk * w.cg * w.Z;
  if (blocks > kI32Max) return false;
  w.num_blocks = (int)blocks;
  q->kind = PLAN_MFMA;
  q->wf32 = true;
  q->wf32_tw = tw;
  q->wf32_nb = nb;
  q->cb = kWf32Cb;
  q->z = w.Z * w.cg;
  q->blocks = w.num_blocks;
  q->wf = w;
  return true;
}

// Packed fp8 MFMA filter-gradient plan (e4m3 / e5m2 operands): false if
// the kernel does not apply.  The slicing of plan_wgrad_mfma; staging in
// bytes, four columns of one channel per LDS dword: X rows at a pitch of an
// odd number of 16-byte units, dY rows zero-padded so that every lane's
// 36-byte band read stays in its row, and zero rows up to a multiple of
// four output rows (one MFMA sums four).
bool plan_wgrad_mfma8(const dwc_problem* p, int64_t oh, int64_t ow, Plan* q) {
  const int dt = p->in_dtype;
  if ((dt != DT_E4M3 && dt != DT_E5M2) || p->stride_h != 1 || p->stride_w != 1 || p->fw > 32 ||
      p->fh > 32 || p->w > 64 || p->c % kWgmCb != 0)
    return false;
  WgradMfmaArgs w{};
  w.N = (int)p->n; w.IH = (int)p->h; w.IW = (int)p->w; w.C = (int)p->c;
  w.OH = (int)oh; w.OW = (int)ow;
  w.FH = p->fh; w.FW = p->fw; w.PH = p->pad_h; w.PW = p->pad_w;
  const int nfm = (p->fw + 15) / 16, nfn = (p->fh + 15) / 16, nk = (int)((p->w + 31) / 32);
  w.cblk = w.C / kWgmCb;
  w.xr = w.IH + 1;
  w.xp = 32 * nk + 16;  // an odd number of 16-byte units per row
  // lane m's band starts at byte 32 kc - 16 fm - m + pw + dpad >= 0 of a
  // staged dY row
  w.dpad = std::max(0, 16 * (nfm - 1) + 15 - w.PW);
  // staging items: column quads of the image (X) and the staged dY quads
  // holding at least one real column
  w.hx = (w.IW + 3) / 4;
  w.ix = w.IH * w.hx;
  w.e_lo = w.dpad / 4;
  w.hd = (w.dpad + w.OW - 1) / 4 - w.e_lo + 1;
  w.id = w.OH * w.hd;
  w.dyp = (std::max(32 * nk + w.PW + w.dpad + 4, 4 * (w.e_lo + w.hd)) + 15) / 16 * 16;
  const int items = std::max(w.ix, w.id);
  const int pf = (items + 64 * kMfmaWaves - 1) / (64 * kMfmaWaves);
  if (pf > kWgmMaxPf) return false;
  const int ohp = (w.OH + 3) / 4 * 4;
  const int64_t stage = (int64_t)kWgmCb * ((int64_t)w.xr * w.xp + (int64_t)ohp * w.dyp);
  const int64_t part = (int64_t)p->fh * p->fw * kWgmCb * 4;
  const int64_t lds = std::max(stage, part);
  if (lds > kMfmaMaxLds) return false;
  w.lds_bytes = (int)lds;
  // slices of whole images, chosen as in plan_wgrad_mfma
  const int64_t per_cu =
      std::max<int64_t>(1, std::min<int64_t>(kLdsPerCu / lds, wgm8_waves_per_eu(pf) / 2));
  const int64_t resident = (int64_t)device_cus() * per_cu;
  const int64_t nn = std::max<int64_t>(p->n, 1);
  const int64_t z = wgm_slices(p, nn, w.cblk, resident, elem_bytes(dt));
  w.ipb = (int)((nn + z - 1) / z);
  w.Z = (int)((nn + w.ipb - 1) / w.ipb);
  const int64_t blocks = (int64_t)w.Z * w.cblk;
  if (blocks > kI32Max) return false;
  w.num_blocks = (int)blocks;
  q->kind = PLAN_MFMA;
  q->nfm = nfm;
  q->nfn = nfn;
  q->nk = nk;
  q->pf = pf;
  q->cb = kWgmCb;
  q->z = w.Z;
  q->blocks = w.num_blocks;
  q->wm = w;
  return true;
}

}  // namespace

void set_last_error(const std::string& msg) { g_last_error = msg; }

void set_device_cus_hook(int (*hook)()) { g_cus_hook = hook; }

int device_cus() {
  const int c = g_cus_hook ? g_cus_hook() : 0;
  return c > 0 ? c : kCus;
}

// Checks of the problem itself, shared by every entry point (not which
// kernel would run it); on success *oh_out, *ow_out are the output dims.
static int validate(const dwc_problem* p, int64_t* oh_out, int64_t* ow_out, std::string* err) {
  if (!p) return fail(err, DWC_ERR_BAD_PARAM, "problem pointer is NULL");
  if (p->n < 0 || p->h < 1 || p->w < 1 || p->c < 1)
    return fail(err, DWC_ERR_BAD_PARAM, "need n >= 0 and h, w, c >= 1");
  if (p->fh < 1 || p->fw < 1) return fail(err, DWC_ERR_BAD_PARAM, "need fh, fw >= 1");
  if (p->stride_h < 1 || p->stride_w < 1)
    return fail(err, DWC_ERR_BAD_PARAM, "need stride_h, stride_w >= 1");
  if (p->pad_h < 0 || p->pad_w < 0) return fail(err, DWC_ERR_BAD_PARAM, "need pad_h, pad_w >= 0");
  if (p->in_dtype < DWC_F32 || p->in_dtype > DWC_FP8_E5M2)
    return fail(err, DWC_ERR_BAD_PARAM,
                "in_dtype must be DWC_F32, DWC_BF16, DWC_F16, DWC_FP8_E4M3 or DWC_FP8_E5M2");
  if (p->out_dtype != DWC_F32)
    return fail(err, DWC_ERR_UNSUPPORTED, "outputs are fp32 only (out_dtype must be DWC_F32)");
  if (p->algo < DWC_ALGO_AUTO || p->algo > DWC_ALGO_HYBRID)
    return fail(err, DWC_ERR_BAD_PARAM, "unknown algo");
  if (p->wgrad_split < 0) return fail(err, DWC_ERR_BAD_PARAM, "wgrad_split must be >= 0");
  const int64_t a = p->h + 2 * (int64_t)p->pad_h - p->fh;
  const int64_t b = p->w + 2 * (int64_t)p->pad_w - p->fw;
  if (a < 0 || b < 0)
    return fail(err, DWC_ERR_BAD_PARAM, "filter larger than the padded input (OH or OW < 1)");
  const int64_t oh = a / p->stride_h + 1, ow = b / p->stride_w + 1;
  // 32-bit buffer offsets: one image of every tensor, and the filter, must
  // stay below 2 GiB; counts of rows and work items must fit in int32.
  if (p->h * p->w * p->c * 4 > kI32Max || oh * ow * p->c * 4 > kI32Max ||
      (int64_t)p->fh * p->fw * p->c * 4 > kI32Max || p->n * std::max(oh, p->h) > kI32Max ||
      p->c > kI32Max / 4)
    return fail(err, DWC_ERR_UNSUPPORTED, "tensor too large for 32-bit per-image offsets");
  *oh_out = oh;
  *ow_out = ow;
  return DWC_OK;
}

int make_plan(const dwc_problem* p, int op, Plan* pl, std::string* err) {
  if (op < DWC_OP_FWD || op > DWC_OP_BWD_FILTER)
    return fail(err, DWC_ERR_BAD_PARAM, "unknown operation code");
  int64_t oh = 0, ow = 0;
  const int vst = validate(p, &oh, &ow, err);
  if (vst != DWC_OK) return vst;

  const int dt = p->in_dtype;
  const int64_t eb = elem_bytes(dt);

  Plan q;
  q.op = op;
  q.dt = dt;
  q.oh = oh;
  q.ow = ow;
  q.empty = p->n == 0;
  const int C = (int)p->c;
  const int cblocks = (C + kWaveChannels - 1) / kWaveChannels;

  // Direct kernels: instantiated filter width, equal strides of 1 or 2 (the
  // data gradient: stride 1, where it is a forward map with the filter
  // turned by 180 degrees).
  const bool square_stride = p->stride_h == p->stride_w && p->stride_w <= 2;
  // Strided data gradient: the phase kernel, for equal strides >= 2 whose
  // sub-filters fit the largest instantiated size.
  int phase_km = 0;
  if (op == DWC_OP_BWD_DATA && p->stride_h == p->stride_w && p->stride_h >= 2) {
    const int need = (std::max(p->fh, p->fw) + p->stride_h - 1) / p->stride_h;
#define DWC_PICK(K) \
  if (phase_km == 0 && need <= K) phase_km = K;
    DWC_PHASE_KM_LIST(DWC_PICK)
#undef DWC_PICK
  }
  // Widths between the instantiated ones run on the next wider body (11 on
  // 13: 18% more FMAs, against a generic kernel ~50x slower).
  q.kfw = direct_kfw(p->fw);
  bool can_direct = q.kfw > 0 && square_stride;
  if (op == DWC_OP_BWD_DATA) can_direct = (can_direct && p->stride_w == 1) || phase_km > 0;
  if (p->algo == DWC_ALGO_DIRECT && !can_direct)
    return fail(err, DWC_ERR_UNSUPPORTED,
                "no direct kernel for this filter width / stride (use DWC_ALGO_AUTO)");
  const bool direct = p->algo != DWC_ALGO_GENERIC && can_direct;
  q.kind = direct ? PLAN_DIRECT : PLAN_GENERIC;
  // Sweep kernels: stride 1, square filter up to 9x9.
  const bool sweep_ok = p->stride_h == 1 && p->fh == p->fw && sweep_f(p->fw);
  // AUTO keeps the sweeps for the smallest filters with any operand type:
  // the packed matrix-core kernels lose there (MI355X, bf16 N=128 28x28
  // C=512 3x3 / 5x5 / 7x7: forward 64 / 68 / 93 against 96 / 97 / 98 us,
  // filter gradient 47 / 52 / 80 against 97 / 94 / 92 us; e4m3 N=64 7x7
  // C=1024 3x3 forward 12 against 47 us; from 9x9 on the matrix cores win)
  const bool sweep_auto = p->algo == DWC_ALGO_AUTO && sweep_ok && direct_fw(p->fw) &&
                          p->fw <= kSweepAutoMaxF && p->in_dtype != DT_F32;
  // ... and the vector kernels for the other filters up to 5x5 (bf16, N=64:
  // forward 1x1 26 against 35 us at 56x56 C=128, 3x5 11.0 against 18.5 us
  // at 14x14 C=512; filter gradient 3x5 23.6 against 27.5 us at 28x28
  // C=256; e4m3 forward 1x1 25 against 54 us at 56x56).  fp8 filter
  // gradients only up to 5 taps: from 3x5 on its packed kernel is ahead.
  const bool vec_auto =
      p->algo == DWC_ALGO_AUTO && p->in_dtype != DT_F32 && can_direct && !sweep_ok &&
      p->fh <= kVecAutoMaxF && p->fw <= kVecAutoMaxF &&
      (op != DWC_OP_BWD_FILTER || elem_bytes(p->in_dtype) == 2 || p->fh * p->fw <= 5);
  const bool vector_auto = sweep_auto || vec_auto;
  const bool hybrid = p->algo == DWC_ALGO_HYBRID;
  if (hybrid && (op != DWC_OP_BWD_FILTER || dt != DT_F16 || !sweep_ok))
    return fail(err, DWC_ERR_UNSUPPORTED,
                "hybrid accumulation is for the filter gradient of fp16 operands at stride 1 "
                "with a square 3x3, 5x5, 7x7 or 9x9 filter");

  if (op == DWC_OP_FWD || op == DWC_OP_BWD_DATA) {
    // The data gradient runs the forward map on dY with the filter turned
    // by 180 degrees and padding FH-1-pad (§5.1); its "input" is dY.
    const bool bwd = op == DWC_OP_BWD_DATA;
    FwdArgs f{};
    f.N = (int)p->n;
    f.C = C;
    f.FH = p->fh;
    f.FW = p->fw;
    f.IH = bwd ? (int)oh : (int)p->h;
    f.IW = bwd ? (int)ow : (int)p->w;
    f.OH = bwd ? (int)p->h : (int)oh;
    f.OW = bwd ? (int)p->w : (int)ow;
    f.SH = p->stride_h;
    f.SW = p->stride_w;
    f.PH = bwd ? p->fh - 1 - p->pad_h : p->pad_h;
    f.PW = bwd ? p->fw - 1 - p->pad_w : p->pad_w;
    // Packed MFMA for half-precision operands (the stride-1 data gradient
    // too: stride 1 is part of the kernel's conditions).
    if ((p->algo == DWC_ALGO_AUTO && !vector_auto) || p->algo == DWC_ALGO_MFMA) {
      if (plan_mfma_h4(f, dt, bwd, &q) || plan_mfma_batch(f, dt, bwd, &q) || plan_mfma(f, dt, bwd, &q) ||
          plan_mfma8(f, dt, bwd, &q) ||
          plan_mfma_f32(f, dt, bwd, p->algo == DWC_ALGO_MFMA, &q)) {
        *pl = q;
        return DWC_OK;
      }
      if (p->algo == DWC_ALGO_MFMA)
        return fail(err, DWC_ERR_UNSUPPORTED,
                    "no packed-MFMA kernel for this problem (needs bf16/fp16 with C % 8 == 0, "
                    "fp8 with C % 16 == 0 or fp32 with C % 16 == 0 and FW <= 31, stride 1, "
                    "FW <= 32, output width <= 64)");
    }
    if (direct && bwd && p->stride_h > 1) {
      const int S = p->stride_h;
      DgradPhaseArgs g{};
      g.N = (int)p->n; g.IH = (int)p->h; g.IW = (int)p->w; g.C = C;
      g.OH = (int)oh; g.OW = (int)ow;
      g.FH = p->fh; g.FW = p->fw; g.S = S; g.PH = p->pad_h; g.PW = p->pad_w;
      g.tiles_i = (int)(((p->h + S - 1) / S + kFwdRows - 1) / kFwdRows);
      g.tiles_j = (int)(((p->w + S - 1) / S + kPhaseTmw - 1) / kPhaseTmw);
      g.cblocks = cblocks;
      const int64_t items = p->n * cblocks * (int64_t)g.tiles_i * g.tiles_j * S * S;
      if (items > kI32Max - kWavesPerBlock)
        return fail(err, DWC_ERR_UNSUPPORTED, "too many work items for one launch");
      g.num_items = (int)items;
      q.kind = PLAN_PHASE;
      q.km = phase_km;
      q.blocks = (int)((items + kWavesPerBlock - 1) / kWavesPerBlock);
      q.pa = g;
      *pl = q;
      return DWC_OK;
    }
    if (direct) {
      q.flip = bwd;
      q.sweep = sweep_ok;
      f.cblocks = cblocks;
      if (q.sweep) {
        SweepArgs w{};
        w.N = f.N; w.IH = f.IH; w.IW = f.IW; w.C = C; w.OH = f.OH; w.OW = f.OW;
        w.F = p->fw;
        w.P = f.PH;
        w.PW = f.PW;
        q.tmw = p->fw >= 7 ? 7 : strip_override("DWC_FWD_STRIP", pick_strip(f.OW));
        w.tiles_w = (f.OW + q.tmw - 1) / q.tmw;
        w.cbg = cblocks;
        const int64_t cpi = sweep_chunks((int64_t)f.N * w.cbg * w.tiles_w, f.OH, p->fw);
        w.R = (int)((f.OH + cpi - 1) / cpi);
        if (const char* v = getenv("DWC_SWEEP_ROWS")) w.R = std::max(1, std::min(f.OH, atoi(v)));
        w.cpi = (f.OH + w.R - 1) / w.R;
        const int64_t waves = (int64_t)f.N * w.cpi * w.cbg * w.tiles_w;
        if (waves > kI32Max - kWavesPerBlock)
          return fail(err, DWC_ERR_UNSUPPORTED, "too many work items for one launch");
        w.num_items = (int)waves;
        q.blocks = (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
        q.sa = w;
        q.fa = f;
        *pl = q;
        return DWC_OK;
      }
      q.tmw = strip_override("DWC_FWD_STRIP", pick_strip(f.OW));
      f.tiles_w = (f.OW + q.tmw - 1) / q.tmw;
      f.tiles_h = (f.OH + kFwdRows - 1) / kFwdRows;
      const int64_t items = (int64_t)f.N * cblocks * f.tiles_h * f.tiles_w;
      if (items > kI32Max - kWavesPerBlock)
        return fail(err, DWC_ERR_UNSUPPORTED, "too many work items for one launch");
      f.num_items = (int)items;
      q.blocks = (int)((items + kWavesPerBlock - 1) / kWavesPerBlock);
      q.fa = f;
    } else {
      GenericArgs g{};
      g.N = (int)p->n;
      g.C = C;
      g.FH = p->fh;
      g.FW = p->fw;
      g.SH = p->stride_h;
      g.SW = p->stride_w;
      if (!bwd) {
        g.IH = (int)p->h; g.IW = (int)p->w; g.OH = (int)oh; g.OW = (int)ow;
        g.PH = p->pad_h; g.PW = p->pad_w;
        q.gen_kind = 0;  // GEN_FWD
        g.total = p->n * oh * ow * p->c;
      } else {
        // gather form for any stride; IH/IW = dX dims, OH/OW = dY dims
        g.IH = (int)p->h; g.IW = (int)p->w; g.OH = (int)oh; g.OW = (int)ow;
        g.PH = p->pad_h; g.PW = p->pad_w;
        q.gen_kind = 2;  // GEN_DGRAD
        g.total = p->n * p->h * p->w * p->c;
      }
      q.ga = g;
    }
  } else {
    if (p->wgrad_split > 0 && p->n * oh > 0 && p->wgrad_split > p->n * oh)
      return fail(err, DWC_ERR_BAD_PARAM, "wgrad_split larger than N*OH");
    if ((p->algo == DWC_ALGO_AUTO && !vector_auto) || p->algo == DWC_ALGO_MFMA) {
      if (plan_wgrad_mfma(p, oh, ow, &q) || plan_wgrad_mfma8(p, oh, ow, &q) ||
          plan_wgrad_mfma_f32(p, oh, ow, p->algo == DWC_ALGO_MFMA, &q)) {
        const int64_t m = (int64_t)p->fh * p->fw * p->c;
        q.ws_bytes = ((size_t)q.z * (size_t)m * 4 + 255) / 256 * 256;
        *pl = q;
        return DWC_OK;
      }
      if (p->algo == DWC_ALGO_MFMA)
        return fail(err, DWC_ERR_UNSUPPORTED,
                    "no packed-MFMA filter-gradient kernel for this problem (needs bf16/fp16 "
                    "with W <= 64 and C % 8 == 0, or fp32 with C % 16 == 0; stride 1, FH and "
                    "FW <= 32)");
    }
    const int64_t rows = p->n * oh;
    const int64_t m = (int64_t)p->fh * p->fw * p->c;
    const double flops = 2.0 * (double)p->n * oh * ow * p->c * p->fh * p->fw;
    const double bytes = (double)eb * ((double)p->n * p->h * p->w * p->c + (double)rows * ow * p->c);
    if (direct) {
      WgradArgs w{};
      w.N = (int)p->n; w.IH = (int)p->h; w.IW = (int)p->w; w.C = C;
      w.OH = (int)oh; w.OW = (int)ow;
      w.FH = p->fh; w.FW = p->fw; w.SH = p->stride_h; w.SW = p->stride_w;
      w.PH = p->pad_h; w.PW = p->pad_w;
      w.cblocks = cblocks;
      w.rows = (int)rows;
      q.sweep = sweep_ok;
      int64_t items = 0;
      if (q.sweep) {
        SweepArgs sw{};
        sw.N = (int)p->n; sw.IH = (int)p->h; sw.IW = (int)p->w; sw.C = C;
        sw.OH = (int)oh; sw.OW = (int)ow;
        sw.F = p->fw;
        sw.P = p->pad_h;
        sw.PW = p->pad_w;
        sw.hybrid = hybrid ? 1 : 0;
        q.tj = p->fw >= 7 ? 7 : strip_override("DWC_WGRAD_STRIP", pick_strip(ow));
        q.tfh = p->fh;
        sw.tiles_w = (int)((ow + q.tj - 1) / q.tj);
        sw.cbg = cblocks;
        // chunks per image: from a requested split of the N*OH axis, or
        // enough to fill the GPU
        const int64_t nn = std::max<int64_t>(p->n, 1);
        int64_t cpi = p->wgrad_split > 0 ? (p->wgrad_split + nn - 1) / nn
                                         : sweep_chunks(nn * sw.cbg * sw.tiles_w, oh, p->fw);
        cpi = std::max<int64_t>(1, std::min<int64_t>(cpi, oh));
        sw.R = (int)((oh + cpi - 1) / cpi);
        if (const char* v = getenv("DWC_SWEEP_ROWS"))
          sw.R = (int)std::max<int64_t>(1, std::min<int64_t>(oh, atoi(v)));
        sw.cpi = (int)((oh + sw.R - 1) / sw.R);
        const int64_t groups = (p->n * sw.cpi + kWavesPerBlock - 1) / kWavesPerBlock;
        sw.Z = (int)(groups * sw.tiles_w);
        q.z = rows == 0 ? 1 : std::max(1, sw.Z);
        items = rows == 0 ? 0 : groups * sw.cbg * sw.tiles_w;  // workgroups
        if (items > kI32Max)
          return fail(err, DWC_ERR_UNSUPPORTED, "too many work items for one launch");
        sw.num_items = (int)items;
        q.blocks = (int)items;
        q.sa = sw;
      } else {
        // 7-wide strips keep the dY block, the input strip and the taps of a
        // filter-row chunk within ~128 registers.
        q.tj = strip_override("DWC_WGRAD_STRIP", 7);
        q.tfh = filter_row_chunk(q.kfw);
        w.fh_tiles = (p->fh + q.tfh - 1) / q.tfh;
        const int64_t per_slice = (int64_t)cblocks * w.fh_tiles;
        const int64_t strips = (ow + q.tj - 1) / q.tj;
        q.z = rows == 0 ? 1
                        : (p->wgrad_split > 0 ? p->wgrad_split
                                              : pick_split(rows, per_slice, strips, m, flops, bytes));
        w.Z = q.z;
        items = (int64_t)q.z * per_slice;  // one workgroup each
      }
      if (items > kI32Max)
        return fail(err, DWC_ERR_UNSUPPORTED, "too many work items for one launch");
      w.num_items = (int)items;
      q.blocks = (int)items;
      q.wa = w;
    } else {
      GenericArgs g{};
      g.N = (int)p->n; g.IH = (int)p->h; g.IW = (int)p->w; g.C = C;
      g.OH = (int)oh; g.OW = (int)ow;
      g.FH = p->fh; g.FW = p->fw; g.SH = p->stride_h; g.SW = p->stride_w;
      g.PH = p->pad_h; g.PW = p->pad_w;
      g.rows = (int)rows;
      // one lane per (slice, tap, channel): enough slices for ~512K lanes
      const int64_t fill = std::max<int64_t>(1, (524288 + m - 1) / m);
      q.z = rows == 0 ? 1
                      : (p->wgrad_split > 0 ? p->wgrad_split
                                            : (int)std::min<int64_t>({fill, rows, 4096}));
      g.Z = q.z;
      g.total = (int64_t)q.z * m;
      q.gen_kind = 3;  // GEN_WGRAD
      q.ga = g;
    }
    q.ws_bytes = q.z > 1 ? (size_t)q.z * (size_t)m * 4 : 0;
    q.ws_bytes = (q.ws_bytes + 255) / 256 * 256;
  }
  *pl = q;
  return DWC_OK;
}

namespace {

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace

int check_pointers(const dwc_problem* p, const Plan& pl, const void* in0, const void* in1,
                   const void* out, const void* ws, size_t ws_bytes, std::string* err) {
  const size_t eb = elem_bytes(pl.dt);
  const size_t nx = (size_t)p->n * p->h * p->w * p->c;
  const size_t ny = (size_t)p->n * pl.oh * pl.ow * p->c;
  const size_t nw = (size_t)p->fh * p->fw * p->c;
  size_t in0_bytes = 0, in1_bytes = 0, out_bytes = 0;
  if (pl.op == DWC_OP_FWD) {
    in0_bytes = nx * eb; in1_bytes = nw * eb; out_bytes = ny * 4;
  } else if (pl.op == DWC_OP_BWD_DATA) {
    in0_bytes = ny * eb; in1_bytes = nw * eb; out_bytes = nx * 4;
  } else {
    in0_bytes = nx * eb; in1_bytes = ny * eb; out_bytes = nw * 4;
  }
  const bool need_inputs = !pl.empty;
  // A tensor with no elements may have a NULL address.
  if (!out && out_bytes > 0) return fail(err, DWC_ERR_BAD_PARAM, "output pointer is NULL");
  if (need_inputs && (!in0 || !in1)) return fail(err, DWC_ERR_BAD_PARAM, "input pointer is NULL");
  if (((uintptr_t)out) % 4) return fail(err, DWC_ERR_MISALIGNED, "output not 4-byte aligned");
  if (need_inputs && ((((uintptr_t)in0) % eb) || (((uintptr_t)in1) % eb)))
    return fail(err, DWC_ERR_MISALIGNED, "input not aligned to its element size");
  if (need_inputs &&
      (overlap(out, out_bytes, in0, in0_bytes) || overlap(out, out_bytes, in1, in1_bytes)))
    return fail(err, DWC_ERR_ALIAS, "output overlaps an input");
  if (pl.op == DWC_OP_BWD_FILTER && pl.ws_bytes > 0 && !pl.empty) {
    if (!ws || ws_bytes < pl.ws_bytes)
      return fail(err, DWC_ERR_WORKSPACE, "workspace missing or smaller than required (" +
                                              std::to_string(pl.ws_bytes) + " bytes)");
    if (((uintptr_t)ws) % 4) return fail(err, DWC_ERR_MISALIGNED, "workspace not 4-byte aligned");
    if (overlap(ws, pl.ws_bytes, out, out_bytes) || overlap(ws, pl.ws_bytes, in0, in0_bytes) ||
        overlap(ws, pl.ws_bytes, in1, in1_bytes))
      return fail(err, DWC_ERR_ALIAS, "workspace overlaps a tensor");
  }
  return DWC_OK;
}

int check_prologue(const dwc_problem* p, const Plan& pl, const void* out, const float* scale,
                   const float* shift, std::string* err) {
  if (pl.empty) return DWC_OK;
  if (!scale || !shift) return fail(err, DWC_ERR_BAD_PARAM, "scale or shift pointer is NULL");
  if (((uintptr_t)scale) % 4 || ((uintptr_t)shift) % 4)
    return fail(err, DWC_ERR_MISALIGNED, "scale or shift not 4-byte aligned");
  const size_t out_bytes = (size_t)p->n * pl.oh * pl.ow * p->c * 4;
  const size_t vec_bytes = (size_t)p->c * 4;
  if (overlap(out, out_bytes, scale, vec_bytes) || overlap(out, out_bytes, shift, vec_bytes))
    return fail(err, DWC_ERR_ALIAS, "output overlaps scale or shift");
  return DWC_OK;
}

std::string describe(const Plan& pl) {
  static const char* ops[] = {"fwd", "bwd_data", "bwd_filter"};
  char buf[512];
  if (pl.kind == PLAN_PHASE) {
    const DgradPhaseArgs& g = pl.pa;
    snprintf(buf, sizeof buf,
             "%s phase dt=%s fh=%d fw=%d s=%d km=%d tiles_i=%d tiles_j=%d cblocks=%d items=%d "
             "blocks=%d",
             ops[pl.op], dt_name(pl.dt), g.FH, g.FW, g.S, pl.km, g.tiles_i, g.tiles_j, g.cblocks,
             g.num_items, pl.blocks);
    return buf;
  }
  if (pl.kind == PLAN_MFMA && pl.op == DWC_OP_BWD_FILTER && pl.wf32) {
    const WgradF32Args& w = pl.wf;
    snprintf(buf, sizeof buf,
             "%s mfma dt=%s fw=%d fh=%d f32=1 tw=%d nb=%d cg=%d nw=%d rps=%d zr=%d z=%d cblk=%d "
             "lds=%d blocks=%d ws_bytes=%zu",
             ops[pl.op], dt_name(pl.dt), w.FW, w.FH, pl.wf32_tw, pl.wf32_nb, w.cg, w.nw, w.rps,
             w.Z, pl.z, w.cblk, w.lds_bytes, pl.blocks, pl.ws_bytes);
    return buf;
  }
  if (pl.kind == PLAN_MFMA && pl.op == DWC_OP_BWD_FILTER) {
    const WgradMfmaArgs& w = pl.wm;
    snprintf(buf, sizeof buf,
             "%s mfma dt=%s fw=%d fh=%d nfm=%d nfn=%d nk=%d pf=%d cb=%d xr=%d xp=%d dyp=%d "
             "dpad=%d hx=%d ix=%d e_lo=%d hd=%d id=%d lds=%d z=%d ipb=%d cblk=%d blocks=%d "
             "ws_bytes=%zu",
             ops[pl.op], dt_name(pl.dt), w.FW, w.FH, pl.nfm, pl.nfn, pl.nk, pl.pf, pl.cb, w.xr,
             w.xp, w.dyp, w.dpad, w.hx, w.ix, w.e_lo, w.hd, w.id, w.lds_bytes, w.Z, w.ipb,
             w.cblk, pl.blocks, pl.ws_bytes);
    return buf;
  }
  if (pl.kind == PLAN_MFMA && pl.h4m) {
    const MfmaF32Args& m = pl.mf;
    snprintf(buf, sizeof buf,
             "%s mfma dt=%s fw=%d fh=%d flip=%d h4=1 fwi=%d t=%d rg=%d cg=%d tiles=%d "
             "nw=%d same=%d cblk=%d lds=%d blocks=%d",
             ops[pl.op], dt_name(pl.dt), m.FW, m.FH, (int)pl.flip, pl.h4m_fwi, pl.h4m_t, m.rg,
             m.cg, m.tiles, m.nw, m.same, m.cblk, m.lds_bytes, pl.blocks);
    return buf;
  }
  if (pl.kind == PLAN_MFMA && pl.f32m) {
    const MfmaF32Args& m = pl.mf;
    snprintf(buf, sizeof buf,
             "%s mfma dt=%s fw=%d fh=%d flip=%d f32=1 fwi=%d t=%d img=%d rg=%d cg=%d tiles=%d "
             "nw=%d same=%d cblk=%d lds=%d blocks=%d",
             ops[pl.op], dt_name(pl.dt), m.FW, m.FH, (int)pl.flip, pl.f32m_fwi, pl.f32m_t,
             (int)pl.f32m_img, m.rg, m.cg, m.tiles, m.nw, m.same, m.cblk, m.lds_bytes, pl.blocks);
    return buf;
  }
  if (pl.kind == PLAN_MFMA && pl.batch) {
    const MfmaBatchArgs& m = pl.mb;
    snprintf(buf, sizeof buf,
             "%s mfma dt=%s fw=%d fh=%d flip=%d batch=1 cb=%d imgs=%d rows=%d ng=%d "
             "rch=%d cblk=%d nq=%d lds=%d blocks=%d",
             ops[pl.op], dt_name(pl.dt), m.FW, m.FH, (int)pl.flip, m.cb, pl.bimg,
             pl.bimg == kB16Img ? kB16Rows : kBatchRows, m.ng, m.rch, m.cblk, m.nq, m.lds_bytes,
             pl.blocks);
    if (pl.bimg == kB16Img) {
      const size_t k = strlen(buf);
      snprintf(buf + k, sizeof buf - k, " ocg=%d orows=%d", pl.bng, m.orows);
    }
    return buf;
  }
  if (pl.kind == PLAN_MFMA) {
    const MfmaArgs& m = pl.ma;
    snprintf(buf, sizeof buf,
             "%s mfma dt=%s fw=%d fh=%d flip=%d nf=%d cb=%d gt=%d tiles=%d rblk=%d "
             "xr=%d wt=%d wp=%d lds=%d rch=%d cblk=%d blocks=%d",
             ops[pl.op], dt_name(pl.dt), m.FW, m.FH, (int)pl.flip, pl.nf, pl.cb, m.gt, pl.tiles,
             m.rblk, m.xr, m.wt, m.wp, m.lds_bytes, m.rch, m.cblk, pl.blocks);
    return buf;
  }
  if (pl.kind == PLAN_DIRECT && pl.sweep) {
    const SweepArgs& w = pl.sa;
    snprintf(buf, sizeof buf,
             "%s sweep dt=%s f=%d strip=%d tiles_w=%d rows=%d cpi=%d cblocks=%d "
             "items=%d blocks=%d z=%d ws_bytes=%zu%s",
             ops[pl.op], dt_name(pl.dt), w.F, pl.op == DWC_OP_BWD_FILTER ? pl.tj : pl.tmw,
             w.tiles_w, w.R, w.cpi, w.cbg, w.num_items, pl.blocks,
             pl.op == DWC_OP_BWD_FILTER ? pl.z : 0, pl.ws_bytes, w.hybrid ? " hybrid=1" : "");
  } else if (pl.kind == PLAN_DIRECT && pl.op != DWC_OP_BWD_FILTER) {
    snprintf(buf, sizeof buf,
             "%s %s dt=%s fw=%d kfw=%d sw=%d flip=%d tmw=%d rows=%d tiles_w=%d tiles_h=%d "
             "cblocks=%d items=%d blocks=%d",
             ops[pl.op], "direct", dt_name(pl.dt), pl.fa.FW, pl.kfw, pl.fa.SW,
             (int)pl.flip, pl.tmw, kFwdRows,
             pl.fa.tiles_w, pl.fa.tiles_h, pl.fa.cblocks, pl.fa.num_items, pl.blocks);
  } else if (pl.kind == PLAN_DIRECT) {
    snprintf(buf, sizeof buf,
             "%s %s dt=%s fw=%d kfw=%d sw=%d tj=%d tfh=%d fh_tiles=%d rows=%d cblocks=%d z=%d "
             "items=%d blocks=%d ws_bytes=%zu",
             ops[pl.op], "direct", dt_name(pl.dt), pl.wa.FW, pl.kfw, pl.wa.SW, pl.tj,
             pl.tfh, pl.wa.fh_tiles, kWgradRows, pl.wa.cblocks, pl.z,
             pl.wa.num_items, pl.blocks, pl.ws_bytes);
  } else {
    snprintf(buf, sizeof buf, "%s generic dt=%s kind=%d z=%d total=%lld ws_bytes=%zu",
             ops[pl.op], dt_name(pl.dt), pl.gen_kind, pl.z, (long long)pl.ga.total, pl.ws_bytes);
  }
  return buf;
}

}  // namespace dwc

using namespace dwc;

extern "C" {

int dwc_version(void) { return DWC_VERSION; }

const char* dwc_status_string(int s) {
  switch (s) {
    case DWC_OK: return "ok";
    case DWC_ERR_BAD_PARAM: return "bad parameter";
    case DWC_ERR_UNSUPPORTED: return "unsupported";
    case DWC_ERR_MISALIGNED: return "misaligned pointer";
    case DWC_ERR_WORKSPACE: return "workspace too small";
    case DWC_ERR_ALIAS: return "output aliases an input";
    case DWC_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* dwc_last_error(void) { return g_last_error.c_str(); }

int dwc_output_dims(const dwc_problem* p, int64_t* oh, int64_t* ow) {
  std::string err;
  int64_t h = 0, w = 0;
  const int st = validate(p, &h, &w, &err);
  if (st) {
    set_last_error(err);
    return st;
  }
  if (oh) *oh = h;
  if (ow) *ow = w;
  return DWC_OK;
}

int dwc_check(const dwc_problem* p, int op) {
  Plan pl;
  std::string err;
  const int st = make_plan(p, op, &pl, &err);
  if (st) set_last_error(err);
  return st;
}

int dwc_plan_describe(const dwc_problem* p, int op, char* buf, size_t len) {
  Plan pl;
  std::string err;
  const int st = make_plan(p, op, &pl, &err);
  if (st) {
    set_last_error(err);
    return st;
  }
  if (buf && len) {
    const std::string s = describe(pl);
    const size_t k = std::min(len - 1, s.size());
    s.copy(buf, k);
    buf[k] = 0;
  }
  return DWC_OK;
}

int dwc_bwd_filter_workspace_size(const dwc_problem* p, size_t* bytes) {
  Plan pl;
  std::string err;
  const int st = make_plan(p, DWC_OP_BWD_FILTER, &pl, &err);
  if (st) {
    set_last_error(err);
    return st;
  }
  if (!bytes) {
    set_last_error("bytes pointer is NULL");
    return DWC_ERR_BAD_PARAM;
  }
  size_t need = pl.empty ? 0 : pl.ws_bytes;
  // AUTO may fall back from the packed-MFMA kernels to the vector kernels
  // at call time (tensors not 16-byte aligned): cover both plans
  if (pl.kind == PLAN_MFMA && p->algo == DWC_ALGO_AUTO && !pl.empty) {
    dwc_problem d = *p;
    d.algo = DWC_ALGO_DIRECT;
    Plan alt;
    int s2 = make_plan(&d, DWC_OP_BWD_FILTER, &alt, &err);
    if (s2 == DWC_ERR_UNSUPPORTED) {
      d.algo = DWC_ALGO_GENERIC;
      s2 = make_plan(&d, DWC_OP_BWD_FILTER, &alt, &err);
    }
    if (s2 == DWC_OK) need = std::max(need, alt.ws_bytes);
  }
  *bytes = need;
  return DWC_OK;
}

}  // extern "C"
