// dwc_kernels.h -- HIP kernels of libdwc for gfx950 (MI355X).
//
// Operations (Flash-DWC, TACO): forward DWC (§2.1), the stride-1 data
// gradient as the forward map of dY with the filter turned by 180 degrees
// (§5.1), and the filter gradient split along the N*OH accumulation axis
// (§5.1).  Layouts are channel-last (§2.3).
//
// Mapping shared by the direct kernels: one channel per lane, 64 channels per
// wave, so every load of one pixel is one contiguous 256-byte (fp32) or
// 128-byte (bf16/fp16) segment, and every lane owns a strip of outputs in
// registers.  Zero padding is read through buffer-resource range checks:
// an out-of-range offset returns 0, so the FMA loops have no branches.
#pragma once

#include "dwc_device.h"

namespace dwc {

// Loads one operand element through a buffer resource.  `voff` is the
// lane's byte offset (the channel), `soff` the wave-uniform byte offset of
// the pixel.  Reads through a resource of zero bytes return 0.
template <int DT>
__device__ __forceinline__ float ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (DT == DT_F32) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
  } else if constexpr (DT == DT_BF16) {
    uint32_t b = __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
    return __uint_as_float(b << 16);
  } else if constexpr (DT == DT_F16) {
    unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
    return (float)__builtin_bit_cast(_Float16, h);
  } else {
    return fp8_to_f32<DT>(__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0));
  }
}

// Byte offsets, per lane, of the pixels col0 .. col0+SPAN-1 of an image row
// relative to pixel col0, plus the lane's channel.  Columns outside
// [0, cols) and channels >= C get an offset no resource covers, so they read
// as zero (implicit zero padding).  Computed once per strip and shared by
// every row the strip visits.
template <int SPAN>
__device__ __forceinline__ void column_offsets(uint32_t (&o)[SPAN], int col0, int cols,
                                               uint32_t pix_bytes, int c, int C, int eb) {
#pragma unroll
  for (int j = 0; j < SPAN; ++j) {
    const bool ok = (unsigned)(col0 + j) < (unsigned)cols && c < C;
    o[j] = ok ? (uint32_t)j * pix_bytes + (uint32_t)c * eb : kOOB;
  }
}

// The strip of SPAN pixels of image row `row` starting at column col0, one
// channel per lane.  A row outside [0, rows) reads as zero.
template <int DT, int SPAN>
__device__ __forceinline__ void load_strip(float (&v)[SPAN], const char* img, int row, int rows,
                                           int col0, int cols, uint32_t pix_bytes,
                                           const uint32_t (&o)[SPAN]) {
  const bool row_ok = (unsigned)row < (unsigned)rows;
  const char* base = img + ((ptrdiff_t)row * cols + col0) * (ptrdiff_t)pix_bytes;
  const auto r = make_rsrc(base, row_ok ? (uint32_t)SPAN * pix_bytes : 0u);
#pragma unroll
  for (int j = 0; j < SPAN; ++j) v[j] = ld<DT>(r, o[j], 0);
}

// t * sigmoid(t) = t / (1 + e^-t), with e^-t = 2^(-t log2 e) from the
// hardware's base-2 exponential and 1 / (1 + e^-t) from its reciprocal.
__device__ __forceinline__ float silu_f(float t) {
  const float e = __builtin_amdgcn_exp2f(-t * 1.44269504088896341f);
  return t * __builtin_amdgcn_rcpf(1.0f + e);
}

// The fused prologue on a strip as it is consumed: t = act(v * s + b) for
// the pixels inside the image; a row or column outside stays 0 (the zero
// padding surrounds X', not X).  row, col0 and p are wave-uniform.
template <int SPAN>
__device__ __forceinline__ void apply_prologue(float (&v)[SPAN], int row, int rows, int col0,
                                               int cols, float s, float b, const Prologue& p) {
  if ((unsigned)row >= (unsigned)rows) return;
  if (p.silu) {
#pragma unroll
    for (int j = 0; j < SPAN; ++j) {
      const float t = silu_f(fminf(fmaxf(fmaf(v[j], s, b), p.lo), p.hi));
      v[j] = (unsigned)(col0 + j) < (unsigned)cols ? t : 0.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < SPAN; ++j) {
      const float t = fminf(fmaxf(fmaf(v[j], s, b), p.lo), p.hi);
      v[j] = (unsigned)(col0 + j) < (unsigned)cols ? t : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// Forward-type direct kernel ("row streaming").
//
// A wave owns 64 channels x TR output rows x TMW output columns; each lane
// keeps its TR x TMW outputs in registers.  The filter is processed in
// chunks of FHC rows held in registers: filter reuse across all TR x TMW
// outputs (§3.2).  For each chunk the wave streams the (TR-1)*S+FHC input
// rows the chunk touches; each row's strip of (TMW-1)*S+FW pixels is loaded
// once and feeds every (output row, filter row) pair that reads it, and
// along the width consecutive taps share TMW-1 of their inputs (the
// width-first reuse of §3.3, run as 1-D filters along the width accumulated
// over filter rows).  All loop bounds are compile-time, so every accumulator
// and tap is a register.  FLIP reads the filter turned by 180 degrees, which
// makes this the stride-1 data gradient (§5.1).  PAD runs a filter a.FW < FW
// columns wide on the FW-wide body: its taps a.FW .. FW-1 take no products
// (a zero tap times an inf input would give NaN).  Taps that may be past
// a.FW keep the accumulator by a select, not a branch, so the whole row body
// stays one block that the compiler schedules loads across.
// ---------------------------------------------------------------------------
template <int DT, int FW, int S, int TMW, bool FLIP, bool PRO = false, bool PAD = false>
__global__ __launch_bounds__(kBlockThreads) void fwd_rows(FwdArgs a) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int TR = kFwdRows;
  constexpr int FHC = filter_row_chunk(FW);
  constexpr int SPAN = (TMW - 1) * S + FW;
  constexpr int MSPAN = (TR - 1) * S + FHC;
  constexpr int FWLO = PAD ? direct_fw_below(FW) + 1 : FW;  // taps always real
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int item = xcd_logical_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wave;
  if (item >= a.num_items) return;
  int t = item;
  const int tw = t % a.tiles_w;
  t /= a.tiles_w;
  const int th = t % a.tiles_h;
  t /= a.tiles_h;
  const int cb = t % a.cblocks;
  const int n = t / a.cblocks;
  const int c = cb * kWaveChannels + lane;
  const uint32_t voff = c < a.C ? (uint32_t)c * EB : kOOB;
  const uint32_t Cb = (uint32_t)a.C * EB;
  const char* img = (const char*)a.in + (size_t)n * a.IH * a.IW * Cb;
  const auto zero = make_rsrc(a.in, 0);
  float ps = 1.f, pb = 0.f;  // this lane's prologue scale and shift
  if constexpr (PRO) {
    if (c < a.C) {
      ps = a.pro.scale[c];
      pb = a.pro.shift[c];
    }
  }
  const int fwn = PAD ? a.FW : FW;  // the filter's real width
  const auto wrs = make_rsrc(a.filt, (uint32_t)(a.FH * fwn) * Cb);
  const int oh0 = th * TR, ow0 = tw * TMW;
  const int ih_base = oh0 * S - a.PH;
  // Odd row tiles walk their input rows bottom-up, so two neighbouring
  // tiles read the rows they share at about the same time and the second
  // read hits L2.  Bottom-up is the same computation on the tile mirrored
  // vertically: input row m stands for row MSPAN-1-m of the chunk, filter
  // row k for FHC-1-k and accumulator row r for output row TR-1-r.
  const bool up = (th & 1) != 0;
  const int iw0 = ow0 * S - a.PW;
  uint32_t coff[SPAN];
  column_offsets<SPAN>(coff, iw0, a.IW, Cb, c, a.C, EB);

  float acc[TR][TMW];
#pragma unroll
  for (int r = 0; r < TR; ++r)
#pragma unroll
    for (int q = 0; q < TMW; ++q) acc[r][q] = 0.f;

  for (int fh0 = 0; fh0 < a.FH; fh0 += FHC) {
    // chunk rows k in [klo, khi) are filter rows; the last chunk's others
    // are past FH and take no products (a zero tap times an inf input would
    // be NaN, where the definition has no such term)
    const int nk = a.FH - fh0;
    const int klo = up ? FHC - nk : 0, khi = up ? FHC : nk;
    float wv[FHC][FW];
#pragma unroll
    for (int k = 0; k < FHC; ++k) {
      const int fh = fh0 + (up ? FHC - 1 - k : k);
      const bool ok = fh < a.FH;
      const int fhe = FLIP ? a.FH - 1 - fh : fh;
#pragma unroll
      for (int fw = 0; fw < FW; ++fw) {
        const bool okw = ok && (!PAD || fw < fwn);
        const int fwe = FLIP ? fwn - 1 - fw : fw;
        wv[k][fw] = ld<DT>(okw ? wrs : zero, voff, okw ? (uint32_t)(fhe * fwn + fwe) * Cb : 0u);
      }
    }
#pragma unroll
    for (int m = 0; m < MSPAN; ++m) {
      const int ih = ih_base + fh0 + (up ? MSPAN - 1 - m : m);
      if ((unsigned)ih >= (unsigned)a.IH) continue;  // a padding row: contributes 0
      float xv[SPAN];
      load_strip<DT, SPAN>(xv, img, ih, a.IH, iw0, a.IW, Cb, coff);
      if constexpr (PRO) apply_prologue<SPAN>(xv, ih, a.IH, iw0, a.IW, ps, pb, a.pro);
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const int k = m - r * S;
        if (k < 0 || k >= FHC || k < klo || k >= khi) continue;
#pragma unroll
        for (int fw = 0; fw < FW; ++fw) {
          if (fw < FWLO) {
#pragma unroll
            for (int q = 0; q < TMW; ++q) acc[r][q] = fmaf(xv[q * S + fw], wv[k][fw], acc[r][q]);
          } else {
            const bool real = fw < fwn;
#pragma unroll
            for (int q = 0; q < TMW; ++q) {
              const float v = fmaf(xv[q * S + fw], wv[k][fw], acc[r][q]);
              acc[r][q] = real ? v : acc[r][q];
            }
          }
        }
      }
    }
  }

  if (c < a.C) {
    float* out = a.out + (size_t)n * a.OH * a.OW * a.C + c;
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      const int oh = oh0 + (up ? TR - 1 - r : r);
      if (oh >= a.OH) continue;
#pragma unroll
      for (int q = 0; q < TMW; ++q) {
        const int ow = ow0 + q;
        if (ow < a.OW) store_nt(&out[((size_t)oh * a.OW + ow) * a.C], acc[r][q]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Strided data gradient (stride S >= 2 in both dimensions) by output phase.
//
// dX[ih][iw] gathers dY[oh][ow] * W[fh][fw] over oh*S - PH + fh = ih and
// ow*S - PW + fw = iw (the adjoint of the strided forward map).  For the dX
// pixels ih = a + S i, iw = b + S j of phase (a, b), only the taps
// fh = f0h + S k and fw = f0w + S l contribute, with oh = i + ch - k and
// ow = j + cw - l (f0h = (a + PH) mod S, ch = (a + PH - f0h) / S; likewise
// for columns): a stride-1 correlation of dY with that sub-filter, which
// runs like fwd_rows -- TR x TMW outputs per lane, sub-filter rows in
// registers in chunks of KC, one dY strip per row feeding every output row
// that reads it, width-first reuse along the strip.  KM bounds the
// sub-filter's rows and columns; taps past its real size are zeros.  The
// S*S phases of a tile are consecutive waves of one workgroup, so they read
// the same dY rows at the same time.
// ---------------------------------------------------------------------------
template <int DT, int KM, int TMW>
__global__ __launch_bounds__(kBlockThreads) void dgrad_phase(DgradPhaseArgs a) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int TR = kFwdRows;
  constexpr int KC = KM <= 8 ? KM : 4;  // sub-filter rows held at once
  constexpr int SPAN = TMW + KM - 1;
  constexpr int MSPAN = TR + KC - 1;
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int item = xcd_logical_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wave;
  if (item >= a.num_items) return;
  const int S = a.S;
  int t = item;
  const int ph = t % (S * S);
  t /= S * S;
  const int tj = t % a.tiles_j;
  t /= a.tiles_j;
  const int ti = t % a.tiles_i;
  t /= a.tiles_i;
  const int cb = t % a.cblocks;
  const int n = t / a.cblocks;
  const int pa = ph / S, pb = ph - pa * S;  // row and column phase
  const int f0h = (pa + a.PH) % S, f0w = (pb + a.PW) % S;
  const int ch = (pa + a.PH - f0h) / S, cw = (pb + a.PW - f0w) / S;
  const int kh = f0h < a.FH ? (a.FH - f0h + S - 1) / S : 0;  // sub-filter rows
  const int kw = f0w < a.FW ? (a.FW - f0w + S - 1) / S : 0;  // and columns
  const int c = cb * kWaveChannels + lane;
  const uint32_t voff = c < a.C ? (uint32_t)c * EB : kOOB;
  const uint32_t Cb = (uint32_t)a.C * EB;
  const char* img = (const char*)a.dy + (size_t)n * a.OH * a.OW * Cb;
  const auto zero = make_rsrc(a.filt, 0);
  const auto wrs = make_rsrc(a.filt, (uint32_t)(a.FH * a.FW) * Cb);
  const int i0 = ti * TR, j0 = tj * TMW;  // first phase row / column of the tile
  // strip of dY columns ow0 .. ow0+SPAN-1: output column q, tap l reads
  // strip element q - l + KM - 1
  const int ow0 = j0 + cw - (KM - 1);
  uint32_t coff[SPAN];
  column_offsets<SPAN>(coff, ow0, a.OW, Cb, c, a.C, EB);

  float acc[TR][TMW];
#pragma unroll
  for (int r = 0; r < TR; ++r)
#pragma unroll
    for (int q = 0; q < TMW; ++q) acc[r][q] = 0.f;

  for (int k0 = 0; k0 < kh; k0 += KC) {
    float wv[KC][KM];
#pragma unroll
    for (int k = 0; k < KC; ++k)
#pragma unroll
      for (int l = 0; l < KM; ++l) {
        const bool ok = k0 + k < kh && l < kw;
        const int e = (f0h + S * (k0 + k)) * a.FW + f0w + S * l;
        wv[k][l] = ld<DT>(ok ? wrs : zero, voff, ok ? (uint32_t)e * Cb : 0u);
      }
    // dY row ohb + m feeds output row r through chunk row k = r + KC - 1 - m
    const int ohb = i0 + ch - (k0 + KC - 1);
#pragma unroll
    for (int m = 0; m < MSPAN; ++m) {
      const int oh = ohb + m;
      if ((unsigned)oh >= (unsigned)a.OH) continue;  // no such dY row: contributes 0
      float yv[SPAN];
      load_strip<DT, SPAN>(yv, img, oh, a.OH, ow0, a.OW, Cb, coff);
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const int k = r + KC - 1 - m;
        // sub-filter rows past kh and columns past kw are zero taps: they
        // take no products (zero times an inf dY would be NaN)
        if (k < 0 || k >= KC || k0 + k >= kh) continue;
#pragma unroll
        for (int l = 0; l < KM; ++l) {
          if (l >= kw) continue;  // not break: a loop exit leaves acc in scratch memory
#pragma unroll
          for (int q = 0; q < TMW; ++q)
            acc[r][q] = fmaf(yv[q - l + KM - 1], wv[k][l], acc[r][q]);
        }
      }
    }
  }

  if (c < a.C) {
    float* out = a.dx + (size_t)n * a.IH * a.IW * a.C + c;
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      const int ih = pa + S * (i0 + r);
      if (ih >= a.IH) break;
#pragma unroll
      for (int q = 0; q < TMW; ++q) {
        const int iw = pb + S * (j0 + q);
        if (iw < a.IW) store_nt(&out[((size_t)ih * a.IW + iw) * a.C], acc[r][q]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Filter-gradient direct kernel (§5.1 "accumulation-axis parallelism").
//
// A workgroup owns 64 channels x a chunk of TFH filter rows x all FW taps
// and one slice [r0, r1) of the flattened N*OH axis; each lane keeps its
// TFH x FW taps in registers.  The slice is cut into units of up to RY
// consecutive output rows of one image x one strip of TJ columns, dealt
// round-robin to the 4 waves.  For a unit, the RY x TJ dY values stay in
// registers and each of the (RY-1)*S+TFH input rows it touches is loaded
// once as a strip of (TJ-1)*S+FW pixels, which feeds every (dY row, filter
// row) pair that reads it; along the width each input pixel meets every tap
// whose window covers it (width-first reuse, §3.3).  The 4 waves add their
// sums through LDS in a fixed order and one partial per slice is written;
// reduce_partials adds the slices in slice order.  Deterministic.  A filter
// a.FW < FW columns wide runs on the FW-wide body; its taps a.FW .. FW-1 are
// summed but not written, and the partials have a.FW taps per filter row.
// ---------------------------------------------------------------------------
template <int DT, int FW, int S, int TJ>
__global__ __launch_bounds__(kBlockThreads) void wgrad_rows(WgradArgs a) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int TFH = filter_row_chunk(FW);
  constexpr int RY = kWgradRows;
  constexpr int SPAN = (TJ - 1) * S + FW;
  constexpr int MSPAN = (RY - 1) * S + TFH;
  __shared__ float red[2][TFH * FW][64];

  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_items) return;  // the whole workgroup leaves together
  int t = blk;
  const int ft = t % a.fh_tiles;
  t /= a.fh_tiles;
  const int cb = t % a.cblocks;
  const int z = t / a.cblocks;
  const int c = cb * kWaveChannels + lane;
  const uint32_t Cb = (uint32_t)a.C * EB;
  const int q0 = a.rows / a.Z, rem = a.rows % a.Z;
  const int r0 = z * q0 + (z < rem ? z : rem);
  const int r1 = r0 + q0 + (z < rem ? 1 : 0);
  const int fh0 = ft * TFH;
  const int strips = (a.OW + TJ - 1) / TJ;

  float acc[TFH][FW];
#pragma unroll
  for (int k = 0; k < TFH; ++k)
#pragma unroll
    for (int fw = 0; fw < FW; ++fw) acc[k][fw] = 0.f;

  int unit = 0;  // running index of (row group, strip) units in this slice
  for (int row = r0; row < r1;) {
    const int n = row / a.OH, oh0 = row - n * a.OH;
    int cnt = r1 - row;
    if (cnt > RY) cnt = RY;
    if (cnt > a.OH - oh0) cnt = a.OH - oh0;
    const char* ximg = (const char*)a.x + (size_t)n * a.IH * a.IW * Cb;
    const char* dimg = (const char*)a.dy + (size_t)n * a.OH * a.OW * Cb;
    for (int s = 0; s < strips; ++s, ++unit) {
      if ((unit & 3) != wave) continue;
      const int ow0 = s * TJ;
      const int ih_base = oh0 * S - a.PH + fh0;
      const int iw0 = ow0 * S - a.PW;
      float dv[RY][TJ];
      {
        uint32_t doff[TJ];
        column_offsets<TJ>(doff, ow0, a.OW, Cb, c, a.C, EB);
#pragma unroll
        for (int r = 0; r < RY; ++r)
          load_strip<DT, TJ>(dv[r], dimg, r < cnt ? oh0 + r : -1, a.OH, ow0, a.OW, Cb, doff);
      }
      uint32_t xoff[SPAN];
      column_offsets<SPAN>(xoff, iw0, a.IW, Cb, c, a.C, EB);
#pragma unroll
      for (int m = 0; m < MSPAN; ++m) {
        const int ih = ih_base + m;
        if ((unsigned)ih >= (unsigned)a.IH) continue;  // padding row: contributes 0
        float xv[SPAN];
        load_strip<DT, SPAN>(xv, ximg, ih, a.IH, iw0, a.IW, Cb, xoff);
#pragma unroll
        for (int r = 0; r < RY; ++r) {
          const int k = m - r * S;
          if (k < 0 || k >= TFH) continue;
#pragma unroll
          for (int q = 0; q < TJ; ++q)
#pragma unroll
            for (int fw = 0; fw < FW; ++fw) acc[k][fw] = fmaf(xv[q * S + fw], dv[r][q], acc[k][fw]);
        }
      }
    }
    row += cnt;
  }

  // (w0 + w2) + (w1 + w3), then one store of the slice partial.
  if (wave >= 2) {
#pragma unroll
    for (int k = 0; k < TFH; ++k)
#pragma unroll
      for (int fw = 0; fw < FW; ++fw) red[wave - 2][k * FW + fw][lane] = acc[k][fw];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int k = 0; k < TFH; ++k)
#pragma unroll
      for (int fw = 0; fw < FW; ++fw) acc[k][fw] += red[wave][k * FW + fw][lane];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int k = 0; k < TFH; ++k)
#pragma unroll
      for (int fw = 0; fw < FW; ++fw) red[0][k * FW + fw][lane] = acc[k][fw];
  }
  __syncthreads();
  if (wave == 0 && c < a.C) {
    float* ws = a.ws + (size_t)z * a.FH * a.FW * a.C + c;
#pragma unroll
    for (int k = 0; k < TFH; ++k) {
      const int fh = fh0 + k;
      if (fh >= a.FH) break;
#pragma unroll
      for (int fw = 0; fw < FW; ++fw)  // (a guard, not a break: a loop exit
                                       // would leave acc in scratch memory)
        if (fw < a.FW) ws[((size_t)fh * a.FW + fw) * a.C] = acc[k][fw] + red[0][k * FW + fw][lane];
    }
  }
}

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

// Number of input-row strips a sweep wave keeps in registers: the row in
// use plus two in flight, so each row's loads have two steps of FMAs to
// arrive.
constexpr int kSweepBufs = 3;

// ---------------------------------------------------------------------------
// Forward-type sweep kernel: stride 1, square filter F <= 9.
//
// A wave owns 64 channels x TMW output columns x R consecutive output rows
// of one image and walks down them.  The whole F x F filter stays in
// registers (filter reuse, §3.2).  Input rows are read in order, each once
// per wave: input row i feeds output rows i-F+1 .. i (one per filter row),
// whose accumulators live in a ring of F register rows; when an output row
// has seen all F filter rows it is stored and its ring slot reused.  Along
// the width one strip of TMW+F-1 pixels serves all F taps of every filter
// row (the width-first reuse and 1-D row decomposition of §3.3).  Rows are
// loaded two steps ahead into a ring of three strip buffers.  The body is
// unrolled over lcm(F, 3) rows, so every ring index is a compile-time
// constant.  FLIP reads the filter turned by 180 degrees: the stride-1 data
// gradient.
// ---------------------------------------------------------------------------
template <int DT, int F, int TMW, bool FLIP, bool PRO = false>
__global__ __launch_bounds__(kBlockThreads) void fwd_sweep(SweepArgs a) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int SPAN = TMW + F - 1;
  constexpr int NB = kSweepBufs;
  constexpr int L = lcm_c(F, NB);
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int item = xcd_logical_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wave;
  if (item >= a.num_items) return;
  int t = item;
  const int tw = t % a.tiles_w;
  t /= a.tiles_w;
  const int rc = t % a.cpi;
  t /= a.cpi;
  const int cb = t % a.cbg;
  const int n = t / a.cbg;
  const int c = cb * kWaveChannels + lane;
  const uint32_t Cb = (uint32_t)a.C * EB;
  const char* img = (const char*)a.in + (size_t)n * a.IH * a.IW * Cb;
  const int ow0 = tw * TMW;
  const int o_start = rc * a.R;
  const int o_cnt = uniform(a.OH - o_start < a.R ? a.OH - o_start : a.R);
  const int iw0 = ow0 - a.PW;
  // Odd chunks walk up from their last row: neighbouring chunks then reach
  // the F-1 input rows they share at the same time and the second read
  // hits L2.  Walking up is the same ring with the filter rows reversed:
  // step i reads input row i_first + dir * i and output row o_rel is
  // o_first + dir * o_rel.
  const bool up = (rc & 1) != 0;
  const int dir = up ? -1 : 1;
  const int i_first = uniform(up ? o_start + o_cnt - 1 - a.P + F - 1 : o_start - a.P);
  const int o_first = up ? o_start + o_cnt - 1 : o_start;

  uint32_t coff[SPAN];
  column_offsets<SPAN>(coff, iw0, a.IW, Cb, c, a.C, EB);
  float ps = 1.f, pb = 0.f;  // this lane's prologue scale and shift
  if constexpr (PRO) {
    if (c < a.C) {
      ps = a.pro.scale[c];
      pb = a.pro.shift[c];
    }
  }
  float xb[NB][SPAN];
  load_strip<DT, SPAN>(xb[0], img, i_first, a.IH, iw0, a.IW, Cb, coff);
  load_strip<DT, SPAN>(xb[1], img, i_first + dir, a.IH, iw0, a.IW, Cb, coff);

  float wv[F][F];
  {
    const auto wrs = make_rsrc(a.in2, (uint32_t)(F * F) * Cb);
    const uint32_t voff = c < a.C ? (uint32_t)c * EB : kOOB;
#pragma unroll
    for (int fh = 0; fh < F; ++fh)
#pragma unroll
      for (int fw = 0; fw < F; ++fw) {
        const int fr = up ? F - 1 - fh : fh;  // filter row of ring offset fh
        const int e = FLIP ? (F - 1 - fr) * F + (F - 1 - fw) : fr * F + fw;
        wv[fh][fw] = ld<DT>(wrs, voff, (uint32_t)e * Cb);
      }
  }
  uint32_t ooff[TMW];  // output pixel offsets within a row, from column ow0
#pragma unroll
  for (int q = 0; q < TMW; ++q)
    ooff[q] = (ow0 + q < a.OW && c < a.C) ? (uint32_t)(q * a.C + c) * 4u : kOOB;
  float acc[F][TMW];  // ring: slot s holds output row o with o = s (mod F)
#pragma unroll
  for (int r = 0; r < F; ++r)
#pragma unroll
    for (int q = 0; q < TMW; ++q) acc[r][q] = 0.f;

  float* out_img = a.out + (size_t)n * a.OH * a.OW * a.C;
  const int steps = o_cnt + F - 1;  // input rows i_first + dir * (0 .. steps-1)
  for (int g = 0; g < steps; g += L) {
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const int i_rel = g + u;  // = u (mod F) and (mod NB)
      if (i_rel >= steps) break;
      load_strip<DT, SPAN>(xb[(u + 2) % NB], img, i_first + dir * (i_rel + 2), a.IH, iw0, a.IW, Cb,
                           coff);
      // the prologue runs on a row when it is used, after its loads arrive
      if constexpr (PRO)
        apply_prologue<SPAN>(xb[u % NB], i_first + dir * i_rel, a.IH, iw0, a.IW, ps, pb, a.pro);
      const float(&xv)[SPAN] = xb[u % NB];
      const bool row_in = (unsigned)(i_first + dir * i_rel) < (unsigned)a.IH;
#pragma unroll
      for (int fh = 0; fh < F; ++fh) {
        const int slot = ((u - fh) % F + F) % F;  // output row i_rel - fh
        // Only products of an image row with an output row of this chunk
        // count: padding rows add zero and the halo's rows are not stored
        // (a wave-uniform branch).
        if (!row_in || (unsigned)(i_rel - fh) >= (unsigned)o_cnt) continue;
#pragma unroll
        for (int fw = 0; fw < F; ++fw)
#pragma unroll
          for (int q = 0; q < TMW; ++q)
            acc[slot][q] = fmaf(xv[q + fw], wv[fh][fw], acc[slot][q]);
      }
      // Output row i_rel-F+1 has seen all F filter rows: store it (rows
      // outside [0, o_cnt) write nowhere) and free its slot.
      const int done = (u + 1) % F;
      const int o_rel = i_rel - (F - 1);
      const bool ok = o_rel >= 0 && o_rel < o_cnt;
      const float* orow = out_img + ((ptrdiff_t)(o_first + dir * o_rel) * a.OW + ow0) * a.C;
      const auto ors = make_rsrc(orow, ok ? (uint32_t)(TMW * a.C) * 4u : 0u);
#pragma unroll
      for (int q = 0; q < TMW; ++q) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[done][q]), ors, (int)ooff[q], 0, kStoreNT);
        acc[done][q] = 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Filter-gradient sweep kernel: stride 1, square filter F <= 9.
//
// A wave owns 64 channels x all F x F taps (registers) x one strip of TJ
// columns x one chunk of R consecutive dY rows of one image, and walks down
// the chunk.  Input rows are read in order, each once: input row i pairs
// with dY rows i-F+1 .. i (one per filter row), held in a ring of F
// register rows; each step does F*F*TJ FMAs on one input strip of TJ+F-1
// pixels and one new dY strip.  Both strips are loaded two steps ahead.
// The workgroup's 4 waves take 4 consecutive chunks of the same strip, add
// their taps through LDS in a fixed order, and write one partial per
// (strip, chunk group); reduce_partials sums the partials in order (the
// split of §5.1, deterministic).
// ---------------------------------------------------------------------------
template <int DT, int F, int TJ>
__global__ __launch_bounds__(kBlockThreads) void wgrad_sweep(SweepArgs a) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int SPAN = TJ + F - 1;
  constexpr int NB = kSweepBufs;
  constexpr int L = lcm_c(F, NB);
  __shared__ float red[2][F * F][64];
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_items) return;  // the whole workgroup leaves together
  int t = blk;
  const int s = t % a.tiles_w;
  t /= a.tiles_w;
  const int cb = t % a.cbg;
  const int cg = t / a.cbg;
  const int z = cg * a.tiles_w + s;
  const int c = cb * kWaveChannels + lane;
  const uint32_t Cb = (uint32_t)a.C * EB;
  const int chunk = cg * kWavesPerBlock + wave;
  int n = 0, rc = 0, o_start = 0, o_cnt = 0;
  if (chunk < a.N * a.cpi) {
    n = chunk / a.cpi;
    rc = chunk - n * a.cpi;
    o_start = rc * a.R;
    o_cnt = a.OH - o_start < a.R ? a.OH - o_start : a.R;
  }
  o_cnt = uniform(o_cnt);
  const int ow0 = s * TJ;
  const int iw0 = ow0 - a.PW;
  // Odd chunks walk up from their last row (see fwd_sweep): step i reads
  // input row i_first + dir * i and dY row o_first + dir * i, and ring
  // offset fh then stands for filter row F-1-fh.
  const bool up = (rc & 1) != 0;
  const int dir = up ? -1 : 1;
  const int i_first = uniform(up ? o_start + o_cnt - 1 - a.P + F - 1 : o_start - a.P);
  const int o_first = up ? o_start + o_cnt - 1 : o_start;
  const char* ximg = (const char*)a.in + (size_t)n * a.IH * a.IW * Cb;
  const char* dimg = (const char*)a.in2 + (size_t)n * a.OH * a.OW * Cb;
  uint32_t doff[TJ], xoff[SPAN];
  column_offsets<TJ>(doff, ow0, a.OW, Cb, c, a.C, EB);
  column_offsets<SPAN>(xoff, iw0, a.IW, Cb, c, a.C, EB);
  auto drow = [&](int i) { return i < o_cnt ? o_first + dir * i : -1; };  // dY row of step i

  float xb[NB][SPAN], db[NB][TJ];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    load_strip<DT, SPAN>(xb[k], ximg, i_first + dir * k, a.IH, iw0, a.IW, Cb, xoff);
    load_strip<DT, TJ>(db[k], dimg, drow(k), a.OH, ow0, a.OW, Cb, doff);
  }
  float acc[F][F];
  float dv[F][TJ];  // ring: slot s holds dY row o with o = s (mod F)
#pragma unroll
  for (int k = 0; k < F; ++k) {
#pragma unroll
    for (int fw = 0; fw < F; ++fw) acc[k][fw] = 0.f;
#pragma unroll
    for (int q = 0; q < TJ; ++q) dv[k][q] = 0.f;
  }

  const int steps = o_cnt > 0 ? o_cnt + F - 1 : 0;
  for (int g = 0; g < steps; g += L) {
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const int i_rel = g + u;  // = u (mod F) and (mod NB)
      if (i_rel >= steps) break;
      load_strip<DT, SPAN>(xb[(u + 2) % NB], ximg, i_first + dir * (i_rel + 2), a.IH, iw0, a.IW, Cb,
                           xoff);
      load_strip<DT, TJ>(db[(u + 2) % NB], dimg, drow(i_rel + 2), a.OH, ow0, a.OW, Cb, doff);
#pragma unroll
      for (int q = 0; q < TJ; ++q) dv[u % F][q] = db[u % NB][q];  // newest dY row: o = i_rel
      const float(&xv)[SPAN] = xb[u % NB];
      const bool row_in = (unsigned)(i_first + dir * i_rel) < (unsigned)a.IH;
#pragma unroll
      for (int fh = 0; fh < F; ++fh) {
        const int slot = ((u - fh) % F + F) % F;  // dY row i_rel - fh
        // Only an image row times a dY row of this chunk adds anything
        // (a wave-uniform branch).
        if (!row_in || (unsigned)(i_rel - fh) >= (unsigned)o_cnt) continue;
#pragma unroll
        for (int q = 0; q < TJ; ++q)
#pragma unroll
          for (int fw = 0; fw < F; ++fw) acc[fh][fw] = fmaf(xv[q + fw], dv[slot][q], acc[fh][fw]);
      }
    }
  }

  if (up) {  // ring offset k held filter row F-1-k
#pragma unroll
    for (int k = 0; k < F / 2; ++k)
#pragma unroll
      for (int fw = 0; fw < F; ++fw) {
        const float v = acc[k][fw];
        acc[k][fw] = acc[F - 1 - k][fw];
        acc[F - 1 - k][fw] = v;
      }
  }

  // (w0 + w2) + (w1 + w3), then one store of the partial.
  if (wave >= 2) {
#pragma unroll
    for (int k = 0; k < F; ++k)
#pragma unroll
      for (int fw = 0; fw < F; ++fw) red[wave - 2][k * F + fw][lane] = acc[k][fw];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int k = 0; k < F; ++k)
#pragma unroll
      for (int fw = 0; fw < F; ++fw) acc[k][fw] += red[wave][k * F + fw][lane];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int k = 0; k < F; ++k)
#pragma unroll
      for (int fw = 0; fw < F; ++fw) red[0][k * F + fw][lane] = acc[k][fw];
  }
  __syncthreads();
  if (wave == 0 && c < a.C) {
    float* ws = a.out + (size_t)z * F * F * a.C + c;
#pragma unroll
    for (int k = 0; k < F; ++k)
#pragma unroll
      for (int fw = 0; fw < F; ++fw)
        ws[((size_t)k * F + fw) * a.C] = acc[k][fw] + red[0][k * F + fw][lane];
  }
}

// ---------------------------------------------------------------------------
// Filter-gradient sweep with hybrid accumulation (Flash-DWC §5.1, "hybrid
// accumulation"; fp16 operands only).  The same walk as wgrad_sweep, but the
// operands stay fp16 and each step accumulates into fp16 sub-unit sums with
// packed FMAs (two adjacent taps fw, fw+1 per instruction, exact products
// and one rounding per FMA).  Every HS input rows -- at most 63 products
// per tap -- the fp16 sums are added into fp32 accumulators and cleared, so
// rounding error grows only within a short sub-unit; the cross-wave
// reduction and the partials are fp32 as in wgrad_sweep.  An fp16 sub-unit
// sum can overflow (|sum| > 65504) where fp32 would not: the option is for
// activations and gradients of ordinary magnitude.
// ---------------------------------------------------------------------------
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

template <int SPAN>
__device__ __forceinline__ void load_strip_h(_Float16 (&v)[SPAN], const char* img, int row,
                                             int rows, int col0, int cols, uint32_t pix_bytes,
                                             const uint32_t (&o)[SPAN]) {
  const bool row_ok = (unsigned)row < (unsigned)rows;
  const char* base = img + ((ptrdiff_t)row * cols + col0) * (ptrdiff_t)pix_bytes;
  const auto r = make_rsrc(base, row_ok ? (uint32_t)SPAN * pix_bytes : 0u);
#pragma unroll
  for (int j = 0; j < SPAN; ++j)
    v[j] = __builtin_bit_cast(_Float16, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(
                                            r, (int)o[j], 0, 0));
}

template <int F, int TJ>
__global__ __launch_bounds__(kBlockThreads) void wgrad_sweep_hyb(SweepArgs a) {
  constexpr int EB = 2;
  constexpr int SPAN = TJ + F - 1;
  constexpr int NB = kSweepBufs;
  constexpr int L = lcm_c(F, NB);
  constexpr int HP = (F + 1) / 2;   // tap pairs per filter row
  constexpr int HS = 63 / TJ;       // input rows per fp16 sub-unit
  __shared__ float red[2][F * F][64];
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_items) return;  // the whole workgroup leaves together
  int t = blk;
  const int s = t % a.tiles_w;
  t /= a.tiles_w;
  const int cb = t % a.cbg;
  const int cg = t / a.cbg;
  const int z = cg * a.tiles_w + s;
  const int c = cb * kWaveChannels + lane;
  const uint32_t Cb = (uint32_t)a.C * EB;
  const int chunk = cg * kWavesPerBlock + wave;
  int n = 0, rc = 0, o_start = 0, o_cnt = 0;
  if (chunk < a.N * a.cpi) {
    n = chunk / a.cpi;
    rc = chunk - n * a.cpi;
    o_start = rc * a.R;
    o_cnt = a.OH - o_start < a.R ? a.OH - o_start : a.R;
  }
  o_cnt = uniform(o_cnt);
  const int ow0 = s * TJ;
  const int iw0 = ow0 - a.PW;
  // odd chunks walk up from their last row (see wgrad_sweep)
  const bool up = (rc & 1) != 0;
  const int dir = up ? -1 : 1;
  const int i_first = uniform(up ? o_start + o_cnt - 1 - a.P + F - 1 : o_start - a.P);
  const int o_first = up ? o_start + o_cnt - 1 : o_start;
  const char* ximg = (const char*)a.in + (size_t)n * a.IH * a.IW * Cb;
  const char* dimg = (const char*)a.in2 + (size_t)n * a.OH * a.OW * Cb;
  uint32_t doff[TJ], xoff[SPAN];
  column_offsets<TJ>(doff, ow0, a.OW, Cb, c, a.C, EB);
  column_offsets<SPAN>(xoff, iw0, a.IW, Cb, c, a.C, EB);
  auto drow = [&](int i) { return i < o_cnt ? o_first + dir * i : -1; };

  _Float16 xb[NB][SPAN], db[NB][TJ];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    load_strip_h<SPAN>(xb[k], ximg, i_first + dir * k, a.IH, iw0, a.IW, Cb, xoff);
    load_strip_h<TJ>(db[k], dimg, drow(k), a.OH, ow0, a.OW, Cb, doff);
  }
  float acc[F][F];
  h2_t hacc[F][HP];
  _Float16 dv[F][TJ];  // ring: slot s holds dY row o with o = s (mod F)
#pragma unroll
  for (int k = 0; k < F; ++k) {
#pragma unroll
    for (int fw = 0; fw < F; ++fw) acc[k][fw] = 0.f;
#pragma unroll
    for (int j = 0; j < HP; ++j) hacc[k][j] = h2_t{(_Float16)0.f, (_Float16)0.f};
#pragma unroll
    for (int q = 0; q < TJ; ++q) dv[k][q] = (_Float16)0.f;
  }
  auto merge = [&]() {  // fp16 sub-unit sums into the fp32 accumulators
#pragma unroll
    for (int k = 0; k < F; ++k)
#pragma unroll
      for (int j = 0; j < HP; ++j) {
        acc[k][2 * j] += (float)hacc[k][j].x;
        if (2 * j + 1 < F) acc[k][2 * j + 1] += (float)hacc[k][j].y;
        hacc[k][j] = h2_t{(_Float16)0.f, (_Float16)0.f};
      }
  };

  const int steps = o_cnt > 0 ? o_cnt + F - 1 : 0;
  for (int g = 0; g < steps; g += L) {
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const int i_rel = g + u;
      if (i_rel >= steps) break;
      load_strip_h<SPAN>(xb[(u + 2) % NB], ximg, i_first + dir * (i_rel + 2), a.IH, iw0, a.IW, Cb,
                         xoff);
      load_strip_h<TJ>(db[(u + 2) % NB], dimg, drow(i_rel + 2), a.OH, ow0, a.OW, Cb, doff);
#pragma unroll
      for (int q = 0; q < TJ; ++q) dv[u % F][q] = db[u % NB][q];
      const _Float16(&xv)[SPAN] = xb[u % NB];
      const bool row_in = (unsigned)(i_first + dir * i_rel) < (unsigned)a.IH;
#pragma unroll
      for (int fh = 0; fh < F; ++fh) {
        const int slot = ((u - fh) % F + F) % F;
        if (!row_in || (unsigned)(i_rel - fh) >= (unsigned)o_cnt) continue;
#pragma unroll
        for (int q = 0; q < TJ; ++q) {
          const h2_t d2 = h2_t{dv[slot][q], dv[slot][q]};
#pragma unroll
          for (int j = 0; j < HP; ++j) {
            const h2_t x2 = h2_t{xv[q + 2 * j], 2 * j + 1 < F ? xv[q + 2 * j + 1] : (_Float16)0.f};
            hacc[fh][j] = x2 * d2 + hacc[fh][j];
          }
        }
      }
      if ((i_rel + 1) % HS == 0) merge();
    }
  }
  merge();
  if (up) {  // ring offset k held filter row F-1-k
#pragma unroll
    for (int k = 0; k < F / 2; ++k)
#pragma unroll
      for (int fw = 0; fw < F; ++fw) {
        const float v = acc[k][fw];
        acc[k][fw] = acc[F - 1 - k][fw];
        acc[F - 1 - k][fw] = v;
      }
  }

  // (w0 + w2) + (w1 + w3), then one store of the partial (as wgrad_sweep).
  if (wave >= 2) {
#pragma unroll
    for (int k = 0; k < F; ++k)
#pragma unroll
      for (int fw = 0; fw < F; ++fw) red[wave - 2][k * F + fw][lane] = acc[k][fw];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int k = 0; k < F; ++k)
#pragma unroll
      for (int fw = 0; fw < F; ++fw) acc[k][fw] += red[wave][k * F + fw][lane];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int k = 0; k < F; ++k)
#pragma unroll
      for (int fw = 0; fw < F; ++fw) red[0][k * F + fw][lane] = acc[k][fw];
  }
  __syncthreads();
  if (wave == 0 && c < a.C) {
    float* ws = a.out + (size_t)z * F * F * a.C + c;
#pragma unroll
    for (int k = 0; k < F; ++k)
#pragma unroll
      for (int fw = 0; fw < F; ++fw)
        ws[((size_t)k * F + fw) * a.C] = acc[k][fw] + red[0][k * F + fw][lane];
  }
}

// ---------------------------------------------------------------------------
// Generic kernels: one output element per lane, any filter size and stride.
// Element index i runs channel-fastest, so a wave reads 64 consecutive
// channels of one pixel.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float load_at(const void* p, int64_t i) {
  if constexpr (DT == DT_F32) {
    return ((const float*)p)[i];
  } else if constexpr (DT == DT_BF16) {
    return __uint_as_float((uint32_t)((const unsigned short*)p)[i] << 16);
  } else if constexpr (DT == DT_F16) {
    return (float)((const _Float16*)p)[i];
  } else {
    return fp8_to_f32<DT>(((const unsigned char*)p)[i]);
  }
}

// Forward map, or (FLIP) the stride-1 data gradient as the forward map of dY
// with the rotated filter and padding FH-1-ph.
template <int DT, bool FLIP>
__global__ __launch_bounds__(256) void fwd_generic(GenericArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.total) return;
  const int c = (int)(i % a.C);
  int64_t p = i / a.C;
  const int ow = (int)(p % a.OW);
  p /= a.OW;
  const int oh = (int)(p % a.OH);
  const int64_t n = p / a.OH;
  float s = 0.f;
  for (int fh = 0; fh < a.FH; ++fh) {
    const int ih = oh * a.SH - a.PH + fh;
    if (ih < 0 || ih >= a.IH) continue;
    const int fhe = FLIP ? a.FH - 1 - fh : fh;
    for (int fw = 0; fw < a.FW; ++fw) {
      const int iw = ow * a.SW - a.PW + fw;
      if (iw < 0 || iw >= a.IW) continue;
      const int fwe = FLIP ? a.FW - 1 - fw : fw;
      s = fmaf(load_at<DT>(a.a, ((n * a.IH + ih) * a.IW + iw) * a.C + c),
               load_at<DT>(a.b, ((int64_t)fhe * a.FW + fwe) * a.C + c), s);
    }
  }
  store_nt(&a.out[i], s);
}

// Data gradient for any stride: every (tap, output) pair whose window reads
// input pixel (ih, iw).  IH/IW are the input (dX) dims, OH/OW the dY dims.
template <int DT>
__global__ __launch_bounds__(256) void dgrad_generic(GenericArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.total) return;
  const int c = (int)(i % a.C);
  int64_t p = i / a.C;
  const int iw = (int)(p % a.IW);
  p /= a.IW;
  const int ih = (int)(p % a.IH);
  const int64_t n = p / a.IH;
  float s = 0.f;
  for (int fh = 0; fh < a.FH; ++fh) {
    const int th = ih + a.PH - fh;
    if (th < 0 || th % a.SH) continue;
    const int oh = th / a.SH;
    if (oh >= a.OH) continue;
    for (int fw = 0; fw < a.FW; ++fw) {
      const int tw = iw + a.PW - fw;
      if (tw < 0 || tw % a.SW) continue;
      const int ow = tw / a.SW;
      if (ow >= a.OW) continue;
      s = fmaf(load_at<DT>(a.a, ((n * a.OH + oh) * a.OW + ow) * a.C + c),
               load_at<DT>(a.b, ((int64_t)fh * a.FW + fw) * a.C + c), s);
    }
  }
  store_nt(&a.out[i], s);
}

// Filter gradient partials: work item (z, fh, fw, c), channel fastest; the
// item sums X * dY over the rows of slice z.
template <int DT>
__global__ __launch_bounds__(256) void wgrad_generic(GenericArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.total) return;
  const int c = (int)(i % a.C);
  int64_t p = i / a.C;
  const int fw = (int)(p % a.FW);
  p /= a.FW;
  const int fh = (int)(p % a.FH);
  const int z = (int)(p / a.FH);
  const int q0 = a.rows / a.Z, rem = a.rows % a.Z;
  const int r0 = z * q0 + (z < rem ? z : rem);
  const int r1 = r0 + q0 + (z < rem ? 1 : 0);
  float s = 0.f;
  for (int row = r0; row < r1; ++row) {
    const int64_t n = row / a.OH;
    const int oh = row - (int)n * a.OH;
    const int ih = oh * a.SH - a.PH + fh;
    if (ih < 0 || ih >= a.IH) continue;
    for (int ow = 0; ow < a.OW; ++ow) {
      const int iw = ow * a.SW - a.PW + fw;
      if (iw < 0 || iw >= a.IW) continue;
      s = fmaf(load_at<DT>(a.a, ((n * a.IH + ih) * a.IW + iw) * a.C + c),
               load_at<DT>(a.b, ((n * a.OH + oh) * a.OW + ow) * a.C + c), s);
    }
  }
  store_nt(&a.out[i], s);
}

}  // namespace dwc
