// dwc_mfma8.h -- packed-MFMA forward-type kernel of libdwc for fp8 operands
// (OCP e4m3 / e5m2 codes; gfx950 v_mfma_f32_16x16x128_f8f6f4, fp32
// accumulation).
//
// Low-bit operands (Flash-DWC, TACO, §7, low-bit data types) on the
// GEMV-to-GEMM packing of §4.2 (Fig. 8).  The 16x16x32 form of the packing
// (one filter row and one 16-tap fragment per MFMA) carries over; the fp8
// matrix core takes K = 128 per instruction, so one MFMA here is four of
// those products side by side along K, one per filter row:
//   A[m][32 s + k] = x[row_m + s][16 g_m + 16 f + k - pw]   (s = 0..3, k < 32)
//   B[32 s + k][j] = w[4 h + s][16 f + k - j]  if 0 <= k - j < 16, else 0
//   D[m][j] += sum over s, k = rows 4h .. 4h+3 of fragment f of the filter
// so each of the ceil(FH / 4) MFMAs per fragment covers four filter rows
// (rows past FH are zero fragments).  The lanes of K slice s (lanes
// 16 s .. 16 s + 15) hold row s of the four: A is 32 consecutive staged
// columns of input row row_m + s, B the band of filter row 4h + s.
//
// Staging (channel-major, one byte per element, as in the 16-bit kernel):
//   * the input tile [c][row][col] with one shared zero row for every
//     padding row; the row pitch is an odd number of 16-byte units, so lanes
//     reading consecutive rows hit distinct banks;
//   * the filter in compact zero-padded fragment rows: per (channel, filter
//     row, fragment) 16 zero bytes then the 16 taps, rows padded to a
//     multiple of four with zeros; lane (s, j) takes bytes [16 - j, 48 - j)
//     of its row: nine dwords from the dword at or below, shifted by
//     v_alignbit in whole bytes;
//   * from filter rows 4h .. 4h+3 to 4h+4 .. 4h+7, combination (g, r) needs
//     the input row that (g, r + 4) used: a DPP row shift by four lanes moves
//     it, and only the last four rows of each group read LDS again.
// Zero padding of the image: out-of-image pixels read as 0 through the
// buffer resource's range check.
#pragma once

#include "dwc_device.h"

namespace dwc {

typedef int mf8_i32x8 __attribute__((ext_vector_type(8)));
typedef float mf8_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mf8_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfma8Batch = 4;  // staging items a thread keeps in flight

template <int DT>
__device__ __forceinline__ mf8_f32x4 mfma_f8(const mf8_i32x8& a, const mf8_i32x8& b,
                                             mf8_f32x4 c) {
  // operand format: 0 = e4m3, 1 = e5m2 (both operands alike); no scaling
  constexpr int fmt = DT == DT_E4M3 ? 0 : 1;
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, fmt, fmt, 0, 0, 0, 0);
}

// DPP row_shl:4 -- lane i of each 16-lane row takes the value of lane i+4;
// the last four lanes of a row keep their own value.
__device__ __forceinline__ int row_shift_down4(int v) {
  return __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0xF, false);
}

// Bytes (p0[j], p1[j], p2[j], p3[j]) of four 16-channel pixels, for
// channels j = 4 w .. 4 w + 3 of dword w: out[i] holds channel 4 w + i.
__device__ __forceinline__ void transpose4(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                           uint32_t (&out)[4]) {
  const uint32_t lo01 = __builtin_amdgcn_perm(p1, p0, 0x05010400u);  // p0b0 p1b0 p0b1 p1b1
  const uint32_t hi01 = __builtin_amdgcn_perm(p1, p0, 0x07030602u);  // p0b2 p1b2 p0b3 p1b3
  const uint32_t lo23 = __builtin_amdgcn_perm(p3, p2, 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(p3, p2, 0x07030602u);
  out[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// kMfma8Cb channels per workgroup of kMfmaWaves waves (two per wave), NF
// 16-tap fragments per filter row, TILES tiles of 16 combinations per
// channel.  FLIP stages the filter turned by 180 degrees: the stride-1 data
// gradient.  Geometry in MfmaArgs, in bytes (= elements).
template <int DT, int NF, int TILES, bool FLIP>
__global__ __launch_bounds__(64 * kMfmaWaves) void fwd_mfma8(MfmaArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int NT = 64 * kMfmaWaves;
  constexpr int CB = kMfma8Cb;
  constexpr int CPW = CB / kMfmaWaves;
  static_assert(CB % kMfmaWaves == 0, "whole channels per wave");
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_blocks) return;  // the whole workgroup leaves together
  int t = blk;
  const int rc = t % a.rch;
  t /= a.rch;
  const int cbk = t % a.cblk;
  const int n = t / a.cblk;
  const int c0 = cbk * CB;
  const int oh0 = rc * a.rblk;
  const int XR = a.xr, WP = a.wp;
  const int FH = a.FH, FW = a.FW;
  const int G4 = (FH + 3) / 4;  // MFMAs per fragment: four filter rows each
  const int FHP = 4 * G4;
  // image rows [r_lo, r_hi) feed this block; LDS row 0 is the zero row and
  // image row ir sits at LDS row ir - r_lo + 1
  const int s_top = oh0 - a.PH;  // image row of staged index 0
  const int r_lo = s_top > 0 ? s_top : 0;
  const int r_end = s_top + a.rblk + FH - 1;
  const int r_hi = r_end < a.IH ? r_end : a.IH;
  const int nrow = r_hi > r_lo ? r_hi - r_lo : 0;
  unsigned char* xs = lds;                           // [CB][XR][WP]
  unsigned char* zt = xs + CB * XR * WP;             // [CB][FHP][NF][kZ8Row] + tail
  float* os = (float*)lds;                           // [rblk * OW][CB + 4], after compute
  constexpr int OSP = CB + 4;
  const int zlen = (CB * FHP * NF + kZ8Tail) * kZ8Row;  // a multiple of 16

  // ---- zero the filter-fragment rows (taps are written after a barrier)
  for (int i = tid; i < zlen / 16; i += NT) ((mf8_u32x4*)zt)[i] = mf8_u32x4{0u, 0u, 0u, 0u};

  // ---- stage the input tile: LDS rows 0 .. nrow, wt columns from -PW.
  // Thread tid owns column quad e (4 pixels x 16 channels, four 16-byte
  // loads) of a row and visits every rs-th row, kMfma8Batch rows of loads
  // in flight before any LDS write.  LDS row 0 loads out of range: zeros.
  {
    const uint32_t Cb = (uint32_t)a.C;  // bytes per pixel
    const char* img = (const char*)a.in + (size_t)n * a.IH * a.IW * Cb;
    const auto rsrc = make_rsrc(img, (uint32_t)(a.IH * a.IW) * Cb);
    const int e = tid & (a.e2 - 1);
    const int r0 = tid >> a.e2_log;
    const int rs = NT >> a.e2_log;
    const int iw = 4 * e - a.PW;
    const bool e_in = e < a.e_items;
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ok[i] = e_in && (unsigned)(iw + i) < (unsigned)a.IW;
    const uint32_t col0 = (uint32_t)iw * Cb + (uint32_t)c0;
    const uint32_t rowb = (uint32_t)a.IW * Cb;
    const int plane4 = XR * WP / 4;  // dwords per channel plane
    uint32_t* dst0 = (uint32_t*)xs + e;
    for (int rb = r0; rb <= nrow; rb += rs * kMfma8Batch) {
      mf8_u32x4 v[kMfma8Batch][4];
#pragma unroll
      for (int b = 0; b < kMfma8Batch; ++b) {
        const int r = rb + b * rs;  // LDS row
        const bool rok = r >= 1 && r <= nrow;
        const uint32_t off = (uint32_t)(r_lo + r - 1) * rowb + col0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[b][i] = __builtin_bit_cast(
              mf8_u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                             rsrc, (int)(rok && ok[i] ? off + (uint32_t)i * Cb : kOOB), 0, 0));
      }
#pragma unroll
      for (int b = 0; b < kMfma8Batch; ++b) {
        const int r = rb + b * rs;
        if (r > nrow || !e_in) continue;
        uint32_t* d = dst0 + r * (WP / 4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t ch[4];
          transpose4(v[b][0][w], v[b][1][w], v[b][2][w], v[b][3][w], ch);
#pragma unroll
          for (int i = 0; i < 4; ++i) d[(4 * w + i) * plane4] = ch[i];
        }
      }
    }
  }
  __syncthreads();  // zt is zero
  // ---- filter taps into their fragment rows, turned by 180 degrees for FLIP
  {
    const auto rsrc = make_rsrc(a.filt, (uint32_t)(FH * FW) * (uint32_t)a.C);
    const int taps = FH * FW;
    for (int i0 = 0; i0 < taps; i0 += NT * kMfma8Batch) {
      mf8_u32x4 v[kMfma8Batch];
#pragma unroll
      for (int b = 0; b < kMfma8Batch; ++b) {
        const int te = i0 + b * NT + tid;  // staged tap (fh, fw)
        const int src = FLIP ? taps - 1 - te : te;
        const uint32_t off = te < taps ? (uint32_t)src * (uint32_t)a.C + (uint32_t)c0 : kOOB;
        v[b] = __builtin_bit_cast(mf8_u32x4,
                                  __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 0));
      }
#pragma unroll
      for (int b = 0; b < kMfma8Batch; ++b) {
        const int te = i0 + b * NT + tid;
        if (te >= taps) continue;
        const int fh = te / FW, fw = te - fh * FW;
        const int f = fw >> 4;
        unsigned char* d = zt + (fh * NF + f) * kZ8Row + 16 + fw - 16 * f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          d[j * FHP * NF * kZ8Row] = (unsigned char)(v[b][j >> 2] >> (8 * (j & 3)));
      }
    }
  }
  __syncthreads();

  // ---- compute.  Lane (s, m): K slice s (filter row 4h + s of the
  // instruction's four); A row m, B column m; D: lane (s, j) holds
  // D[4s .. 4s+3][j].  The wave's CPW channels run together.
  const int s = lane >> 4, m = lane & 15;
  const int RT = 16 / a.gt;
  const int gA = m / RT, rA = m % RT;
  const bool reload = rA >= RT - 4;
  const unsigned char* xbase = xs + (wave * CPW) * XR * WP + 16 * gA;
  // B: lane (s, j = m) reads bytes [16 - m, 48 - m) of its fragment row
  const int u0 = 16 - m;
  const uint32_t bshift = (uint32_t)(u0 & 3) * 8u;
  const uint32_t* zbase = (const uint32_t*)(zt + (wave * CPW) * FHP * NF * kZ8Row) + (u0 >> 2);
  auto read_b = [&](int k, int h, int f) -> mf8_i32x8 {
    const uint32_t* p = zbase + ((k * FHP + 4 * h + s) * NF + f) * (kZ8Row / 4);
    uint32_t d[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) d[i] = p[i];
    mf8_i32x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (int)__builtin_amdgcn_alignbit(d[i + 1], d[i], bshift);
    return r;
  };
  // LDS row of staged index si (image row s_top + si): the zero row outside
  // the image
  auto lds_row = [&](int si) -> int {
    const int ir = s_top + si;
    return (ir >= r_lo && ir < r_hi) ? ir - r_lo + 1 : 0;
  };
  auto read_a = [&](int k, int row, int f) -> mf8_i32x8 {
    const mf8_u32x4* p = (const mf8_u32x4*)(xbase + (k * XR + row) * WP + 16 * f);
    const mf8_u32x4 lo = p[0], hi = p[1];
    return mf8_i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  mf8_f32x4 acc[CPW][TILES];
  mf8_i32x8 A[CPW][TILES][NF];
  mf8_i32x8 B[CPW][NF];
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) {
      acc[k][tt] = mf8_f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = lds_row(tt * RT + rA + s);
#pragma unroll
      for (int f = 0; f < NF; ++f) A[k][tt][f] = read_a(k, row, f);
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) B[k][f] = read_b(k, 0, f);
  }
  // One uniform body per group of four filter rows: the operands of group
  // h+1 are formed in the last iteration too (from rows that exist, never
  // used), which keeps the accumulators in place across iterations.
  for (int h = 0; h < G4; ++h) {
#pragma unroll
    for (int k = 0; k < CPW; ++k)
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[k][tt] = mfma_f8<DT>(A[k][tt][f], B[k][f], acc[k][tt]);
    const int hn = h + 1 < G4 ? h + 1 : h;
#pragma unroll
    for (int k = 0; k < CPW; ++k)
#pragma unroll
      for (int f = 0; f < NF; ++f) B[k][f] = read_b(k, hn, f);
#pragma unroll
    for (int k = 0; k < CPW; ++k)
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int v = 0; v < 8; ++v) A[k][tt][f][v] = row_shift_down4(A[k][tt][f][v]);
    if (reload) {
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt) {
        const int row = lds_row(tt * RT + rA + s + 4 * (h + 1));
#pragma unroll
        for (int k = 0; k < CPW; ++k)
#pragma unroll
          for (int f = 0; f < NF; ++f) A[k][tt][f] = read_a(k, row, f);
      }
    }
  }

  // ---- outputs: registers -> LDS [pixel][channel] -> channel-contiguous stores
  __syncthreads();  // every wave is done with the staged operands
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
    const int cc = wave * CPW + k;
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mm = 4 * s + r;
        const int ol = tt * RT + mm % RT;
        const int ow = 16 * (mm / RT) + m;
        if (ow < a.OW) os[(ol * a.OW + ow) * OSP + cc] = acc[k][tt][r];
      }
  }
  __syncthreads();
  {
    constexpr int QU = CB / 4;
    const int items = a.rblk * a.OW * QU;
    float* out_img = a.out + (size_t)n * a.OH * a.OW * a.C;
    for (int i0 = 0; i0 < items; i0 += NT * kMfma8Batch) {
      mf8_f32x4 v[kMfma8Batch];
#pragma unroll
      for (int b = 0; b < kMfma8Batch; ++b) {
        const int i = i0 + b * NT + tid;
        const int p = i / QU;
        v[b] = i < items ? *(const mf8_f32x4*)(os + p * OSP + 4 * (i % QU)) : mf8_f32x4{};
      }
#pragma unroll
      for (int b = 0; b < kMfma8Batch; ++b) {
        const int i = i0 + b * NT + tid;
        const int q4 = i % QU;
        const int p = i / QU;
        const int oh = oh0 + p / a.OW;
        const int c = c0 + 4 * q4;
        if (i < items && oh < a.OH && c < a.C)
          *(mf8_f32x4*)(out_img + ((size_t)oh * a.OW + p % a.OW) * a.C + c) = v[b];
      }
    }
  }
}

}  // namespace dwc
