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
  // image rows [r_lo, r_hi) feed this block: image row ir sits at LDS row
  // ir - r_lo + 1, between the zero rows 0 and nrow + 1 that stand for
  // every row above and below
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

  // ---- filter taps: 16-byte loads (16 channels of one tap) of
  // kMfma8Batch taps per thread.  The first batch is issued before the input
  // tile's loads, so the two wait for memory together; the taps go into
  // their zero-padded fragment rows (turned by 180 degrees for FLIP) after
  // the barrier that ends the zero fill.
  const auto frsrc = make_rsrc(a.filt, (uint32_t)(FH * FW) * (uint32_t)a.C);
  const int ftaps = FH * FW;
  auto load_taps = [&](int i0, mf8_u32x4 (&v)[kMfma8Batch]) {
#pragma unroll
    for (int b = 0; b < kMfma8Batch; ++b) {
      if (i0 + b * NT >= ftaps) break;  // uniform: no tap left in this batch
      const int te = i0 + b * NT + tid;  // staged tap (fh, fw)
      const int src = FLIP ? ftaps - 1 - te : te;
      const uint32_t off = te < ftaps ? (uint32_t)src * (uint32_t)a.C + (uint32_t)c0 : kOOB;
      v[b] = __builtin_bit_cast(mf8_u32x4,
                                __builtin_amdgcn_raw_buffer_load_b128(frsrc, (int)off, 0, 0));
    }
  };
  auto store_taps = [&](int i0, const mf8_u32x4 (&v)[kMfma8Batch]) {
#pragma unroll
    for (int b = 0; b < kMfma8Batch; ++b) {
      if (i0 + b * NT >= ftaps) break;
      const int te = i0 + b * NT + tid;
      if (te >= ftaps) continue;
      const int fh = fast_div(te, a.fw_magic), fw = te - fh * FW;
      const int f = fw >> 4;
      const int zstep = FHP * NF * kZ8Row;  // bytes from one channel's rows to the next
      unsigned char* d = zt + (fh * NF + f) * kZ8Row + 16 + fw - 16 * f;
#pragma unroll
      for (int j = 0; j < 16; ++j, d += zstep)
        *d = (unsigned char)(v[b][j >> 2] >> (8 * (j & 3)));
    }
  };
  mf8_u32x4 fv0[kMfma8Batch];
  load_taps(0, fv0);

  // ---- zero the filter-fragment rows (taps are written after a barrier)
  for (int i = tid; i < zlen / 16; i += NT) ((mf8_u32x4*)zt)[i] = mf8_u32x4{0u, 0u, 0u, 0u};

  // ---- stage the input tile: LDS rows 0 .. nrow + 1 (0 and nrow + 1 are
  // zeros), wt columns from -PW.
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
    // byte offset of LDS row r's pixel quad is (r_lo + r - 1) * rowb + col0;
    // LDS dwords of row r start at dst0 + r * (WP / 4).  Both advance by
    // fixed steps from row to row.
    const uint32_t row_step = (uint32_t)rs * rowb;
    uint32_t off_rb = (uint32_t)(r_lo + r0 - 1) * rowb + col0;
    for (int rb = r0; rb <= nrow + 1; rb += rs * kMfma8Batch, off_rb += kMfma8Batch * row_step) {
      mf8_u32x4 v[kMfma8Batch][4];
#pragma unroll
      for (int b = 0; b < kMfma8Batch; ++b) {
        const int r = rb + b * rs;  // LDS row
        const bool rok = r >= 1 && r <= nrow;
        const uint32_t off = off_rb + (uint32_t)b * row_step;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[b][i] = __builtin_bit_cast(
              mf8_u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                             rsrc, (int)(rok && ok[i] ? off + (uint32_t)i * Cb : kOOB), 0, 0));
      }
#pragma unroll
      for (int b = 0; b < kMfma8Batch; ++b) {
        const int r = rb + b * rs;
        if (r > nrow + 1 || !e_in) continue;
        uint32_t* d = dst0 + rb * (WP / 4) + b * (rs * (WP / 4));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t ch[4];
          transpose4(v[b][0][w], v[b][1][w], v[b][2][w], v[b][3][w], ch);
#pragma unroll
          for (int i = 0; i < 4; ++i, d += plane4) *d = ch[i];
        }
      }
    }
  }
  __syncthreads();  // zt is zero
  store_taps(0, fv0);
  for (int i0 = NT * kMfma8Batch; i0 < ftaps; i0 += NT * kMfma8Batch) {
    mf8_u32x4 v[kMfma8Batch];
    load_taps(i0, v);
    store_taps(i0, v);
  }
  __syncthreads();

  // ---- compute.  Lane (s, m): K slice s (filter row 4h + s of the
  // instruction's four); A row m, B column m; D: lane (s, j) holds
  // D[4s .. 4s+3][j].  The wave's CPW channels run together.
  const int s = lane >> 4, m = lane & 15;
  const int RT = 1 << a.rt_log;
  const int gA = m >> a.rt_log, rA = m & (RT - 1);
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
  // A of tile tt in row group h is staged row tt * RT + rA + s + 4h, at
  // byte offset clamp((s_top - r_lo + 1 + row) * WP, 0, (nrow + 1) * WP) of
  // the channel's plane: rows above the image clamp to zero row 0, rows
  // below to zero row nrow + 1.
  const int top_b = (nrow + 1) * WP;
  const int a0 = (s_top - r_lo + 1 + rA + s) * WP;
  auto read_a = [&](int k, int tt, int f, int h) -> mf8_i32x8 {
    const int o = min(max(a0 + (tt * RT + 4 * h) * WP, 0), top_b);
    const mf8_u32x4* p = (const mf8_u32x4*)(xbase + k * XR * WP + o + 16 * f);
    const mf8_u32x4 lo = p[0], hi = p[1];
    return mf8_i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  constexpr int TD = TILES / 2;  // tiles whose A moves by DPP row shifts
  mf8_f32x4 acc[CPW][TILES];
  mf8_i32x8 A[CPW][TILES][NF];
  mf8_i32x8 B[CPW][NF];
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) {
      acc[k][tt] = mf8_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < NF; ++f) A[k][tt][f] = read_a(k, tt, f, 0);
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
    // Tiles below TD move A down four combinations with DPP row shifts and
    // reload the last four of each row group; tiles from TD on read all of
    // A again from LDS (eight DPP instructions per MFMA alone take longer
    // to issue than the MFMA; a full re-read costs 2 KB of LDS bandwidth).
#pragma unroll
    for (int k = 0; k < CPW; ++k)
#pragma unroll
      for (int tt = 0; tt < TD; ++tt)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int v = 0; v < 8; ++v) A[k][tt][f][v] = row_shift_down4(A[k][tt][f][v]);
    if (reload) {
#pragma unroll
      for (int tt = 0; tt < TD; ++tt)
#pragma unroll
        for (int k = 0; k < CPW; ++k)
#pragma unroll
          for (int f = 0; f < NF; ++f) A[k][tt][f] = read_a(k, tt, f, h + 1);
    }
#pragma unroll
    for (int tt = TD; tt < TILES; ++tt)
#pragma unroll
      for (int k = 0; k < CPW; ++k)
#pragma unroll
        for (int f = 0; f < NF; ++f) A[k][tt][f] = read_a(k, tt, f, h + 1);
  }

  // ---- outputs: registers -> LDS [pixel][channel] -> channel-contiguous stores
  __syncthreads();  // every wave is done with the staged operands
  // Lane (s, m) holds row mm = 4s + r of every tile at column m: output
  // row tt * RT + (mm mod RT), column 16 (mm / RT) + m.  One address and one
  // bounds test per mm; tiles and the wave's channels are fixed offsets.
  {
    const int tile_step = RT * a.OW * OSP;  // floats from one tile to the next
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = 4 * s + r;
      const int ow = 16 * (mm >> a.rt_log) + m;
      if (ow < a.OW) {
        float* p = os + ((mm & (RT - 1)) * a.OW + ow) * OSP + wave * CPW;
#pragma unroll
        for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
          for (int k = 0; k < CPW; ++k) p[tt * tile_step + k] = acc[k][tt][r];
      }
    }
  }
  __syncthreads();
  // The block's output rows are consecutive, so staged pixel p is output
  // pixel oh0 * OW + p.  Thread tid keeps one 16-byte channel quad sq of
  // pixels pt, pt + PSTEP, ...
  {
    constexpr int QU = CB / 4;      // channel quads per pixel
    constexpr int PSTEP = NT / QU;  // pixels per pass of the workgroup
    const int rows = a.OH - oh0 < a.rblk ? a.OH - oh0 : a.rblk;
    const int npix = rows * a.OW;
    const int sq = tid % QU, pt = tid / QU;
    const bool c_ok = c0 + 4 * sq < a.C;
    const float* src = os + pt * OSP + 4 * sq;
    float* dst = a.out + ((size_t)n * a.OH * a.OW + (size_t)oh0 * a.OW + pt) * a.C + c0 + 4 * sq;
    for (int p0 = 0; p0 < npix; p0 += PSTEP * kMfma8Batch) {
      mf8_f32x4 v[kMfma8Batch];
#pragma unroll
      for (int b = 0; b < kMfma8Batch; ++b) {
        const int pb = p0 + b * PSTEP;  // uniform
        v[b] = pb + pt < npix ? *(const mf8_f32x4*)(src + pb * OSP) : mf8_f32x4{};
      }
#pragma unroll
      for (int b = 0; b < kMfma8Batch; ++b) {
        const int pb = p0 + b * PSTEP;
        if (pb + pt < npix && c_ok) store_nt((mf8_f32x4*)(dst + (size_t)pb * a.C), v[b]);
      }
    }
  }
}

}  // namespace dwc

namespace dwc {

// ---------------------------------------------------------------------------
// Packed fp8 MFMA filter gradient (e4m3 / e5m2 operands, stride 1).
//
// The 16x16x32 product of the 16-bit filter-gradient kernel (A: the band of
// one zero-padded dY row, 16 taps fw x 32 columns; B: 16 consecutive input
// rows fh over the same 32 columns), four output rows side by side along
// the fp8 MFMA's K = 128:
//   A[m][32 s + k] = dY[oh + s][32 kc + k - (16 fm + m) + pw]
//   B[32 s + k][n] = X[oh + s + 16 fn + n - ph][32 kc + k]
//   D[m][n] += contributions to dW[16 fn + n][16 fm + m] of output rows
//              oh .. oh + 3 (rows past OH are zero rows of the staged dY)
// K slice s (lanes 16 s .. 16 s + 15) holds output row oh + s.  A is read
// like the forward kernel's filter band: nine dwords from the dword at or
// below the lane's first byte, shifted by v_alignbit.  B moves down four
// rows per step: a DPP row shift by four lanes, the last four lanes of each
// row group reading LDS again.  A workgroup owns kWgmCb channels (one per
// wave) and a slice of ipb images, stages each image's X and dY rows in LDS
// channel-major (one dword = four columns of one channel), and writes the
// same channel-blocked partial as the 16-bit kernel.
// ---------------------------------------------------------------------------
template <int DT, int NFM, int NFN, int NK, int PF>
__global__ __launch_bounds__(64 * kMfmaWaves, wgm8_waves_per_eu(PF)) void wgrad_mfma8(
    WgradMfmaArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int NT = 64 * kMfmaWaves;
  constexpr int CB = kWgmCb;
  static_assert(CB == kMfmaWaves, "one channel per wave");
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_blocks) return;  // the whole workgroup leaves together
  const int cbk = blk % a.cblk;
  const int z = blk / a.cblk;
  const int n0 = z * a.ipb;
  const int n1 = n0 + a.ipb < a.N ? n0 + a.ipb : a.N;
  const int c0 = cbk * CB;
  const int XR = a.xr, XP = a.xp, DYP = a.dyp, OH = a.OH;
  const int OHP = 4 * ((OH + 3) / 4);  // staged dY rows: whole groups of four
  const int taps = a.FH * a.FW;
  unsigned char* xs = lds;              // [CB][XR][XP]
  unsigned char* dz = xs + CB * XR * XP;  // [CB][OHP][DYP]
  float* pst = (float*)lds;             // [taps][CB], after the last image
  const uint32_t Cb = (uint32_t)a.C;    // bytes per pixel

  // ---- zero both staging regions once: per image only the pixels of the
  // image are written, so the zero row, the columns past the image, the dY
  // padding and the dY rows past OH stay zero for every image of the slice
  {
    const int units = CB * (XR * XP + OHP * DYP) / 16;
    for (int i = tid; i < units; i += NT) ((mf8_u32x4*)lds)[i] = mf8_u32x4{0u, 0u, 0u, 0u};
  }

  // ---- this thread's staging items, the same for every image: item i of
  // X is the column quad (4e .. 4e+3) of row r; item i of dY is the staged
  // column quad e, i.e. dY columns 4e - dpad .. 4e + 3 - dpad.  Byte
  // offsets of the four pixels within the image (kOOB: zero) and the LDS
  // dword of channel 0 (-1: no item).
  uint32_t xo[PF][4], dof[PF][4];
  int xw[PF], dw[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int i = tid + k * NT;
    xw[k] = dw[k] = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) xo[k][j] = dof[k][j] = kOOB;
    if (i < a.ix) {
      const int r = i / a.hx, e = i - r * a.hx;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * e + j < a.IW) xo[k][j] = (uint32_t)(r * a.IW + 4 * e + j) * Cb + (uint32_t)c0;
      xw[k] = ((r + 1) * XP) / 4 + e;
    }
    if (i < a.id) {
      const int r = i / a.hd, e = a.e_lo + (i - r * a.hd);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t0 = 4 * e + j - a.dpad;
        if ((unsigned)t0 < (unsigned)a.OW) dof[k][j] = (uint32_t)(r * a.OW + t0) * Cb + (uint32_t)c0;
      }
      dw[k] = (r * DYP) / 4 + e;
    }
  }
  u32x2 vx[PF][4], vd[PF][4];
  auto fetch = [&](int n) {  // global -> registers, in flight during compute
    const auto rx = make_rsrc((const char*)a.x + (size_t)n * a.IH * a.IW * Cb,
                              (uint32_t)(a.IH * a.IW) * Cb);
    const auto rd = make_rsrc((const char*)a.dy + (size_t)n * OH * a.OW * Cb,
                              (uint32_t)(OH * a.OW) * Cb);
#pragma unroll
    for (int k = 0; k < PF; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vx[k][j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rx, (int)xo[k][j], 0, 0));
        vd[k][j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rd, (int)dof[k][j], 0, 0));
      }
  };
  auto commit = [&]() {  // registers -> LDS, transposed to channel-major
    const int px = XR * XP / 4, pd = OHP * DYP / 4;  // dwords per channel plane
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      if (xw[k] >= 0) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          uint32_t ch[4];
          transpose4(vx[k][0][w], vx[k][1][w], vx[k][2][w], vx[k][3][w], ch);
#pragma unroll
          for (int i = 0; i < 4; ++i) ((uint32_t*)xs)[xw[k] + (4 * w + i) * px] = ch[i];
        }
      }
      if (dw[k] >= 0) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          uint32_t ch[4];
          transpose4(vd[k][0][w], vd[k][1][w], vd[k][2][w], vd[k][3][w], ch);
#pragma unroll
          for (int i = 0; i < 4; ++i) ((uint32_t*)dz)[dw[k] + (4 * w + i) * pd] = ch[i];
        }
      }
    }
  };

  // ---- per-lane constants.  Lane (s, m): K slice s (output row oh + s);
  // A row m, B column m; D: lane (s, j) holds D[4s .. 4s+3][j].
  const int s = lane >> 4, m = lane & 15;
  const int cc = wave;
  // A starts at staged dY byte 32 kc - 16 fm - m + pw + dpad of row oh + s
  const int ua = a.PW + a.dpad - m;
  const uint32_t ashift = (uint32_t)(ua & 3) * 8u;
  const uint32_t* dzl = (const uint32_t*)(dz + cc * OHP * DYP + s * DYP) + (ua >> 2);
  auto read_a = [&](int oh, int fm, int kc) -> mf8_i32x8 {
    const uint32_t* p = dzl + (oh * DYP + 32 * kc - 16 * fm) / 4;
    uint32_t d[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) d[i] = p[i];
    mf8_i32x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (int)__builtin_amdgcn_alignbit(d[i + 1], d[i], ashift);
    return r;
  };
  const unsigned char* xl = xs + cc * XR * XP;
  // LDS row of input row r: row 0 is zeros, image row r sits at r + 1
  auto x_row = [&](int r) -> int { return (unsigned)r < (unsigned)a.IH ? r + 1 : 0; };
  auto read_b = [&](int row, int kc) -> mf8_i32x8 {
    const mf8_u32x4* p = (const mf8_u32x4*)(xl + row * XP + 32 * kc);
    const mf8_u32x4 lo = p[0], hi = p[1];
    return mf8_i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  mf8_f32x4 acc[NFM][NFN];
#pragma unroll
  for (int fm = 0; fm < NFM; ++fm)
#pragma unroll
    for (int fn = 0; fn < NFN; ++fn) acc[fm][fn] = mf8_f32x4{0.f, 0.f, 0.f, 0.f};

  if (n0 < n1) fetch(n0);
  for (int n = n0; n < n1; ++n) {
    __syncthreads();  // the zero fill, or the previous image's reads, are done
    commit();
    __syncthreads();
    if (n + 1 < n1) fetch(n + 1);

    mf8_i32x8 A[NFM][NK], B[NFN][NK];
#pragma unroll
    for (int fn = 0; fn < NFN; ++fn) {
      const int row = x_row(s + 16 * fn + m - a.PH);
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) B[fn][kc] = read_b(row, kc);
    }
#pragma unroll
    for (int fm = 0; fm < NFM; ++fm)
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) A[fm][kc] = read_a(0, fm, kc);
    // One uniform body per group of four output rows: the operands of the
    // next group are formed in the last iteration too (from staged rows,
    // never used).
    for (int oh = 0; oh < OH; oh += 4) {
#pragma unroll
      for (int kc = 0; kc < NK; ++kc)
#pragma unroll
        for (int fm = 0; fm < NFM; ++fm)
#pragma unroll
          for (int fn = 0; fn < NFN; ++fn)
            acc[fm][fn] = mfma_f8<DT>(A[fm][kc], B[fn][kc], acc[fm][fn]);
      const int on = oh + 4 < OHP ? oh + 4 : oh;
#pragma unroll
      for (int fm = 0; fm < NFM; ++fm)
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) A[fm][kc] = read_a(on, fm, kc);
#pragma unroll
      for (int fn = 0; fn < NFN; ++fn)
#pragma unroll
        for (int kc = 0; kc < NK; ++kc)
#pragma unroll
          for (int v = 0; v < 8; ++v) B[fn][kc][v] = row_shift_down4(B[fn][kc][v]);
      if (m >= 12) {
#pragma unroll
        for (int fn = 0; fn < NFN; ++fn) {
          const int row = x_row(oh + 4 + s + 16 * fn + m - a.PH);
#pragma unroll
          for (int kc = 0; kc < NK; ++kc) B[fn][kc] = read_b(row, kc);
        }
      }
    }
  }

  // ---- the slice's partial: registers -> LDS [tap][channel] -> one
  // contiguous run of taps * CB floats
  __syncthreads();
#pragma unroll
  for (int fm = 0; fm < NFM; ++fm)
#pragma unroll
    for (int fn = 0; fn < NFN; ++fn)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int fw = 16 * fm + 4 * s + r, fh = 16 * fn + m;
        if (fw < a.FW && fh < a.FH) pst[(fh * a.FW + fw) * CB + cc] = acc[fm][fn][r];
      }
  __syncthreads();
  float* dst = a.ws + ((size_t)z * a.cblk + cbk) * taps * CB;
  for (int i = tid; i < taps * CB / 4; i += NT)
    *(mf8_f32x4*)(dst + 4 * i) = *(const mf8_f32x4*)(pst + 4 * i);
}

}  // namespace dwc
