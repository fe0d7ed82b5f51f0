// dwc_mfma.h -- packed-MFMA forward-type kernel of libdwc for bf16/fp16
// operands (gfx950 v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulation).
//
// The GEMV-to-GEMM packing of Flash-DWC (§4.2 "Transforming GEMV into
// GEMM", Fig. 8), re-sized for the 16x16x32 CDNA4 MFMA.  Per channel, the
// 1-D convolution of one input row with one filter row is a product of two
// small matrices:
//   A[m][k] = x[row_m][16 g_m + 16 f + k - pw]   (16 x 32, input windows)
//   B[k][j] = w[fh][16 f + k - j]  if 0 <= k - j < 16, else 0   (32 x 16)
//   D[m][j] += sum_k A[m][k] B[k][j] = sum_{t in fragment f} x[..][16 g_m + j + t - pw] w[fh][t]
// so D[m][j] is output column 16 g_m + j of the output row behind
// combination m.  Filter taps are cut into 16-wide fragments f (B is a band
// of 16 diagonals: 16/32 = 50% of each MFMA is useful at a full fragment);
// the filter rows run as a loop of accumulating MFMAs.  The 16 combinations
// m of a tile are gt column groups x 16/gt consecutive output rows.
//
// Operand staging (all in LDS; §4.3 keeps the repeated filter in compact
// form and reuses overlapping input rows):
//   * the input tile is stored channel-major, [c][row][col], so one lane's
//     8 consecutive columns of A are one 16-byte LDS read.  Only real image
//     rows are stored, after one shared zero row that stands for every
//     padding row;
//   * going from filter row fh to fh+1, combination (g, r) needs the input
//     row that combination (g, r+1) used: a DPP row shift by one lane moves
//     it, and only the last row of each group reads LDS again;
//   * B is not stored as a 32 x 16 matrix: each (channel, filter row,
//     fragment) keeps its 16 taps once, z[u] = w[16f + u - 16] for u in
//     [16, 32), with 16 zeros before them, and lane (q, j) takes its 8
//     values z[16 + 8q - j .. +7] (the zeros around the taps are the band's
//     mask).  Rows follow each other every 32 elements, so the zeros after
//     a row's taps are the next row's leading zeros.  A lane reads 5
//     4-byte-aligned dwords from the even element at or below its start and
//     shifts them by 0 or 16 bits (v_alignbit): 2-byte-aligned 16-byte LDS
//     reads run at a quarter of the speed;
//   * outputs pass through LDS so that global stores are channel-contiguous.
// Zero padding of the image: the staging loads read out-of-image pixels as
// 0 through the buffer resource's range check.
#pragma once

#include "dwc_device.h"

namespace dwc {

typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 mf_f16x8 __attribute__((ext_vector_type(8)));
typedef float mf_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mf_u32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ mf_f32x4 mfma_16x16x32(mf_u32x4 a, mf_u32x4 b, mf_f32x4 c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, a),
                                                   __builtin_bit_cast(mf_bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mf_f16x8, a),
                                                  __builtin_bit_cast(mf_f16x8, b), c, 0, 0, 0);
  }
}

// DPP row_shl:1 -- lane i of each 16-lane row takes the value of lane i+1;
// the last lane of a row keeps its own value.
__device__ __forceinline__ uint32_t row_shift_down(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x101, 0xF, 0xF, false);
}

// Staging items (16-byte loads, 16-byte output stores) each thread keeps in
// flight before it writes them on.
constexpr int kStageBatch = 4;
// Elements between consecutive filter-row fragments (16 zeros, 16 taps);
// lane (q, j) reads elements [16 + 8q - j, +8) of a row, which end inside
// the next row's leading zeros.  Two zero rows follow the last one.
constexpr int kZRow = 32;
constexpr int kZTail = 2;

// CB channels per workgroup of kMfmaWaves waves (CB / kMfmaWaves per wave),
// NF 16-tap fragments per filter row, TILES tiles of 16 combinations per
// channel.  FLIP stages the filter turned by 180 degrees: the stride-1 data
// gradient.
template <int DT, int NF, int CB, int TILES, bool FLIP>
__global__ __launch_bounds__(64 * kMfmaWaves) void fwd_mfma(MfmaArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int NT = 64 * kMfmaWaves;
  constexpr int CPW = CB / kMfmaWaves;
  static_assert(CPW >= 1 && CB % kMfmaWaves == 0, "whole channels per wave");
  constexpr int OCT = CB / 8;  // 16-byte channel octets per pixel
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
  // Image rows [r_lo, r_hi) feed this block: image row ir sits at LDS row
  // ir - r_lo + 1, between two zero rows (0 and nrow + 1) that stand for
  // every row above and below.
  const int s_top = oh0 - a.PH;  // image row of staged index 0
  const int r_lo = s_top > 0 ? s_top : 0;
  const int r_end = s_top + a.rblk + FH - 1;
  const int r_hi = r_end < a.IH ? r_end : a.IH;
  const int nrow = r_hi > r_lo ? r_hi - r_lo : 0;
  uint16_t* xs = (uint16_t*)lds;                     // [CB][XR][WP]
  uint16_t* zt = xs + CB * XR * WP;                  // [CB][FH][NF][kZRow] + tail
  float* os = (float*)lds;                           // [rblk * OW][CB + 4], after compute
  constexpr int OSP = CB + 4;                        // floats per staged output pixel
  const int zlen = (CB * FH * NF + kZTail) * kZRow;  // elements of zt (a multiple of 8)

  // ---- filter taps: 16-byte loads of kStageBatch items per thread.  The
  // first batch is issued before the input tile's loads, so the two wait
  // for memory together; the taps go into their zero-padded fragment rows
  // (turned by 180 degrees for FLIP) after the barrier that ends the zero
  // fill.
  const auto frsrc = make_rsrc(a.filt, (uint32_t)(FH * FW) * (uint32_t)a.C * 2u);
  const int ftaps = FH * FW;
  const int fitems = ftaps * OCT;
  auto load_taps = [&](int i0, mf_u32x4 (&v)[kStageBatch]) {
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      if (i0 + b * NT >= fitems) break;  // uniform: no item left in this batch
      const int i = i0 + b * NT + tid;
      const int c = c0 + 8 * (i % OCT);
      const int te = i / OCT;  // staged tap (fh, fw)
      const int src = FLIP ? ftaps - 1 - te : te;
      const uint32_t off =
          i < fitems && c < a.C ? ((uint32_t)src * (uint32_t)a.C + (uint32_t)c) * 2u : kOOB;
      v[b] = __builtin_bit_cast(mf_u32x4,
                                __builtin_amdgcn_raw_buffer_load_b128(frsrc, (int)off, 0, 0));
    }
  };
  auto store_taps = [&](int i0, const mf_u32x4 (&v)[kStageBatch]) {
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      if (i0 + b * NT >= fitems) break;
      const int i = i0 + b * NT + tid;
      if (i >= fitems) continue;
      const int te = i / OCT;
      const int fh = fast_div(te, a.fw_magic), fw = te - fh * FW;
      const int f = fw >> 4;
      const int zstep = FH * NF * kZRow;  // elements from one channel's rows to the next
      uint16_t* d = zt + ((8 * (i % OCT)) * FH * NF + fh * NF + f) * kZRow + 16 + fw - 16 * f;
#pragma unroll
      for (int j = 0; j < 8; ++j, d += zstep)
        *d = (uint16_t)((v[b][j >> 1] >> (16 * (j & 1))) & 0xffffu);
    }
  };
  mf_u32x4 fv0[kStageBatch];
  load_taps(0, fv0);

  // ---- zero the filter-fragment rows (their taps are written after a barrier)
  for (int i = tid; i < zlen / 8; i += NT) ((mf_u32x4*)zt)[i] = mf_u32x4{0u, 0u, 0u, 0u};

  // ---- stage the input tile: LDS rows 0 .. nrow + 1, wt columns from -PW,
  // CB channels (rows 0 and nrow + 1 are zeros).  Thread tid owns one (column pair, channel octet) e of a row
  // and visits every rs-th row; it issues kStageBatch rows of loads before
  // writing any of them to LDS.  LDS row 0 loads out of range: zeros.
  {
    const uint32_t Cb = (uint32_t)a.C * 2u;
    const char* img = (const char*)a.in + (size_t)n * a.IH * a.IW * Cb;
    const auto rsrc = make_rsrc(img, (uint32_t)(a.IH * a.IW) * Cb);
    const int e = tid & (a.e2 - 1);
    const int r0 = tid >> a.e2_log;
    const int rs = NT >> a.e2_log;
    const int o = e % OCT, cp = e / OCT;
    const int iw = 2 * cp - a.PW;
    const int c = c0 + 8 * o;
    const bool e_in = e < a.e_items;
    const bool e_ok = e_in && c < a.C;
    const bool ok0 = e_ok && (unsigned)iw < (unsigned)a.IW;
    const bool ok1 = e_ok && (unsigned)(iw + 1) < (unsigned)a.IW;
    const uint32_t col0 = ((uint32_t)iw * (uint32_t)a.C + (uint32_t)c) * 2u;
    const uint32_t rowb = (uint32_t)a.IW * Cb;  // bytes per image row
    const int plane2 = XR * WP / 2;             // dwords per channel plane
    uint32_t* dst0 = (uint32_t*)xs + (8 * o) * plane2 + cp;
    // byte offset of LDS row r's pixel pair is (r_lo + r - 1) * rowb + col0;
    // LDS dwords of row r start at dst0 + r * (WP / 2).  Both advance by
    // fixed steps from row to row.
    const uint32_t row_step = (uint32_t)rs * rowb;
    uint32_t off_rb = (uint32_t)(r_lo + r0 - 1) * rowb + col0;
    for (int rb = r0; rb <= nrow + 1; rb += rs * kStageBatch, off_rb += kStageBatch * row_step) {
      mf_u32x4 v0[kStageBatch], v1[kStageBatch];
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        const int r = rb + b * rs;  // LDS row
        const bool rok = r >= 1 && r <= nrow;
        const uint32_t off = off_rb + (uint32_t)b * row_step;
        v0[b] = __builtin_bit_cast(mf_u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rsrc, (int)(rok && ok0 ? off : kOOB), 0, 0));
        v1[b] = __builtin_bit_cast(mf_u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rsrc, (int)(rok && ok1 ? off + Cb : kOOB), 0, 0));
      }
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        const int r = rb + b * rs;
        if (r > nrow + 1 || !e_in) continue;
        // channel j of a pixel is half (j & 1) of dword j / 2; the LDS dword
        // of channel j holds (pixel 0, pixel 1)
        uint32_t* d = dst0 + rb * (WP / 2) + b * (rs * (WP / 2));
#pragma unroll
        for (int j = 0; j < 8; ++j, d += plane2)
          *d = __builtin_amdgcn_perm(v1[b][j >> 1], v0[b][j >> 1],
                                                (j & 1) ? 0x07060302u : 0x05040100u);
      }
    }
  }
  __syncthreads();  // zt is zero
  store_taps(0, fv0);
  for (int i0 = NT * kStageBatch; i0 < fitems; i0 += NT * kStageBatch) {
    mf_u32x4 v[kStageBatch];
    load_taps(i0, v);
    store_taps(i0, v);
  }
  __syncthreads();

  // ---- compute.  A: lane (q, m) holds A[m][8q .. 8q+7]; B: lane (q, j=m)
  // holds B[8q .. 8q+7][j]; D: lane (q, j) holds D[4q .. 4q+3][j].  The
  // wave's CPW channels run together in the filter-row loop, and the B
  // operands of row fh+1 are read while the MFMAs of row fh execute.
  const int q = lane >> 4, m = lane & 15;
  const int RT = 1 << a.rt_log;
  const int gA = m >> a.rt_log, rA = m & (RT - 1);
  const bool reload = rA == RT - 1;
  // A of tile tt at filter row fh is staged row s = tt * RT + rA + fh, at
  // byte offset clamp((s_top - r_lo + 1 + s) * 2 WP, 0, (nrow + 1) * 2 WP)
  // of the channel's plane: rows above the image clamp to zero row 0, rows
  // below to zero row nrow + 1.
  const int rowb2 = 2 * WP;
  const int top_b = (nrow + 1) * rowb2;
  const int a0 = (s_top - r_lo + 1 + rA) * rowb2;
  const unsigned char* xb8 =
      (const unsigned char*)(xs + (wave * CPW) * XR * WP + 16 * gA + 8 * q);
  auto a_at = [&](int k, int tt, int f, int fh) -> mf_u32x4 {
    const int o = min(max(a0 + (tt * RT + fh) * rowb2, 0), top_b);
    return *(const mf_u32x4*)(xb8 + k * XR * rowb2 + o + 32 * f);
  };
  // B: lane (q, j = m) starts at element 16 + 8q - m of a fragment row; it
  // reads from the even element at or below and shifts odd starts by 16 bits
  const int u0 = 16 + 8 * q - m;
  const uint32_t bshift = (uint32_t)(u0 & 1) * 16u;
  const uint32_t* zbase = (const uint32_t*)(zt + (wave * CPW) * FH * NF * kZRow + (u0 & ~1));
  auto read_b = [&](int row) -> mf_u32x4 {  // row: fragment row of this wave
    const uint32_t* p = zbase + row * (kZRow / 2);
    mf_u32x4 d;
    __builtin_memcpy(&d, p, 16);
    const uint32_t d4 = p[4];
    return mf_u32x4{__builtin_amdgcn_alignbit(d[1], d[0], bshift),
                    __builtin_amdgcn_alignbit(d[2], d[1], bshift),
                    __builtin_amdgcn_alignbit(d[3], d[2], bshift),
                    __builtin_amdgcn_alignbit(d4, d[3], bshift)};
  };
  constexpr int TD = TILES / 2;  // tiles whose A moves by DPP row shifts
  mf_f32x4 acc[CPW][TILES];
  mf_u32x4 A[CPW][TILES][NF];
  mf_u32x4 B[CPW][NF];
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) {
      acc[k][tt] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < NF; ++f) A[k][tt][f] = a_at(k, tt, f, 0);
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) B[k][f] = read_b(k * FH * NF + f);
  }
  // One uniform body per filter row: the operands for row fh+1 are formed
  // in the last iteration too (from rows that exist, never used), which
  // keeps the accumulators in place across iterations.
  for (int fh = 0; fh < FH; ++fh) {
#pragma unroll
    for (int k = 0; k < CPW; ++k)
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[k][tt] = mfma_16x16x32<DT>(A[k][tt][f], B[k][f], acc[k][tt]);
    const int fn = fh + 1 < FH ? fh + 1 : fh;
#pragma unroll
    for (int k = 0; k < CPW; ++k)
#pragma unroll
      for (int f = 0; f < NF; ++f) B[k][f] = read_b((k * FH + fn) * NF + f);
    // Tiles below TD move A down one combination with DPP row shifts (VALU)
    // and reload only the last combination of each row group; tiles from
    // TD on read all of A again (LDS).  The split keeps both pipes below
    // the MFMA time: DPP alone costs four VALU instructions per MFMA.
#pragma unroll
    for (int k = 0; k < CPW; ++k)
#pragma unroll
      for (int tt = 0; tt < TD; ++tt)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int v = 0; v < 4; ++v) A[k][tt][f][v] = row_shift_down(A[k][tt][f][v]);
    if (reload) {
#pragma unroll
      for (int tt = 0; tt < TD; ++tt)
#pragma unroll
        for (int k = 0; k < CPW; ++k)
#pragma unroll
          for (int f = 0; f < NF; ++f) A[k][tt][f] = a_at(k, tt, f, fh + 1);
    }
#pragma unroll
    for (int tt = TD; tt < TILES; ++tt)
#pragma unroll
      for (int k = 0; k < CPW; ++k)
#pragma unroll
        for (int f = 0; f < NF; ++f) A[k][tt][f] = a_at(k, tt, f, fh + 1);
  }

  // ---- outputs: registers -> LDS [pixel][channel] -> channel-contiguous stores
  __syncthreads();  // every wave is done with the staged input
  // Lane (q, m) holds row mm = 4q + r of every tile at column m: output
  // row tt * RT + (mm mod RT), column 16 (mm / RT) + m.  One address and one
  // bounds test per mm; tiles and the wave's channels are fixed offsets.
  {
    const int tile_step = RT * a.OW * OSP;  // floats from one tile to the next
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = 4 * q + r;
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
    for (int p0 = 0; p0 < npix; p0 += PSTEP * kStageBatch) {
      mf_f32x4 v[kStageBatch];
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        const int pb = p0 + b * PSTEP;  // uniform
        v[b] = pb + pt < npix ? *(const mf_f32x4*)(src + pb * OSP) : mf_f32x4{};
      }
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        const int pb = p0 + b * PSTEP;
        if (pb + pt < npix && c_ok) store_nt((mf_f32x4*)(dst + (size_t)pb * a.C), v[b]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Packed-MFMA filter gradient (bf16 / fp16 operands, stride 1).
//
// Per channel and output row oh (the split of the accumulation axis of
// Flash-DWC §5.1, with the GEMV-to-GEMM packing of §4.2 applied to the
// filter gradient):
//   A[m][k] = dY[oh][32 kc + k - (16 fm + m) + pw]   (16 taps fw x 32 columns)
//   B[k][n] = X[oh + 16 fn + n - ph][32 kc + k]        (32 columns x 16 rows fh)
//   D[m][n] += sum_k A[m][k] B[k][n]  =  dW[16 fn + n][16 fm + m] contributions
// so one 16x16x32 MFMA covers up to 16 x 16 taps over 32 input columns.  A is
// the Toeplitz band of the zero-padded dY row (read like the forward kernel's
// filter band: 4-byte-aligned dwords and v_alignbit); B is 16 consecutive
// input rows, which move down one row per output row by a DPP row shift plus
// one reloaded lane.  A workgroup owns kWgmCb channels (one per wave) and a
// slice of ipb images, stages each image's X and dY rows in LDS
// channel-major, and writes one channel-blocked partial per slice.
// ---------------------------------------------------------------------------
template <int DT, int NFM, int NFN, int NK, int PF>
__global__ __launch_bounds__(64 * kMfmaWaves, wgm_waves_per_eu(NFM, NFN, NK, PF)) void wgrad_mfma(
    WgradMfmaArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int NT = 64 * kMfmaWaves;
  constexpr int CB = kWgmCb;
  static_assert(CB == kMfmaWaves, "one channel per wave");
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
  const int taps = a.FH * a.FW;
  uint16_t* xs = (uint16_t*)lds;        // [CB][XR][XP]
  uint16_t* dz = xs + CB * XR * XP;     // [CB][OH][DYP]
  float* pst = (float*)lds;             // [taps][CB], after the last image
  const uint32_t Cb = (uint32_t)a.C * 2u;

  // ---- zero both staging regions once: per image only the pixels of the
  // image are written, so the zero row, the columns past the image and the
  // dY padding stay zero for every image of the slice
  {
    const int units = CB * (XR * XP + OH * DYP) / 8;  // 16-byte units
    for (int i = tid; i < units; i += NT) ((mf_u32x4*)lds)[i] = mf_u32x4{0u, 0u, 0u, 0u};
  }

  // ---- this thread's staging items, the same for every image: item i of
  // X is the pixel pair (2e, 2e+1) of row r; item i of dY is the pair of
  // staged columns (2e, 2e+1), i.e. dY columns 2e - dpad and 2e + 1 - dpad.
  // Global byte offsets within the image (kOOB: zero) and the LDS dword of
  // channel 0 (-1: no item).
  uint32_t xo0[PF], xo1[PF], do0[PF], do1[PF];
  int xw[PF], dw[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int i = tid + k * NT;
    xo0[k] = xo1[k] = do0[k] = do1[k] = kOOB;
    xw[k] = dw[k] = -1;
    if (i < a.ix) {
      const int r = i / a.hx, e = i - r * a.hx;
      xo0[k] = (uint32_t)(r * a.IW + 2 * e) * Cb + (uint32_t)c0 * 2u;
      if (2 * e + 1 < a.IW) xo1[k] = xo0[k] + Cb;
      xw[k] = (r + 1) * (XP / 2) + e;
    }
    if (i < a.id) {
      const int r = i / a.hd, e = a.e_lo + (i - r * a.hd);
      const int t0 = 2 * e - a.dpad;
      const uint32_t base = (uint32_t)(r * a.OW) * Cb + (uint32_t)c0 * 2u;
      if ((unsigned)t0 < (unsigned)a.OW) do0[k] = base + (uint32_t)t0 * Cb;
      if ((unsigned)(t0 + 1) < (unsigned)a.OW) do1[k] = base + (uint32_t)(t0 + 1) * Cb;
      dw[k] = r * (DYP / 2) + e;
    }
  }
  mf_u32x4 vx0[PF], vx1[PF], vd0[PF], vd1[PF];
  auto fetch = [&](int n) {  // global -> registers, in flight during compute
    const auto rx = make_rsrc((const char*)a.x + (size_t)n * a.IH * a.IW * Cb,
                              (uint32_t)(a.IH * a.IW) * Cb);
    const auto rd = make_rsrc((const char*)a.dy + (size_t)n * OH * a.OW * Cb,
                              (uint32_t)(OH * a.OW) * Cb);
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      vx0[k] = __builtin_bit_cast(mf_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)xo0[k], 0, 0));
      vx1[k] = __builtin_bit_cast(mf_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)xo1[k], 0, 0));
      vd0[k] = __builtin_bit_cast(mf_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, (int)do0[k], 0, 0));
      vd1[k] = __builtin_bit_cast(mf_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, (int)do1[k], 0, 0));
    }
  };
  auto commit = [&]() {  // registers -> LDS, transposed to channel-major
    const int px = XR * XP / 2, pd = OH * DYP / 2;  // dwords per channel plane
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      if (xw[k] >= 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          ((uint32_t*)xs)[xw[k] + j * px] = __builtin_amdgcn_perm(
              vx1[k][j >> 1], vx0[k][j >> 1], (j & 1) ? 0x07060302u : 0x05040100u);
      }
      if (dw[k] >= 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          ((uint32_t*)dz)[dw[k] + j * pd] = __builtin_amdgcn_perm(
              vd1[k][j >> 1], vd0[k][j >> 1], (j & 1) ? 0x07060302u : 0x05040100u);
      }
    }
  };

  // ---- per-lane constants.  A: lane (q, m) holds A[m][8q .. 8q+7]; B:
  // lane (q, n = m) holds B[8q .. 8q+7][n]; D: lane (q, j) holds
  // D[4q .. 4q+3][j].
  const int q = lane >> 4, m = lane & 15;
  const int cc = wave;
  // A starts at staged dY element 32 kc + 8q - 16 fm - m + pw + dpad of its
  // row: five dwords from the even element at or below, odd starts shifted
  // by 16 bits
  const int ua = 8 * q - m + a.PW + a.dpad;
  const uint32_t ashift = (uint32_t)(ua & 1) * 16u;
  const uint32_t* dzl = (const uint32_t*)(dz + cc * OH * DYP + (ua & ~1));
  const int dyp2 = DYP / 2;
  auto read_a = [&](int oh, int fm, int kc) -> mf_u32x4 {
    const uint32_t* p = dzl + oh * dyp2 + 16 * kc - 8 * fm;
    // dword reads (paired by the compiler): a 16-byte LDS read at these
    // lane-varying 4-byte-aligned starts runs at about a sixth of the speed
    mf_u32x4 d;
    __builtin_memcpy(&d, p, 16);
    const uint32_t d4 = p[4];
    return mf_u32x4{__builtin_amdgcn_alignbit(d[1], d[0], ashift),
                    __builtin_amdgcn_alignbit(d[2], d[1], ashift),
                    __builtin_amdgcn_alignbit(d[3], d[2], ashift),
                    __builtin_amdgcn_alignbit(d4, d[3], ashift)};
  };
  const uint16_t* xl = xs + cc * XR * XP + 8 * q;
  // LDS row of input row r: row 0 is zeros, image row r sits at r + 1
  auto x_row = [&](int r) -> int { return (unsigned)r < (unsigned)a.IH ? r + 1 : 0; };

  mf_f32x4 acc[NFM][NFN];
#pragma unroll
  for (int fm = 0; fm < NFM; ++fm)
#pragma unroll
    for (int fn = 0; fn < NFN; ++fn) acc[fm][fn] = mf_f32x4{0.f, 0.f, 0.f, 0.f};

  if (n0 < n1) fetch(n0);
  for (int n = n0; n < n1; ++n) {
    __syncthreads();  // the zero fill, or the previous image's reads, are done
    commit();
    __syncthreads();
    if (n + 1 < n1) fetch(n + 1);

    // ---- accumulate over the image's output rows.  B of row oh+1 is B of
    // row oh moved down one lane (DPP row shift) with lane 15 of each row
    // group taking input row oh+1 + 16 fn + 15 - ph, read one row ahead into
    // R (the DPP "old" operand, kept where the shift has no source lane).
    mf_u32x4 A[NFM][NK], B[NFN][NK], R[NFN][NK];
#pragma unroll
    for (int fn = 0; fn < NFN; ++fn) {
      const int row = x_row(16 * fn + m - a.PH);
      const int rrow = uniform(x_row(1 + 16 * fn + 15 - a.PH));
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) {
        B[fn][kc] = *(const mf_u32x4*)(xl + row * XP + 32 * kc);
        R[fn][kc] = *(const mf_u32x4*)(xl + rrow * XP + 32 * kc);
      }
    }
#pragma unroll
    for (int fm = 0; fm < NFM; ++fm)
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) A[fm][kc] = read_a(0, fm, kc);
    // One uniform body per output row: the operands of row oh+1 (and R of
    // row oh+2) are formed in the last iterations too, from rows that exist
    // (the zero row past the image), and never used.
    auto row_step = [&](int oh) {
#pragma unroll
      for (int kc = 0; kc < NK; ++kc)
#pragma unroll
        for (int fm = 0; fm < NFM; ++fm)
#pragma unroll
          for (int fn = 0; fn < NFN; ++fn)
            acc[fm][fn] = mfma_16x16x32<DT>(A[fm][kc], B[fn][kc], acc[fm][fn]);
      const int on = oh + 1 < OH ? oh + 1 : oh;
#pragma unroll
      for (int fm = 0; fm < NFM; ++fm)
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) A[fm][kc] = read_a(on, fm, kc);
#pragma unroll
      for (int fn = 0; fn < NFN; ++fn) {
        const int rrow = uniform(x_row(oh + 2 + 16 * fn + 15 - a.PH));
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            B[fn][kc][v] = __builtin_amdgcn_update_dpp(R[fn][kc][v], B[fn][kc][v], 0x101, 0xF,
                                                       0xF, false);
          R[fn][kc] = *(const mf_u32x4*)(xl + rrow * XP + 32 * kc);
        }
      }
    };
    // Two rows per iteration: the shifted B lands in the registers R held
    // (the DPP keeps its destination's old value where no lane feeds it),
    // so B and R trade registers every row and are back in place after two.
    int oh = 0;
    for (; oh + 1 < OH; oh += 2) {
      row_step(oh);
      row_step(oh + 1);
    }
    if (oh < OH) row_step(oh);
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
        const int fw = 16 * fm + 4 * q + r, fh = 16 * fn + m;
        if (fw < a.FW && fh < a.FH) pst[(fh * a.FW + fw) * CB + cc] = acc[fm][fn][r];
      }
  __syncthreads();
  float* dst = a.ws + ((size_t)z * a.cblk + cbk) * taps * CB;
  for (int i = tid; i < taps * CB / 4; i += NT)
    *(mf_f32x4*)(dst + 4 * i) = *(const mf_f32x4*)(pst + 4 * i);
}

}  // namespace dwc
