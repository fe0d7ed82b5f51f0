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
// Operand staging (all in LDS, §4.3 keeps the repeated filter in compact
// form and reuses overlapping input rows):
//   * the input tile is stored channel-major, [c][row][col], so one lane's
//     8 consecutive columns of A are one 16-byte LDS read;
//   * going from filter row fh to fh+1, combination (g, r) needs the input
//     row that combination (g, r+1) used: a DPP row shift by one lane moves
//     it, and only the last row of each group reads LDS again;
//   * B is built per filter row from one packed tap pair per lane,
//     (w[i-1], w[i]), gathered with ds_bpermute -- the filter row is held
//     once, not as a 32 x 16 matrix;
//   * outputs pass through LDS so that global stores are channel-contiguous.
// Zero padding: the staging loads read out-of-image pixels as 0 through the
// buffer resource's range check.
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

// CB channels per workgroup (CB/4 per wave), NF 16-tap fragments per filter
// row, TILES tiles of 16 combinations per channel.  FLIP stages the filter
// turned by 180 degrees: the stride-1 data gradient.
template <int DT, int NF, int CB, int TILES, bool FLIP>
__global__ __launch_bounds__(kBlockThreads) void fwd_mfma(MfmaArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int CPW = CB / kWavesPerBlock;
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
  const int XR = a.xr, WT = a.wt;
  const int FH = a.FH, FW = a.FW;
  uint16_t* xs = (uint16_t*)lds;                   // [CB][XR][WT]
  uint16_t* wsh = xs + CB * XR * WT;               // [CB][FH][FW]
  float* os = (float*)lds;                         // [rblk * OW][CB + 4], after compute
  constexpr int OSP = CB + 4;                      // floats per staged output pixel

  // ---- stage the input tile: rows oh0-PH .., columns -PW .., CB channels.
  // Each thread issues the loads of kStageBatch items before writing any of
  // them to LDS, so that many loads are in flight per workgroup.
  {
    const uint32_t Cb = (uint32_t)a.C * 2u;
    const char* img = (const char*)a.in + (size_t)n * a.IH * a.IW * Cb;
    const auto rs = make_rsrc(img, (uint32_t)(a.IH * a.IW) * Cb);
    const int ih0 = oh0 - a.PH, iw0 = -a.PW;
    const int half = WT / 2;
    const int items = XR * half * OCT;
    const int plane = XR * WT;  // elements per channel plane
    for (int i0 = 0; i0 < items; i0 += kBlockThreads * kStageBatch) {
      mf_u32x4 v0[kStageBatch], v1[kStageBatch];
      int dst[kStageBatch];
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        const int i = i0 + b * kBlockThreads + tid;
        const int o = i % OCT;
        const int cp = (i / OCT) % half;
        const int r = i / (OCT * half);
        const int ih = ih0 + r, iw = iw0 + 2 * cp;
        const int c = c0 + 8 * o;
        const bool rok = i < items && (unsigned)ih < (unsigned)a.IH && c < a.C;
        const uint32_t base = (uint32_t)(ih * a.IW) * Cb + (uint32_t)c * 2u;
        const uint32_t off0 =
            rok && (unsigned)iw < (unsigned)a.IW ? base + (uint32_t)iw * Cb : kOOB;
        const uint32_t off1 =
            rok && (unsigned)(iw + 1) < (unsigned)a.IW ? base + (uint32_t)(iw + 1) * Cb : kOOB;
        v0[b] = __builtin_bit_cast(mf_u32x4,
                                   __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off0, 0, 0));
        v1[b] = __builtin_bit_cast(mf_u32x4,
                                   __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off1, 0, 0));
        // LDS dword (channel 8o, row r, columns 2cp, 2cp+1); -1: no item
        dst[b] = i < items ? (((8 * o) * XR + r) * WT + 2 * cp) / 2 : -1;
      }
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        if (dst[b] < 0) continue;
        // channel j of a pixel is half (j & 1) of dword j / 2; the LDS dword
        // of channel j holds (pixel 0, pixel 1)
        uint32_t* d = (uint32_t*)xs + dst[b];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t lo = (v0[b][j >> 1] >> (16 * (j & 1))) & 0xffffu;
          const uint32_t hi = (v1[b][j >> 1] >> (16 * (j & 1))) & 0xffffu;
          d[j * (plane / 2)] = lo | (hi << 16);
        }
      }
    }
  }
  // ---- stage the filter: [cc][fh][fw], turned by 180 degrees for FLIP.
  {
    const auto rs = make_rsrc(a.filt, (uint32_t)(FH * FW) * (uint32_t)a.C * 2u);
    const int taps = FH * FW;
    const int items = taps * OCT;
    for (int i = tid; i < items; i += kBlockThreads) {
      const int o = i % OCT;
      const int e = i / OCT;
      const int c = c0 + 8 * o;
      const uint32_t off = c < a.C ? ((uint32_t)e * (uint32_t)a.C + (uint32_t)c) * 2u : kOOB;
      const mf_u32x4 v = __builtin_bit_cast(
          mf_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
      const int ed = FLIP ? taps - 1 - e : e;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        wsh[(8 * o + j) * taps + ed] = (uint16_t)((v[j >> 1] >> (16 * (j & 1))) & 0xffffu);
    }
  }
  __syncthreads();

  // ---- compute.  A: lane (q, m) holds A[m][8q .. 8q+7]; B: lane (q, j=m)
  // holds B[8q .. 8q+7][j]; D: lane (q, j) holds D[4q .. 4q+3][j].  The
  // wave's CPW channels run together in the filter-row loop, and the B
  // operands of row fh+1 are gathered while the MFMAs of row fh execute.
  const int q = lane >> 4, m = lane & 15;
  const int RT = 16 / a.gt;
  const int gA = m / RT, rA = m % RT;
  const bool reload = rA == RT - 1;
  // B gather: register v of fragment f holds taps (16f + d, 16f + d + 1)
  // with d = 8q + 2v - j, from lane 16f + d + 1 of the tap-pair vector; the
  // mask drops taps outside the fragment's diagonal band.
  uint32_t bsrc[NF][4], bmask[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int d = 8 * q + 2 * v - m;
    bmask[v] = ((d >= 0 && d < 16) ? 0x0000ffffu : 0u) |
               ((d + 1 >= 0 && d + 1 < 16) ? 0xffff0000u : 0u);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      int s = 16 * f + d + 1;
      s = s < 0 ? 0 : (s > 63 ? 63 : s);
      bsrc[f][v] = (uint32_t)s * 4u;
    }
  }
  // tap pair of lane i: (w[i-1], w[i]), zero outside [0, FW); the reads are
  // clamped into the row and masked afterwards
  const int lo_i = lane - 1 < 0 ? 0 : (lane - 1 >= FW ? FW - 1 : lane - 1);
  const int hi_i = lane >= FW ? FW - 1 : lane;
  const uint32_t lo_m = (lane >= 1 && lane - 1 < FW) ? 0xffffu : 0u;
  const uint32_t hi_m = lane < FW ? 0xffffu : 0u;
  const uint16_t* wbase = wsh + (wave * CPW) * FH * FW;
  auto tap_pair = [&](int k, int fh) -> uint32_t {
    const uint16_t* row = wbase + (k * FH + fh) * FW;
    const uint32_t lo = row[lo_i], hi = row[hi_i];
    return (lo & lo_m) | ((hi & hi_m) << 16);
  };
  const uint16_t* xbase = xs + (wave * CPW) * XR * WT;
  // lane's element offset in a channel plane for tile tt, fragment f, at
  // staged row `row` of its combination
  const int col_off = 16 * gA + 8 * q;

  mf_f32x4 acc[CPW][TILES];
  mf_u32x4 A[CPW][TILES][NF];
  mf_u32x4 B[CPW][NF];
  uint32_t pair[CPW];
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) {
      acc[k][tt] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < NF; ++f)
        A[k][tt][f] = *(const mf_u32x4*)(xbase + (k * XR + tt * RT + rA) * WT + col_off + 16 * f);
    }
    pair[k] = tap_pair(k, 0);
  }
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        B[k][f][v] = (uint32_t)__builtin_amdgcn_ds_bpermute((int)bsrc[f][v], (int)pair[k]) & bmask[v];
    pair[k] = tap_pair(k, FH > 1 ? 1 : 0);
  }
  // One uniform body per filter row: the operands for row fh+1 are formed
  // in the last iteration too (from clamped rows of the staged tile, never
  // used), which keeps the accumulators in place across iterations.
  for (int fh = 0; fh < FH; ++fh) {
#pragma unroll
    for (int k = 0; k < CPW; ++k)
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[k][tt] = mfma_16x16x32<DT>(A[k][tt][f], B[k][f], acc[k][tt]);
    const int fpair = fh + 2 < FH ? fh + 2 : FH - 1;
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          B[k][f][v] =
              (uint32_t)__builtin_amdgcn_ds_bpermute((int)bsrc[f][v], (int)pair[k]) & bmask[v];
      pair[k] = tap_pair(k, fpair);
    }
#pragma unroll
    for (int k = 0; k < CPW; ++k)
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int v = 0; v < 4; ++v) A[k][tt][f][v] = row_shift_down(A[k][tt][f][v]);
    if (reload) {
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt) {
        // staged row of this tile's last combination at filter row fh+1
        int row = tt * RT + RT + fh;
        row = row < XR ? row : XR - 1;
#pragma unroll
        for (int k = 0; k < CPW; ++k)
#pragma unroll
          for (int f = 0; f < NF; ++f)
            A[k][tt][f] = *(const mf_u32x4*)(xbase + (k * XR + row) * WT + col_off + 16 * f);
      }
    }
  }
  __syncthreads();  // every wave is done with the staged input

  // ---- outputs: registers -> LDS [pixel][channel] -> channel-contiguous stores
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
    const int cc = wave * CPW + k;
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mm = 4 * q + r;
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
    for (int i0 = 0; i0 < items; i0 += kBlockThreads * kStageBatch) {
      mf_f32x4 v[kStageBatch];
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        const int i = i0 + b * kBlockThreads + tid;
        const int p = i / QU;
        v[b] = i < items ? *(const mf_f32x4*)(os + p * OSP + 4 * (i % QU)) : mf_f32x4{};
      }
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        const int i = i0 + b * kBlockThreads + tid;
        const int s = i % QU;
        const int p = i / QU;
        const int oh = oh0 + p / a.OW;
        const int c = c0 + 4 * s;
        if (i < items && oh < a.OH && c < a.C)
          *(mf_f32x4*)(out_img + ((size_t)oh * a.OW + p % a.OW) * a.C + c) = v[b];
      }
    }
  }
}

}  // namespace dwc
