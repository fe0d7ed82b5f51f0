// dwc_mfma_h4.h -- forward-type kernel of libdwc for bf16/fp16 operands on
// the 16-block 4x4x4 matrix instructions (gfx950
// v_mfma_f32_4x4x4_16b_{f16,bf16}, fp32 accumulation), 4 images as the
// matrix rows.
//
// The GEMV-to-GEMM packing of Flash-DWC (§4.2, Fig. 8) with the narrowest
// 16-bit matrix operation: per block b, D[i][j] += sum_k A[i][k] B[k][j]
// over K = 4.  Here
//   block b      = channel c0 + b (16 channels per wave),
//   row i        = image n0 + i (4 images),
//   column j     = output column ow0 + 4m + j of tile m (T tiles per wave),
//   the K step s = input columns 4(m + s) .. 4(m + s) + 3 of the wave's
//                  window (window column u is input column ow0 - PW + u), at
//                  input row r and filter row fh = r - oh + PH:
//   A[i][k]      = x[n0 + i][r][ow0 - PW + 4(m + s) + k]
//   B[k][j]      = w[fh][4s + k - j]                 (0 outside 0 .. FW-1)
// Output column 4m + j reads window columns 4m + j + fw, so the S =
// ceil((FW + 3) / 4) steps cover every tap (13 / 16 of the work is useful at
// FW = 13).  The window is NG = T + S - 1 groups of 4 columns; group g
// serves step s of tile g - s, so one A register pair serves up to S tiles
// and one B pair (per filter row and s) all T tiles.
//
// A wave owns RR = 4 consecutive output rows of its 4 images and 4T
// columns: it streams the input rows that reach them, each loaded once and
// applied to every output row it feeds (an accumulator ring of RR x T
// tiles); padding rows are skipped, and MFMAs whose 4 input columns are all
// padding are skipped in the first and last column groups (compile-time
// edge variants).  An input row of the window (4 images x NA columns x 16
// channels) comes in as 16-byte loads of 8 channels of one pixel, which the
// wave writes to its own LDS row buffer ([image][column][channel], the row
// pitch padded so that the 4 images fall on different banks); each lane
// then reads its 4 columns per group as 2-byte LDS reads.  Gathering the
// operands straight from memory (2 bytes per lane, 4 images per lane quad)
// kept the texture units busy about 30 cycles per 128-byte instruction,
// against about 85 per kilobyte in the 16-byte form (MI355X counters).  The
// next row's loads are in flight while the current row's MFMAs run;
// columns outside the image read 0 through the range check.
//
// The band sits in LDS as [FH][S][16 channels][4 columns j] entries of 4
// taps (8 bytes): lane (b, j) reads its B for (fh, s) as one 8-byte entry,
// 64 consecutive entries per wave (conflict-free).  The workgroup's waves
// share it and take the same channel block; the row buffers follow it.
// Outputs are fp32.
#pragma once

#include <type_traits>

#include "dwc_device.h"

namespace dwc {

typedef float h4m_f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4m_f16x4 __attribute__((ext_vector_type(4)));
typedef short h4m_s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t h4m_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t h4m_u32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ h4m_f32x4 mfma_4x4x4(h4m_u32x2 a, h4m_u32x2 b, h4m_f32x4 c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(h4m_s16x4, a),
                                                  __builtin_bit_cast(h4m_s16x4, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4m_f16x4, a),
                                              __builtin_bit_cast(h4m_f16x4, b), c, 0, 0, 0);
  }
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void h4m_static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    h4m_static_for<B + 1, E>(f);
  }
}

// K steps of a filter of width FWI: ceil((FWI + 3) / 4)
constexpr int h4m_steps(int fwi) { return (fwi + 6) / 4; }

template <int DT, int FWI, int T, bool FLIP>
__global__ __launch_bounds__(64 * kH4mMaxWaves) void fwd_mfma_h4n(MfmaF32Args a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int RR = kH4mRows;           // output rows per wave (accumulator ring)
  constexpr int S = h4m_steps(FWI);      // K steps per tile
  constexpr int NG = T + S - 1;          // 4-column groups of the window
  constexpr int NA = 4 * NG;             // window columns
  constexpr int NAP = NA + ((2 - NA % 8) + 8) % 8;  // staged row pitch: NAP % 8 == 2
  constexpr int NCH = 8 * NA;            // 16-byte chunks of a staged row
  constexpr int CPL = (NCH + 63) / 64;   // chunks per lane
  h4m_u32x2* band = reinterpret_cast<h4m_u32x2*>(lds);  // [FH][S][16][4]
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_blocks) return;  // the whole workgroup leaves together
  const int cbk = blk % a.cblk;
  const int grp = blk / a.cblk;
  const int c0 = cbk * kH4mCb;
  const int FH = a.FH, FW = a.FW, C = a.C;

  // ---- band: entry (fh, s, b, j) holds w[fh][4s + k - j] of channel c0 + b
  // for k = 0 .. 3 (the filter turned by 180 degrees under FLIP), zeros
  // outside the filter read as 0 through the range check
  {
    const int items = FH * S * 64;
    const int taps = FH * FW;
    const auto frs = make_rsrc(a.filt, (uint32_t)taps * (uint32_t)C * 2u);
    for (int e0 = 0; e0 < items; e0 += kH4mStageBatch * nthr) {
      uint32_t v[kH4mStageBatch][4];
#pragma unroll
      for (int jb = 0; jb < kH4mStageBatch; ++jb) {
        const int e = e0 + jb * nthr + tid;
        const int j = e & 3, bb = (e >> 2) & 15, fs = e >> 6;
        const int fh = fs / S, s = fs - fh * S;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int fw = 4 * s + k - j;
          const bool ok = e < items && fw >= 0 && fw < FW;
          const int tap = FLIP ? taps - 1 - (fh * FW + fw) : fh * FW + fw;
          const uint32_t off = ok ? ((uint32_t)tap * (uint32_t)C + (uint32_t)(c0 + bb)) * 2u : kOOB;
          v[jb][k] = __builtin_amdgcn_raw_buffer_load_b16(frs, (int)off, 0, 0);
        }
      }
#pragma unroll
      for (int jb = 0; jb < kH4mStageBatch; ++jb) {
        const int e = e0 + jb * nthr + tid;
        if (e < items) band[e] = h4m_u32x2{v[jb][0] | (v[jb][1] << 16), v[jb][2] | (v[jb][3] << 16)};
      }
    }
  }
  __syncthreads();

  // ---- the wave's tile: images n0 .. n0 + 3, output rows oh0 .. oh0 + 3,
  // columns ow0 .. ow0 + 4T - 1 (column groups, then row groups, then image
  // groups; the last column group ends at the right edge)
  const int wave = uniform(tid >> 6);
  const int tile = grp * a.nw + wave;
  if (tile >= a.tiles) return;
  int rest = tile;
  const int cgi = rest % a.cg;
  rest /= a.cg;
  const int rgi = rest % a.rg;
  const int n0 = (rest / a.rg) * 4;
  const int oh0 = rgi * RR;
  const int ow0 = a.OW >= 4 * T ? min(cgi * 4 * T, a.OW - 4 * T) : 0;
  const int lane = tid & 63, b = lane >> 2, q = lane & 3;
  const int IH = a.IH, IW = a.IW, PH = a.PH, PW = a.PW;
  const uint32_t img_bytes = (uint32_t)IH * (uint32_t)IW * (uint32_t)C * 2u;
  const auto xrs = make_rsrc(reinterpret_cast<const uint16_t*>(a.in) + (size_t)n0 * IH * IW * C,
                             (uint32_t)(a.N - n0) * img_bytes);  // images n0 .. N - 1
  // the wave's row buffer: [4 images][NAP columns][16 channels] of 2 bytes
  unsigned char* xs = lds + FH * S * 512 + wave * (4 * NAP * 32);
  // 16-byte chunk e = lane + 64 t of a row: image e / 2NA, column, half
  uint32_t vo[CPL];  // global byte offset within the row's images (kOOB: 0)
  uint32_t wo[CPL];  // LDS byte offset (kNoChunk: past the row)
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const int e = lane + 64 * t;
    const int im = e / (2 * NA), rem = e - im * (2 * NA);
    const int col = rem >> 1, half = rem & 1;
    const int ic = ow0 - PW + col;  // input column
    const bool ok = e < NCH && n0 + im < a.N && ic >= 0 && ic < IW;
    vo[t] = ok ? (uint32_t)im * img_bytes + (uint32_t)((ic * C + c0 + 8 * half) * 2) : kOOB;
    wo[t] = (uint32_t)((im * NAP + col) * 32 + half * 16);
  }
  const unsigned char* xr = xs + (q * NAP * 32 + b * 2);  // lane (b, i): image i, channel b
  const uint32_t row_bytes = (uint32_t)IW * (uint32_t)C * 2u;

  h4m_f32x4 D[RR][T];
#pragma unroll
  for (int j = 0; j < RR; ++j)
#pragma unroll
    for (int m = 0; m < T; ++m) D[j][m] = h4m_f32x4{0.f, 0.f, 0.f, 0.f};
  // input rows that reach the wave's output rows and are not padding
  const int r_lo = max(0, oh0 - PH);
  const int r_hi = min(IH, oh0 + RR - 1 + FH - PH);  // exclusive
  const h4m_u32x2* bl = band + lane;

  auto run = [&](auto lc, auto rc) {
    constexpr int L = decltype(lc)::value, R = decltype(rc)::value;
    // groups that hold at least one real column
    constexpr int GLO = L / 4;
    constexpr int GHI = (NA - R + 3) / 4;
    h4m_u32x4 G[CPL];
    auto load_row = [&](int r) {
      const int so = (int)((uint32_t)r * row_bytes);
#pragma unroll
      for (int t = 0; t < CPL; ++t)
        G[t] = __builtin_bit_cast(h4m_u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)vo[t], so, 0));
    };
    if (r_lo < r_hi) load_row(r_lo);
    for (int r = r_lo; r < r_hi; ++r) {
      // this row into the buffer (the previous row's reads have returned:
      // their registers fed the MFMAs), then the next row's loads go out
#pragma unroll
      for (int t = 0; t < CPL; ++t)
        if (t < CPL - 1 || lane + 64 * t < NCH) *reinterpret_cast<h4m_u32x4*>(xs + wo[t]) = G[t];
      load_row(min(r + 1, r_hi - 1));  // the last row loads itself again: no branch
      h4m_u32x2 A[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g < GLO || g >= GHI) {
          A[g] = h4m_u32x2{0u, 0u};
          continue;
        }
        uint32_t hh[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) hh[k] = *reinterpret_cast<const uint16_t*>(xr + (4 * g + k) * 32);
        A[g] = h4m_u32x2{__builtin_amdgcn_perm(hh[1], hh[0], 0x05040100u),
                         __builtin_amdgcn_perm(hh[3], hh[2], 0x05040100u)};
      }
#pragma unroll
      for (int j = 0; j < RR; ++j) {
        const int fh = r - oh0 - j + PH;
        if (fh < 0 || fh >= FH) continue;  // uniform
        const h4m_u32x2* bk = bl + fh * (S * 64);
        h4m_static_for<0, S>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          const h4m_u32x2 bv = bk[s * 64];
          constexpr int mlo = GLO - s > 0 ? GLO - s : 0;
          constexpr int mhi = GHI - s < T ? GHI - s : T;
#pragma unroll
          for (int m = mlo; m < mhi; ++m) D[j][m] = mfma_4x4x4<DT>(A[m + s], bv, D[j][m]);
        });
      }
    }
  };
  {
    using Z = std::integral_constant<int, 0>;
    using P = std::integral_constant<int, (FWI - 1) / 2>;
    using PR = std::integral_constant<int, NA - 4 * T - (FWI - 1) / 2>;
    const bool el = a.same && ow0 == 0, er = a.same && ow0 + 4 * T == a.OW;
    if (el && er) run(P{}, PR{});
    else if (el) run(P{}, Z{});
    else if (er) run(Z{}, PR{});
    else run(Z{}, Z{});
  }

  // ---- outputs: register i of D[j][m] is image n0 + i, row oh0 + j,
  // column ow0 + 4m + q
  // The last column group, moved left to end at the right edge, writes only
  // the columns that no other group owns: its K steps group the taps of a
  // column differently, so a second write could differ in the last bits
  // (and the last writer would decide)
  const int own0 = cgi * 4 * T;
  const uint32_t orowb = (uint32_t)a.OW * (uint32_t)C * 4u;
  const uint32_t ooff = (uint32_t)(((ow0 + q) * C + c0 + b) * 4);
  const uint32_t sstep = (uint32_t)C * 16u;
  uint32_t mo[T];
#pragma unroll
  for (int m = 0; m < T; ++m) mo[m] = ow0 + 4 * m + q >= own0 ? ooff + (uint32_t)m * sstep : kOOB;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (n0 + i >= a.N) break;  // uniform
    float* yimg = a.out + (size_t)(n0 + i) * a.OH * a.OW * C;
#pragma unroll
    for (int j = 0; j < RR; ++j) {
      const int oh = oh0 + j;
      if (oh >= a.OH) break;  // uniform
      const auto ors = make_rsrc(yimg + (size_t)oh * a.OW * C, orowb);
#pragma unroll
      for (int m = 0; m < T; ++m) {
        // the element is copied out first: this compiler's __builtin_bit_cast
        // of a vector element expression reads element 0
        const float v = D[j][m][i];
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ors, (int)mo[m], 0, 0);
      }
    }
  }
}

}  // namespace dwc
