// dwc_mfma_f32.h -- fp32 matrix-core forward-type kernel of libdwc (gfx950
// v_mfma_f32_4x4x1_16b_f32, fp32 operands and accumulation).
//
// The GEMV-to-GEMM packing of Flash-DWC (§4.2, Fig. 8) turns one filter row
// into a Toeplitz band so that adjacent outputs share one matrix operation.
// On the fp32 matrix cores the narrowest such operation is the 16-block
// 4x4x1 form: per block b, D[i][j] += A[i] * B[j].  Here
//   block b      = channel c0 + b (16 channels per wave),
//   row i        = output row oh0 + i (4 consecutive rows),
//   column j     = output column ow0 + 4m + j of tile m (T tiles per wave),
//   the K step   = one input column u, at filter row fh:
//   A[i]         = x[oh0 + i + fh - PH][ow0 - PW + u]   (the same column, 4 rows)
//   B[j]         = w[fh][u - 4m - j]                   (0 outside 0 .. FW-1)
// A tile's 4 columns read the input columns u = 4m .. 4m + FW + 2, so
// FW + 3 instructions cover 4 x FW taps: 31 / 34 of the work is useful at
// FW = 31 (a 16-wide tile would keep 31 / 46).  The band depends on t = u - 4m
// only, so one B register (per filter row and t) serves all T tiles, and
// one A register (per input column) serves every tile whose taps reach it.
//
// Registers: A holds the wave's NA = 4T + FWI - 1 input columns for its 4
// rows at the current filter row; moving to the next filter row shifts
// every column down one row inside each lane quad (DPP) and brings the new
// bottom row in, loaded 4 columns per instruction one filter row ahead.
// The band (per filter row: 3 zeros, the taps, zeros to FWI + 3) sits in
// LDS, shared by the workgroup's waves, which all take the same channels;
// lane (b, j) reads its B at t as one dword, 64 lanes on 64 banks.
// Instructions whose input column is padding are skipped (a uniform
// branch); padding rows are never loaded (the row's buffer range is 0).
// The waves need no barrier after the band is staged.
#pragma once

#include <type_traits>

#include "dwc_device.h"

namespace dwc {

typedef float f32m_x4 __attribute__((ext_vector_type(4)));

// Calls f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void f32m_static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    f32m_static_for<B + 1, E>(f);
  }
}

// One filter row down in a quad of rows: lanes 0-2 take lanes 1-3 of a,
// lane 3 takes lane K of n (keep = 1, put = 0 in lanes 0-2; the reverse in
// lane 3).  Two VALU instructions: a v_mul_f32 with the rotation as its DPP
// source (the compiler folds the move into it), then a v_fmac_f32 with the
// broadcast of n as its DPP source, which the compiler does not form.  The
// products by 1 and 0 are exact, so are the sums with one zero term, for
// finite operands.  The fmac's DPP operand comes from a load (no VALU
// write before a DPP read), its accumulator from the preceding VALU
// instruction (not a DPP operand).
template <int K>
__device__ __forceinline__ float quad_shift_in(float a, float n, float keep, float put) {
  float x = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a),
                                                                  0x39, 0xF, 0xF, true)) * keep;
  asm("v_fmac_f32_dpp %0, %1, %2 quad_perm:[%3,%3,%3,%3] row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(x)
      : "v"(n), "v"(put), "i"(K));
  return x;
}

// One input row on in a quad of dY rows (lane j holds row r - j): lanes 1-3
// take lanes 0-2 of a, lane 0 takes lane K of n (keep = 0 in lane 0, 1
// elsewhere; put the reverse).  The same two instructions as quad_shift_in,
// with the rotation the other way.
template <int K>
__device__ __forceinline__ float quad_shift_up_in(float a, float n, float keep, float put) {
  float x = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a),
                                                                  0x93, 0xF, 0xF, true)) * keep;
  asm("v_fmac_f32_dpp %0, %1, %2 quad_perm:[%3,%3,%3,%3] row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(x)
      : "v"(n), "v"(put), "i"(K));
  return x;
}

// Four consecutive 16-bit operand elements (bf16 or fp16, two per dword) as
// fp32: exact.
template <int DT>
__device__ __forceinline__ f32m_x4 wf32_widen4(uint32_t lo, uint32_t hi) {
  if constexpr (DT == DT_BF16) {
    return f32m_x4{__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                   __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
  } else {
    return f32m_x4{(float)__builtin_bit_cast(_Float16, (unsigned short)(lo & 0xffffu)),
                   (float)__builtin_bit_cast(_Float16, (unsigned short)(lo >> 16)),
                   (float)__builtin_bit_cast(_Float16, (unsigned short)(hi & 0xffffu)),
                   (float)__builtin_bit_cast(_Float16, (unsigned short)(hi >> 16))};
  }
}

// One operand element (fp32, bf16 or fp16) at a lane offset, as fp32:
// exact.  Offsets past the resource read 0.
template <int DT>
__device__ __forceinline__ float f32m_ld1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (DT == DT_F32) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
  } else {
    const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    if constexpr (DT == DT_BF16) return __uint_as_float(h << 16);
    else return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
  }
}

// Four consecutive operand elements (one 16- or 8-byte load) as fp32.
template <int DT>
__device__ __forceinline__ f32m_x4 f32m_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (DT == DT_F32) {
    return __builtin_bit_cast(f32m_x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    return wf32_widen4<DT>(v.x, v.y);
  }
}

// DT: the operand type of the input and filter (fp32, or bf16 / fp16
// widened to fp32 as they are loaded).
template <int DT, int FWI, int T, bool FLIP>
__global__ __launch_bounds__(64 * kF32mMaxWaves) void fwd_mfma_f32(MfmaF32Args a) {
  constexpr int EB = DT == DT_F32 ? 4 : 2;  // operand bytes
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int NT = FWI + 3;            // K steps (taps t) of one 4-column tile
  constexpr int NA = 4 * T + FWI - 1;    // input columns a wave holds
  constexpr int NS = (NA + 3) / 4;       // 4-column loads of a new row
  constexpr int ZP = FWI + 6;            // band entries per filter row
  float* band = reinterpret_cast<float*>(lds);  // [FH][ZP][kF32mCb]
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_blocks) return;  // the whole workgroup leaves together
  // Logical ids run over the channel blocks first: neighbouring blocks read
  // the two halves of the same 128-byte lines of a pixel.
  const int cbk = blk % a.cblk;
  const int grp = blk / a.cblk;
  const int c0 = cbk * kF32mCb;
  const int FH = a.FH, FW = a.FW, C = a.C;

  // ---- the band: zeros, then the taps (turned by 180 degrees for FLIP),
  // 4 channels per 16-byte load, kF32mStageBatch loads in flight per thread
  const int bn = FH * ZP * kF32mCb / 4;
  for (int e = tid; e < bn; e += nthr)
    reinterpret_cast<f32m_x4*>(band)[e] = f32m_x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  {
    const int taps = FH * FW;
    const int items = taps * (kF32mCb / 4);
    const auto frs = make_rsrc(a.filt, (uint32_t)taps * (uint32_t)C * EB);
    for (int e0 = 0; e0 < items; e0 += kF32mStageBatch * nthr) {
      f32m_x4 v[kF32mStageBatch];
#pragma unroll
      for (int j = 0; j < kF32mStageBatch; ++j) {
        const int e = e0 + j * nthr + tid;
        const int tap = e >> 2, c4 = (e & 3) * 4;
        const int src = FLIP ? taps - 1 - tap : tap;
        const uint32_t off = e < items ? ((uint32_t)src * (uint32_t)C + (uint32_t)(c0 + c4)) * EB : kOOB;
        v[j] = f32m_ld4<DT>(frs, off);
      }
#pragma unroll
      for (int j = 0; j < kF32mStageBatch; ++j) {
        const int e = e0 + j * nthr + tid;
        if (e < items) {
          const int tap = e >> 2, c4 = (e & 3) * 4;
          const int fh = fast_div(tap, a.fw_magic), fw = tap - fh * FW;
          *reinterpret_cast<f32m_x4*>(band + (fh * ZP + fw + 3) * kF32mCb + c4) = v[j];
        }
      }
    }
  }
  __syncthreads();

  // ---- the wave's tile: image n, output rows oh0 .. oh0 + 3, columns
  // ow0 .. ow0 + 4T - 1 (tiles of a channel block run over column groups,
  // then row groups, then images).  The last column group ends at the
  // image's right edge (it may overlap the one before it, whose shared
  // columns both compute alike).
  const int wave = uniform(tid >> 6);
  const int tile = grp * a.nw + wave;
  if (tile >= a.tiles) return;
  int rest = tile;
  const int cgi = rest % a.cg;
  rest /= a.cg;
  const int rgi = rest % a.rg;
  const int n = rest / a.rg;
  const int oh0 = rgi * kF32mRows;
  const int ow0 = a.OW >= 4 * T ? min(cgi * 4 * T, a.OW - 4 * T) : 0;
  const int lane = tid & 63, b = lane >> 2, q = lane & 3;
  const int IH = a.IH, IW = a.IW, PH = a.PH, PW = a.PW;

  const char* ximg = reinterpret_cast<const char*>(a.in) + (size_t)n * IH * IW * C * EB;
  const uint32_t rowb = (uint32_t)IW * (uint32_t)C * EB;
  // Lane (b, q) of a 4-column load takes column ow0 - PW + 4s + q of a row;
  // negative columns wrap to offsets past any row's range.
  const uint32_t loff = (uint32_t)(((ow0 - PW + q) * C + c0 + b) * EB);
  const uint32_t istep = (uint32_t)C * 4u * EB;  // 4 input columns
  const uint32_t sstep = (uint32_t)C * 16u;       // 4 output columns

  // Filter rows whose 4 input rows are not all padding.
  const int k_lo = max(0, PH - oh0 - (kF32mRows - 1));
  const int k_hi = min(FH, IH + PH - oh0);

  f32m_x4 D[T];
#pragma unroll
  for (int m = 0; m < T; ++m) D[m] = f32m_x4{0.f, 0.f, 0.f, 0.f};

  // The filter rows of the tile.  L (R) leading (trailing) input columns of
  // the window are known to be padding: their instructions are not issued.
  auto run = [&](auto lc, auto rc) {
    constexpr int L = decltype(lc)::value, R = decltype(rc)::value;
    float A[NA];
    {
      // lane q: input row oh0 + q + k_lo - PH, every column of the window
      const int r = oh0 + q + k_lo - PH;
      const bool ok = r >= 0 && r < IH;
      const auto irs = make_rsrc(ximg, (uint32_t)IH * rowb);
      const uint32_t rbase = ok ? (uint32_t)r * rowb + (uint32_t)(c0 + b) * EB : kOOB;
#pragma unroll
      for (int u = 0; u < NA; ++u) {
        const int col = ow0 - PW + u;
        A[u] = 0.f;
        if (u >= L && u < NA - R && col >= 0 && col < IW)
          A[u] = f32m_ld1<DT>(irs, rbase + (uint32_t)col * (uint32_t)C * EB);
      }
    }
    // every load above has landed before the loop (whose first instructions
    // would otherwise wait for the loads it issues itself)
    __builtin_amdgcn_s_waitcnt(0);
    float nv[NS];
    // 1 in lanes 0-2 of each quad, 0 in lane 3; and the reverse
    const float keep = q == kF32mRows - 1 ? 0.f : 1.f, put = 1.f - keep;
    // lane (b, j): band entry t - j + 3 of channel b
    const float* bl = band + (3 - q) * kF32mCb + b;
    for (int k = k_lo; k < k_hi; ++k) {
      const bool more = k + 1 < k_hi;
      if (more) {
        // the row that enters next: oh0 + 4 + k - PH for lane 3
        const int r = oh0 + kF32mRows + k - PH;
        const bool ok = r >= 0 && r < IH;
        const auto rs = make_rsrc(ximg + (size_t)(ok ? r : 0) * IW * C * EB, ok ? rowb : 0u);
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) nv[s2] = f32m_ld1<DT>(rs, loff + (uint32_t)s2 * istep);
      }
      const float* bk = bl + k * (ZP * kF32mCb);
      float bcur = bk[0];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float bnext = t + 1 < NT ? bk[(t + 1) * kF32mCb] : 0.f;
#pragma unroll
        for (int m = 0; m < T; ++m) {
          const int u = 4 * m + t;
          if (u >= L && u < NA - R)
            D[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(A[u], bcur, D[m], 0, 0, 0);
        }
        bcur = bnext;
      }
      if (more) {
        // lane q takes lane q + 1's row; lane 3 the new row (through lane 0:
        // Y = new row in lane 0, then a rotation of the quad)
        f32m_static_for<L, NA - R>([&](auto uc) {
          constexpr int u = decltype(uc)::value;
          A[u] = quad_shift_in<u & 3>(A[u], nv[u >> 2], keep, put);
        });
      }
    }
  };
  if (k_lo < k_hi) {
    using Z = std::integral_constant<int, 0>;
    using P = std::integral_constant<int, (FWI - 1) / 2>;
    const bool el = a.same && ow0 == 0, er = a.same && ow0 + 4 * T == a.OW;
    if (el && er) run(P{}, P{});
    else if (el) run(P{}, Z{});
    else if (er) run(Z{}, P{});
    else run(Z{}, Z{});
  }

  // ---- outputs: register i of tile m is row oh0 + i, column ow0 + 4m + q
  float* yimg = a.out + (size_t)n * a.OH * a.OW * C;
  const uint32_t orowb = (uint32_t)a.OW * (uint32_t)C * 4u;
  const uint32_t ooff = (uint32_t)(((ow0 + q) * C + c0 + b) * 4);
#pragma unroll
  for (int i = 0; i < kF32mRows; ++i) {
    const int oh = oh0 + i;
    if (oh >= a.OH) break;  // uniform
    const auto ors = make_rsrc(yimg + (size_t)oh * a.OW * C, orowb);
#pragma unroll
    for (int m = 0; m < T; ++m) {
      // the element is copied out first: this compiler's __builtin_bit_cast
      // of a vector element expression reads element 0
      const float v = D[m][i];
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ors,
                                            (int)(ooff + (uint32_t)m * sstep), 0, 0);
    }
  }
}

// ---- forward-type kernel with 4 images as the matrix rows: per block b
// (channel c0 + b), D[i][j] of tile m and ring row q is output pixel
// (n0 + i, oh0 + q, ow0 + 4m + j); the K step is one input column u of one
// input row r, A[i] = x[n0 + i][r][ow0 - PW + u] (the same column of 4
// images: no data moves between lanes) and B[j] = w[r - oh0 - q + PH][u -
// 4m - j], the band row of that ring row.  A wave streams the FH + RR - 1
// input rows of its RR output rows, loading each once; padding rows are
// skipped.  The band staging, the edge variants and the output layout are
// those of fwd_mfma_f32.
template <int FWI, int T, bool FLIP>
__global__ __launch_bounds__(64 * kF32mMaxWaves) void fwd_mfma_f32n(MfmaF32Args a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int RR = kF32mRows;          // output rows per wave (accumulator ring)
  constexpr int NT = FWI + 3;
  constexpr int NA = 4 * T + FWI - 1;
  constexpr int ZP = FWI + 6;
  float* band = reinterpret_cast<float*>(lds);  // [FH][ZP][kF32mCb]
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_blocks) return;  // the whole workgroup leaves together
  const int cbk = blk % a.cblk;
  const int grp = blk / a.cblk;
  const int c0 = cbk * kF32mCb;
  const int FH = a.FH, FW = a.FW, C = a.C;

  const int bn = FH * ZP * kF32mCb / 4;
  for (int e = tid; e < bn; e += nthr)
    reinterpret_cast<f32m_x4*>(band)[e] = f32m_x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  {
    const int taps = FH * FW;
    const int items = taps * (kF32mCb / 4);
    const auto frs = make_rsrc(a.filt, (uint32_t)taps * (uint32_t)C * 4u);
    for (int e0 = 0; e0 < items; e0 += kF32mStageBatch * nthr) {
      f32m_x4 v[kF32mStageBatch];
#pragma unroll
      for (int j = 0; j < kF32mStageBatch; ++j) {
        const int e = e0 + j * nthr + tid;
        const int tap = e >> 2, c4 = (e & 3) * 4;
        const int src = FLIP ? taps - 1 - tap : tap;
        const uint32_t off = e < items ? ((uint32_t)src * (uint32_t)C + (uint32_t)(c0 + c4)) * 4u : kOOB;
        v[j] = __builtin_bit_cast(f32m_x4, __builtin_amdgcn_raw_buffer_load_b128(frs, (int)off, 0, 0));
      }
#pragma unroll
      for (int j = 0; j < kF32mStageBatch; ++j) {
        const int e = e0 + j * nthr + tid;
        if (e < items) {
          const int tap = e >> 2, c4 = (e & 3) * 4;
          const int fh = fast_div(tap, a.fw_magic), fw = tap - fh * FW;
          *reinterpret_cast<f32m_x4*>(band + (fh * ZP + fw + 3) * kF32mCb + c4) = v[j];
        }
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
  // lane (b, i): image n0 + i (kOOB past the batch), channel c0 + b
  const uint32_t img_bytes = (uint32_t)IH * (uint32_t)IW * (uint32_t)C * 4u;
  const uint32_t loff = n0 + q < a.N ? (uint32_t)q * img_bytes + (uint32_t)(c0 + b) * 4u : kOOB;
  const auto xrs = make_rsrc(reinterpret_cast<const float*>(a.in) + (size_t)n0 * IH * IW * C,
                             (uint32_t)(a.N - n0) * img_bytes);  // images n0 .. N - 1

  f32m_x4 D[RR][T];
#pragma unroll
  for (int j = 0; j < RR; ++j)
#pragma unroll
    for (int m = 0; m < T; ++m) D[j][m] = f32m_x4{0.f, 0.f, 0.f, 0.f};
  // input rows that reach the wave's output rows and are not padding
  const int r_lo = max(0, oh0 - PH);
  const int r_hi = min(IH, oh0 + RR - 1 + FH - PH);  // exclusive
  const float* bl = band + (3 - q) * kF32mCb + b;

  auto run = [&](auto lc, auto rc) {
    constexpr int L = decltype(lc)::value, R = decltype(rc)::value;
    for (int r = r_lo; r < r_hi; ++r) {
      // the row's columns of the window, one load each: the lane offset
      // (image, channel) is the same for all, the pixel's offset goes in the
      // scalar offset (a padding column is not loaded)
      float A[NA];
      int so = (r * IW + ow0 - PW) * C * 4;  // bytes to column u
      int col = ow0 - PW;                    // column u
#pragma unroll
      for (int u = 0; u < NA; ++u) {
        A[u] = 0.f;
        if (u >= L && u < NA - R && col >= 0 && col < IW)
          A[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xrs, (int)loff, so, 0));
        so += C * 4;
        ++col;
        // scalar adds per column: keep the compiler from holding every
        // column's offset and bounds in scalar registers across the row loop
        asm volatile("" : "+s"(so), "+s"(col));
      }
#pragma unroll
      for (int j = 0; j < RR; ++j) {
        const int fh = r - oh0 - j + PH;
        if (fh < 0 || fh >= FH) continue;  // uniform
        const float* bk = bl + fh * (ZP * kF32mCb);
        f32m_static_for<0, NT>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          const float bv = bk[t * kF32mCb];
          constexpr int mlo = (L - t + 3) / 4 > 0 ? (L - t + 3) / 4 : 0;
          constexpr int mhi0 = (NA - R - t + 3) / 4;
          constexpr int mhi = mhi0 < T ? mhi0 : T;
#pragma unroll
          for (int m = mlo; m < mhi; ++m)
            D[j][m] = __builtin_amdgcn_mfma_f32_4x4x1f32(A[4 * m + t], bv, D[j][m], 0, 0, 0);
        });
      }
    }
  };
  {
    using Z = std::integral_constant<int, 0>;
    using P = std::integral_constant<int, (FWI - 1) / 2>;
    const bool el = a.same && ow0 == 0, er = a.same && ow0 + 4 * T == a.OW;
    if (el && er) run(P{}, P{});
    else if (el) run(P{}, Z{});
    else if (er) run(Z{}, P{});
    else run(Z{}, Z{});
  }

  // ---- outputs: register i of D[j][m] is image n0 + i, row oh0 + j,
  // column ow0 + 4m + q
  const uint32_t orowb = (uint32_t)a.OW * (uint32_t)C * 4u;
  const uint32_t ooff = (uint32_t)(((ow0 + q) * C + c0 + b) * 4);
  const uint32_t sstep = (uint32_t)C * 16u;
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
        const float v = D[j][m][i];  // copied out: see fwd_mfma_f32's store
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ors,
                                              (int)(ooff + (uint32_t)m * sstep), 0, 0);
      }
    }
  }
}

// ---- filter gradient (layout and mapping: WgradF32Args).  DT: the operand
// type of x and dY; 16-bit operands are widened to fp32 as they are loaded
// (X on its way to the LDS, dY into the register window), so the matrix
// cores see the same fp32 values the oracle multiplies.
template <int DT, int TW, int NB>
__global__ __launch_bounds__(64 * kWf32MaxWaves, 4) void wgrad_mfma_f32(WgradF32Args a) {
  constexpr int EB = DT == DT_F32 ? 4 : 2;  // operand bytes
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  using XRaw = std::conditional_t<DT == DT_F32, f32m_x4, u32x2>;
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int OWW = 4 * NB;             // output columns per wave
  constexpr int NU = OWW + 4 * TW - 3;    // 4-column X windows u
  constexpr int XP = NU + 3;              // staged pixels per X row
  float* xb = reinterpret_cast<float*>(lds);  // [2][XP][kWf32Cb]
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_blocks) return;  // the whole workgroup leaves together
  // channel blocks first (neighbours share the lines of a pixel), then
  // column groups, then row slices
  const int cbk = blk % a.cblk;
  int rest = blk / a.cblk;
  const int cgi = rest % a.cg;
  const int z = rest / a.cg;
  const int c0 = cbk * kWf32Cb;
  const int ow0 = cgi * OWW;
  const int h = uniform(tid >> 6);        // the wave's filter-row tile
  const int lane = tid & 63, b = lane >> 2, q = lane & 3;
  const int C = a.C, IH = a.IH, IW = a.IW, OH = a.OH, OW = a.OW, PH = a.PH, PW = a.PW;
  const int npairs = a.N * IH;
  const int p0 = z * a.rps;
  const int p1 = min(p0 + a.rps, npairs);
  const uint32_t xrow = (uint32_t)IW * (uint32_t)C * EB;

  // ---- X staging: item e = (pixel e / 4, channels 4 (e % 4) .. + 3) of the
  // row; pixel p is input column ow0 - PW + p
  const int items = XP * (kWf32Cb / 4);
  XRaw xv[kWf32StageItems];
  auto x_fetch = [&](int n, int r) {
    const auto rs = make_rsrc(reinterpret_cast<const char*>(a.x) +
                                  ((size_t)n * IH + r) * IW * C * EB,
                              xrow);
#pragma unroll
    for (int k = 0; k < kWf32StageItems; ++k) {
      const int e = tid + k * nthr;
      const int col = ow0 - PW + (e >> 2);
      const uint32_t off = e < items ? (uint32_t)((col * C + c0 + (e & 3) * 4) * EB) : kOOB;
      if constexpr (DT == DT_F32)
        xv[k] = __builtin_bit_cast(f32m_x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
      else
        xv[k] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0));
    }
  };
  auto x_commit = [&](int buf) {
#pragma unroll
    for (int k = 0; k < kWf32StageItems; ++k) {
      const int e = tid + k * nthr;
      if (e < items) {
        f32m_x4 v;
        if constexpr (DT == DT_F32) v = xv[k];
        else v = wf32_widen4<DT>(xv[k].x, xv[k].y);
        *reinterpret_cast<f32m_x4*>(xb + (buf * XP + (e >> 2)) * kWf32Cb + (e & 3) * 4) = v;
      }
    }
  };

  // ---- dY rows: lane (b, j) of Bw[o] holds dy[r - 4h - j + PH][ow0 + o]
  float Bw[OWW];
  float nv[NB];
  const float keep = q != 0 ? 1.f : 0.f, put = 1.f - keep;
  // Each load below has its own buffer resource (scalar registers) starting
  // at its column, so that all of them share one lane offset register; the
  // resource's range still ends at the row's (image's) end.
  const char* dyc = reinterpret_cast<const char*>(a.dy) + (size_t)ow0 * C * EB;  // column ow0
  const int wcols = OW - ow0;  // columns of the row from ow0 on
  const uint32_t qoff = (uint32_t)((q * C + c0 + b) * EB);
  auto dy_fetch = [&](int n, int row) {  // row `row` of image n, 4 columns per load
    const bool ok = row >= 0 && row < OH;
    const char* rp = dyc + ((size_t)n * OH + (ok ? row : 0)) * OW * C * EB;
#pragma unroll
    for (int s2 = 0; s2 < NB; ++s2) {
      const int left = wcols - 4 * s2;  // columns of the row from this load's first on
      const auto rs = make_rsrc(rp + (size_t)(4 * s2) * C * EB,
                                ok && left > 0 ? (uint32_t)(left * C) * EB : 0u);
      nv[s2] = f32m_ld1<DT>(rs, qoff);
    }
  };
  auto dy_shift = [&]() {  // the fetched row into lane 0, the others one lane on
    f32m_static_for<0, OWW>([&](auto oc) {
      constexpr int o = decltype(oc)::value;
      Bw[o] = quad_shift_up_in<o & 3>(Bw[o], nv[o >> 2], keep, put);
    });
  };
  // the window of image n at input row r: its 4 rows shifted in, the
  // highest last
  auto dy_init = [&](int n, int r) {
#pragma unroll
    for (int o = 0; o < OWW; ++o) Bw[o] = 0.f;
    for (int j = 3; j >= 0; --j) {
      dy_fetch(n, r - 4 * h - j + PH);
      dy_shift();
    }
  };

  f32m_x4 D[TW];
#pragma unroll
  for (int f = 0; f < TW; ++f) D[f] = f32m_x4{0.f, 0.f, 0.f, 0.f};
  if (p0 < p1) {
    int n = p0 / IH, r = p0 - (p0 / IH) * IH;
    x_fetch(n, r);
    x_commit(0);
    dy_init(n, r);
    // every load above has landed before the loop (whose first instructions
    // would otherwise wait for the loads it issues itself)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // lane (b, i) of window u reads staged pixel u + i, channel b
    const float* xl = xb + q * kWf32Cb + b;
    for (int p = p0; p < p1; ++p) {
      const int buf = (p - p0) & 1;
      const bool more = p + 1 < p1;
      const bool same_img = r + 1 < IH;
      if (more) {
        x_fetch(same_img ? n : n + 1, same_img ? r + 1 : 0);
        if (same_img) dy_fetch(n, r + 1 - 4 * h + PH);
      }
      // this wave's 4 dY rows r - 4h - 3 + PH .. r - 4h + PH
      const int hi = r - 4 * h + PH;
      if (hi >= 0 && hi - 3 < OH && 4 * h < a.FH) {
        const float* xr = xl + buf * (XP * kWf32Cb);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const float xa = xr[u * kWf32Cb];
#pragma unroll
          for (int f = 0; f < TW; ++f) {
            const int o = u - 4 * f;
            if (o >= 0 && o < OWW) D[f] = __builtin_amdgcn_mfma_f32_4x4x1f32(xa, Bw[o], D[f], 0, 0, 0);
          }
        }
      }
      if (more) {
        x_commit(buf ^ 1);
        if (same_img) {
          dy_shift();
          ++r;
        } else {
          ++n;
          r = 0;
          dy_init(n, 0);
          __builtin_amdgcn_s_waitcnt(0);
        }
      }
      __syncthreads();
    }
  }

  // ---- the slice's partial: register i of tile f is dW[4h + q][4f + i]
  const int taps = a.FH * a.FW;
  float* part = a.ws + ((size_t)(z * a.cg + cgi) * a.cblk + cbk) * taps * kWf32Cb + b;
  const int fh = 4 * h + q;
  if (fh < a.FH) {
#pragma unroll
    for (int f = 0; f < TW; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int fw = 4 * f + i;
        if (fw < a.FW) part[(fh * a.FW + fw) * kWf32Cb] = D[f][i];
      }
  }
}

}  // namespace dwc
